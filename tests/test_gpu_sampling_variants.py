"""GPU parity of the sampling variant with siblings drawn without replacement
(sv_problem.sampling = SV_SAMPLE_DISTINCT) against the oracle's
without_replacement walk, through the C ABI: stage-isolated sampling fed the
oracle's logits, many rounds on one context, the whole step end to end, and
the input check on duplicate siblings. Tolerances and exclusions are those of
the default variant (tests/parity_util.py)."""
import numpy as np
import pytest
import torch

from oracle import verify as ov
from speculative_decoding_tree_amd import lib, synth
from speculative_decoding_tree_amd.runner import DeviceBatch

from parity_util import (MARGIN_STAGE, TOL_PROB, compare_rounds, path_excluded, widened)
from test_gpu_parity import (MINI, _check_probabilities, _compare_e2e, _oracle_logits, _run,
                             _sample_with_logits)

pytestmark = pytest.mark.gpu


def _distinct(name_or_wl):
    wl = synth.WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    return wl.with_(name=wl.name + "_distinct", children="distinct")


def _stage(inp):
    W = inp.workload
    logits32 = _oracle_logits(inp).astype(np.float32)
    res = _sample_with_logits(inp, logits32)
    logits64 = logits32.astype(np.float64)
    rounds, _, _, _ = ov.sample_batch(logits64, inp.draft_logits.astype(np.float64), inp.parent,
                                      inp.node_token, inp.uniforms, inp.temperature, W.n_nodes,
                                      without_replacement=True)
    npath, nfin, excl, bad = compare_rounds(rounds, inp.temperature, res["accept_len"],
                                            res["accept_path"], res["out_tokens"], W.n_nodes,
                                            margin=MARGIN_STAGE)
    print(f"{W.name}: paths {npath}, final tokens {nfin}, excluded {excl}", flush=True)
    assert not bad, bad[:3]
    assert (res["seq_status"] & lib.SEQ_ERR_MASK == 0).all()
    assert _check_probabilities(inp, logits64, res, rounds) <= TOL_PROB
    for b, r in enumerate(rounds):
        if path_excluded(r, float(inp.temperature[b])):
            continue
        for t in r.tests:
            g = res["node_ratio"][b * W.n_nodes + t.node]
            assert abs(g - t.ratio) <= 1e-4 * max(1.0, abs(t.ratio)), (b, t, g)
    return npath, nfin


@pytest.mark.parametrize("wl", [MINI, "eagle1_7b_t1", "share_70b", "gqa_8b"],
                         ids=lambda w: w if isinstance(w, str) else w.name)
def test_distinct_sampling_stage_matches_oracle(wl):
    _stage(synth.generate(_distinct(wl), seed=3))


@pytest.mark.parametrize("name,copies", [("eagle1_7b_t1", 48), ("share_70b", 48)])
def test_distinct_sampling_many_rounds(name, copies):
    base = synth.generate(_distinct(name), seed=21)
    inp = synth.replicate_rounds(base, copies, seed=22)
    npath, nfin = _stage(inp)
    assert npath >= 0.9 * copies and nfin >= 0.5 * copies


def test_distinct_verify_end_to_end():
    inp = synth.generate(_distinct(MINI), seed=4)
    W = inp.workload
    _, res = _run(inp)
    w = widened(inp)
    ref = ov.verify_batch(w["node_hidden"], w["kv"], inp.kv_offset, inp.prefix_len, inp.parent,
                          inp.node_token, w["lm_head"], inp.draft_logits, inp.uniforms,
                          inp.temperature, W.n_nodes, W.n_q_heads, W.n_kv_heads, W.head_dim,
                          with_attention=False, without_replacement=True)
    _compare_e2e(inp, ref, res)
    assert (res["seq_status"] & lib.SEQ_ERR_MASK == 0).all()


def test_duplicate_siblings_are_an_input_error_only_when_distinct():
    inp = synth.generate(_distinct(MINI), seed=5)
    W = inp.workload
    N = W.n_nodes
    # sequence 2 (T > 0): give two root children the same token
    par = inp.parent[2 * N:3 * N]
    kids = [j for j in range(N) if par[j] == -1]
    assert len(kids) >= 2
    inp.node_token[2 * N + kids[1]] = inp.node_token[2 * N + kids[0]]
    _, res = _run(inp)
    assert res["seq_status"][2] & lib.SEQ_ERR_TOKEN
    assert res["accept_len"][2] == -1
    assert (res["seq_status"][:2] & lib.SEQ_ERR_MASK == 0).all()
    # the same tokens with siblings declared i.i.d. are valid input
    inp.workload = W.with_(children="iid")
    _, res = _run(inp)
    assert (res["seq_status"] & lib.SEQ_ERR_MASK == 0).all()
