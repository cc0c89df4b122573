"""GPU parity of top-k / top-p warping (sv_problem.top_k / top_p) against the
oracle's warped walk, through the C ABI: stage-isolated sampling fed the
oracle's logits over several workloads and settings (top-k alone, top-p
alone, both, top_k = 1), logits with many exact ties (the cut inside a tie
group), many rounds on one context, siblings drawn without replacement,
the whole step end to end, and bitwise reruns.

Drafted tokens come from the warped draft distribution (synth draws them
so). Rounds are compared unless a walked test, the final draw or a warped
row's top-p cut lies within its stated tolerance of flipping
(tests/parity_util.py); the kept masses the GPU reports for the rows it
visited are checked against the oracle's to 1e-5 relative.
"""
import numpy as np
import pytest
import torch

from oracle import verify as ov
from speculative_decoding_tree_amd import lib, synth

from parity_util import MARGIN_STAGE, compare_rounds, path_excluded, widened
from test_gpu_parity import MINI, _compare_e2e, _oracle_logits, _run, _sample_with_logits

pytestmark = pytest.mark.gpu


def _warped(wl, k, tp, children="iid"):
    wl = synth.WORKLOADS[wl] if isinstance(wl, str) else wl
    return wl.with_(name=f"{wl.name}_k{k}_p{tp}_{children}", top_k=k, top_p=tp,
                    children=children)


def _tp(W):
    """top_p as the C ABI carries it (fp32); the oracle gets the same value."""
    return float(np.float32(W.top_p))


def _kept_mass(z, T, k, tp):
    """Sum over the oracle's kept set of exp((z - max z) / T)."""
    p = ov.softmax_t(z, T)
    w = ov.warp(p, k, tp)
    e = np.exp((z - z.max()) / T)
    return float(e[w > 0].sum())


def _stage(inp, logits32=None, check_mass=True):
    W = inp.workload
    if logits32 is None:
        logits32 = _oracle_logits(inp).astype(np.float32)
    print(f"warp stage: {W.name} B={W.batch} V={W.vocab} k={W.top_k} p={W.top_p}", flush=True)
    res = _sample_with_logits(inp, logits32)
    logits64 = logits32.astype(np.float64)
    draft64 = inp.draft_logits.astype(np.float64)
    rounds, _, _, _ = ov.sample_batch(logits64, draft64, inp.parent, inp.node_token, inp.uniforms,
                                      inp.temperature, W.n_nodes,
                                      without_replacement=W.children == "distinct",
                                      top_k=W.top_k, top_p=_tp(W))
    npath, nfin, excl, bad = compare_rounds(rounds, inp.temperature, res["accept_len"],
                                            res["accept_path"], res["out_tokens"], W.n_nodes,
                                            margin=MARGIN_STAGE)
    print(f"{W.name}: paths {npath}, final tokens {nfin}, excluded {excl}", flush=True)
    assert not bad, bad[:3]
    assert (res["seq_status"] & lib.SEQ_ERR_MASK == 0).all(), res["seq_status"]
    R, N = W.rows, W.n_nodes
    for b, r in enumerate(rounds):
        T = float(inp.temperature[b])
        if T == 0.0 or path_excluded(r, T):
            continue
        for t in r.tests:
            g = res["node_ratio"][b * N + t.node]
            if np.isinf(t.ratio):
                assert np.isinf(g), (b, t, g)
            else:
                assert abs(g - t.ratio) <= 1e-4 * max(1.0, abs(t.ratio)), (b, t, g)
        if not check_mass:
            continue
        for s in r.visited:
            row = b * R + s
            want = _kept_mass(logits64[row], T, W.top_k, _tp(W))
            got = float(res["slot_stats"][row, 1])
            assert abs(got - want) <= 1e-5 * want, (b, s, got, want)
            if any(int(inp.parent[b * N + j]) == s - 1 for j in range(N)):
                want = _kept_mass(draft64[row], T, W.top_k, _tp(W))
                got = float(res["slot_stats"][row, 3])
                assert abs(got - want) <= 1e-5 * want, (b, s, "draft", got, want)
    return npath, nfin, res


SETTINGS = [(20, 1.0), (0, 0.9), (50, 0.8), (1, 1.0), (4000, 0.95)]


@pytest.mark.parametrize("k,tp", SETTINGS, ids=lambda v: str(v))
@pytest.mark.parametrize("wl", [MINI, "eagle1_7b_t1", "share_70b"],
                         ids=lambda w: w if isinstance(w, str) else w.name)
def test_warped_sampling_stage_matches_oracle(wl, k, tp):
    inp = synth.generate(_warped(wl, k, tp), seed=3)
    if inp.workload.batch == 1:
        inp = synth.replicate_rounds(inp, 8, seed=4)    # several rounds on the context
    npath, _, _ = _stage(inp)
    assert npath >= 1


@pytest.mark.parametrize("k,tp", [(50, 0.9), (0, 0.95)])
def test_warped_sampling_gqa_8b(k, tp):
    _stage(synth.generate(_warped("gqa_8b", k, tp), seed=3))


def _quantised(inp, step):
    """Logits rounded to multiples of `step` (many exact ties), draft tokens
    redrawn from the rounded, warped draft rows."""
    inp.draft_logits = (np.round(inp.draft_logits / step) * step).astype(np.float32)
    return _redrawn(inp)


def _redrawn(inp):
    """Draft tokens drawn again from the (edited) draft rows, warped."""
    W = inp.workload
    N, R = W.n_nodes, W.rows
    rng = np.random.default_rng(99)
    toks = []
    for b in range(W.batch):
        toks.append(synth._draw_tokens(rng, inp.draft_logits[b * R:(b + 1) * R],
                                       inp.parent[b * N:(b + 1) * N], float(inp.temperature[b]),
                                       W.children == "distinct", W.top_k, W.top_p))
    inp.node_token = np.concatenate(toks).astype(np.int32)
    return inp


@pytest.mark.parametrize("k,tp", [(7, 1.0), (100, 1.0), (0, 0.5), (300, 0.9)])
def test_warped_sampling_with_tied_logits(k, tp):
    """Logits on a grid of 0.25 (target) and 0.5 (draft): the cut falls inside
    groups of equal logits, which the GPU orders by id in its last pass."""
    inp = _quantised(synth.generate(_warped(MINI, k, tp), seed=7), 0.5)
    logits32 = (np.round(_oracle_logits(inp) * 4.0) / 4.0).astype(np.float32)
    _stage(inp, logits32)


@pytest.mark.parametrize("name,k,tp", [("eagle1_7b_t1", 30, 0.9), ("share_70b", 0, 0.8)])
def test_warped_sampling_many_rounds(name, k, tp):
    base = synth.generate(_warped(name, k, tp), seed=21)
    inp = synth.replicate_rounds(base, 48, seed=22)
    npath, nfin, _ = _stage(inp)
    assert npath >= 0.9 * 48 and nfin >= 0.5 * 48


@pytest.mark.parametrize("k,tp", [(50, 1.0), (0, 0.95)])
def test_warped_distinct_siblings(k, tp):
    _stage(synth.generate(_warped(MINI, k, tp, children="distinct"), seed=5))


def test_warped_verify_end_to_end():
    inp = synth.generate(_warped(MINI, 40, 0.9), seed=4)
    W = inp.workload
    _, res = _run(inp)
    w = widened(inp)
    ref = ov.verify_batch(w["node_hidden"], w["kv"], inp.kv_offset, inp.prefix_len, inp.parent,
                          inp.node_token, w["lm_head"], inp.draft_logits, inp.uniforms,
                          inp.temperature, W.n_nodes, W.n_q_heads, W.n_kv_heads, W.head_dim,
                          with_attention=False, top_k=W.top_k, top_p=_tp(W))
    _compare_e2e(inp, ref, res)
    assert (res["seq_status"] & lib.SEQ_ERR_MASK == 0).all()


def test_warped_reruns_are_bitwise_equal():
    inp = synth.generate(_warped("eagle1_7b_t1", 30, 0.9), seed=8)
    logits32 = _oracle_logits(inp).astype(np.float32)
    a = _sample_with_logits(inp, logits32)
    b = _sample_with_logits(inp, logits32)
    for key in ("accept_len", "accept_path", "out_tokens", "seq_status", "slot_stats"):
        np.testing.assert_array_equal(a[key], b[key])
    torch.cuda.synchronize()


@pytest.mark.parametrize("k,tp", [(2000, 1.0), (0, 0.5), (5000, 0.7)])
def test_warped_sampling_huge_tie_groups(k, tp):
    """V = 32000 with logits rounded to whole numbers: a few thousand tokens
    share each value, so the cut bin and even its sub-bin hold more than the
    1024 candidates the sort takes; the GPU falls back to its key-byte
    histograms and orders the final tie group by id."""
    base = synth.generate(_warped("eagle1_7b_t1", k, tp), seed=12)
    inp = _quantised(synth.replicate_rounds(base, 6, seed=13), 1.0)
    logits32 = np.round(_oracle_logits(inp)).astype(np.float32)
    _stage(inp, logits32)


@pytest.mark.parametrize("k,tp", [(300, 1.0), (0, 0.6)])
def test_warped_sampling_tie_block_in_one_workgroup(k, tp):
    """600 tokens with ids 0..599 share the largest logit of every target and
    draft row: they all fall in the first workgroup's vocabulary share, whose
    candidate list (256 entries) overflows, so the selection takes the
    fallback path even though the bin is small enough to sort."""
    inp = synth.generate(_warped(MINI, k, tp), seed=14)
    W = inp.workload
    top = float(np.abs(inp.draft_logits).max()) + 3.0
    inp.draft_logits[:, :600] = top
    inp = _redrawn(inp)
    logits32 = _oracle_logits(inp).astype(np.float32)
    logits32[:, :600] = float(logits32.max()) + 3.0
    _stage(inp, logits32)
