"""sv_sample_noalloc, the variant of sv_sample whose scratch is the library's
static device array, against sv_sample with a caller-supplied workspace,
through the C ABI: every output bitwise equal, on calls in a row whose
problems shrink (the scratch keeps the previous call's contents)."""
import numpy as np
import pytest
import torch

from speculative_decoding_tree_amd import lib, synth
from speculative_decoding_tree_amd.runner import DeviceBatch

pytestmark = pytest.mark.gpu

MINI = synth.Workload(
    name="mini_noalloc", batch=3, n_nodes=12, n_q_heads=8, n_kv_heads=2, head_dim=128,
    vocab=5000, dtype=synth.BF16, prefix=("list", (1, 77, 300)), tree=("seeded", 4), w_std=0.05,
    draft=("perturbed", 0.5), temperature=("list", (0.0, 0.7, 1.3)))

OUTS = ("accept_len", "accept_path", "out_tokens", "seq_status")


def _logits(db):
    """Target logits from the library's own LM head (both calls read the
    same array; the comparison is between the two sampling entry points)."""
    W = db.inp.workload
    lg = torch.empty((W.batch * W.rows, W.vocab), dtype=torch.float32, device="cuda")
    lib.sv_lm_head(db.prob, W.batch * W.rows, db.t["node_hidden"], db.t["lm_head"], lg)
    return lg


def _sample(db, lg, noalloc):
    t = db.t
    out = {k: torch.full_like(t[k], -7) for k in OUTS}
    dbg = db.debug_buffers()
    dbg.pop("logits")
    args = (db.prob, t["parent"], t["node_token"], lg, t["draft_logits"], t["uniforms"],
            t["temperature"], out["accept_len"], out["accept_path"], out["out_tokens"],
            out["seq_status"])
    if noalloc:
        lib.sv_sample_noalloc(*args, dbg=dbg)
    else:
        lib.sv_sample(*args, dbg=dbg, workspace=db.workspace)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res.update({k: v.cpu().numpy() for k, v in dbg.items()})
    return res


def _check_equal(db, lg, label):
    print(f"[no-alloc] {label}: batch {db.prob.batch}, vocab {db.prob.vocab}", flush=True)
    a = _sample(db, lg, noalloc=False)
    b = _sample(db, lg, noalloc=True)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"{label}: {k}")
    assert (b["seq_status"] & lib.SEQ_ERR_MASK == 0).all(), b["seq_status"]
    assert (b["accept_len"] >= 0).all()


def test_noalloc_matches_workspace_calls_in_a_row():
    # call 1: the batched workload at full size (32 sequences, V = 128256)
    big = DeviceBatch.create(synth.generate("batch32_8b", seed=0))
    lg = _logits(big)
    _check_equal(big, lg, "batch32_8b")
    del lg
    # call 2: a smaller problem on the same scratch
    small = DeviceBatch.create(synth.generate(MINI, seed=3))
    _check_equal(small, _logits(small), "mini")
    # call 3: smaller still, with top-k / top-p warping (its selection buffers)
    warped_wl = MINI.with_(name="mini_noalloc_warped", batch=2, vocab=3000, top_k=40, top_p=0.9,
                           temperature=("list", (1.0, 0.8)))
    warped = DeviceBatch.create(synth.generate(warped_wl, seed=4))
    _check_equal(warped, _logits(warped), "mini warped")


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    db = DeviceBatch.create(synth.generate(MINI, seed=5))
    lg = _logits(db)
    t = db.t
    big = lib.make_problem(1000, 60, 32, 8, 128, 128256, lib.SV_BF16, 8192, 4)
    with pytest.raises(lib.SVError) as ei:
        lib.sv_sample_noalloc(big, t["parent"], t["node_token"], lg, t["draft_logits"],
                              t["uniforms"], t["temperature"], t["accept_len"],
                              t["accept_path"], t["out_tokens"], t["seq_status"])
    assert ei.value.code == 7
