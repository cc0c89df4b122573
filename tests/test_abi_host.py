"""The C ABI library on the host: it loads, exports every declared symbol, and
its argument checks return the documented codes without touching a device."""
import ctypes
import os

import pytest

from speculative_decoding_tree_amd import lib, synth
from speculative_decoding_tree_amd.runner import problem_for

pytestmark = pytest.mark.skipif(not os.path.exists(lib.LIB_PATH),
                                reason="libspecverify.so not built")


def _prob(**kw):
    base = dict(batch=1, n_nodes=10, n_q_heads=32, n_kv_heads=32, head_dim=128, vocab=32000,
                dtype=lib.SV_BF16, max_prefix=1024, max_children=4)
    base.update(kw)
    return lib.make_problem(**base)


def test_exports_every_declared_symbol():
    L = lib.load()
    names = lib.header_symbols()
    for must in ("sv_verify_tree", "sv_tree_attention", "sv_lm_head", "sv_sample",
                 "sv_compact_cache", "sv_workspace_size", "sv_status_string",
                 "sv_seq_status_string", "sv_version"):
        assert must in names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings():
    assert lib.sv_version() == lib.ABI_VERSION == 200
    assert lib.sv_status_string(0) == "ok"
    assert "NULL" in lib.sv_status_string(1)
    assert "unknown" in lib.sv_status_string(99)
    assert "parent" in lib.sv_seq_status_string(lib.SEQ_ERR_TREE)
    assert "clamped" in lib.sv_seq_status_string(lib.SEQ_WARN_UNIFORM)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workspace_size_of_every_workload(name):
    wl = synth.WORKLOADS[name]
    prob = lib.make_problem(batch=wl.batch, n_nodes=wl.n_nodes, n_q_heads=wl.n_q_heads,
                            n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim, vocab=wl.vocab,
                            dtype=lib.SV_BF16 if wl.dtype == "bf16" else lib.SV_F32,
                            max_prefix=8192 if wl.prefix[0] == "uniform" else wl.prefix[1],
                            max_children=4)
    n = lib.sv_workspace_size(prob)
    # the logits of every slot alone take B*R*V*4 bytes
    assert n >= wl.batch * wl.rows * wl.vocab * 4
    assert n % 256 == 0


def test_warping_sizes_its_selection_buffers():
    base = dict(batch=8, n_nodes=10, n_q_heads=8, n_kv_heads=8, head_dim=128, vocab=1000,
                dtype=lib.SV_BF16, max_prefix=64, max_children=4)
    plain = lib.sv_workspace_size(lib.make_problem(**base))
    # no cut (top_k >= V, top_p 0 or 1) keeps the plain plan
    for k, tp in ((1000, 1.0), (5000, 0.0), (0, 1.0)):
        assert lib.sv_workspace_size(lib.make_problem(**base, top_k=k, top_p=tp)) == plain
    for k, tp in ((10, 1.0), (0, 0.9), (999, 0.5)):
        n = lib.sv_workspace_size(lib.make_problem(**base, top_k=k, top_p=tp))
        # per sequence: 2 phases x 16 workgroups x 2 rows x 256 bins x (4 + 8) bytes
        assert n >= plain + 8 * 2 * 16 * 2 * 256 * 12


def test_problem_for_synthetic_batch():
    inp = synth.generate("chain_v1k", seed=0)
    prob = problem_for(inp)
    assert (prob.batch, prob.n_nodes, prob.hidden, prob.vocab, prob.dtype) == (1, 4, 256, 1024, 1)
    assert prob.max_prefix == 128 and prob.max_children == 1


@pytest.mark.parametrize("kw,code", [
    (dict(n_nodes=65), 2), (dict(n_nodes=-1), 2), (dict(batch=0), 2),
    (dict(n_kv_heads=5), 2), (dict(head_dim=96, hidden=32 * 96), 2), (dict(hidden=4000), 2),
    (dict(vocab=0), 2), (dict(dtype=7), 3), (dict(max_prefix=0), 2), (dict(max_children=0), 2),
    (dict(max_children=65), 2), (dict(batch=2000, n_nodes=60), 2),
    (dict(sampling=2), 2), (dict(top_k=-1), 2), (dict(top_p=-0.1), 2), (dict(top_p=1.5), 2),
    (dict(top_p=float("nan")), 2),
])
def test_shape_checks(kw, code):
    with pytest.raises(lib.SVError) as e:
        lib.sv_workspace_size(_prob(**kw))
    assert e.value.code == code


def _call_verify(prob, ptrs, ws_ptr, ws_bytes, dbg=None):
    L = lib.load()
    return L.sv_verify_tree(ctypes.byref(prob), *ptrs, dbg, ws_ptr, ws_bytes, None)


FAKE = 1 << 20        # aligned dummy addresses: never dereferenced by a failing check


def test_verify_null_problem_and_pointers():
    L = lib.load()
    ptrs = [FAKE] * 14
    assert L.sv_verify_tree(None, *ptrs, None, FAKE, 1 << 40, None) == 1
    prob = _prob()
    for i in range(14):
        p = list(ptrs)
        p[i] = None
        rc = _call_verify(prob, p, FAKE, 1 << 40)
        assert rc == 1, i


def test_verify_alignment_and_workspace():
    prob = _prob()
    need = lib.sv_workspace_size(prob)
    ptrs = [FAKE] * 14
    p = list(ptrs)
    p[0] = FAKE + 8        # kv misaligned
    assert _call_verify(prob, p, FAKE, need) == 6
    assert _call_verify(prob, ptrs, FAKE, need - 1) == 4
    assert _call_verify(prob, ptrs, None, need) == 4
    assert _call_verify(prob, ptrs, FAKE + 64, need) == 6     # workspace not 256-aligned


def test_sample_and_lm_head_checks():
    L = lib.load()
    prob = _prob()
    assert L.sv_sample(ctypes.byref(prob), *([None] * 10), None, FAKE, 1 << 40, None) == 1
    assert L.sv_lm_head(ctypes.byref(prob), 0, FAKE, FAKE, FAKE, None) == 2
    assert L.sv_lm_head(None, 4, FAKE, FAKE, FAKE, None) == 1
    bad = _prob(dtype=9)
    assert L.sv_lm_head(ctypes.byref(bad), 4, FAKE, FAKE, FAKE, None) == 3
    assert L.sv_lm_head(ctypes.byref(prob), 4, FAKE + 4, FAKE, FAKE, None) == 6
    assert L.sv_tree_attention(ctypes.byref(prob), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               1 << 40, None) == 1


def test_binding_refuses_host_tensors():
    import torch
    prob = _prob()
    with pytest.raises(ValueError):
        lib.sv_lm_head(prob, 4, torch.zeros(4), torch.zeros(4), torch.zeros(4))


def _compact(cache=FAKE, stride=1 << 20, layers=2, row_bytes=4096, batch=3, n=10,
             ptrs=(FAKE,) * 6):
    return lib.load().sv_compact_cache(cache, stride, layers, row_bytes, batch, n, *ptrs, None)


@pytest.mark.parametrize("kw", [
    dict(batch=-1), dict(batch=65536), dict(n=65), dict(n=-1), dict(layers=0),
    dict(layers=65536), dict(row_bytes=0), dict(row_bytes=6), dict(stride=-4),
])
def test_compact_cache_shape_checks(kw):
    assert _compact(**kw) == 2


def test_compact_cache_null_and_alignment_checks():
    # every call below fails a host check before any HIP call
    assert _compact(batch=0, ptrs=(None,) * 6) == 0     # nothing to do, nothing touched
    assert _compact(cache=None) == 1
    # kv_offset, prefix_len, accept_len, accept_path (N > 0), new_prefix_len
    for i in (0, 1, 2, 3, 4):
        p = [FAKE] * 6
        p[i] = None
        assert _compact(ptrs=tuple(p)) == 1, i
    assert _compact(cache=FAKE + 2) == 6
    assert _compact(stride=(1 << 20) + 2) == 6
    assert "compaction" in lib.sv_seq_status_string(lib.SEQ_ERR_PATH)


def test_tree_build_checks():
    # every call below fails a host check before any HIP call
    L = lib.load()
    P = [FAKE] * 9        # draft_logits, frontier, frontier_count, 5 pool arrays, status
    WS = (FAKE, 1 << 30)  # workspace, bytes
    # sv_tree_init(batch, K, frontier, frontier_count, pool_count, status, stream)
    assert L.sv_tree_init(0, 4, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert L.sv_tree_init(2, 17, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert L.sv_tree_init(2, 4, None, FAKE, FAKE, FAKE, None) == 1
    # sv_tree_workspace_size(batch, K, V, &bytes)
    assert lib.sv_tree_workspace_size(32, 10, 128256) >= 32 * 10 * 4 * 16 * 8
    with pytest.raises(lib.SVError):
        lib.sv_tree_workspace_size(0, 10, 100)
    with pytest.raises(lib.SVError):
        lib.sv_tree_workspace_size(2, 10, (1 << 20) + 1)
    # sv_tree_expand(batch, V, K, C, P, 9 pointers, workspace, bytes, stream)
    for args in ((0, 100, 4, 4, 64), (2, 100, 0, 4, 64), (2, 100, 17, 4, 64),
                 (2, 100, 4, 17, 64), (2, 3, 4, 4, 64), (2, 100, 4, 4, 0),
                 (2, 100, 4, 4, 1025), (2, (1 << 20) + 1, 4, 4, 64)):
        assert L.sv_tree_expand(*args, *P, *WS, None) == 2, args
    for i in range(9):
        p = list(P)
        p[i] = None
        assert L.sv_tree_expand(2, 100, 4, 4, 64, *p, *WS, None) == 1, i
    assert L.sv_tree_expand(2, 100, 4, 4, 64, FAKE + 2, *P[1:], *WS, None) == 6
    need = lib.sv_tree_workspace_size(2, 4, 100)
    assert L.sv_tree_expand(2, 100, 4, 4, 64, *P, FAKE, need - 1, None) == 4
    assert L.sv_tree_expand(2, 100, 4, 4, 64, *P, None, need, None) == 4
    assert L.sv_tree_expand(2, 100, 4, 4, 64, *P, FAKE + 4, need, None) == 6
    # sv_tree_finalize(batch, P, m, 9 pointers, stream)
    for args in ((0, 64, 8), (2, 0, 8), (2, 1025, 8), (2, 64, 0), (2, 64, 65)):
        assert L.sv_tree_finalize(*args, *([FAKE] * 9), None) == 2, args
    for i in range(9):
        p = [FAKE] * 9
        p[i] = None
        assert L.sv_tree_finalize(2, 64, 8, *p, None) == 1, i
    assert "pool" in lib.sv_seq_status_string(lib.SEQ_ERR_POOL)


def test_layer_share_checks():
    # every call below fails a host check before any HIP call
    L = lib.load()
    prob = _prob(n_kv_heads=8)
    need = lib.sv_layer_workspace_size(prob)
    assert need > 0
    ptrs = [FAKE] * 5                     # hidden, wq, wk, wv, wo

    def call(p=prob, ptrs=ptrs, theta=10000.0, kv=FAKE, off=FAKE, par=FAKE, out=FAKE,
             attn=None, st=FAKE, ws=FAKE, nbytes=None):
        return L.sv_layer_share(ctypes.byref(p), *ptrs, theta, kv, off, par, out, attn, st, ws,
                                need if nbytes is None else nbytes, None)
    assert call(p=_prob(dtype=lib.SV_F32, head_dim=64, hidden=32 * 64)) == 3
    assert call(p=_prob(head_dim=64, hidden=32 * 64)) == 2
    assert call(theta=0.0) == 2 and call(theta=float("inf")) == 2 and call(theta=float("nan")) == 2
    for i in range(5):
        p = list(ptrs)
        p[i] = None
        assert call(ptrs=p) == 1, i
    assert call(kv=None) == 1 and call(off=None) == 1 and call(par=None) == 1
    assert call(out=None) == 1 and call(st=None) == 1
    assert call(ptrs=[FAKE + 2] + ptrs[1:]) == 6
    assert call(attn=FAKE + 4) == 6
    assert call(nbytes=need - 1) == 4 and call(ws=None) == 4
    assert call(ws=FAKE + 16) == 6


def test_sample_noalloc_rejects_problems_beyond_its_scratch():
    """sv_sample_noalloc checks its arguments and the static scratch's size on
    the host, before any HIP call: a problem whose sampling buffers exceed
    SV_NOALLOC_SCRATCH_BYTES gets SV_ERR_SCRATCH, a missing pointer
    SV_ERR_NULL, a bad shape SV_ERR_SHAPE."""
    L = lib.load()
    fake = [256] * 10      # never dereferenced: the call returns before any launch
    big = _prob(batch=1000, n_nodes=60, n_q_heads=32, n_kv_heads=8, vocab=128256)
    assert L.sv_sample_noalloc(ctypes.byref(big), *fake, None, None) == 7
    assert "scratch" in lib.sv_status_string(7)
    ok = _prob(batch=32, n_nodes=60, n_q_heads=32, n_kv_heads=8, vocab=128256)
    nulls = list(fake)
    nulls[2] = None        # logits
    assert L.sv_sample_noalloc(ctypes.byref(ok), *nulls, None, None) == 1
    bad = _prob(n_nodes=65)
    assert L.sv_sample_noalloc(ctypes.byref(bad), *fake, None, None) == 2
