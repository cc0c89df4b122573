"""GPU parity of sv_layer_share (projections, rotary positions by tree depth,
tree attention, output projection, residual) with the oracle
(oracle/layer.py), through the C ABI.

Tolerances: the GPU rounds q, k, v, the attention output and h' to bf16 and
accumulates in fp32, the oracle works in fp64 on the same bf16 inputs. Each
bf16 rounding is within 2^-9 relative, so per (row, head) relative L2 errors
stay well under the attention tolerance of 1e-2 used for the written K/V
rows, the attention output and the layer output.
"""
import numpy as np
import pytest
import torch

from oracle import layer as ol
from speculative_decoding_tree_amd import lib, synth
from speculative_decoding_tree_amd.runner import problem_for

from parity_util import TOL_ATTN

pytestmark = pytest.mark.gpu

MINI = synth.Workload(
    name="mini_layer", batch=3, n_nodes=12, n_q_heads=8, n_kv_heads=2, head_dim=128,
    vocab=5000, dtype=synth.BF16, prefix=("list", (1, 77, 300)), tree=("seeded", 4), w_std=0.05,
    draft=("perturbed", 0.5), temperature=("list", (0.0, 0.7, 1.3)))


def _weights(seed, Hq, Hkv, D, d, std=0.02):
    rng = np.random.default_rng(seed)
    mk = lambda n, k: synth.to_bf16_bits((rng.standard_normal((n, k)) * std).astype(np.float32))
    return mk(Hq * D, d), mk(Hkv * D, d), mk(Hkv * D, d), mk(d, Hq * D)


def _dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _rel(a, b):
    """Largest relative L2 error over the rows of the last axis."""
    a = a.reshape(-1, a.shape[-1]).astype(np.float64)
    b = b.reshape(-1, b.shape[-1]).astype(np.float64)
    num = np.linalg.norm(a - b, axis=1)
    den = np.maximum(np.linalg.norm(b, axis=1), 1e-12)
    return float((num / den).max())


def _run_gpu(inp, w, theta, with_attn=True):
    W = inp.workload
    prob = problem_for(inp)
    B, R, d = W.batch, W.rows, W.hidden
    kv = _dev16(inp.kv)
    out = torch.empty((B * R, d), dtype=torch.int16, device="cuda")
    attn = (torch.empty((B * R, W.n_q_heads, W.head_dim), dtype=torch.float32, device="cuda")
            if with_attn else None)
    st = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(lib.sv_layer_workspace_size(prob), dtype=torch.uint8, device="cuda")
    print(f"layer share: {W.name} B={B} N={W.n_nodes} d={d} attn_out={with_attn}", flush=True)
    lib.sv_layer_share(prob, _dev16(inp.node_hidden), *[_dev16(x) for x in w], theta, kv,
                       torch.from_numpy(inp.kv_offset.astype(np.int32)).cuda(),
                       torch.from_numpy(inp.parent.astype(np.int32)).cuda(), out, st,
                       attn_out=attn, workspace=ws)
    torch.cuda.synchronize()
    return (kv.cpu().numpy().view(np.uint16), out.cpu().numpy().view(np.uint16),
            attn.cpu().numpy() if with_attn else None, st.cpu().numpy())


def _check(inp, w, theta, seqs, got):
    W = inp.workload
    N, R, Hkv = W.n_nodes, W.rows, W.n_kv_heads
    kv_g, out_g, attn_g, st = got
    assert (st & lib.SEQ_ERR_MASK == 0).all()
    wf = [synth.widen(x, W.dtype) for x in w]
    for b in seqs:
        r0, r1 = int(inp.kv_offset[b]), int(inp.kv_offset[b + 1])
        L = int(inp.prefix_len[b])
        rows = slice(b * R, (b + 1) * R)
        h = synth.widen(inp.node_hidden[rows], W.dtype)
        kv = synth.widen(inp.kv[r0:r1], W.dtype)
        h_out, kv_out, attn = ol.layer_share_sequence(h, *wf, kv, L,
                                                      inp.parent[b * N:(b + 1) * N], Hkv, theta)
        np.testing.assert_array_equal(kv_g[r0:r0 + L], inp.kv[r0:r0 + L])   # prefix untouched
        e_kv = _rel(synth.widen(kv_g[r0 + L:r1], W.dtype), kv_out[L:])
        e_at = _rel(attn_g[rows], attn)
        e_out = _rel(synth.widen(out_g[rows], W.dtype), h_out)
        print(f"seq {b}: L={L} kv {e_kv:.2e} attn {e_at:.2e} out {e_out:.2e}", flush=True)
        assert e_kv <= TOL_ATTN and e_at <= TOL_ATTN and e_out <= TOL_ATTN


@pytest.mark.parametrize("theta", [10000.0, 500000.0])
def test_layer_share_mini_ragged(theta):
    inp = synth.generate(MINI, seed=2)
    W = inp.workload
    w = _weights(5, W.n_q_heads, W.n_kv_heads, W.head_dim, W.hidden)
    _check(inp, w, theta, range(W.batch), _run_gpu(inp, w, theta))


def test_layer_share_gqa_8b_shape():
    inp = synth.generate(synth.workload("gqa_8b"), seed=1)
    W = inp.workload
    w = _weights(6, W.n_q_heads, W.n_kv_heads, W.head_dim, W.hidden)
    _check(inp, w, 500000.0, [0], _run_gpu(inp, w, 500000.0))


def test_layer_share_batched_workload_full_size():
    """The batched workload (32 sequences, prefixes up to 8192); the oracle
    recomputes the shortest and the longest sequence. The benchmark's own
    call (no attn_out, so attention writes only the bf16 input of the O
    projection) gives the same output rows, cache and status bit for bit."""
    inp = synth.generate("batch32_8b", seed=0)
    W = inp.workload
    w = _weights(7, W.n_q_heads, W.n_kv_heads, W.head_dim, W.hidden)
    got = _run_gpu(inp, w, 500000.0)
    L = inp.prefix_len
    _check(inp, w, 500000.0, sorted({int(np.argmin(L)), int(np.argmax(L))}), got)
    bare = _run_gpu(inp, w, 500000.0, with_attn=False)
    for i, name in ((0, "kv"), (1, "out_hidden"), (3, "seq_status")):
        np.testing.assert_array_equal(bare[i], got[i], err_msg=name)


def test_layer_share_without_attn_out_mini():
    """No attn_out on the ragged mini batch: the same output rows, cache and
    status as with it, bit for bit."""
    inp = synth.generate(MINI, seed=2)
    W = inp.workload
    w = _weights(5, W.n_q_heads, W.n_kv_heads, W.head_dim, W.hidden)
    got = _run_gpu(inp, w, 10000.0)
    bare = _run_gpu(inp, w, 10000.0, with_attn=False)
    for i, name in ((0, "kv"), (1, "out_hidden"), (3, "seq_status")):
        np.testing.assert_array_equal(bare[i], got[i], err_msg=name)
