"""GPU parity of sv_compact_cache (KV-cache compaction after acceptance) with
the oracle (oracle/cache.py), through the C ABI: bit-exact bytes, new prefix
lengths and status, on ragged batches, several layers, every move width, the
degenerate and invalid cases, the batched workload's shape at full size, and
after a real verification step."""
import numpy as np
import pytest
import torch

from oracle import cache as oc
from oracle import verify as ov
from speculative_decoding_tree_amd import lib, synth
from speculative_decoding_tree_amd.runner import DeviceBatch

from parity_util import path_excluded

pytestmark = pytest.mark.gpu


def _random_path(rng, parent, stop=0.2):
    kids = {}
    for j, p in enumerate(parent):
        kids.setdefault(int(p), []).append(j)
    path, cur = [], -1
    while kids.get(cur):
        if path and rng.random() < stop:
            break
        cur = int(rng.choice(kids[cur]))
        path.append(cur)
    return path


def _gpu_compact(cache, kv_offset, prefix_len, accept_len, accept_path, N, layer_stride_rows):
    """cache: uint8 [layers, rows_alloc, row_bytes] host array. Returns the
    GPU's (cache, new_prefix_len, status) as host arrays."""
    layers, _, row_bytes = cache.shape
    dc = torch.from_numpy(np.ascontiguousarray(cache)).cuda()
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    B = len(prefix_len)
    new_len = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    status = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    print(f"compact: B={B} N={N} layers={layers} row_bytes={row_bytes}", flush=True)
    lib.sv_compact_cache(dc, layer_stride_rows * row_bytes, layers, row_bytes, B, N,
                         i32(kv_offset), i32(prefix_len), i32(accept_len),
                         i32(accept_path if len(accept_path) else [0]), new_len, status)
    torch.cuda.synchronize()
    return dc.cpu().numpy(), new_len.cpu().numpy(), status.cpu().numpy()


def _ragged_case(seed, row_bytes, layers=3, B=10, N=20):
    rng = np.random.default_rng(seed)
    L = rng.integers(1, 40, B).astype(np.int32)
    kv_offset = np.zeros(B + 1, dtype=np.int32)
    kv_offset[1:] = np.cumsum(L + N)
    rows_alloc = int(kv_offset[-1]) + 5                  # spare rows past the last region
    cache = rng.integers(0, 256, (layers, rows_alloc, row_bytes), dtype=np.uint8)
    acc = np.zeros(B, dtype=np.int32)
    paths = np.full(B * N, -1, dtype=np.int32)
    for b in range(B):
        parent = synth.seeded_tree(rng, N, depth=6)
        p = _random_path(rng, parent)
        acc[b] = len(p)
        paths[b * N: b * N + len(p)] = p
    # degenerate and invalid sequences
    acc[0] = 0                                            # nothing accepted
    acc[1] = -1                                           # flagged by the verifier
    acc[2], paths[2 * N: 2 * N + 4] = 4, [0, 2, 5, 9]     # row 2 read, then written
    acc[3], paths[3 * N: 3 * N + 2] = 2, [4, 4]           # not strictly increasing
    acc[4], paths[4 * N] = 1, N                           # outside [0, N)
    acc[5] = N + 1                                        # longer than the tree
    L[6] += 1                                             # tree rows past the region
    acc[7], paths[7 * N: 8 * N] = N, np.arange(N)        # a chain accepted in full
    return cache, kv_offset, L, acc, paths, rows_alloc


@pytest.mark.parametrize("row_bytes", [4096, 2052, 256, 16, 4])
def test_compact_ragged_batch_matches_oracle(row_bytes):
    N = 20
    cache, kv_offset, L, acc, paths, rows_alloc = _ragged_case(row_bytes, row_bytes, N=N)
    want, want_len, want_st = oc.compact_cache(cache, kv_offset, L, acc, paths, N)
    got, got_len, got_st = _gpu_compact(cache, kv_offset, L, acc, paths, N, rows_alloc)
    np.testing.assert_array_equal(got_len, want_len)
    np.testing.assert_array_equal(got_st != 0, want_st != 0)
    assert list(np.nonzero(got_st)[0]) == [3, 4, 5, 6]
    assert (got_st[got_st != 0] == lib.SEQ_ERR_PATH).all()
    np.testing.assert_array_equal(got, want)


def test_compact_without_status_and_empty_tree():
    rng = np.random.default_rng(5)
    B, N, rb = 4, 0, 64
    L = np.array([3, 1, 7, 2], dtype=np.int32)
    kv_offset = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cache = rng.integers(0, 256, (1, int(kv_offset[-1]), rb), dtype=np.uint8)
    acc = np.array([0, -1, 0, 0], dtype=np.int32)
    dc = torch.from_numpy(cache).cuda()
    new_len = torch.empty(B, dtype=torch.int32, device="cuda")
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()
    lib.sv_compact_cache(dc, int(kv_offset[-1]) * rb, 1, rb, B, N, i32(kv_offset), i32(L),
                         i32(acc), None, new_len, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(new_len.cpu().numpy(), L)
    np.testing.assert_array_equal(dc.cpu().numpy(), cache)


def test_compact_batched_workload_full_size():
    """The batched workload's cache shape (32 sequences, prefixes uniform on
    [512, 8192], 60-node trees of depth 6, 8 KV heads x 128 in bf16 = 4 KB per
    row) in two layers with a gap between them."""
    rng = np.random.default_rng(32)
    B, N, row_bytes = 32, 60, 2 * 8 * 128 * 2
    L = rng.integers(512, 8193, B).astype(np.int32)
    kv_offset = np.zeros(B + 1, dtype=np.int32)
    kv_offset[1:] = np.cumsum(L + N)
    rows = int(kv_offset[-1])
    stride_rows = rows + 64
    cache = np.frombuffer(rng.bytes(2 * stride_rows * row_bytes), dtype=np.uint8)
    cache = cache.reshape(2, stride_rows, row_bytes)
    acc = np.zeros(B, dtype=np.int32)
    paths = np.full(B * N, -1, dtype=np.int32)
    for b in range(B):
        p = _random_path(rng, synth.seeded_tree(rng, N, depth=6), stop=0.1)
        acc[b] = len(p)
        paths[b * N: b * N + len(p)] = p
    got, got_len, got_st = _gpu_compact(cache, kv_offset, L, acc, paths, N, stride_rows)
    assert (got_st == 0).all()
    np.testing.assert_array_equal(got_len, L + acc)
    # the oracle on each sequence's region; everything outside the tree rows
    # (prefixes, the gap between layers) must be untouched
    for b in range(B):
        r0, r1 = int(kv_offset[b]), int(kv_offset[b + 1])
        for layer in range(2):
            want, nl, st = oc.compact_sequence(cache[layer, r0:r1], L[b], N, acc[b],
                                               paths[b * N:(b + 1) * N])
            np.testing.assert_array_equal(got[layer, r0:r1], want)
    np.testing.assert_array_equal(got[:, rows:], cache[:, rows:])


@pytest.mark.parametrize("name", ["eagle1_7b_t1", "share_70b", "chain_v1k"])
def test_compact_after_verification(name):
    """Verify on the GPU, then compact its KV cache by its own accept path; the
    oracle verifies and compacts the same inputs. Rounds whose path the parity
    rule excludes (a test within 1e-5 of its threshold) are skipped."""
    inp = synth.generate(synth.workload(name, batch=4) if name != "chain_v1k" else name, seed=9)
    W = inp.workload
    B, N = W.batch, W.n_nodes
    db = DeviceBatch.create(inp)
    db.verify()
    t = db.t
    row_bytes = t["kv"][0].numel() * t["kv"].element_size()
    new_len = torch.empty(B, dtype=torch.int32, device="cuda")
    status = torch.empty(B, dtype=torch.int32, device="cuda")
    prefix = torch.from_numpy(inp.prefix_len.astype(np.int32)).cuda()
    lib.sv_compact_cache(t["kv"], 0, 1, row_bytes, B, N, t["kv_offset"], prefix,
                         t["accept_len"], t["accept_path"], new_len, status)
    torch.cuda.synchronize()
    w = {"kv": synth.widen(inp.kv, W.dtype), "node_hidden": synth.widen(inp.node_hidden, W.dtype),
         "lm_head": synth.widen(inp.lm_head, W.dtype)}
    ref = ov.verify_batch(w["node_hidden"], w["kv"], inp.kv_offset, inp.prefix_len, inp.parent,
                          inp.node_token, w["lm_head"], inp.draft_logits, inp.uniforms,
                          inp.temperature, N, W.n_q_heads, W.n_kv_heads, W.head_dim,
                          with_attention=False)
    raw = inp.kv.reshape(1, inp.kv.shape[0], -1).view(np.uint8)
    want, want_len, want_st = oc.compact_cache(raw, inp.kv_offset, inp.prefix_len,
                                               ref.accept_len, ref.accept_path, N)
    got = t["kv"].cpu().numpy().reshape(1, inp.kv.shape[0], -1).view(np.uint8)
    got_len = new_len.cpu().numpy()
    assert (status.cpu().numpy() == 0).all() and (want_st == 0).all()
    compared = 0
    for b in range(B):
        if path_excluded(ref.rounds[b], float(inp.temperature[b])):
            continue
        compared += 1
        r0, r1 = int(inp.kv_offset[b]), int(inp.kv_offset[b + 1])
        assert got_len[b] == want_len[b]
        np.testing.assert_array_equal(got[0, r0:r1], want[0, r0:r1])
    print(f"{name}: {compared} of {B} sequences compared", flush=True)
    assert compared >= 1
