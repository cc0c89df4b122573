"""CPU oracle for the cache step that follows verification: keep the accepted
path's rows, drop the rest of the draft tree.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module. The product path
never calls it, and it imports nothing from that path.

Sources (titles of the pages this restates):
  [E1]  "EAGLE / EAGLE-2" translated excerpts (modelers.csdn.net), sec. 1.3.2:
        after the tree is verified, the accepted tokens (and their features)
        are kept for the next drafting round.
  [EQ]  "EAGLE (ICML 2024) close reading" (edgeai1.github.io), sec. 5: after a
        rejection both caches (the target's and the draft decoder's) are cut
        back, and cache reordering is a cost of its own, next to tree
        verification and the sampling kernel.
  [SPS] "LLM speculative decoding: EAGLE" blog (jingming.pro), sec. 4.2: the
        draft tree is packed after the prefix, one row per node, and a node
        attends to the prefix and to its ancestors; so the rows of a
        root-to-node path, in order, are exactly the rows a plain causal
        decode of those tokens would have appended.

Readings where the pages are silent:
  - The cache region of sequence b starts at row kv_offset[b]; its prefix
    holds prefix_len[b] rows and node j's row is prefix_len[b] + j. Rows are
    opaque bytes (K and V of every head, or any per-token record such as the
    draft decoder's features), so the step is a byte copy.
  - Accepted node accept_path[b][i] moves to row prefix_len[b] + i, for
    i < accept_len[b]; the new prefix length is prefix_len[b] + accept_len[b].
    Rows past it are left as they are (free for the next tree). The corrected
    or bonus token has no row yet: the next forward computes it.
  - accept_len[b] = -1 (a sequence the verifier flagged) leaves the region
    untouched and the prefix length unchanged.
  - A path that is not strictly increasing, leaves [0, N), or does not fit the
    region is rejected for that sequence (region untouched, status flagged).
    A valid accepted path is a root-to-node chain of the packed tree, whose
    indices increase because every parent precedes its children.
"""
from __future__ import annotations

import numpy as np

STATUS_BAD_PATH = 1   # the sequence's accept path or region was not valid


def path_is_valid(path, n: int, n_nodes: int) -> bool:
    """Strictly increasing node indices inside [0, n_nodes)."""
    prev = -1
    for i in range(n):
        j = int(path[i])
        if j <= prev or j >= n_nodes:
            return False
        prev = j
    return True


def compact_sequence(rows, prefix_len: int, n_nodes: int, accept_len: int, accept_path):
    """One sequence's region, rows [prefix_len + n_nodes (+ spare), ...].

    Returns (new_rows, new_prefix_len, status). new_rows is a copy; its rows
    prefix_len + i hold the original rows prefix_len + accept_path[i].
    """
    out = np.array(rows, copy=True)
    L = int(prefix_len)
    n = int(accept_len)
    if n == -1:
        return out, L, 0
    if n < -1 or n > n_nodes or L < 0 or L + n_nodes > len(rows) \
            or not path_is_valid(accept_path, n, n_nodes):
        return out, L, STATUS_BAD_PATH
    for i in range(n):
        out[L + i] = rows[L + int(accept_path[i])]
    return out, L + n, 0


def compact_cache(cache, kv_offset, prefix_len, accept_len, accept_path, n_nodes: int):
    """Batch form over a cache of shape [layers, rows, row_bytes] (any dtype).

    accept_path is [B * n_nodes] (-1 padded). Every layer moves the same rows.
    Returns (new_cache, new_prefix_len[B], status[B]).
    """
    cache = np.asarray(cache)
    out = cache.copy()
    B = len(prefix_len)
    new_len = np.empty(B, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        r0, r1 = int(kv_offset[b]), int(kv_offset[b + 1])
        path = accept_path[b * n_nodes:(b + 1) * n_nodes]
        for layer in range(cache.shape[0]):
            region, nl, st = compact_sequence(cache[layer, r0:r1], prefix_len[b], n_nodes,
                                              accept_len[b], path)
            out[layer, r0:r1] = region
        new_len[b] = nl
        status[b] = st
    return out, new_len, status
