"""CPU oracle for the full verify-layer share: projections, rotary positions
by tree depth, tree attention, output projection and the residual that feeds
the LM head.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module. The product path
never calls it, and it imports nothing from that path.

Sources (titles of the pages this restates):
  [SPS] "LLM speculative decoding: EAGLE" blog (jingming.pro), sec. 3.1 (the
        LM head maps the last layer's feature of each position to logits) and
        sec. 4.2 (the draft tree is packed into one sequence; a node attends
        to the prefix and its own ancestors, so along any root-to-node path
        the computation is that of ordinary decoding).
  [EQ]  "EAGLE (ICML 2024) close reading" (edgeai1.github.io), sec. 5: the
        tree's position ids must be set correctly at inference.

Readings where the pages are silent:
  - One decoder layer's attention block, without norms or MLP: q = h Wq^T,
    k = h Wk^T, v = h Wv^T per slot, rotary embedding on q and k, tree
    attention, o = attn Wo^T, and h' = h + o is the LM head's input.
  - Positions: the root slot (the last committed token, prefix row L - 1)
    has position L - 1; node j has position L - 1 + depth(j), depth(root
    child) = 1. So every root-to-node path gets the positions a causal
    decode of that path would use. The root's K/V is the cache's row L - 1
    (computed by the previous step) and is not recomputed; each node's
    rotated K and its V are written to cache row L + j.
  - Rotary embedding: dimension pairs (i, i + D/2), i < D/2, rotate by
    angle pos * theta^(-2i/D) (the "rotate half" layout).
  - Scores q.k / sqrt(D); query head h reads KV head h // (Hq / Hkv).
"""
from __future__ import annotations

import math

import numpy as np

from . import verify as _verify


def rope(x, pos, theta: float):
    """Rotate every head vector of x [..., D] at position pos (scalar or
    broadcastable over the leading axes)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    inv = theta ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv        # [..., half]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def positions(parent, prefix_len: int):
    """Position of every slot: root L - 1, node j at L - 1 + depth(j)."""
    N = len(parent)
    pos = np.empty(N + 1, dtype=np.int64)
    pos[0] = prefix_len - 1
    for j in range(N):
        pos[j + 1] = prefix_len - 1 + _verify.depth_of(parent, j)
    return pos


def layer_share_sequence(h, wq, wk, wv, wo, kv, prefix_len: int, parent, n_kv_heads: int,
                         theta: float):
    """One sequence.

    h [R, d] slot hidden states (slot 0 = root); wq [Hq*D, d], wk / wv
    [Hkv*D, d], wo [d, Hq*D]; kv [L + N, 2, Hkv, D] with the prefix rows
    filled (node rows are overwritten). Returns (h_out [R, d], kv_out,
    attn [R, Hq, D]), all fp64.
    """
    h = np.asarray(h, dtype=np.float64)
    wq, wk, wv, wo = (np.asarray(w, dtype=np.float64) for w in (wq, wk, wv, wo))
    L = int(prefix_len)
    N = len(parent)
    R = N + 1
    Hkv = n_kv_heads
    D = kv.shape[-1]
    Hq = wq.shape[0] // D
    pos = positions(parent, L)
    q = rope((h @ wq.T).reshape(R, Hq, D), pos[:, None], theta)
    k_node = rope((h[1:] @ wk.T).reshape(N, Hkv, D), pos[1:, None], theta)
    v_node = (h[1:] @ wv.T).reshape(N, Hkv, D)
    kv_out = np.array(kv, dtype=np.float64, copy=True)
    kv_out[L:L + N, 0] = k_node
    kv_out[L:L + N, 1] = v_node
    attn = _verify.tree_attention_sequence(q, kv_out[:, 0], kv_out[:, 1], L, parent, Hkv)
    h_out = h + attn.reshape(R, Hq * D) @ wo.T
    return h_out, kv_out, attn
