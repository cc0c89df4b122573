"""Pins of the verify-layer-share oracle (oracle/layer.py).

  - The rotary embedding equals multiplying each dimension pair, read as a
    complex number, by numpy's complex exponential of the angle; position 0
    is the identity; scores of rotated vectors depend only on the position
    difference.
  - The central one: along every root-to-node path of a tree, the layer's
    outputs equal a plain causal decode of that path, one token at a time,
    with the usual consecutive positions and a growing cache (what the tree
    mask and depth positions are for).
  - A chain tree's positions are consecutive; projections and the residual
    are checked against numpy matmuls on a one-node tree.
"""
import math

import numpy as np
import pytest

from oracle import layer as ol
from speculative_decoding_tree_amd import synth


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(0)
    D, theta = 16, 10000.0
    x = rng.normal(0, 1, (5, 3, D))
    pos = np.array([0, 1, 7, 100, 4095])
    got = ol.rope(x, pos[:, None], theta)
    half = D // 2
    z = x[..., :half] + 1j * x[..., half:]
    w = np.exp(1j * pos[:, None, None] * theta ** (-np.arange(half) * 2.0 / D))
    want = z * w
    np.testing.assert_allclose(got[..., :half], want.real, atol=1e-12)
    np.testing.assert_allclose(got[..., half:], want.imag, atol=1e-12)
    np.testing.assert_allclose(ol.rope(x, 0, theta), x, atol=0)


def test_rope_scores_depend_on_position_difference():
    rng = np.random.default_rng(1)
    D = 32
    q, k = rng.normal(0, 1, D), rng.normal(0, 1, D)
    for delta in (0, 1, 5, 300):
        s = [ol.rope(q, m + delta, 500000.0) @ ol.rope(k, m, 500000.0) for m in (0, 3, 1000)]
        np.testing.assert_allclose(s, s[0], rtol=1e-10)


def _causal_decode(h_path, wq, wk, wv, wo, kv_prefix, L, Hkv, theta):
    """Decode the path tokens one at a time after the prefix: token t (the
    root first) sits at position L - 1 + t. Returns the per-token output h'."""
    D = kv_prefix.shape[-1]
    Hq = wq.shape[0] // D
    G = Hq // Hkv
    K = [kv_prefix[r, 0] for r in range(L)]
    Vv = [kv_prefix[r, 1] for r in range(L)]
    outs = []
    for t, hv in enumerate(h_path):
        p = L - 1 + t
        if t > 0:                       # the root's K/V is the cache's row L - 1
            K.append(ol.rope((hv @ wk.T).reshape(Hkv, D), p, theta))
            Vv.append((hv @ wv.T).reshape(Hkv, D))
        q = ol.rope((hv @ wq.T).reshape(Hq, D), p, theta)
        Ks, Vs = np.stack(K), np.stack(Vv)
        o = np.empty((Hq, D))
        for h in range(Hq):
            sc = Ks[:, h // G] @ q[h] / math.sqrt(D)
            w = np.exp(sc - sc.max())
            o[h] = (w / w.sum()) @ Vs[:, h // G]
        outs.append(hv + o.reshape(-1) @ wo.T)
    return np.stack(outs)


@pytest.mark.parametrize("seed", range(4))
def test_every_path_equals_a_causal_decode(seed):
    rng = np.random.default_rng(10 + seed)
    Hq, Hkv, D, L, N, theta = 4, 2, 8, 6, 10, 10000.0
    d = Hq * D
    parent = synth.seeded_tree(rng, N, depth=4)
    h = rng.normal(0, 1, (N + 1, d))
    wq, wk, wv = (rng.normal(0, 0.3, (n, d)) for n in (Hq * D, Hkv * D, Hkv * D))
    wo = rng.normal(0, 0.3, (d, Hq * D))
    kv = rng.normal(0, 1, (L + N, 2, Hkv, D))
    h_out, kv_out, _ = ol.layer_share_sequence(h, wq, wk, wv, wo, kv, L, parent, Hkv, theta)
    np.testing.assert_array_equal(kv_out[:L], kv[:L])
    leaves = [j for j in range(N) if j not in set(int(p) for p in parent)]
    for leaf in leaves:
        path, j = [], leaf
        while j >= 0:
            path.append(j)
            j = int(parent[j])
        path.reverse()
        ref = _causal_decode(np.concatenate([h[:1], h[[a + 1 for a in path]]]), wq, wk, wv,
                             wo, kv[:L], L, Hkv, theta)
        np.testing.assert_allclose(h_out[0], ref[0], rtol=1e-10, atol=1e-10)
        for t, a in enumerate(path):
            np.testing.assert_allclose(h_out[a + 1], ref[t + 1], rtol=1e-10, atol=1e-10)


def test_chain_positions_are_consecutive():
    L = 9
    np.testing.assert_array_equal(ol.positions(np.arange(-1, 5), L), np.arange(L - 1, L + 6))
    tree = np.array([-1, -1, 0, 1, 2])
    np.testing.assert_array_equal(ol.positions(tree, L), [8, 9, 9, 10, 10, 11])


def test_single_node_projection_and_residual():
    """N = 1, L = 1: the root attends to its own cached row only and the node
    to the root row and itself; checked with numpy matmuls written out."""
    rng = np.random.default_rng(3)
    Hq = Hkv = 1
    D, theta = 4, 100.0
    h = rng.normal(0, 1, (2, D))
    wq, wk, wv, wo = (rng.normal(0, 1, (D, D)) for _ in range(4))
    kv = rng.normal(0, 1, (2, 2, 1, D))
    h_out, kv_out, attn = ol.layer_share_sequence(h, wq, wk, wv, wo, kv, 1, np.array([-1]),
                                                  Hkv, theta)
    # root: one key (the cached row 0), so attention returns that row's V
    np.testing.assert_allclose(attn[0, 0], kv[0, 1, 0], atol=1e-12)
    np.testing.assert_allclose(h_out[0], h[0] + kv[0, 1, 0] @ wo.T, atol=1e-12)
    # node: K/V written to row 1 (position 1), V unrotated
    np.testing.assert_allclose(kv_out[1, 1, 0], h[1] @ wv.T, atol=1e-12)
    np.testing.assert_allclose(kv_out[1, 0, 0], ol.rope(h[1] @ wk.T, 1, theta), atol=1e-12)
