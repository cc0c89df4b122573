"""Pins of the oracle's inverse-CDF margin and of its batch forms.

The margin of the final draw decides which final tokens the GPU parity tests
compare; the batch forms (sample_batch, tree_attention, verify_batch) decide
where each sequence's results land in the packed output arrays. Both are
checked here against hand-worked values and against independent per-sequence
calls, never against the GPU.

Sources: "LLM speculative decoding: EAGLE" (jingming.pro), sec. 2.3 (the
rejection step resamples from the normalised residual; greedy decoding takes
the target argmax) and sec. 4.2 (each sequence's tree is packed behind its own
prefix).
"""
import math

import numpy as np
import pytest

from oracle import verify as ov


# ---------------------------------------------------------------------------
# inverse CDF: the chosen index and its margin
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("w,u,t,margin", [
    # CDF of [0.2, 0.3, 0.5] steps at 0.2, 0.5, 1.0
    ([0.2, 0.3, 0.5], 0.45, 1, 0.05),   # 0.45 lies in (0.2, 0.5]: 0.25 above, 0.05 below
    ([0.2, 0.3, 0.5], 0.10, 0, 0.10),   # first bin: distance to 0 and to 0.2
    ([0.2, 0.3, 0.5], 0.70, 2, 0.20),   # last bin: 0.2 above 0.5, 0.3 below 1.0
    ([0.2, 0.3, 0.5], 0.95, 2, 0.05),
    ([0.2, 0.3, 0.5], 0.20, 1, 0.00),   # exactly on a step: "exceeds" moves past it
    ([2.0, 3.0, 5.0], 0.45, 1, 0.05),   # unnormalised weights: margin relative to the sum
    ([0.0, 4.0, 0.0, 4.0], 0.5, 3, 0.0),  # on the step between the two positive bins
    ([0.0, 4.0, 0.0, 4.0], 0.25, 1, 0.25),
])
def test_inverse_cdf_margin_hand_worked(w, u, t, margin):
    got_t, got_margin, clamped = ov.inverse_cdf(np.array(w), u)
    assert got_t == t and not clamped
    assert got_margin == pytest.approx(margin, abs=1e-15)


def test_inverse_cdf_margin_is_distance_to_nearest_step():
    """The margin equals the distance from u*S to the nearest cumulative sum
    (0 included), over all steps, relative to S; and moving u by less than
    the margin keeps the draw, by a bit more (towards that step) changes it."""
    rng = np.random.default_rng(7)
    for _ in range(300):
        V = int(rng.integers(1, 40))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0.0:
            w[int(rng.integers(0, V))] = 1.0
        u = float(rng.random())
        t, margin, clamped = ov.inverse_cdf(w, u)
        assert not clamped
        S = w.sum()
        steps = np.concatenate([[0.0], np.cumsum(w)])
        nearest = np.abs(steps - u * S).min() / S
        assert margin == pytest.approx(nearest, abs=1e-12)
        # the brute-force draw: count of steps at or below u*S among C(0..V-1)
        assert t == int(np.sum(np.cumsum(w) <= u * S))
        if margin > 1e-9:
            for du in (-0.999 * margin, 0.999 * margin):
                if 0.0 <= u + du < 1.0:
                    assert ov.inverse_cdf(w, u + du)[0] == t
            lo_gap = u * S - (steps[t] if t >= 0 else 0.0)
            hi_gap = steps[t + 1] - u * S
            if lo_gap / S <= hi_gap / S and u - 1.001 * margin >= 0.0:
                assert ov.inverse_cdf(w, u - 1.001 * margin)[0] != t
            elif hi_gap / S < lo_gap / S and u + 1.001 * margin < 1.0:
                assert ov.inverse_cdf(w, u + 1.001 * margin)[0] != t


# ---------------------------------------------------------------------------
# sample_batch: per-sequence offsets and -1 padding, worked by hand
# ---------------------------------------------------------------------------


def test_sample_batch_packing_hand_example():
    """Two sequences of N = 3 nodes over V = 4 tokens.

    Sequence 0, greedy. Tree: node 0 and node 2 are root children, node 1 is
    node 0's child; tokens [2, 1, 3]. Root argmax 2 = node 0's token (accept),
    slot 1 argmax 1 = node 1's token (accept), slot 2 (node 1, a leaf) argmax
    3 is the corrected token: path [0, 1], emitted [2, 1, 3].

    Sequence 1, T = 1. Tree: nodes 0 and 1 are root children, node 2 is node
    0's child; tokens [0, 1, 2]. Root p = [0.1, 0.6, 0.2, 0.1], q = [0.7, 0.1,
    0.1, 0.1]. Node 0 (x = 0): p/q = 1/7 < u = 0.5, rejected; residual
    max(0, p - q) = [0, 0.5, 0.1, 0], mass 0.6, so p becomes [0, 5/6, 1/6, 0].
    Node 1 (x = 1): (5/6)/0.1 > 1, accepted. Slot 2 (node 1) is a leaf: the
    bonus draw from its p = uniform with u[3] = 0.6 gives token 2 (cumulative
    0.25, 0.5, 0.75 > 0.6). Path [1], emitted [1, 2].
    """
    N, V = 3, 4
    R = N + 1
    parent = np.array([-1, 0, -1, -1, -1, 0], dtype=np.int32)
    tokens = np.array([2, 1, 3, 0, 1, 2], dtype=np.int32)
    zt = np.zeros((2 * R, V))
    zd = np.zeros((2 * R, V))
    zt[0] = [0.0, 1.0, 5.0, 2.0]        # seq 0 root: argmax 2
    zt[1] = [0.0, 3.0, 1.0, 2.0]        # seq 0 slot 1: argmax 1
    zt[2] = [0.0, 1.0, 2.0, 4.0]        # seq 0 slot 2: argmax 3
    zt[R + 0] = np.log([0.1, 0.6, 0.2, 0.1])
    zd[R + 0] = np.log([0.7, 0.1, 0.1, 0.1])
    zt[R + 2] = np.log([0.25, 0.25, 0.25, 0.25])
    u = np.array([0.3, 0.3, 0.3, 0.3, 0.5, 0.9, 0.3, 0.6])
    temperature = np.array([0.0, 1.0])
    rounds, acc_len, acc_path, out_tok = ov.sample_batch(zt, zd, parent, tokens, u, temperature, N)
    assert rounds[0].path == [0, 1] and rounds[0].emitted == [2, 1, 3]
    assert rounds[1].path == [1] and rounds[1].emitted == [1, 2]
    assert [t.accepted for t in rounds[1].tests] == [False, True]
    assert rounds[1].tests[0].ratio == pytest.approx(1.0 / 7.0, rel=1e-12)
    assert rounds[1].residual_norms[0] == [pytest.approx(0.6, rel=1e-12)]
    np.testing.assert_array_equal(acc_len, [2, 1])
    np.testing.assert_array_equal(acc_path, [0, 1, -1, 1, -1, -1])
    np.testing.assert_array_equal(out_tok, [2, 1, 3, -1, 1, 2, -1, -1])


# ---------------------------------------------------------------------------
# batch forms against independent per-sequence calls
# ---------------------------------------------------------------------------


def _random_tree(rng, n):
    return np.array([int(rng.integers(-1, j)) for j in range(n)], dtype=np.int32)


def _per_sequence_problems(seed):
    """Three sequences with different prefix lengths, each built on its own
    arrays: queries [R, Hq, D], keys/values [L + N, Hkv, D], tree, tokens."""
    rng = np.random.default_rng(seed)
    N, Hq, Hkv, D, V = 5, 4, 2, 8, 11
    R = N + 1
    seqs = []
    for L in (1, 4, 9):
        seqs.append({
            "L": L,
            "q": rng.normal(0, 1, (R, Hq * D)),
            "k": rng.normal(0, 1, (L + N, Hkv, D)),
            "v": rng.normal(0, 1, (L + N, Hkv, D)),
            "parent": _random_tree(rng, N),
            "tokens": rng.integers(0, V, N).astype(np.int32),
            "zd": rng.normal(0, 2, (R, V)),
            "u": rng.random(R),
        })
    w = rng.normal(0, 0.3, (V, Hq * D))
    return seqs, w, (N, Hq, Hkv, D, V)


def _pack(seqs):
    kv = np.concatenate([np.stack([s["k"], s["v"]], axis=1) for s in seqs])
    lens = [s["L"] for s in seqs]
    N = len(seqs[0]["parent"])
    kv_offset = np.concatenate([[0], np.cumsum([L + N for L in lens])]).astype(np.int32)
    return {
        "kv": kv, "kv_offset": kv_offset, "prefix_len": np.array(lens, dtype=np.int32),
        "hidden": np.concatenate([s["q"] for s in seqs]),
        "parent": np.concatenate([s["parent"] for s in seqs]),
        "tokens": np.concatenate([s["tokens"] for s in seqs]),
        "zd": np.concatenate([s["zd"] for s in seqs]),
        "u": np.concatenate([s["u"] for s in seqs]),
    }


def test_tree_attention_batch_slices_per_sequence():
    seqs, _, (N, Hq, Hkv, D, _) = _per_sequence_problems(3)
    R = N + 1
    pk = _pack(seqs)
    out = ov.tree_attention(pk["hidden"], pk["kv"], pk["kv_offset"], pk["prefix_len"],
                            pk["parent"], N, Hq, Hkv, D)
    assert out.shape == (len(seqs) * R, Hq, D)
    for b, s in enumerate(seqs):
        ref = ov.tree_attention_sequence(s["q"].reshape(R, Hq, D), s["k"], s["v"], s["L"],
                                         s["parent"], Hkv)
        np.testing.assert_array_equal(out[b * R:(b + 1) * R], ref)


@pytest.mark.parametrize("temps", [(1.0, 0.0, 0.7), (0.0, 0.0, 0.0), (1.3, 1.0, 2.0)])
def test_verify_batch_slices_per_sequence(temps):
    seqs, w, (N, Hq, Hkv, D, V) = _per_sequence_problems(4)
    R = N + 1
    pk = _pack(seqs)
    T = np.array(temps)
    res = ov.verify_batch(pk["hidden"], pk["kv"], pk["kv_offset"], pk["prefix_len"], pk["parent"],
                          pk["tokens"], w, pk["zd"], pk["u"], T, N, Hq, Hkv, D)
    for b, s in enumerate(seqs):
        rows = slice(b * R, (b + 1) * R)
        o = ov.tree_attention_sequence(s["q"].reshape(R, Hq, D), s["k"], s["v"], s["L"],
                                       s["parent"], Hkv)
        np.testing.assert_array_equal(res.attn_out[rows], o)
        z = s["q"] @ w.T
        np.testing.assert_allclose(res.logits[rows], z, rtol=1e-13, atol=1e-13)
        r = ov.verify_round(z, s["zd"], s["parent"], s["tokens"], s["u"], float(T[b]))
        assert res.rounds[b].path == r.path and res.rounds[b].token == r.token
        n = len(r.path)
        assert res.accept_len[b] == n
        np.testing.assert_array_equal(res.accept_path[b * N:(b + 1) * N],
                                      r.path + [-1] * (N - n))
        np.testing.assert_array_equal(res.out_tokens[rows], r.emitted + [-1] * (R - n - 1))
        assert 1 <= len(r.emitted) <= N + 1
        assert math.isfinite(r.final_margin) or T[b] == 0.0
