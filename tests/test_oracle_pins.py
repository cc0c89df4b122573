"""Pins of the CPU oracle against what the source pages and mathematics fix.

None of these tests retypes the oracle's own formulas: they use the pages'
printed numbers (tests/golden/worked_examples.json), closed forms, the
distribution-preservation theorem checked by exact enumeration and by a
chi-square test, textbook special cases, and brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import verify as ov

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# worked examples printed on the pages
# ---------------------------------------------------------------------------


def test_blog_example_acceptance_numbers():
    g = _golden()["sps_blog_example"]
    t1, t2 = g["tests"]
    # 0.9 vs 0.7: accepted whatever the uniform draw is
    for u in np.linspace(0.0, 1.0, 1001)[:-1]:
        assert ov.accept_test(t1["p"], t1["q"], u)
    # 0.2 vs 0.8: accepted exactly on u <= 0.25; the printed r = 0.6 rejects
    assert ov.accept_test(t2["p"], t2["q"], t2["acceptance"])
    assert not ov.accept_test(t2["p"], t2["q"], np.nextafter(t2["acceptance"], 1.0))
    assert ov.accept_test(t2["p"], t2["q"], t2["u"]) == t2["accepted"]
    frac = np.mean([ov.accept_test(t2["p"], t2["q"], u)
                    for u in (np.arange(100000) + 0.5) / 100000])
    assert abs(frac - t2["acceptance"]) < 1e-4


def _chain_round_from_probs(p_rows, q_rows, tokens, u):
    """Run the oracle on a chain whose per-slot distributions are given as
    probabilities: logits log(p) at T = 1 reproduce p."""
    zt = np.log(np.asarray(p_rows, dtype=np.float64))
    zd = np.log(np.asarray(q_rows, dtype=np.float64))
    parent = np.arange(-1, len(tokens) - 1)
    return ov.verify_round(zt, zd, parent, tokens, u, 1.0)


def test_blog_example_round():
    g = _golden()["sps_blog_example"]
    # tokens: 0 "ren", 1 "gong", 2 "zhineng", 3 "lei" (the corrected token);
    # slot 1's residual max(0, p - q) is one-hot on token 3, which forces the
    # resample the example describes.
    p = [[0.90, 0.05, 0.03, 0.02], [0.05, 0.20, 0.05, 0.70], [0.25] * 4, [0.25] * 4]
    q = [[0.70, 0.10, 0.10, 0.10], [0.05, 0.80, 0.05, 0.10], [0.25] * 4, [0.25] * 4]
    for u0 in (0.0, 0.5, 0.999):
        for u_final in (0.0, 0.37, 0.999):
            r = _chain_round_from_probs(p, q, [0, 1, 2], [u0, g["tests"][1]["u"], 0.1, u_final])
            assert r.path == [0]
            assert r.emitted == [0, 3]
            assert len(r.emitted) == g["emitted"]
            assert abs(r.tests[1].ratio - g["tests"][1]["acceptance"]) < 1e-12


def test_eagle3_article_example_round():
    g = _golden()["eagle3_article_example"]
    # tokens: 0 "help", 1 "you", 2 "?", 3 "with"; slot 2's residual is
    # one-hot on "with".
    p = [[0.38, 0.30, 0.20, 0.12], [0.20, 0.45, 0.20, 0.15], [0.10, 0.10, 0.12, 0.68],
         [0.25] * 4]
    q = [[0.35, 0.30, 0.20, 0.15], [0.20, 0.42, 0.20, 0.18], [0.15, 0.15, 0.55, 0.15],
         [0.25] * 4]
    r = _chain_round_from_probs(p, q, [0, 1, 2], [0.99, 0.99, 0.5, 0.3])
    assert r.path == [0, 1]
    assert len(r.path) == g["tau"]
    assert r.emitted == [0, 1, 3]
    assert len(r.emitted) == g["emitted"]
    for test, printed in zip(r.tests, g["tests"]):
        alpha = min(1.0, test.ratio)
        assert round(alpha, 2) == pytest.approx(printed["acceptance"])
    assert r.tests[2].accepted is False


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------


def _rand_dist(rng, V, scale=2.0):
    z = rng.normal(0, scale, V)
    e = np.exp(z - z.max())
    return e / e.sum()


def test_residual_mass_is_total_variation():
    rng = np.random.default_rng(1)
    for _ in range(50):
        V = int(rng.integers(2, 300))
        p, q = _rand_dist(rng, V), _rand_dist(rng, V)
        new_p, Z, ok = ov.residual(p, q)
        assert ok
        assert Z == pytest.approx(0.5 * np.abs(p - q).sum(), abs=1e-12)
        assert Z == pytest.approx(1.0 - np.minimum(p, q).sum(), abs=1e-12)
        assert new_p.sum() == pytest.approx(1.0, abs=1e-12)
        # the residual lives where the target exceeds the draft
        assert np.all(new_p[p <= q] == 0)


def test_first_acceptance_probability_is_overlap():
    rng = np.random.default_rng(2)
    V = 50
    p, q = _rand_dist(rng, V), _rand_dist(rng, V)
    n = 200000
    xs = rng.choice(V, size=n, p=q)
    us = rng.random(n)
    acc = np.mean([ov.accept_test(p[x], q[x], u) for x, u in zip(xs, us)])
    expect = np.minimum(p, q).sum()
    sigma = math.sqrt(expect * (1 - expect) / n)
    assert abs(acc - expect) < 5 * sigma


def test_residual_fallback_when_mass_vanishes():
    p = np.array([0.5, 0.5])
    new_p, Z, ok = ov.residual(p, p)
    assert not ok and Z == 0.0
    assert np.array_equal(new_p, p)


# ---------------------------------------------------------------------------
# distribution preservation: exact enumeration with u integrated by bisection
# ---------------------------------------------------------------------------


def _softmax_direct(z, T):
    w = np.exp(np.asarray(z, dtype=np.float64) / T)
    return w / w.sum()


def _threshold(f, lo=0.0, hi=1.0, iters=56):
    """sup{u in [lo, hi) : f(u)} for a predicate true on [lo, t] and false after."""
    if not f(lo):
        return lo
    if f(np.nextafter(hi, 0.0)):
        return hi
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if f(mid):
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _enumerate_outputs(zt, zd, parent, tokens, T, round_fn=None):
    """Exact distribution of (accepted path, emitted tokens) for one round.

    Uses the oracle as a black box: each node test is a threshold in its own
    uniform (accept below, reject above) that bisection locates, and the
    final draw is monotone in the last uniform, so each token's probability
    is the length of its uniform interval. Returns
    {(tuple(path), tuple(emitted)): probability}.
    """
    N = len(parent)
    out = {}

    def run(u):
        if round_fn is not None:
            return round_fn(zt, zd, parent, tokens, u, T)
        return ov.verify_round(zt, zd, parent, tokens, u, T)

    def explore(u, prob, decided):
        r = run(u)
        for t in r.tests:
            if decided[t.node] is None:
                c = t.node

                def acc(x, c=c):
                    uu = list(u)
                    uu[c] = x
                    return any(tt.node == c and tt.accepted for tt in run(uu).tests)

                theta = _threshold(acc)
                for branch, pr in ((True, theta), (False, 1.0 - theta)):
                    if pr <= 0:
                        continue
                    uu = list(u)
                    uu[c] = 0.0 if branch else 0.5 * (theta + 1.0)
                    d2 = list(decided)
                    d2[c] = branch
                    explore(uu, prob * pr, d2)
                return
        # every test on this branch is decided: integrate the final uniform
        V = zt.shape[1]
        edges = []
        for tok in range(V):
            def le(x, tok=tok):
                uu = list(u)
                uu[N] = x
                return run(uu).token <= tok
            edges.append(_threshold(le))
        for tok in range(V):
            width = edges[tok] - (edges[tok - 1] if tok else 0.0)
            if width > 0:
                key = (tuple(r.path), tuple(r.emitted[:-1]) + (tok,))
                out[key] = out.get(key, 0.0) + prob * width

    explore([0.5] * (N + 1), 1.0, [None] * N)
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_exact_enumeration_preserves_target(seed):
    rng = np.random.default_rng(100 + seed)
    V, T = 3, 0.8
    # root with two candidate children; the first of them has two children
    parent = np.array([-1, -1, 0, 0])
    R = len(parent) + 1
    zt = rng.normal(0, 1.5, (R, V))
    zd = rng.normal(0, 1.5, (R, V))
    q = [_softmax_direct(zd[s], T) for s in range(R)]
    first = np.zeros(V)
    second = {0: np.zeros(V), 1: np.zeros(V)}
    mass = {0: 0.0, 1: 0.0}
    # children are i.i.d. draws from their parent slot's q
    for x0 in range(V):
        for x1 in range(V):
            for x2 in range(V):
                for x3 in range(V):
                    tokens = [x0, x1, x2, x3]
                    w = q[0][x0] * q[0][x1] * q[1][x2] * q[1][x3]
                    for (path, emitted), pr in _enumerate_outputs(zt, zd, parent, tokens,
                                                                  T).items():
                        first[emitted[0]] += w * pr
                        if path:
                            mass[path[0]] += w * pr
                            second[path[0]][emitted[1]] += w * pr
    assert first.sum() == pytest.approx(1.0, abs=1e-9)
    # the first emitted token follows the target distribution at the root
    np.testing.assert_allclose(first, _softmax_direct(zt[0], T), atol=1e-9)
    # given that root child c was accepted, the next token follows slot c+1
    for node in (0, 1):
        assert mass[node] > 1e-6
        np.testing.assert_allclose(second[node] / mass[node],
                                   _softmax_direct(zt[node + 1], T), atol=1e-8)


# ---------------------------------------------------------------------------
# distribution preservation: chi-square over seeded rounds
# ---------------------------------------------------------------------------


def _chi_square_first_token(zt, zd, parent, T, rounds, seed):
    rng = np.random.default_rng(seed)
    V = zt.shape[1]
    N = len(parent)
    q = [_softmax_direct(zd[s], T) for s in range(N + 1)]
    counts = np.zeros(V)
    for _ in range(rounds):
        tokens = [int(rng.choice(V, p=q[int(parent[j]) + 1])) for j in range(N)]
        u = rng.random(N + 1)
        r = ov.verify_round(zt, zd, parent, tokens, u, T)
        assert 1 <= len(r.emitted) <= N + 1
        counts[r.emitted[0]] += 1
    expected = _softmax_direct(zt[0], T) * rounds
    # pool bins with expected count below 5
    order = np.argsort(expected)
    obs, exp = [], []
    acc_o = acc_e = 0.0
    for i in order:
        acc_o += counts[i]
        acc_e += expected[i]
        if acc_e >= 5:
            obs.append(acc_o)
            exp.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0:
        obs[-1] += acc_o
        exp[-1] += acc_e
    return stats.chisquare(obs, exp).pvalue


def test_chi_square_tree_v32():
    rng = np.random.default_rng(7)
    V, T = 32, 1.0
    # four candidates at the root, depth 2
    parent = np.array([-1, -1, -1, -1, 0, 0, 1, 2])
    zt = rng.normal(0, 1.0, (len(parent) + 1, V))
    zd = zt + rng.normal(0, 1.0, zt.shape)
    assert _chi_square_first_token(zt, zd, parent, T, 40000, seed=11) >= 1e-3


def test_chi_square_chain_shape_v1024():
    rng = np.random.default_rng(8)
    V, T = 1024, 1.0
    parent = np.array([-1, 0, 1, 2])
    zt = rng.normal(0, 1.28, (5, V))
    zd = rng.normal(0, 2.0, (5, V))
    assert _chi_square_first_token(zt, zd, parent, T, 10000, seed=12) >= 1e-3


# ---------------------------------------------------------------------------
# token-count bounds and greedy
# ---------------------------------------------------------------------------


def _random_tree(rng, n):
    return np.array([int(rng.integers(-1, j)) for j in range(n)])


def test_token_count_bounds():
    rng = np.random.default_rng(3)
    for _ in range(300):
        N = int(rng.integers(0, 12))
        V = int(rng.integers(2, 40))
        parent = _random_tree(rng, N)
        T = float(rng.choice([0.0, 0.5, 1.0, 2.0]))
        zt = rng.normal(0, 2, (N + 1, V))
        zd = zt + rng.normal(0, 0.5, (N + 1, V))
        tokens = rng.integers(0, V, N)
        r = ov.verify_round(zt, zd, parent, tokens, rng.random(N + 1), T)
        depth_max = max([ov.depth_of(parent, j) for j in range(N)], default=0)
        assert 1 <= len(r.emitted) <= depth_max + 1
        # the accepted nodes form a root-to-node path
        prev = -1
        for c in r.path:
            assert parent[c] == prev
            prev = c
        if np.array_equal(parent, np.arange(-1, N - 1)):
            assert len(r.emitted) <= N + 1      # at most gamma + 1 on a chain


def test_greedy_follows_planted_argmax():
    rng = np.random.default_rng(4)
    V, N = 50, 12
    parent = np.array([-1, -1, -1, 0, 0, 1, 3, 3, 6, 6, 2, 8])
    R = N + 1
    planted = [(7 * s + 3) % V for s in range(R)]
    zt = rng.normal(0, 1, (R, V))
    for s in range(R):
        zt[s, planted[s]] = 10.0
    # children whose token matches the planted maximum of their parent slot:
    # node 1 (slot 0), node 3 (slot 2), node 8 (slot 7); others differ
    tokens = [(planted[int(parent[j]) + 1] + 1) % V for j in range(N)]
    tokens[1] = planted[0]
    tokens[2] = planted[0]          # a later sibling with the same token
    tokens[5] = planted[2]
    r = ov.verify_round(zt, zt, parent, tokens, np.zeros(N + 1), 0.0)
    assert r.path == [1, 5]
    assert r.emitted == [planted[0], planted[2], planted[6]]


def test_equal_draft_and_target_accepts_first_child_to_a_leaf():
    rng = np.random.default_rng(5)
    V, N = 20, 9
    parent = np.array([-1, -1, 0, 0, 2, 1, 4, 4, 3])
    z = rng.normal(0, 1, (N + 1, V))
    tokens = rng.integers(0, V, N)
    u = rng.random(N + 1) * 0.999
    r = ov.verify_round(z, z, parent, tokens, u, 1.0)
    kids = {}
    for j, p in enumerate(parent):
        kids.setdefault(int(p), []).append(j)
    expect, s = [], -1
    while s in kids:
        s = kids[s][0]
        expect.append(s)
    assert r.path == expect


def test_argmax_ties_lowest_index():
    a, gap = ov.argmax_lowest([1.0, 3.0, 2.0, 3.0])
    assert a == 1 and gap == 0.0


# ---------------------------------------------------------------------------
# textbook special cases
# ---------------------------------------------------------------------------


def test_no_nodes_is_plain_sampling():
    rng = np.random.default_rng(6)
    for _ in range(200):
        V = int(rng.integers(1, 200))
        T = float(rng.choice([0.3, 1.0, 1.7]))
        z = rng.normal(0, 2, (1, V))
        u = float(rng.random())
        r = ov.verify_round(z, z, np.zeros(0, dtype=int), [], [u], T)
        p = _softmax_direct(z[0], T)
        c = np.cumsum(p)
        expect = min(int(np.searchsorted(c, u * c[-1], side="right")), V - 1)
        assert r.path == [] and r.token == expect


def _textbook_chain(zt, zd, tokens, u, T):
    """Standard speculative sampling on a chain, in the blog's step order:
    test r_i <= p_i(x_i)/q_i(x_i) in turn; on the first rejection resample from
    norm(max(0, p - q)); if all gamma pass, draw the bonus from p_{gamma+1}."""
    gamma = len(tokens)
    out = []
    for i in range(gamma):
        p = _softmax_direct(zt[i], T)
        q = _softmax_direct(zd[i], T)
        x = tokens[i]
        if u[i] <= p[x] / q[x]:
            out.append(x)
            continue
        r = np.maximum(p - q, 0.0)
        c = np.cumsum(r)
        return out + [int(np.searchsorted(c, u[gamma] * c[-1], side="right"))]
    p = _softmax_direct(zt[gamma], T)
    c = np.cumsum(p)
    return out + [int(np.searchsorted(c, u[gamma] * c[-1], side="right"))]


def test_chain_is_textbook_speculative_sampling():
    rng = np.random.default_rng(9)
    agree = 0
    for _ in range(400):
        gamma = int(rng.integers(1, 7))
        V = int(rng.integers(2, 60))
        T = float(rng.choice([0.5, 1.0, 1.5]))
        zt = rng.normal(0, 1.5, (gamma + 1, V))
        zd = zt + rng.normal(0, 1.0, zt.shape)
        tokens = [int(rng.integers(0, V)) for _ in range(gamma)]
        u = rng.random(gamma + 1)
        r = ov.verify_round(zt, zd, np.arange(-1, gamma - 1), tokens, u, T)
        assert r.emitted == _textbook_chain(zt, zd, tokens, u, T)
        agree += 1
    assert agree == 400


def test_inverse_cdf_clamps_to_last_positive():
    w = np.array([0.2, 0.3, 0.5, 0.0, 0.0])
    t, margin, clamped = ov.inverse_cdf(w, 0.0)
    assert t == 0 and not clamped
    t, _, _ = ov.inverse_cdf(w, 0.2)
    assert t == 1               # cumsum 0.2 is not > 0.2
    # a uniform at (or rounding past) the total picks the last positive entry
    t, _, clamped = ov.inverse_cdf(w, 1.0)
    assert t == 2 and clamped


# ---------------------------------------------------------------------------
# tree attention
# ---------------------------------------------------------------------------


def _causal_attention(q, k, v):
    """Plain causal softmax attention over one contiguous sequence.
    q, k, v: [S, H, D] (k, v already expanded to the query heads)."""
    S, H, D = q.shape
    mask = np.tril(np.ones((S, S), dtype=bool))
    out = np.empty_like(q)
    for h in range(H):
        s = q[:, h] @ k[:, h].T / math.sqrt(D)
        s = np.where(mask, s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        out[:, h] = w @ v[:, h]
    return out


def _leaves(parent):
    has_child = set(int(p) for p in parent)
    return [j for j in range(len(parent)) if j not in has_child]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_attention_equals_causal_attention_per_path(seed):
    rng = np.random.default_rng(20 + seed)
    Hq, Hkv, D, L, N = 4, 2, 8, 6, 9
    parent = _random_tree(rng, N)
    q = rng.normal(0, 1, (N + 1, Hq, D))
    k = rng.normal(0, 1, (L + N, Hkv, D))
    v = rng.normal(0, 1, (L + N, Hkv, D))
    O = ov.tree_attention_sequence(q, k, v, L, parent, Hkv)
    G = Hq // Hkv
    for leaf in _leaves(parent) + ([] if N else [None]):
        path = []
        j = leaf
        while j is not None and j >= 0:
            path.append(j)
            j = int(parent[j])
        path = path[::-1]
        # the sequence: prefix rows, then the path's tree rows; the root token
        # is prefix row L-1, so its query sits at position L-1
        rows = list(range(L)) + [L + a for a in path]
        kk = np.repeat(k[rows], G, axis=1)
        vv = np.repeat(v[rows], G, axis=1)
        qq = np.zeros((len(rows), Hq, D))
        qq[L - 1] = q[0]
        for i, a in enumerate(path):
            qq[L + i] = q[a + 1]
        ref = _causal_attention(qq, kk, vv)
        np.testing.assert_allclose(O[0], ref[L - 1], rtol=1e-12, atol=1e-12)
        for i, a in enumerate(path):
            np.testing.assert_allclose(O[a + 1], ref[L + i], rtol=1e-12, atol=1e-12)


def test_tree_attention_dense_mask_from_closure():
    rng = np.random.default_rng(30)
    Hq, Hkv, D, L, N = 6, 3, 4, 5, 12
    parent = _random_tree(rng, N)
    q = rng.normal(0, 1, (N + 1, Hq, D))
    k = rng.normal(0, 1, (L + N, Hkv, D))
    v = rng.normal(0, 1, (L + N, Hkv, D))
    # ancestor-or-self relation as the transitive closure of the parent matrix
    A = np.eye(N, dtype=bool)
    P = np.zeros((N, N), dtype=bool)
    for j, p in enumerate(parent):
        if p >= 0:
            P[j, p] = True
    for _ in range(N):
        A = A | (A.astype(int) @ P.astype(int) > 0)
    mask = np.zeros((N + 1, L + N), dtype=bool)
    mask[:, :L] = True
    mask[1:, L:] = A
    G = Hq // Hkv
    ref = np.empty((N + 1, Hq, D))
    for h in range(Hq):
        s = q[:, h] @ k[:, h // G].T / math.sqrt(D)
        s = np.where(mask, s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        ref[:, h] = w @ v[:, h // G]
    np.testing.assert_allclose(ov.tree_attention_sequence(q, k, v, L, parent, Hkv), ref,
                               rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# LM head
# ---------------------------------------------------------------------------


def test_lm_head_brute_force_and_one_hot():
    rng = np.random.default_rng(40)
    h = rng.normal(0, 1, (3, 5))
    w = rng.normal(0, 1, (7, 5))
    ref = np.zeros((3, 7))
    for r in range(3):
        for v in range(7):
            acc = 0.0
            for k in range(5):
                acc += h[r, k] * w[v, k]
            ref[r, v] = acc
    np.testing.assert_allclose(ov.lm_head(h, w), ref, rtol=1e-13, atol=1e-13)
    e = np.eye(5)[[2]]
    np.testing.assert_array_equal(ov.lm_head(e, w)[0], w[:, 2])


def test_softmax_recovers_probabilities():
    p = np.array([0.1, 0.2, 0.3, 0.4])
    np.testing.assert_allclose(ov.softmax_t(np.log(p), 1.0), p, atol=1e-15)
    np.testing.assert_allclose(ov.softmax_t(0.7 * np.log(p) + 5.0, 0.7), p, atol=1e-15)


def test_oracle_package_exports():
    assert oracle.verify_round is ov.verify_round
