"""Pins of the oracle's top-k / top-p warping (oracle/verify.py, warp and the
walk's top_k / top_p).

  - Worked examples computed by hand (tests/golden/warp_examples.txt).
  - top-k equals keeping the k largest by numpy's stable argsort of -p (ties
    to the lower id); top-p equals the shortest prefix of that order whose
    numpy cumsum reaches top_p times the total (searchsorted); top-k then
    top-p equals top-p applied to the renormalised top-k distribution.
  - Special cases: top_k = 1 and a tiny top_p give the argmax one-hot;
    top_k >= V and top_p = 1 give p back unchanged.
  - Distribution preservation with warped p and q: exact enumeration over
    drafted tokens (drawn from the warped q, i.i.d. or without replacement)
    and over every uniform (the oracle as a black box) gives the warped
    target for the first emitted token and, after an accepted child, the
    child's warped target; a chi-square test at V = 32.
"""
import itertools
import math
from pathlib import Path

import numpy as np
import pytest
from scipy import stats

from oracle import verify as ov

from test_oracle_pins import _enumerate_outputs, _softmax_direct

GOLDEN = Path(__file__).parent / "golden" / "warp_examples.txt"


def _order(p):
    return np.argsort(-np.asarray(p, dtype=np.float64), kind="stable")


def _top_k_library(p, k):
    idx = _order(p)[:k]
    out = np.zeros(len(p))
    out[idx] = np.asarray(p)[idx]
    return out / out.sum()


def _top_p_library(p, top_p):
    p = np.asarray(p, dtype=np.float64)
    order = _order(p)
    c = np.cumsum(p[order])
    cut = int(np.searchsorted(c, top_p * c[-1], side="left")) + 1
    out = np.zeros(len(p))
    out[order[:cut]] = p[order[:cut]]
    return out / out.sum()


def _golden():
    cases = []
    for line in GOLDEN.read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        p, k, tp, want, margin = (f.strip() for f in line.split("|"))
        cases.append(([float(x) for x in p.split()], int(k), float(tp),
                      [float(x) for x in want.split()],
                      math.inf if margin == "inf" else float(margin)))
    return cases


@pytest.mark.parametrize("case", _golden())
def test_worked_examples(case):
    p, k, tp, want, margin = case
    got, m = ov.warp_with_margin(np.array(p), k, tp)
    np.testing.assert_allclose(got, want, atol=1e-12)
    if math.isinf(margin):
        assert math.isinf(m)
    else:
        assert m == pytest.approx(margin, abs=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_top_k_is_stable_argsort(seed):
    rng = np.random.default_rng(seed)
    V = 40
    z = rng.integers(-3, 4, V).astype(np.float64)    # many exact ties
    p = _softmax_direct(z, 1.0)
    for k in (1, 2, 5, 17, 39, 40, 100):
        np.testing.assert_allclose(ov.warp(p, k), _top_k_library(p, min(k, V)), atol=1e-15)
        assert np.count_nonzero(ov.warp(p, k)) == min(k, V)


@pytest.mark.parametrize("seed", range(6))
def test_top_p_is_cumsum_searchsorted(seed):
    rng = np.random.default_rng(10 + seed)
    V = 200
    p = _softmax_direct(rng.normal(0, 2.0, V), 1.0)
    for tp in (1e-9, 0.1, 0.5, 0.9, 0.95, 0.999):
        np.testing.assert_allclose(ov.warp(p, 0, tp), _top_p_library(p, tp), atol=1e-15)


@pytest.mark.parametrize("seed", range(4))
def test_top_k_then_top_p_composes(seed):
    rng = np.random.default_rng(20 + seed)
    p = _softmax_direct(rng.normal(0, 1.5, 300), 1.0)
    for k, tp in ((10, 0.5), (50, 0.9), (300, 0.8), (3, 0.2)):
        got = ov.warp(p, k, tp)
        ref = _top_p_library(_top_k_library(p, k), tp)
        np.testing.assert_allclose(got, ref, atol=1e-14)


def test_special_cases():
    rng = np.random.default_rng(3)
    z = rng.normal(0, 1.0, 64)
    z[[5, 9]] = z.max() + 1.0      # a tie for the largest value
    p = _softmax_direct(z, 0.7)
    one_hot = np.zeros(64)
    one_hot[5] = 1.0
    np.testing.assert_array_equal(ov.warp(p, 1), one_hot)
    np.testing.assert_array_equal(ov.warp(p, 0, 1e-12), one_hot)
    assert ov.warp(p) is not None and np.array_equal(ov.warp(p), p)
    assert np.array_equal(ov.warp(p, 0, 1.0), p)
    np.testing.assert_allclose(ov.warp(p, 64), p, atol=1e-15)
    assert math.isinf(ov.warp_with_margin(p, 7)[1])


def _iid_tuples(q, n):
    support = [v for v in range(len(q)) if q[v] > 0]
    for xs in itertools.product(support, repeat=n):
        yield list(xs), float(np.prod([q[x] for x in xs]))


def _wor_tuples(q, n):
    support = [v for v in range(len(q)) if q[v] > 0]
    for xs in itertools.permutations(support, n):
        pr, left = 1.0, 1.0
        for x in xs:
            pr *= q[x] / left
            left -= q[x]
        yield list(xs), pr


@pytest.mark.parametrize("mode,k,tp,wor", [
    ("top_k", 3, 1.0, False), ("top_p", 0, 0.7, False), ("both", 3, 0.8, False),
    ("top_k_wor", 3, 1.0, True), ("top_p_wor", 0, 0.85, True)])
def test_exact_enumeration_preserves_warped_target(mode, k, tp, wor):
    rng = np.random.default_rng(400 + len(mode) + k)
    V, T = 5, 0.9
    # two candidates at the root; the first has two children
    parent = np.array([-1, -1, 0, 0])
    R = len(parent) + 1
    zt = rng.normal(0, 1.0, (R, V))
    zd = zt + rng.normal(0, 0.7, (R, V))     # a draft close enough that supports overlap
    q = [ov.warp(_softmax_direct(zd[s], T), k, tp) for s in range(R)]
    assert min(np.count_nonzero(q[0]), np.count_nonzero(q[1])) >= 2   # two distinct draws exist
    want = [ov.warp(_softmax_direct(zt[s], T), k, tp) for s in range(R)]
    # the warped targets are library top-k / top-p constructions
    for s in range(R):
        ref = _softmax_direct(zt[s], T)
        if k:
            ref = _top_k_library(ref, k)
        if tp < 1.0:
            ref = _top_p_library(ref, tp)
        np.testing.assert_allclose(want[s], ref, atol=1e-14)
    draws = _wor_tuples if wor else _iid_tuples

    def round_fn(zt_, zd_, parent_, tokens_, u_, T_):
        return ov.verify_round(zt_, zd_, parent_, tokens_, u_, T_, without_replacement=wor,
                               top_k=k, top_p=tp)

    first = np.zeros(V)
    second = np.zeros(V)
    mass0 = 0.0
    for root, w0 in draws(q[0], 2):
        for sub, w1 in draws(q[1], 2):
            tokens = root + sub
            for (path, emitted), pr in _enumerate_outputs(zt, zd, parent, tokens, T,
                                                          round_fn=round_fn).items():
                first[emitted[0]] += w0 * w1 * pr
                if path and path[0] == 0:
                    mass0 += w0 * w1 * pr
                    second[emitted[1]] += w0 * w1 * pr
    assert first.sum() == pytest.approx(1.0, abs=1e-9)
    np.testing.assert_allclose(first, want[0], atol=1e-9)
    assert mass0 > 1e-6
    np.testing.assert_allclose(second / mass0, want[1], atol=1e-8)


def test_chi_square_warped_v32():
    rng = np.random.default_rng(27)
    V, T, k, tp = 32, 1.0, 12, 0.9
    parent = np.array([-1, -1, -1, 0, 0, 1])
    N = len(parent)
    zt = rng.normal(0, 1.0, (N + 1, V))
    zd = zt + rng.normal(0, 1.0, zt.shape)
    q = [ov.warp(_softmax_direct(zd[s], T), k, tp) for s in range(N + 1)]
    counts = np.zeros(V)
    rounds = 30000
    draw = np.random.default_rng(28)
    for _ in range(rounds):
        tokens = [int(draw.choice(V, p=q[int(parent[j]) + 1])) for j in range(N)]
        r = ov.verify_round(zt, zd, parent, tokens, draw.random(N + 1), T, top_k=k, top_p=tp)
        counts[r.emitted[0]] += 1
    expected = ov.warp(_softmax_direct(zt[0], T), k, tp) * rounds
    assert counts[expected == 0].sum() == 0        # nothing outside the kept set
    keep = expected >= 5
    obs = np.append(counts[keep], counts[~keep & (expected > 0)].sum())
    exp = np.append(expected[keep], expected[~keep & (expected > 0)].sum())
    if exp[-1] == 0:
        obs, exp = obs[:-1], exp[:-1]
    assert stats.chisquare(obs, exp).pvalue >= 1e-3


def test_walk_margin_is_the_smallest_row_margin():
    rng = np.random.default_rng(31)
    V, T, tp = 50, 1.0, 0.9
    parent = np.array([-1, -1, 0])
    zt = rng.normal(0, 1.0, (4, V))
    zd = rng.normal(0, 1.0, (4, V))
    tokens = [int(np.argmax(zd[0])), int(np.argsort(-zd[0])[1]), int(np.argmax(zd[1]))]
    r = ov.verify_round(zt, zd, parent, tokens, np.zeros(4), T, top_p=tp)
    assert r.path == [0, 2]          # u = 0 accepts every first child
    rows = [ov.warp_with_margin(_softmax_direct(zt[s], T), 0, tp)[1] for s in (0, 1, 3)]
    rows += [ov.warp_with_margin(_softmax_direct(zd[s], T), 0, tp)[1] for s in (0, 1)]
    assert r.warp_margin == pytest.approx(min(rows), rel=1e-9)
