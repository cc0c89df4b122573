"""Pins of the oracle's sampling variant with children drawn without
replacement (oracle/verify.py, without_replacement=True).

  - Exact enumeration: candidate tuples drawn from q without replacement
    (sequential draws, each renormalised over the tokens not yet drawn), with
    every uniform integrated by bisection of the oracle's own decisions (the
    oracle as a black box): the first emitted token follows the target
    distribution, and after an accepted root child the next token follows
    that child's slot.
  - Chi-square over seeded rounds at V = 32 with four root candidates.
  - Special cases: a single child per slot is standard speculative sampling
    (the variant changes nothing), and a rejected token can never be drawn
    afterwards at that slot.
"""
import itertools

import numpy as np
import pytest
from scipy import stats

from oracle import verify as ov

from test_oracle_pins import _enumerate_outputs, _softmax_direct


def _wor(zt, zd, parent, tokens, u, T):
    return ov.verify_round(zt, zd, parent, tokens, u, T, without_replacement=True)


def _seq_prob(q, xs):
    """Probability of drawing the distinct tokens xs in order without replacement."""
    pr, left = 1.0, 1.0
    for x in xs:
        pr *= q[x] / left
        left -= q[x]
    return pr


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_enumeration_without_replacement(seed):
    rng = np.random.default_rng(300 + seed)
    V, T = 4, 0.9
    # three candidates at the root; the first has two children
    parent = np.array([-1, -1, -1, 0, 0])
    R = len(parent) + 1
    zt = rng.normal(0, 1.5, (R, V))
    zd = rng.normal(0, 1.5, (R, V))
    q = [_softmax_direct(zd[s], T) for s in range(R)]
    first = np.zeros(V)
    second = np.zeros(V)
    mass0 = 0.0
    for root in itertools.permutations(range(V), 3):
        for sub in itertools.permutations(range(V), 2):
            tokens = list(root) + list(sub)
            w = _seq_prob(q[0], root) * _seq_prob(q[1], sub)
            for (path, emitted), pr in _enumerate_outputs(zt, zd, parent, tokens, T,
                                                          round_fn=_wor).items():
                first[emitted[0]] += w * pr
                if path and path[0] == 0:
                    mass0 += w * pr
                    second[emitted[1]] += w * pr
    assert first.sum() == pytest.approx(1.0, abs=1e-9)
    np.testing.assert_allclose(first, _softmax_direct(zt[0], T), atol=1e-9)
    assert mass0 > 1e-6
    np.testing.assert_allclose(second / mass0, _softmax_direct(zt[1], T), atol=1e-8)


def test_chi_square_without_replacement_v32():
    rng = np.random.default_rng(17)
    V, T = 32, 1.0
    parent = np.array([-1, -1, -1, -1, 0, 0, 1])
    N = len(parent)
    zt = rng.normal(0, 1.0, (N + 1, V))
    zd = zt + rng.normal(0, 1.0, zt.shape)
    q = [_softmax_direct(zd[s], T) for s in range(N + 1)]
    kids = ov.children_of(parent)
    counts = np.zeros(V)
    rounds = 40000
    draw = np.random.default_rng(18)
    for _ in range(rounds):
        tokens = np.empty(N, dtype=int)
        for s, ch in enumerate(kids):
            if ch:
                tokens[ch] = draw.choice(V, size=len(ch), replace=False, p=q[s])
        r = _wor(zt, zd, parent, tokens, draw.random(N + 1), T)
        counts[r.emitted[0]] += 1
    expected = _softmax_direct(zt[0], T) * rounds
    keep = expected >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    exp = np.append(expected[keep], expected[~keep].sum())
    if exp[-1] == 0:
        obs, exp = obs[:-1], exp[:-1]
    assert stats.chisquare(obs, exp).pvalue >= 1e-3


def test_single_children_are_unchanged():
    rng = np.random.default_rng(5)
    V, T = 50, 0.8
    parent = np.array([-1, 0, 1, 2])
    zt = rng.normal(0, 1.5, (5, V))
    zd = rng.normal(0, 1.5, (5, V))
    for _ in range(200):
        tokens = rng.integers(0, V, 4)
        u = rng.random(5)
        a = ov.verify_round(zt, zd, parent, tokens, u, T)
        b = _wor(zt, zd, parent, tokens, u, T)
        assert a.path == b.path and a.token == b.token


def test_rejected_token_is_never_drawn_again():
    # after rejecting every sibling, the adjusted target gives zero weight to
    # each rejected token (so the final draw never repeats one)
    rng = np.random.default_rng(6)
    V, T = 6, 1.0
    parent = np.array([-1, -1, -1])
    for _ in range(300):
        zt = rng.normal(0, 2.0, (4, V))
        zd = rng.normal(0, 2.0, (4, V))
        tokens = rng.permutation(V)[:3]
        r = _wor(zt, zd, parent, tokens, np.full(4, 0.999999), T)
        if not r.path:
            assert r.token not in set(int(t) for t in tokens)
