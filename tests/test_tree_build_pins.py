"""Pins of the EAGLE-2 tree-construction oracle (oracle/tree_build.py).

What fixes them, besides the oracle itself:
  - a kept node's value is recomputed as the product of draft probabilities
    (scipy's softmax) along its root path, re-evaluating the draft model at
    every ancestor;
  - with one expanded node and one child per step the tree is the greedy
    draft chain: each token is numpy's argmax of the draft distribution at
    the previous token;
  - a one-step tree is the root distribution sorted by probability;
  - the example the blog tells (a pruned shallow token outranks deeper
    expanded ones and is kept, the deeper ones dropped);
  - top-m optimality, connectivity, parent-first order, and the tie rules
    (shallower first, then creation order).
"""
import hashlib

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import tree_build as tb

V = 50


def _draft_fn(seed, scale=2.0, vocab=V):
    """A deterministic synthetic draft model: the logits at a node depend
    only on the tokens of its root path."""
    def path_tokens(pool, j):
        toks = []
        while j >= 0:
            toks.append(pool.token[j])
            j = pool.parent[j]
        return tuple(reversed(toks))

    def logits_at(tokens):
        h = hashlib.sha256(repr((seed, tokens)).encode()).digest()
        rng = np.random.default_rng(int.from_bytes(h[:8], "little"))
        return rng.normal(0.0, scale, vocab)

    def fn(pool, ids):
        return np.stack([logits_at(path_tokens(pool, j)) for j in ids])
    fn.logits_at = logits_at
    fn.path_tokens = path_tokens
    return fn


@pytest.mark.parametrize("seed", range(5))
def test_values_are_path_products_of_draft_probabilities(seed):
    fn = _draft_fn(seed)
    pool, kept, parent, token = tb.build_tree(fn, depth=5, n_expand=4, n_children=3, m=25)
    for i, j in enumerate(kept):
        # the flattened path from the root to node i
        path = []
        a = i
        while a >= 0:
            path.append(a)
            a = int(parent[a])
        path.reverse()
        val, prefix = 1.0, ()
        for a in path:
            q = sp_softmax(fn.logits_at(prefix))
            val *= q[token[a]]
            prefix = prefix + (int(token[a]),)
        assert abs(val - pool.value[j]) <= 1e-14 * max(1.0, val)
        assert pool.depth[j] == len(path)


@pytest.mark.parametrize("seed", range(4))
def test_single_expansion_single_child_is_greedy_chain(seed):
    fn = _draft_fn(100 + seed)
    D = 6
    pool, kept, parent, token = tb.build_tree(fn, depth=D, n_expand=1, n_children=1, m=D)
    assert list(parent) == list(range(-1, D - 1))
    prefix = ()
    for i in range(D):
        assert token[i] == int(np.argmax(fn.logits_at(prefix)))
        prefix = prefix + (int(token[i]),)


@pytest.mark.parametrize("m", [1, 3, 7, 12])
def test_one_step_tree_is_sorted_root_distribution(m):
    fn = _draft_fn(7)
    pool, kept, parent, token = tb.build_tree(fn, depth=1, n_expand=3, n_children=7, m=m)
    q = sp_softmax(fn.logits_at(()))
    want = np.argsort(-q, kind="stable")[:min(m, 7)]
    assert list(token) == list(want)
    assert (parent == -1).all()


def test_pruned_shallow_token_outranks_deeper_ones():
    """The blog's example, with numbers: the root's children are A (0.6) and
    B (0.4); only A is expanded (k = 1); A's two children get confidence 0.5
    each (value 0.3). Reranking keeps B (0.4) ahead of A's children."""
    eps = 1e-9

    def fn(pool, ids):
        out = []
        for j in ids:
            z = np.full(4, np.log(eps))
            if j < 0:
                z[0], z[1] = np.log(0.6), np.log(0.4)      # tokens 0 = A, 1 = B
            else:
                z[2], z[3] = np.log(0.5), np.log(0.5)
            out.append(z)
        return np.stack(out)

    pool, kept, parent, token = tb.build_tree(fn, depth=2, n_expand=1, n_children=2, m=3)
    assert list(token) == [0, 1, 2]          # A, B, then A's first child
    assert list(parent) == [-1, -1, 0]
    pool, kept, parent, token = tb.build_tree(fn, depth=2, n_expand=1, n_children=2, m=2)
    assert list(token) == [0, 1]             # both of A's children dropped


@pytest.mark.parametrize("seed", range(6))
def test_rerank_is_top_m_connected_and_parent_first(seed):
    rng = np.random.default_rng(seed)
    fn = _draft_fn(200 + seed, scale=float(rng.uniform(0.5, 3.0)))
    K, C, D = int(rng.integers(1, 5)), int(rng.integers(1, 5)), int(rng.integers(1, 6))
    m = int(rng.integers(1, 30))
    pool, kept, parent, token = tb.build_tree(fn, depth=D, n_expand=K, n_children=C, m=m)
    assert len(kept) == min(m, len(pool))
    kept_set = set(kept)
    vals = np.array(pool.value)
    dropped = [j for j in range(len(pool)) if j not in kept_set]
    if dropped and kept:
        assert min(vals[kept]) >= max(vals[dropped])
    for i, j in enumerate(kept):
        assert parent[i] < i
        pj = pool.parent[j]
        assert (pj < 0 and parent[i] == -1) or (pj in kept_set and kept[parent[i]] == pj)
        if pj >= 0:
            assert pool.value[j] <= pool.value[pj]
    # the expansion frontier of each step was the best of its newest layer
    for d in range(1, D):
        layer = [j for j in range(len(pool)) if pool.depth[j] == d]
        expanded = {pool.parent[j] for j in range(len(pool)) if pool.depth[j] == d + 1}
        if not expanded:
            continue
        best = sorted(layer, key=lambda j: (-pool.value[j], j))[:K]
        assert expanded == set(best)


def test_ties_go_to_shallower_then_earlier():
    # every distribution uniform over 2 tokens: root children 0.5 each, their
    # children 0.25, so values tie within a depth
    def fn(pool, ids):
        return np.zeros((len(ids), 2))
    pool, kept, parent, token = tb.build_tree(fn, depth=3, n_expand=2, n_children=2, m=7)
    depths = [pool.depth[j] for j in kept]
    assert depths == sorted(depths)
    for d in set(depths):
        ids = [j for j in kept if pool.depth[j] == d]
        assert ids == sorted(ids)
    assert list(parent[:2]) == [-1, -1] and list(token[:2]) == [0, 1]


def test_equal_values_across_depths_keep_parents_first():
    # one-hot draft distributions: each first child has confidence exactly 1,
    # so a node and its first child have the same value; the shallower node
    # must come first, which keeps every parent ahead of its children
    def fn(pool, ids):
        z = np.full((len(ids), 4), -np.inf)
        z[:, 1] = 0.0
        return z
    pool, kept, parent, token = tb.build_tree(fn, depth=4, n_expand=1, n_children=2, m=4)
    assert [pool.value[j] for j in kept] == [1.0] * 4
    assert list(parent) == [-1, 0, 1, 2]
    assert list(token) == [1, 1, 1, 1]
