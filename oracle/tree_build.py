"""CPU oracle for EAGLE-2's context-aware dynamic draft tree: expansion by
global acceptance value, reranking, flattening.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module. The product path
never calls it, and it imports nothing from that path.

Sources (titles of the pages this restates):
  [SPS] "LLM speculative decoding: EAGLE" blog (jingming.pro), sec. 4.2.1: the
        draft model extends every token of the newest layer in one forward,
        so the tree is pruned: each step expands only the top-k tokens of the
        newest layer by global acceptance probability, the product of the
        token probabilities on the path from the root; after expansion all
        draft tokens are reranked and the top-m by value are kept (a pruned
        shallow token can outrank deeper expanded ones), then laid out as one
        sequence with a tree mask.
  [E1]  "EAGLE / EAGLE-2" translated excerpts (modelers.csdn.net), sec. 2.2
        (the draft model's confidence estimates the acceptance rate), sec.
        2.3.1 (expansion: the most promising nodes of the newest layer go
        through the draft model to form the next layer) and sec. 2.3.2
        (reranking: a node's value never exceeds its parent's; among equal
        values the shallower node goes first, so the top-m form a connected
        tree; flatten to one sequence and mask each token to its ancestors).

Readings where the pages are silent:
  - Confidence of a drafted token is its probability under the draft
    distribution at T = 1: q = softmax(draft logits). The root (the last
    committed token) has value 1; a node's value is its parent's value times
    its own confidence.
  - An expanded node contributes the C most probable tokens of its draft
    distribution as children (ties: lower token id first); every child joins
    the tree. The first step expands the root alone.
  - The next layer's expanded nodes are the K children of highest value
    (ties: earlier creation first). Creation order is the order children are
    generated: by expanded node in frontier order, then by child rank.
  - Reranking orders every tree node by value (higher first), then depth
    (shallower first), then creation order, and keeps the first m. The
    flattened sequence is that order; a parent precedes its children in it
    (a child's value never exceeds its parent's, and ties put the shallower
    first), which is the packed order the verification step reads.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Pool:
    """Every node drafted so far, in creation order (pool id = index)."""
    token: list = field(default_factory=list)
    parent: list = field(default_factory=list)   # pool id, -1 = the root
    value: list = field(default_factory=list)
    depth: list = field(default_factory=list)

    def __len__(self):
        return len(self.token)


def softmax(z):
    z = np.asarray(z, dtype=np.float64)
    w = np.exp(z - z.max())
    return w / w.sum()


def top_tokens(z, c: int):
    """The c most probable tokens of one draft distribution (ties: lower id)."""
    z = np.asarray(z, dtype=np.float64)
    # numpy's sort by (-z, token id): the last key is the primary one
    order = np.lexsort((np.arange(len(z)), -z))
    return [int(v) for v in order[:c]]


def expand(pool: Pool, frontier, frontier_logits, n_expand: int, n_children: int):
    """One expansion step.

    frontier: pool ids of the nodes expanded now (-1 = the root); row i of
    frontier_logits is the draft model's next-token logits at frontier[i].
    Appends n_children children per frontier node to the pool and returns the
    pool ids of the next frontier: the n_expand new children of highest value.
    """
    new = []
    for i, f in enumerate(frontier):
        pv = 1.0 if f < 0 else pool.value[f]
        pd = 0 if f < 0 else pool.depth[f]
        q = softmax(frontier_logits[i])
        for tok in top_tokens(frontier_logits[i], n_children):
            pool.token.append(int(tok))
            pool.parent.append(int(f))
            pool.value.append(pv * q[tok])
            pool.depth.append(pd + 1)
            new.append(len(pool) - 1)
    ranked = sorted(new, key=lambda j: (-pool.value[j], j))
    return ranked[:n_expand]


def rerank(pool: Pool, m: int):
    """Pool ids of the kept nodes in flattened order."""
    order = sorted(range(len(pool)), key=lambda j: (-pool.value[j], pool.depth[j], j))
    return order[:m]


def flatten(pool: Pool, kept):
    """parent[] (indices into the flattened sequence, -1 = root) and tokens."""
    where = {j: i for i, j in enumerate(kept)}
    parent = np.array([-1 if pool.parent[j] < 0 else where[pool.parent[j]] for j in kept],
                      dtype=np.int32)
    token = np.array([pool.token[j] for j in kept], dtype=np.int32)
    return parent, token


def build_tree(draft_logits_fn, depth: int, n_expand: int, n_children: int, m: int):
    """The whole construction for one sequence. draft_logits_fn(pool, ids)
    returns the draft model's logits [len(ids), V] at those nodes (-1 = root).
    Returns (pool, kept, parent, token)."""
    pool = Pool()
    frontier = [-1]
    for _ in range(depth):
        logits = draft_logits_fn(pool, frontier)
        frontier = expand(pool, frontier, logits, n_expand, n_children)
        if not frontier:
            break
    kept = rerank(pool, m)
    parent, token = flatten(pool, kept)
    return pool, kept, parent, token
