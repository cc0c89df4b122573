"""Seeded synthetic inputs for the tree-verification step.

This module only draws random inputs and lays them out the way the C ABI
expects them. It holds none of the verification arithmetic (no attention, no
temperature softmax, no acceptance test, no residual, no inverse-CDF draw):
the CPU oracle and the HIP path both consume the arrays returned here, and
neither is imported by this module.

Workloads (shapes follow the model sizes the source pages discuss: 7B/8B/70B
hidden sizes, 32000/128256 vocabularies, 10-60 node trees, batch 1 to 32):

  chain_v1k      chain of 4 drafted tokens (standard speculative sampling),
                 fp32, vocab 1024, hidden 256 = 4 heads x 64, prefix 128.
  eagle1_7b_t0   EAGLE-1 style 10-node tree of depth 3 with 4 root children
  eagle1_7b_t1   (the 10-token / 3-forward tree of "EAGLE" fig. 6), 7B
                 shapes: hidden 4096 = 32x128 MHA, vocab 32000, prefix 1024,
                 bf16; temperature 0 (greedy) and 1.
  gqa_8b         8B GQA shapes: 32 q / 8 kv heads x 128, vocab 128256,
                 prefix 4096, 60-node seeded tree of depth 6, bf16, T = 1;
                 draft logits are the target logits plus N(0, 1) noise.
  share_70b      70B one-layer share: 64 q / 8 kv heads x 128 (hidden 8192),
                 vocab 32000, prefix 2048, 26-node seeded tree of depth 5,
                 head weights N(0, 0.01), T = 0.7.
  batch32_8b     batched serving: 32 sequences with prefixes uniform on
                 [512, 8192], 8B GQA shapes, 60-node depth-6 tree each,
                 T = 0 for the first 16 sequences and 1 for the rest.

Random streams: ``SeedSequence(seed).spawn(B + 1)`` gives PCG64 stream 0 for
the shared head weights and stream 1 + b for everything that belongs to
sequence b, drawn in this fixed order: prefix length (ragged workloads), tree
(seeded trees), node hidden rows, KV rows, draft logits (or their noise),
candidate-token draws, uniforms.

"N(0, s)" is read as mean 0 and standard deviation s. bf16 values are fp32
normals rounded to nearest even and are stored as raw uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
F32 = "f32"

# Children per node in the seeded trees (branching <= 4).
SEEDED_BRANCHING = 4


@dataclass(frozen=True)
class Workload:
    """Shapes and value distributions of one synthetic verification batch."""

    name: str
    batch: int
    n_nodes: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    dtype: str
    prefix: tuple          # ("fixed", L) | ("uniform", lo, hi) | ("list", (L0, L1, ...))
    tree: tuple            # ("chain",) | ("fixed", parents) | ("seeded", depth) | ("star",)
    w_std: float
    draft: tuple           # ("normal", std) | ("perturbed", noise_std)
    temperature: tuple     # ("all", T) | ("split", T_first_half, T_second_half) | ("list", (...))
    hidden_std: float = 1.0
    kv_std: float = 1.0
    children: str = "iid"  # sampled siblings: "iid" (with replacement) | "distinct"
    top_k: int = 0         # drafter and verifier keep the top_k most probable tokens (0 = all)
    top_p: float = 1.0     # then the shortest prefix reaching this mass (1 = all)

    @property
    def hidden(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def rows(self) -> int:
        """Query / LM-head rows per sequence: the root slot plus one per node."""
        return self.n_nodes + 1

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: dict[str, Workload] = {
    "chain_v1k": Workload(
        name="chain_v1k", batch=1, n_nodes=4, n_q_heads=4, n_kv_heads=4, head_dim=64,
        vocab=1024, dtype=F32, prefix=("fixed", 128), tree=("chain",), w_std=0.02,
        draft=("normal", 2.0), temperature=("all", 1.0)),
    "eagle1_7b_t0": Workload(
        name="eagle1_7b_t0", batch=1, n_nodes=10, n_q_heads=32, n_kv_heads=32, head_dim=128,
        vocab=32000, dtype=BF16, prefix=("fixed", 1024),
        tree=("fixed", (-1, -1, -1, -1, 0, 0, 1, 2, 4, 6)), w_std=0.02,
        draft=("normal", 2.0), temperature=("all", 0.0)),
    "eagle1_7b_t1": Workload(
        name="eagle1_7b_t1", batch=1, n_nodes=10, n_q_heads=32, n_kv_heads=32, head_dim=128,
        vocab=32000, dtype=BF16, prefix=("fixed", 1024),
        tree=("fixed", (-1, -1, -1, -1, 0, 0, 1, 2, 4, 6)), w_std=0.02,
        draft=("normal", 2.0), temperature=("all", 1.0)),
    "gqa_8b": Workload(
        name="gqa_8b", batch=1, n_nodes=60, n_q_heads=32, n_kv_heads=8, head_dim=128,
        vocab=128256, dtype=BF16, prefix=("fixed", 4096), tree=("seeded", 6), w_std=0.02,
        draft=("perturbed", 1.0), temperature=("all", 1.0)),
    "share_70b": Workload(
        name="share_70b", batch=1, n_nodes=26, n_q_heads=64, n_kv_heads=8, head_dim=128,
        vocab=32000, dtype=BF16, prefix=("fixed", 2048), tree=("seeded", 5), w_std=0.01,
        draft=("normal", 2.0), temperature=("all", 0.7)),
    "batch32_8b": Workload(
        name="batch32_8b", batch=32, n_nodes=60, n_q_heads=32, n_kv_heads=8, head_dim=128,
        vocab=128256, dtype=BF16, prefix=("uniform", 512, 8192), tree=("seeded", 6),
        w_std=0.02, draft=("perturbed", 1.0), temperature=("split", 0.0, 1.0)),
}


@dataclass
class Inputs:
    """One verification batch, laid out as the C ABI takes it.

    kv           [sum_b (L_b + N), 2, Hkv, D]; for sequence b, rows
                 kv_offset[b] .. kv_offset[b] + L_b - 1 are the prefix (the last
                 of them is the root, the last committed token) and the next N
                 rows are the K/V of the N packed tree nodes.
    node_hidden  [B * (N + 1), d]; row b*(N+1) is the root slot, row
                 b*(N+1) + 1 + j is node j.
    parent       [B * N] int32, -1 = child of the root, else parent[j] < j.
    node_token   [B * N] int32, the drafted token of each node.
    lm_head      [V, d].
    draft_logits [B * (N + 1), V] fp32; row of slot s is the draft distribution
                 that proposed the children of s.
    uniforms     [B * (N + 1)] fp32 in [0, 1): entry j tests node j, entry N
                 drives the final draw.
    temperature  [B] fp32, 0 = greedy.
    bf16 arrays hold raw uint16 bit patterns; fp32 arrays hold float32.
    """

    workload: Workload
    seed: int
    prefix_len: np.ndarray
    kv_offset: np.ndarray
    kv: np.ndarray
    node_hidden: np.ndarray
    parent: np.ndarray
    node_token: np.ndarray
    lm_head: np.ndarray
    draft_logits: np.ndarray
    uniforms: np.ndarray
    temperature: np.ndarray
    max_children: int
    extra: dict = field(default_factory=dict)

    @property
    def max_prefix(self) -> int:
        return int(self.prefix_len.max())


# ----------------------------------------------------------------------------
# bf16 storage helpers (data format only)
# ----------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, nearest-even, returning uint16 bit patterns.

    Inputs are finite normals, so no NaN special-casing is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 values (exact for both bf16 and fp32 storage)."""
    if dtype == BF16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x32) if dtype == BF16 else np.ascontiguousarray(x32, dtype=np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# ----------------------------------------------------------------------------
# trees
# ----------------------------------------------------------------------------

def chain_tree(n: int) -> np.ndarray:
    return np.arange(-1, n - 1, dtype=np.int32)


def seeded_tree(rng: np.random.Generator, n: int, depth: int,
                branching: int = SEEDED_BRANCHING) -> np.ndarray:
    """Random tree with exactly `depth` levels of nodes and <= `branching` children per node.

    A spine of `depth` nodes is laid first (so the depth is reached), then each
    further node hangs from a uniformly chosen eligible parent (the root
    included): one of depth below `depth` with fewer than `branching` children.
    Nodes are then renumbered level by level (breadth-first, creation order
    within a level), which makes parent[j] < j.
    """
    if n < depth:
        raise ValueError("a tree of depth %d needs at least %d nodes" % (depth, depth))
    # creation-order arrays; parent index -1 is the root, whose depth is 0
    par = []
    dep = []
    kids = {-1: 0}
    for i in range(depth):
        p = i - 1
        par.append(p)
        dep.append(i + 1)
        kids[p] = kids.get(p, 0) + 1
        kids[i] = 0
    while len(par) < n:
        eligible = [-1] if kids[-1] < branching else []
        eligible += [i for i in range(len(par)) if dep[i] < depth and kids[i] < branching]
        p = eligible[int(rng.integers(len(eligible)))]
        i = len(par)
        par.append(p)
        dep.append(1 if p < 0 else dep[p] + 1)
        kids[p] += 1
        kids[i] = 0
    order = sorted(range(n), key=lambda i: (dep[i], i))
    new_id = {old: new for new, old in enumerate(order)}
    out = np.empty(n, dtype=np.int32)
    for old in range(n):
        p = par[old]
        out[new_id[old]] = -1 if p < 0 else new_id[p]
    return out


def children_count(parent: np.ndarray) -> np.ndarray:
    """Children per slot (slot 0 = root, slot j + 1 = node j)."""
    cnt = np.zeros(len(parent) + 1, dtype=np.int64)
    for p in parent:
        cnt[int(p) + 1] += 1
    return cnt


# ----------------------------------------------------------------------------
# candidate tokens (the drafter's choices, emulated)
# ----------------------------------------------------------------------------

def _kept_tokens(z: np.ndarray, temperature: float, top_k: int, top_p: float) -> np.ndarray:
    """Mask of the tokens a top-k / top-p drafter can emit from logits z:
    ranked by logit (ties to the lower id), the first top_k, then the
    shortest prefix whose tempered mass reaches top_p of theirs."""
    z = z.astype(np.float64)
    order = np.argsort(-z, kind="stable")
    if 0 < top_k < len(z):
        order = order[:top_k]
    if 0.0 < top_p < 1.0:
        c = np.cumsum(np.exp((z[order] - z[order[0]]) / temperature))
        order = order[:int(np.searchsorted(c, top_p * c[-1], side="left")) + 1]
    mask = np.zeros(len(z), dtype=bool)
    mask[order] = True
    return mask


def _draw_tokens(rng: np.random.Generator, zd: np.ndarray, parent: np.ndarray,
                 temperature: float, distinct: bool = False, top_k: int = 0,
                 top_p: float = 1.0) -> np.ndarray:
    """Drafted token of each node, from the draft logits of its parent slot.

    Greedy (T = 0): the children of a slot, in ascending index, take the top-k
    distinct tokens of that slot's draft logits in descending order (ties:
    lower index first). Sampling (T > 0): every child is an independent draw
    from the tempered draft distribution, obtained with the Gumbel-max trick
    (argmax of logits / T plus standard Gumbel noise), so siblings are i.i.d.
    with replacement. With `distinct`, the children of a slot are an ordered
    sample without replacement instead: one Gumbel perturbation per slot,
    the k largest perturbed logits in descending order (the Gumbel top-k
    trick), the i-th child taking the i-th. With top_k / top_p, sampled draws
    come from the draft distribution restricted to its kept tokens.
    """
    n = len(parent)
    tok = np.empty(n, dtype=np.int32)
    warped = temperature > 0.0 and (0 < top_k < zd.shape[1] or 0.0 < top_p < 1.0)
    logit_cache = {}

    def tempered(s):
        if s not in logit_cache:
            lt = zd[s].astype(np.float64) / temperature
            if warped:
                lt = np.where(_kept_tokens(zd[s], temperature, top_k, top_p), lt, -np.inf)
            logit_cache[s] = lt
        return logit_cache[s]

    if temperature == 0.0:
        order_cache = {}
        used = {}
        for j in range(n):
            s = int(parent[j]) + 1
            if s not in order_cache:
                order_cache[s] = np.argsort(-zd[s].astype(np.float64), kind="stable")
                used[s] = 0
            tok[j] = order_cache[s][used[s]]
            used[s] += 1
    elif not distinct:
        V = zd.shape[1]
        for j in range(n):
            s = int(parent[j]) + 1
            u = rng.random(V)
            # uniform in (0, 1): guard the (probability ~2^-53) zero draw
            u = np.maximum(u, np.finfo(np.float64).tiny)
            g = -np.log(-np.log(u))
            tok[j] = int(np.argmax(tempered(s) + g))
    else:
        V = zd.shape[1]
        order = {}
        used = {}
        for j in range(n):
            s = int(parent[j]) + 1
            if s not in order:
                u = np.maximum(rng.random(V), np.finfo(np.float64).tiny)
                g = -np.log(-np.log(u))
                order[s] = np.argsort(-(tempered(s) + g), kind="stable")
                used[s] = 0
            tok[j] = order[s][used[s]]
            used[s] += 1
    return tok


# ----------------------------------------------------------------------------
# the generator
# ----------------------------------------------------------------------------

def _temperatures(wl: Workload) -> np.ndarray:
    kind = wl.temperature[0]
    if kind == "all":
        return np.full(wl.batch, wl.temperature[1], dtype=np.float32)
    if kind == "split":
        t = np.full(wl.batch, wl.temperature[2], dtype=np.float32)
        t[: wl.batch // 2] = wl.temperature[1]
        return t
    if kind == "list":
        t = np.asarray(wl.temperature[1], dtype=np.float32)
        assert t.shape == (wl.batch,)
        return t
    raise ValueError(kind)


def generate(wl: Workload | str, seed: int = 0, draft_matmul=None) -> Inputs:
    """Draw one verification batch for workload `wl` from `seed`.

    `draft_matmul(h32, w32) -> z32`, if given, replaces the host fp32 product
    used to build perturbed draft logits (for instance a device matmul when the
    host is slow); any faithful fp32 product serves, since the draft logits are
    an input that both sides of a comparison receive identically.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    B, N, R, d, V = wl.batch, wl.n_nodes, wl.rows, wl.hidden, wl.vocab
    Hkv, D = wl.n_kv_heads, wl.head_dim
    ss = np.random.SeedSequence(seed)
    streams = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(B + 1)]
    temps = _temperatures(wl)

    # stream 0: shared head weights
    w32 = _normal(streams[0], (V, d), wl.w_std)
    lm_head = _store(w32, wl.dtype)
    w_vals = bf16_bits_to_f32(lm_head) if wl.dtype == BF16 else w32
    del w32

    prefix_len = np.empty(B, dtype=np.int32)
    parents, hidden_rows, kv_parts, draft_rows, tokens, uniforms = [], [], [], [], [], []
    for b in range(B):
        rng = streams[1 + b]
        kind = wl.prefix[0]
        if kind == "fixed":
            L = wl.prefix[1]
        elif kind == "uniform":
            L = int(rng.integers(wl.prefix[1], wl.prefix[2] + 1))
        elif kind == "list":
            L = int(wl.prefix[1][b])
        else:
            raise ValueError(kind)
        prefix_len[b] = L

        tk = wl.tree[0]
        if tk == "chain":
            par = chain_tree(N)
        elif tk == "fixed":
            par = np.asarray(wl.tree[1], dtype=np.int32)
            assert len(par) == N
        elif tk == "seeded":
            par = seeded_tree(rng, N, wl.tree[1])
        elif tk == "star":
            par = np.full(N, -1, dtype=np.int32)
        else:
            raise ValueError(tk)
        parents.append(par)

        h32 = _normal(rng, (R, d), wl.hidden_std)
        h = _store(h32, wl.dtype)
        hidden_rows.append(h)
        kv_parts.append(_store(_normal(rng, (L + N, 2, Hkv, D), wl.kv_std), wl.dtype))

        if wl.draft[0] == "normal":
            zd = _normal(rng, (R, V), wl.draft[1])
        elif wl.draft[0] == "perturbed":
            hv = bf16_bits_to_f32(h) if wl.dtype == BF16 else h32
            if draft_matmul is not None:
                base = np.asarray(draft_matmul(hv, w_vals), dtype=np.float32)
            else:
                base = np.matmul(hv, w_vals.T)
            zd = (base + _normal(rng, (R, V), wl.draft[1])).astype(np.float32)
        else:
            raise ValueError(wl.draft[0])
        draft_rows.append(zd)
        tokens.append(_draw_tokens(rng, zd, par, float(temps[b]), wl.children == "distinct",
                                   wl.top_k, wl.top_p))
        uniforms.append(rng.random(N + 1, dtype=np.float32))

    kv_offset = np.zeros(B + 1, dtype=np.int32)
    kv_offset[1:] = np.cumsum(prefix_len.astype(np.int64) + N)
    parent = np.concatenate(parents).astype(np.int32) if N else np.zeros(0, np.int32)
    max_children = max(1, max(int(children_count(p).max()) for p in parents))
    return Inputs(
        workload=wl, seed=seed, prefix_len=prefix_len, kv_offset=kv_offset,
        kv=np.concatenate(kv_parts, axis=0), node_hidden=np.concatenate(hidden_rows, axis=0),
        parent=parent,
        node_token=np.concatenate(tokens).astype(np.int32) if N else np.zeros(0, np.int32),
        lm_head=lm_head, draft_logits=np.concatenate(draft_rows, axis=0),
        uniforms=np.concatenate(uniforms).astype(np.float32), temperature=temps,
        max_children=max_children)


def workload(name: str, **overrides) -> Workload:
    """A registered workload, optionally with some fields replaced (for tests)."""
    wl = WORKLOADS[name]
    return wl.with_(**overrides) if overrides else wl


def replicate_rounds(inp: Inputs, copies: int, seed: int) -> Inputs:
    """`copies` independent rounds on the same context: sequence 0 of `inp`
    repeated, with fresh candidate tokens (drawn as in `generate`) and fresh
    uniforms per copy from PCG64 streams of SeedSequence(seed)."""
    wl = inp.workload
    N, R = wl.n_nodes, wl.rows
    L = int(inp.prefix_len[0])
    rows_kv = L + N
    streams = [np.random.Generator(np.random.PCG64(s))
               for s in np.random.SeedSequence(seed).spawn(copies)]
    par = inp.parent[:N]
    zd = inp.draft_logits[:R]
    T = float(inp.temperature[0])
    tokens, uniforms = [], []
    for c in range(copies):
        rng = streams[c]
        tokens.append(_draw_tokens(rng, zd, par, T, wl.children == "distinct", wl.top_k,
                                   wl.top_p))
        uniforms.append(rng.random(N + 1, dtype=np.float32))
    new_wl = wl.with_(name=f"{wl.name}_x{copies}", batch=copies, prefix=("list", (L,) * copies),
                      temperature=("all", T))
    kv_offset = np.arange(copies + 1, dtype=np.int32) * rows_kv
    return Inputs(
        workload=new_wl, seed=inp.seed, prefix_len=np.full(copies, L, dtype=np.int32),
        kv_offset=kv_offset, kv=np.concatenate([inp.kv[:rows_kv]] * copies, axis=0),
        node_hidden=np.concatenate([inp.node_hidden[:R]] * copies, axis=0),
        parent=np.tile(par, copies).astype(np.int32),
        node_token=np.concatenate(tokens).astype(np.int32) if N else np.zeros(0, np.int32),
        lm_head=inp.lm_head, draft_logits=np.concatenate([zd] * copies, axis=0),
        uniforms=np.concatenate(uniforms).astype(np.float32),
        temperature=np.full(copies, T, dtype=np.float32), max_children=inp.max_children)
