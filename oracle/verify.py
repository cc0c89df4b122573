"""CPU oracle for the verification stage of tree speculative sampling.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module. The product path
(the HIP library behind include/specverify.h) never calls it, and this module
imports nothing from that path: it shares no kernels, helpers, tables or
constants with it. Every function is a plain, slow, fp64 numpy transcription
of what the source pages state, with the steps in the pages' order.

Sources (titles of the pages this restates):
  [SPS]  "LLM speculative decoding: EAGLE" blog (jingming.pro), sec. 2.2-2.4
         (speculative sampling: accept with probability min(1, p/q), on
         rejection resample from norm(max(0, p - q)), bonus draw from
         p_{gamma+1}, 1 to gamma+1 tokens per round, worked example), and
         sec. 4.2 (packing the draft tree into one sequence; the attention
         mask lets a node see the prefix and its own ancestors only).
  [E1]   "EAGLE / EAGLE-2" translated excerpts (modelers.csdn.net), sec. 1.3.2
         (one target forward with tree attention, then recursive speculative
         sampling at every node, SpecInfer-style), sec. 1.7 (multi-round
         speculative sampling: after a rejection the sampler is invoked again
         on the next candidate; only when all candidates are rejected is the
         adjusted distribution sampled; greedy mode takes top-k children),
         sec. 2.3.2 (flatten to 1-D, ancestor-only attention mask).
  [EQ]   "EAGLE (ICML 2024) close reading" (edgeai1.github.io), sec. 3
         (strict speculative sampling per candidate; greedy compares with the
         target argmax) and sec. 5 (fixed-seed statistics, greedy token-by-
         token equality).

Readings where the pages are silent (each is one line of the design notes):
  - Algorithm 1 itself is not printed: after a rejection the adjusted target
    distribution becomes the target for the next sibling, and q stays the
    parent's draft distribution (siblings are i.i.d. draws from q).
  - The ratio test r <= p/q is evaluated as u*q(x) <= p(x) (no division), so
    q(x) = 0 always accepts and a tie accepts.
  - u[j] tests node j; u[N] drives the one final draw; children are tested in
    ascending packed index.
  - A computed residual mass Z <= 0 or non-finite leaves p unchanged and
    flags the round (impossible in exact arithmetic after a rejection).
  - Inverse CDF: the smallest t with cumsum(w)[t] > u * sum(w) on the
    unnormalised weights; if rounding defeats every comparison, the last t
    with w[t] > 0.
  - Argmax ties go to the lowest index. Temperature T divides the logits of
    both p and q; T = 0 means greedy.
  - Top-k / top-p ([SPS] sec. 1 names them among the processing steps whose
    output distribution is preserved, without defining them): p and q get
    the same warping after the temperature; ranks by probability with ties
    to the lower id; top-p is the shortest rank prefix reaching top_p times
    the mass the top-k step kept. Greedy verification is unaffected (the
    argmax is always kept).
  - Children drawn without replacement: the draft distribution is
    renormalised only when another sibling follows; a sibling set that
    exhausts q's support is flagged, not divided by zero.
  - Scores are q.k / sqrt(D); query head h reads KV head h // (Hq / Hkv).
  - The LM head reads each slot's hidden row (not the attention output).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# tree structure  ([SPS] sec. 4.2 "Attention Mask"; [E1] sec. 2.3.2)
# ---------------------------------------------------------------------------


def children_of(parent) -> list:
    """children[s] for slot s: slot 0 is the root (last committed token),
    slot j + 1 is node j. Children are listed in ascending packed index."""
    n = len(parent)
    kids = [[] for _ in range(n + 1)]
    for j in range(n):
        kids[int(parent[j]) + 1].append(j)
    return kids


def ancestors(parent, j: int) -> list:
    """anc(j) = {j} plus the ancestors of parent[j]; the root is not a node."""
    out = []
    while j >= 0:
        out.append(j)
        j = int(parent[j])
    return sorted(out)


def depth_of(parent, j: int) -> int:
    return len(ancestors(parent, j))


# ---------------------------------------------------------------------------
# tree attention  ([SPS] sec. 4.2; [E1] sec. 1.3.2, 2.3.2)
# ---------------------------------------------------------------------------


def tree_attention_sequence(q_rows, k_rows, v_rows, prefix_len, parent, n_kv_heads):
    """Tree attention for one sequence, fp64.

    q_rows : [N + 1, Hq, D]   slot 0 = root, slot j + 1 = node j
    k_rows, v_rows : [L + N, Hkv, D]  rows 0..L-1 prefix (row L-1 = root token),
                     row L + a = node a
    Slot 0 sees prefix rows 0..L-1. Node j sees those and the rows of its
    ancestors, itself included. Returns O [N + 1, Hq, D].
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R, Hq, D = q_rows.shape
    out = np.empty((R, Hq, D), dtype=np.float64)
    for slot in range(R):
        out[slot] = tree_attention_slot(q_rows[slot], k_rows, v_rows, prefix_len, parent, slot,
                                        n_kv_heads)
    return out


def tree_attention_slot(q_slot, k_rows, v_rows, prefix_len, parent, slot, n_kv_heads):
    """Tree attention of one slot, fp64: q_slot [Hq, D], k_rows / v_rows as
    in tree_attention_sequence. Slot 0 sees the prefix; slot j + 1 (node j)
    sees the prefix and the tree rows of node j's ancestors and itself.
    Returns O [Hq, D]."""
    q_slot = np.asarray(q_slot, dtype=np.float64)
    Hq, D = q_slot.shape
    L = int(prefix_len)
    group = Hq // n_kv_heads
    keys = list(range(L))
    if slot > 0:
        keys += [L + a for a in ancestors(parent, slot - 1)]
    K = np.asarray(k_rows[keys], dtype=np.float64)      # [n_keys, Hkv, D]
    V = np.asarray(v_rows[keys], dtype=np.float64)
    out = np.empty((Hq, D), dtype=np.float64)
    for h in range(Hq):
        g = h // group
        scores = K[:, g, :] @ q_slot[h] / math.sqrt(D)
        w = np.exp(scores - scores.max())
        w /= w.sum()
        out[h] = w @ V[:, g, :]
    return out


def tree_attention(node_hidden, kv, kv_offset, prefix_len, parent_all, n_nodes,
                   n_q_heads, n_kv_heads, head_dim):
    """Tree attention over a batch (arrays already widened to float).

    node_hidden [B*(N+1), Hq*D] is read as the queries; kv [rows, 2, Hkv, D].
    Returns O [B*(N+1), Hq, D] fp64.
    """
    B = len(prefix_len)
    R = n_nodes + 1
    out = np.empty((B * R, n_q_heads, head_dim), dtype=np.float64)
    for b in range(B):
        base = int(kv_offset[b])
        L = int(prefix_len[b])
        rows = kv[base: base + L + n_nodes]
        q = np.asarray(node_hidden[b * R:(b + 1) * R], dtype=np.float64).reshape(
            R, n_q_heads, head_dim)
        par = parent_all[b * n_nodes:(b + 1) * n_nodes]
        out[b * R:(b + 1) * R] = tree_attention_sequence(
            q, rows[:, 0], rows[:, 1], L, par, n_kv_heads)
    return out


# ---------------------------------------------------------------------------
# LM head  ([SPS] sec. 3.1: the frozen target head maps a feature to logits)
# ---------------------------------------------------------------------------


def lm_head(hidden, weight):
    """logits[r, v] = sum_k hidden[r, k] * weight[v, k], in fp64."""
    return np.asarray(hidden, dtype=np.float64) @ np.asarray(weight, dtype=np.float64).T


# ---------------------------------------------------------------------------
# speculative sampling pieces  ([SPS] sec. 2.3; [E1] sec. 1.7)
# ---------------------------------------------------------------------------


def softmax_t(z, T: float):
    """Temperature softmax softmax(z / T), max subtracted, fp64."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp((z - z.max()) / T)
    return e / e.sum()


def warp_with_margin(p, top_k: int = 0, top_p: float = 1.0):
    """Top-k / top-p warping of one distribution (reading of "LLM speculative
    decoding: EAGLE" sec. 1: the preserved distribution is the one after the
    temperature, top-k and top-p processing; the draft's q gets the same
    processing, since q must be what the drafted tokens were drawn from).

    Tokens are ranked by probability, ties to the lower id. top_k > 0 keeps
    the first top_k; 0 < top_p < 1 then keeps the shortest prefix of what is
    left whose mass reaches top_p times that mass. The kept probabilities
    are renormalised; everything else is 0. top_k <= 0 and top_p >= 1 leave
    p unchanged (no renormalisation, not even a rounding one).

    Returns (warped, margin): margin is how far the top-p cut lies from
    moving, min(cum_cut - top_p * total, top_p * total - cum_before) with cum
    the running mass in rank order, in units of the largest probability (the
    scale on which a fixed-point mass sum rounds); inf without a top-p cut.
    """
    p = np.asarray(p, dtype=np.float64)
    if top_k <= 0 and not (0.0 < top_p < 1.0):
        return p, math.inf
    order = sorted(range(len(p)), key=lambda v: (-p[v], v))
    keep = order
    if top_k > 0:
        keep = keep[:top_k]
    margin = math.inf
    if 0.0 < top_p < 1.0:
        total = 0.0
        for v in keep:
            total += p[v]
        goal = top_p * total
        acc = 0.0
        cut = len(keep)
        for i, v in enumerate(keep):
            before = acc
            acc += p[v]
            if acc >= goal:
                cut = i + 1
                margin = min(acc - goal, goal - before) / p[order[0]]
                break
        keep = keep[:cut]
    out = np.zeros_like(p)
    idx = np.array(keep, dtype=np.int64)
    out[idx] = p[idx]
    return out / out.sum(), margin


def warp(p, top_k: int = 0, top_p: float = 1.0):
    """The warped distribution alone (see warp_with_margin)."""
    return warp_with_margin(p, top_k, top_p)[0]


def accept_test(p_x: float, q_x: float, u: float) -> bool:
    """Accept the drafted token when r <= p/q, evaluated as u*q <= p."""
    return float(u) * float(q_x) <= float(p_x)


def residual(p, q):
    """Adjusted distribution after a rejection: norm(max(0, p - q)).

    Returns (new_p, Z, ok). If the residual mass Z is not positive and finite
    the distribution is returned unchanged with ok = False.
    """
    r = np.maximum(0.0, np.asarray(p, dtype=np.float64) - np.asarray(q, dtype=np.float64))
    Z = float(r.sum())
    if not (Z > 0.0 and math.isfinite(Z)):
        return np.asarray(p, dtype=np.float64), Z, False
    return r / Z, Z, True


def inverse_cdf(w, u: float):
    """Smallest t with cumsum(w)[t] > u * sum(w); the last t with w[t] > 0 if
    rounding defeats every comparison. Returns (t, margin, clamped) where
    margin = min(u*S - C(t-1), C(t) - u*S) / S measures how far u*S lies from
    the nearest CDF step (fp64)."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    S = float(c[-1])
    target = float(u) * S
    t = -1
    for i in range(len(c)):
        if c[i] > target:
            t = i
            break
    clamped = False
    if t < 0:
        positive = np.nonzero(w > 0)[0]
        t = int(positive[-1]) if len(positive) else len(w) - 1
        clamped = True
    lo = c[t - 1] if t > 0 else 0.0
    margin = min(target - lo, c[t] - target) / S if S > 0 else 0.0
    return t, margin, clamped


def argmax_lowest(z):
    """Index of the largest value, lowest index among ties; also the gap
    between the largest and the second-largest value (inf when V = 1)."""
    z = np.asarray(z, dtype=np.float64)
    a = int(np.argmax(z))          # numpy returns the first maximal index
    if len(z) == 1:
        return a, math.inf
    rest = np.delete(z, a)
    return a, float(z[a] - rest.max())


# ---------------------------------------------------------------------------
# one round on one sequence
# ---------------------------------------------------------------------------


@dataclass
class NodeTest:
    node: int
    slot: int
    rank: int           # 1-based position among the slot's children
    ratio: float        # p_{s,rank-1}(x) / q_s(x) (inf when q_s(x) = 0)
    u: float
    accepted: bool


@dataclass
class RoundResult:
    path: list
    token: int
    path_tokens: list = field(default_factory=list)  # drafted tokens of the accepted nodes
    tests: list = field(default_factory=list)
    visited: list = field(default_factory=list)     # slots whose distribution was used
    final_margin: float = math.inf
    final_clamped: bool = False
    residual_fallback: bool = False
    greedy_gap: float = math.inf                   # min top-2 gap over visited slots
    terminal_slot: int = 0
    terminal_rejections: int = 0
    residual_norms: dict = field(default_factory=dict)   # slot -> [Z_1, Z_2, ...]
    warp_margin: float = math.inf                  # min top-p cut margin over warped rows

    @property
    def emitted(self) -> list:
        """Tokens the round emits: the accepted drafted tokens, then the drawn one."""
        return list(self.path_tokens) + [self.token]


def walk_sampling(zt, zd, parent, tokens, u, T: float,
                  without_replacement: bool = False, top_k: int = 0,
                  top_p: float = 1.0) -> RoundResult:
    """Multi-round speculative sampling down the packed tree, T > 0.

    zt, zd : [N + 1, V] target and draft logits per slot.
    At slot s the target distribution is p = softmax(zt[s]/T) and the draft
    distribution that proposed s's children is q = softmax(zd[s]/T). Each
    child c (ascending index) with token x is accepted when u[c]*q(x) <= p(x);
    the walk then moves to slot c + 1. A rejected child replaces p by
    norm(max(0, p - q)) and the next child is tested against it. When no
    child is accepted (or s is a leaf), one token is drawn from the current p
    with the final uniform u[N].

    without_replacement: the siblings were drawn from q without replacement,
    so after a rejected token x the next sibling's draft distribution is q
    with x removed and renormalised (q <- q * [v != x] / (1 - q(x))); the
    residual step uses the draft distribution the rejected sibling was drawn
    from ("EAGLE / EAGLE-2" excerpts, sec. 1.7: non-greedy children are k
    sampled tokens).

    top_k, top_p: p and q are warped (see warp) before anything else.
    """
    N = len(parent)
    kids = children_of(parent)
    res = RoundResult(path=[], token=-1)
    s = 0
    while True:
        res.visited.append(s)
        p, wm = warp_with_margin(softmax_t(zt[s], T), top_k, top_p)
        res.warp_margin = min(res.warp_margin, wm)
        accepted = None
        norms = []
        if kids[s]:
            q, wm = warp_with_margin(softmax_t(zd[s], T), top_k, top_p)
            res.warp_margin = min(res.warp_margin, wm)
            for rank, c in enumerate(kids[s], start=1):
                x = int(tokens[c])
                ratio = p[x] / q[x] if q[x] > 0 else math.inf
                ok = accept_test(p[x], q[x], u[c])
                res.tests.append(NodeTest(c, s, rank, float(ratio), float(u[c]), ok))
                if ok:
                    accepted = c
                    break
                p, Z, good = residual(p, q)
                norms.append(Z)
                if not good:
                    res.residual_fallback = True
                if without_replacement and rank < len(kids[s]):
                    # the next sibling's draft distribution: x removed, renormalised
                    rest = q.copy()
                    rest[x] = 0.0
                    mass = float(rest.sum())
                    if mass > 0.0:
                        q = rest / mass
                    else:
                        res.residual_fallback = True
        if norms:
            res.residual_norms[s] = norms
        if accepted is not None:
            res.path.append(accepted)
            res.path_tokens.append(int(tokens[accepted]))
            s = accepted + 1
            continue
        res.terminal_slot = s
        res.terminal_rejections = len(norms)
        t, margin, clamped = inverse_cdf(p, u[N])
        res.token = t
        res.final_margin = margin
        res.final_clamped = clamped
        return res


def walk_greedy(zt, parent, tokens) -> RoundResult:
    """Greedy verification (T = 0): at slot s take a = argmax zt[s]; the first
    child (ascending index) whose token is a is accepted and the walk moves
    on; otherwise a is the corrected token."""
    kids = children_of(parent)
    res = RoundResult(path=[], token=-1)
    s = 0
    while True:
        res.visited.append(s)
        a, gap = argmax_lowest(zt[s])
        res.greedy_gap = min(res.greedy_gap, gap)
        nxt = None
        for c in kids[s]:
            if int(tokens[c]) == a:
                nxt = c
                break
        if nxt is None:
            res.token = a
            res.terminal_slot = s
            return res
        res.path.append(nxt)
        res.path_tokens.append(int(tokens[nxt]))
        s = nxt + 1


def verify_round(zt, zd, parent, tokens, u, T: float,
                 without_replacement: bool = False, top_k: int = 0,
                 top_p: float = 1.0) -> RoundResult:
    """One verification round for one sequence (T = 0: greedy, which no
    warping changes: the argmax is always kept)."""
    if T == 0.0:
        return walk_greedy(zt, parent, tokens)
    return walk_sampling(zt, zd, parent, tokens, u, T, without_replacement, top_k, top_p)


# ---------------------------------------------------------------------------
# the whole step over a batch
# ---------------------------------------------------------------------------


@dataclass
class BatchResult:
    attn_out: np.ndarray | None
    logits: np.ndarray | None
    rounds: list
    accept_len: np.ndarray
    accept_path: np.ndarray
    out_tokens: np.ndarray


def sample_batch(logits, draft_logits, parent_all, tokens_all, uniforms, temperature,
                 n_nodes: int, without_replacement: bool = False, top_k: int = 0,
                 top_p: float = 1.0) -> tuple:
    """Rounds for every sequence from given target/draft logits.

    Returns (rounds, accept_len [B], accept_path [B*N] (-1 padded),
    out_tokens [B*(N+1)] (accepted tokens, then the drawn token, -1 padded)).
    """
    B = len(temperature)
    N = n_nodes
    R = N + 1
    rounds = []
    acc_len = np.zeros(B, dtype=np.int32)
    acc_path = np.full(B * N, -1, dtype=np.int32)
    out_tok = np.full(B * R, -1, dtype=np.int32)
    for b in range(B):
        par = parent_all[b * N:(b + 1) * N]
        tok = tokens_all[b * N:(b + 1) * N]
        r = verify_round(logits[b * R:(b + 1) * R], draft_logits[b * R:(b + 1) * R],
                         par, tok, uniforms[b * R:(b + 1) * R], float(temperature[b]),
                         without_replacement, top_k, top_p)
        rounds.append(r)
        acc_len[b] = len(r.path)
        acc_path[b * N: b * N + len(r.path)] = r.path
        em = r.emitted
        out_tok[b * R: b * R + len(em)] = em
    return rounds, acc_len, acc_path, out_tok


def verify_batch(node_hidden, kv, kv_offset, prefix_len, parent, node_token, lm_weight,
                 draft_logits, uniforms, temperature, n_nodes, n_q_heads, n_kv_heads,
                 head_dim, with_attention=True, without_replacement=False, top_k=0,
                 top_p=1.0) -> BatchResult:
    """The full step: tree attention, LM head, speculative sampling (fp64).

    Float arrays must already be widened to float (bf16 storage widened
    exactly); node_hidden serves as the queries and as the LM-head input.
    """
    attn = None
    if with_attention:
        attn = tree_attention(node_hidden, kv, kv_offset, prefix_len, parent, n_nodes,
                              n_q_heads, n_kv_heads, head_dim)
    logits = lm_head(node_hidden, lm_weight)
    rounds, acc_len, acc_path, out_tok = sample_batch(
        logits, np.asarray(draft_logits, dtype=np.float64), parent, node_token, uniforms,
        temperature, n_nodes, without_replacement, top_k, top_p)
    return BatchResult(attn, logits, rounds, acc_len, acc_path, out_tok)
