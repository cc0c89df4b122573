"""Shared helpers of the GPU parity tests: widen inputs for the oracle and
apply the comparison rules (tolerances and round exclusions)."""
from __future__ import annotations

import numpy as np

from oracle import verify as ov
from speculative_decoding_tree_amd import synth

# tolerances stated for this hot path
TOL_RATIO = 1e-5      # node test excluded when |u - p/q| <= this
TOL_CDF = 1e-5        # final draw excluded when its fp64 CDF margin is below this
TOL_GAP = 1e-3        # greedy round excluded when a visited slot's top-2 logits differ less
TOL_LOGIT = 1e-2      # max abs logit error
TOL_PROB = 1e-5       # max abs probability error
TOL_ATTN = 1e-2       # per (row, head) relative L2 error of the attention output
# Round excluded when a warped row's top-p cut lies within TOL_WARP of moving,
# in units of the row's largest probability. The GPU sums per-token masses
# relative to the row max, each formed in fp64 and truncated to a multiple of
# 2^-S with S = min(52, 63 - ceil(log2 V)): a running mass is short by less
# than V * 2^-S (2^-29 < 1.9e-9 for V <= 2^17) plus fp64 rounding, so a cut
# with more margin than 1e-8 lands where the oracle's fp64 sum puts it.
TOL_WARP = 1e-8


def widened(inp: synth.Inputs) -> dict:
    dt = inp.workload.dtype
    return {
        "kv": synth.widen(inp.kv, dt),
        "node_hidden": synth.widen(inp.node_hidden, dt),
        "lm_head": synth.widen(inp.lm_head, dt),
    }


# Final-draw margin of stage-isolated runs. They feed both sides the same fp32
# logits, so only fp32-vs-fp64 softmax/residual/prefix-sum rounding separates
# their CDFs: a few ulp per term over <= 4096-term chunk sums and <= 64 chunk
# masses stays below 4e-6 of the total. End-to-end runs add the windows
# derived from the measured logit error below.
MARGIN_STAGE = 4e-6


def path_excluded(r: ov.RoundResult, T: float) -> bool:
    """The accepted path is compared unless a walked node test is within
    1e-5 of its threshold (greedy: a visited slot's top-2 gap < 1e-3), or a
    warped row's top-p cut is within TOL_WARP of moving (the kept set is then
    a floating-point decision: the GPU forms fp32 masses, the oracle fp64)."""
    if T == 0.0:
        return r.greedy_gap < TOL_GAP
    if r.warp_margin < TOL_WARP:
        return True
    return any(abs(t.u - t.ratio) <= TOL_RATIO for t in r.tests)


def excluded(r: ov.RoundResult, T: float, margin: float = MARGIN_STAGE) -> bool:
    """The whole round (path and final token) is compared unless the path is
    excluded or the final draw lies within `margin` of a CDF step."""
    if path_excluded(r, T):
        return True
    return T != 0.0 and r.final_margin < margin


def compare_rounds(rounds, T, gpu_len, gpu_path, gpu_tok, N, margin=MARGIN_STAGE):
    """Bit-exact comparison of accept lengths, paths and emitted tokens.

    Paths are compared on every round whose walked tests are clear of their
    thresholds; the final token also needs its CDF margin above `margin`.
    Returns (paths_compared, finals_compared, excluded, mismatches)."""
    R = N + 1
    n_paths = n_finals = excl = 0
    bad = []
    for b, r in enumerate(rounds):
        Tb = float(T[b])
        if path_excluded(r, Tb):
            excl += 1
            continue
        n_paths += 1
        n = len(r.path)
        path = list(gpu_path[b * N: b * N + N]) if N else []
        toks = list(gpu_tok[b * R: b * R + R])
        exp_path = list(r.path) + [-1] * (N - n)
        if gpu_len[b] != n or path != exp_path or toks[:n] != r.emitted[:n]:
            bad.append(("path", b, n, int(gpu_len[b]), r.emitted, toks[: n + 1]))
            continue
        if Tb == 0.0 or r.final_margin >= margin:
            n_finals += 1
            if toks[n] != r.token or any(t != -1 for t in toks[n + 1:]):
                bad.append(("final", b, r.token, toks[n], r.final_margin))
    return n_paths, n_finals, excl, bad


# ---------------------------------------------------------------------------
# end to end: windows derived from the measured logit error
# ---------------------------------------------------------------------------
#
# End to end, the GPU's target logits z' differ from the oracle's fp64 z by
# at most delta = max |z' - z| over a sequence's rows (measured). Per slot and
# token, softmax(z'/T)(v) / softmax(z/T)(v) then lies in [e^(-2 delta/T),
# e^(2 delta/T)]: p(v) moves by at most b0(v) = eps0 p(v) with
# eps0 = e^(2 delta/T) - 1 (e^(4 delta/T) - 1 with warping, which restricts
# and renormalises, provided the kept set is the same on both sides; that is
# checked separately). A rejection step r = (p - q)+ moves r(v) by at most
# b(v) ((.)+ is 1-Lipschitz) and the mass Z by at most e = sum b, so the
# normalised residual p_new = r / Z moves by at most
# b_new(v) = (b(v) + p_new(v) e) / (Z - e) at every v. The i-th sibling's
# test value p_{i-1}(x) / q(x) therefore moves by at most b_{i-1}(x) / q(x),
# and the final draw's normalised CDF by at most sum b at the terminal slot.
# The bounds are recomputed along the oracle's own walk, from its logits.


def logit_delta(gpu_rows, ref_rows) -> float:
    """max |z_gpu - z_ref| over the given rows (fp64)."""
    return float(np.abs(np.asarray(gpu_rows, dtype=np.float64) - ref_rows).max())


def e2e_exclusions(r: ov.RoundResult, T: float, delta: float, zt_rows, zd_rows,
                   tokens: np.ndarray, without_replacement: bool = False, top_k: int = 0,
                   top_p: float = 1.0):
    """(path_excluded, final_excluded) for one oracle round compared with a
    GPU round whose target logits are within `delta` of the oracle's.

    zt_rows / zd_rows: the oracle's target and the draft logits of the
    sequence's slots (indexable by slot). Greedy: the argmax cannot move when
    the top-2 gap exceeds 2 delta, so the stated gap rule (1e-3) applies with
    the gap widened to 2 delta if that is larger. T > 0: a node test is
    excluded when |u - ratio| is within TOL_RATIO plus the bound on how far
    its ratio can move; the final draw when its margin is below MARGIN_STAGE
    plus the bound on how far the terminal CDF can move."""
    if T == 0.0:
        ex = r.greedy_gap < max(TOL_GAP, 2.0 * delta)
        return ex, ex
    if r.warp_margin < TOL_WARP:
        return True, True
    warped = top_k > 0 or 0.0 < top_p < 1.0
    eps0 = np.expm1((4.0 if warped else 2.0) * delta / T)
    final_l1 = eps0
    for s in r.visited:
        p = ov.warp(ov.softmax_t(zt_rows[s], T), top_k, top_p)
        b = eps0 * p
        tests = sorted((t for t in r.tests if t.slot == s), key=lambda t: t.rank)
        if tests:
            q = ov.warp(ov.softmax_t(zd_rows[s], T), top_k, top_p)
            n_kids = max(t.rank for t in tests)
            for t in tests:
                x = int(tokens[t.node])
                bound = b[x] / q[x] if q[x] > 0.0 else 0.0
                if abs(t.u - t.ratio) <= TOL_RATIO + bound:
                    return True, True
                if t.accepted:
                    break
                rr = np.maximum(0.0, p - q)
                Z, e = float(rr.sum()), float(b.sum())
                if not Z - e > 0.0:
                    return True, True
                p = rr / Z
                b = (b + p * e) / (Z - e)
                if without_replacement and t.rank < n_kids:
                    q = q.copy()
                    q[x] = 0.0
                    if q.sum() > 0.0:
                        q = q / q.sum()
        if s == r.terminal_slot:
            final_l1 = float(b.sum())
    return False, bool(r.final_margin < MARGIN_STAGE + final_l1)


def compare_rounds_e2e(rounds, T, gpu_len, gpu_path, gpu_tok, N, deltas, zt, zd, tokens,
                       without_replacement=False, top_k=0, top_p=1.0):
    """Bit-exact comparison against the full fp64 oracle with exclusion
    windows from the measured per-sequence logit error (see e2e_exclusions).
    zt: the oracle's target logits [B*R, V], or a list with one slot-indexable
    object per sequence; zd [B*R, V] draft logits; tokens [B*N]. Returns the
    counts of compare_rounds: (paths_compared, finals_compared, excluded,
    mismatches)."""
    R = N + 1
    n_paths = n_finals = excl = 0
    bad = []
    for b, r in enumerate(rounds):
        Tb = float(T[b])
        zt_b = zt[b] if isinstance(zt, list) else zt[b * R:(b + 1) * R]
        pex, fex = e2e_exclusions(r, Tb, deltas[b], zt_b, zd[b * R:(b + 1) * R],
                                  tokens[b * N:(b + 1) * N], without_replacement, top_k, top_p)
        if pex:
            excl += 1
            continue
        n_paths += 1
        n = len(r.path)
        path = list(gpu_path[b * N: b * N + N]) if N else []
        toks = list(gpu_tok[b * R: b * R + R])
        if gpu_len[b] != n or path != list(r.path) + [-1] * (N - n) or toks[:n] != r.emitted[:n]:
            bad.append(("path", b, n, int(gpu_len[b]), r.emitted, toks[: n + 1]))
            continue
        if not fex:
            n_finals += 1
            if toks[n] != r.token or any(t != -1 for t in toks[n + 1:]):
                bad.append(("final", b, r.token, toks[n], r.final_margin))
    return n_paths, n_finals, excl, bad


def attn_rel_err(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    """max over (row, head) of ||o_gpu - o_ref|| / ||o_ref||."""
    num = np.linalg.norm(o_gpu.astype(np.float64) - o_ref, axis=-1)
    den = np.linalg.norm(o_ref, axis=-1)
    return float((num / np.maximum(den, 1e-30)).max())
