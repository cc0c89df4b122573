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


# Final-draw margins. Stage-isolated runs feed both sides the same fp32
# logits, so only fp32-vs-fp64 softmax/residual/prefix-sum rounding separates
# their CDFs: a few ulp per term over <= 4096-term chunk sums and <= 64 chunk
# masses stays below 4e-6 of the total. End to end the GPU's logits also carry
# its fp32 accumulation error: K/32 MFMA accumulator updates, each rounding a
# running sum of a few logit standard deviations, bound it by about
# (K/32) * 2^-24 * 4 * std(z); p moves by at most twice that over T.
MARGIN_STAGE = 4e-6


def margin_end_to_end(K: int, logits_std: float, T: float) -> float:
    dz = (K / 32) * 2.0 ** -24 * 4.0 * logits_std
    return MARGIN_STAGE + 2.0 * dz / T


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


def attn_rel_err(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    """max over (row, head) of ||o_gpu - o_ref|| / ||o_ref||."""
    num = np.linalg.norm(o_gpu.astype(np.float64) - o_ref, axis=-1)
    den = np.linalg.norm(o_ref, axis=-1)
    return float((num / np.maximum(den, 1e-30)).max())
