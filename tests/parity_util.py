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


def widened(inp: synth.Inputs) -> dict:
    dt = inp.workload.dtype
    return {
        "kv": synth.widen(inp.kv, dt),
        "node_hidden": synth.widen(inp.node_hidden, dt),
        "lm_head": synth.widen(inp.lm_head, dt),
    }


def excluded(r: ov.RoundResult, T: float) -> bool:
    if T == 0.0:
        return r.greedy_gap < TOL_GAP
    if any(abs(t.u - t.ratio) <= TOL_RATIO for t in r.tests):
        return True
    return r.final_margin < TOL_CDF


def compare_rounds(rounds, T, gpu_len, gpu_path, gpu_tok, N):
    """Bit-exact comparison of accept lengths, paths and emitted tokens on
    every round not excluded. Returns (compared, excluded, mismatches)."""
    R = N + 1
    compared = excl = 0
    bad = []
    for b, r in enumerate(rounds):
        if excluded(r, float(T[b])):
            excl += 1
            continue
        compared += 1
        n = len(r.path)
        path = list(gpu_path[b * N: b * N + N]) if N else []
        toks = list(gpu_tok[b * R: b * R + R])
        exp_path = list(r.path) + [-1] * (N - n)
        exp_tok = r.emitted + [-1] * (R - n - 1)
        if gpu_len[b] != n or path != exp_path or toks != exp_tok:
            bad.append((b, n, int(gpu_len[b]), r.emitted, toks[: n + 1]))
    return compared, excl, bad


def attn_rel_err(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    """max over (row, head) of ||o_gpu - o_ref|| / ||o_ref||."""
    num = np.linalg.norm(o_gpu.astype(np.float64) - o_ref, axis=-1)
    den = np.linalg.norm(o_ref, axis=-1)
    return float((num / np.maximum(den, 1e-30)).max())
