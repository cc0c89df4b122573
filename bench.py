#!/usr/bin/env python3
"""Benchmark of the tree-verification step on one MI355X.

A step is one sv_verify_tree call over one batch: tree-masked attention, LM
head for every slot, and multi-round speculative sampling. The default
workload is the batched-serving shape (32 sequences, prefixes uniform on
[512, 8192], 8B GQA shapes, vocab 128256, 60-node depth-6 tree each, half
greedy and half T = 1). Inputs are seeded synthetic data resident in HBM
before the timed region.

Warmup: --warmup W runs W untimed steps; by default the steps run until half
a second has passed (at least 5), which brings the GPU's clocks to the level
of a continuously busy serving loop, and the JSON line reports the count.

Prints one JSON line on stdout; progress goes to stderr.
  value      verified draft-tree nodes per second = B * N / step time, the
             step time from the host clock around the timed steps, which
             record one HIP event pair around the LM-head stage (the
             roofline's per-launch time)
  ms_per_step_all_stages_timed  the same steps run again, untimed for value,
             with an event pair around every stage: stages_ms and the
             spread below come from this run
  ms_per_step_no_events  the same steps run once more with no events
  step_ms_p10/p50/p90  spread of the per-step device time (HIP events
             around each step on its stream)
  stage_roofline  every stage against the resource that bounds it, from its
             algorithmic bytes or flops (attention: K/V read once, Q read, O
             written; LM head: 2 R V d flops; sampling: the target rows the
             walk visited and the draft rows of its visited internal slots,
             read once), and the whole step against the sum of those floors
  roofline   the dominant kernel (the LM-head GEMM): achieved vs peak, with
             the per-launch duration taken from HIP events the library
             records around that kernel on the call's stream during the
             timed steps; traffic from rocprofv3 counters when they were
             taken on the current kernel source (else null)
  cpu_baseline  the CPU oracle timed on the host on a bounded sample of the
             same workload
  lm_head_vendor_reference  the same GEMM shape through torch (hipBLASLt),
             bf16 and fp32 output, timed the same way: what the vendor library
             reaches on this chip, for context (not part of the step)
  input_copies  how many copies of the inputs the timed steps rotate over:
             inputs smaller than 1 GiB (the batch-1 workloads) are uploaded
             several times so back-to-back steps do not read them from the
             256 MB Infinity Cache
  next_rows  steps beside the timed step, each timed on its own with HIP
             events and reported against its roofline (not part of value):
             kv_compact = sv_compact_cache over a 32-layer cache of the
             workload's KV shape, driven by the accept paths of the last
             timed step (the step that follows acceptance); tree_build =
             EAGLE-2 draft-tree construction for the workload's batch (top-k
             10 expanded, 10 children each, depth 6, 60 nodes kept) from
             random draft logits, init + 6 expansion steps + finalize (the
             step that precedes verification; the draft model's forwards
             between steps are not part of it); layer_share = the full
             verify-layer share on the workload (Q/K/V projections, rotary
             positions by tree depth, node K/V into the cache, tree
             attention, O projection, residual) with random bf16 weights;
             sampling_variants = the whole step again with siblings drawn
             without replacement, and with top-k 50 / top-p 0.9 warping of p
             and q (drafted tokens redrawn from the matching draft process),
             the sampling stage reported against the HBM bytes of the rows
             the walk had to read (each visited target row, and the draft
             row of each visited slot with children, once)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft-tree nodes/sec (attn+LM head+sampling); % of HBM/MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "lm_head_gemm_batch32_8b_counters.txt")
LM_HEAD_SRC = os.path.join(ROOT, "speculative_decoding_tree_amd", "csrc", "lm_head.hip")
ROTATE_BYTES = 1 << 30         # inputs rotated until the copies exceed this
WARMUP_SECONDS = 0.5          # default warmup: untimed steps for this long ...
WARMUP_MIN = 5                # ... and at least this many


def lm_kernel_for(M: int, K: int, dtype: str) -> str:
    """The kernel sv_verify_tree launches for the LM head at M rows and hidden K."""
    if dtype != "bf16":
        return "k_gemm_f32 (fp32 LM head)"
    if M >= 512:
        return "k_gemm_bf16_big<true> (LM-head GEMM with fused row statistics)"
    if M <= 32 and K % 64 == 0 and K >= 1024:
        bm = 16 if M <= 16 else 32
        ks = 1024 if bm == 16 else 512
        if K % ks == 0:
            return (f"k_gemm_stream_lds<16,{bm},8,{ks},4> (LM head, M <= 32: weight rows "
                    "streamed into registers, X staged in LDS per K segment)")
        return f"k_gemm_stream<NU,{bm},D> (LM head, M <= 32: weight rows streamed into registers)"
    if M <= 32:
        return "k_gemm_bf16<2,4,1,4> (LM head, M <= 32)" if M > 16 else \
            "k_gemm_bf16<1,4,1,4> (LM head, M <= 16)"
    if M <= 64:
        return "k_gemm_bf16<4,4,1,4> (LM head, M <= 64)"
    return "k_gemm_bf16<4,8,2,2> (LM head, M < 512)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def lm_head_source_hash() -> str:
    with open(LM_HEAD_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(launch_rows: int, vocab: int):
    """Measured HBM bytes per LM-head launch from the committed counter
    summary, or None when it is absent or was taken on other kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    with open(COUNTERS) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("lm_head_source_sha256_16") != lm_head_source_hash():
        return None
    try:
        if int(kv["rows"]) != launch_rows or int(kv["vocab"]) != vocab:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, budget_s: float):
    """Time the oracle, whole sequences at a time, until the budget is used."""
    import numpy as np
    from oracle import verify as ov
    from speculative_decoding_tree_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    W = inp.workload
    N, R = W.n_nodes, W.rows
    dt = W.dtype
    w_lm = synth.widen(inp.lm_head, dt)
    done = 0
    t0 = time.perf_counter()
    order = list(range(W.batch))
    for b in order:
        rows = slice(b * R, (b + 1) * R)
        h = synth.widen(inp.node_hidden[rows], dt)
        base = int(inp.kv_offset[b])
        L = int(inp.prefix_len[b])
        kv = synth.widen(inp.kv[base: base + L + N], dt)
        par = inp.parent[b * N:(b + 1) * N]
        ov.tree_attention_sequence(h.reshape(R, W.n_q_heads, W.head_dim), kv[:, 0], kv[:, 1], L,
                                   par, W.n_kv_heads)
        z = ov.lm_head(h, w_lm)
        ov.verify_round(z, inp.draft_logits[rows].astype(np.float64), par,
                        inp.node_token[b * N:(b + 1) * N], inp.uniforms[rows],
                        float(inp.temperature[b]))
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {
        "value": done * N / el, "unit": "nodes/s", "cores": blas_threads or cores,
        "host_cores_visible": cores, "kind": "oracle",
        "sample": f"{done} of {W.batch} sequences of {W.name} (sequences 0..{done - 1}), each "
                  f"whole: fp64 tree attention, fp64 LM head, sampling walk; {el:.1f} s",
    }


def time_compaction(torch, lib, db, inp, layers: int, reps: int) -> dict:
    """sv_compact_cache over a `layers`-layer cache with the workload's rows,
    driven by the last step's accept paths. HBM-bound: every accepted row is
    read once and written once per layer. Repeated calls move the same rows
    (the contents do not matter for the time)."""
    import numpy as np
    W = inp.workload
    t = db.t
    rows = int(inp.kv_offset[-1])
    row_bytes = t["kv"][0].numel() * t["kv"].element_size()
    cache = torch.empty((layers, rows, row_bytes), dtype=torch.uint8, device="cuda")
    prefix = torch.from_numpy(inp.prefix_len.astype(np.int32)).cuda()
    new_len = torch.empty(W.batch, dtype=torch.int32, device="cuda")
    status = torch.empty(W.batch, dtype=torch.int32, device="cuda")
    moved = int(np.clip(t["accept_len"].cpu().numpy(), 0, None).sum())

    def call():
        lib.sv_compact_cache(cache, rows * row_bytes, layers, row_bytes, W.batch, W.n_nodes,
                             t["kv_offset"], prefix, t["accept_len"], t["accept_path"], new_len,
                             status)
    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    alg = 2.0 * moved * row_bytes * layers
    achieved = alg / (us * 1e-6) / 1e9
    del cache
    return {"kernel": "k_compact_cache", "layers": layers, "row_bytes": row_bytes,
            "rows_moved_per_layer": moved, "algorithmic_bytes": alg,
            "per_launch_us": round(us, 2), "bound": "hbm", "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}


def time_tree_build(torch, lib, B: int, V: int, reps: int, K: int = 10, C: int = 10,
                    depth: int = 6, m: int = 60) -> dict:
    """A whole EAGLE-2 build per timed repetition. HBM-bound: each step reads
    the draft logits of every frontier row once (1 row at the root, then K)."""
    P = C + (depth - 1) * K * C
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    logits = torch.randn((B, K, V), device="cuda", generator=gen) * 3.0
    pool = lib.TreePool(B, K, P, V)
    out = [torch.empty(B * m, dtype=torch.int32, device="cuda") for _ in range(3)]
    n_kept = torch.empty(B, dtype=torch.int32, device="cuda")

    def build():
        lib.sv_tree_init(pool)
        for _ in range(depth):
            lib.sv_tree_expand(pool, V, C, logits)
        lib.sv_tree_finalize(pool, m, *out, n_kept)
    for _ in range(3):
        build()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        build()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    ok = bool((pool.status == 0).all().item()) and bool((n_kept == m).all().item())
    rows = B * (1 + (depth - 1) * K)
    alg = 4.0 * rows * V
    achieved = alg / (us * 1e-6) / 1e9
    return {"kernels": "k_tree_init, k_expand_seg, k_expand_merge, k_tree_finalize",
            "batch": B, "vocab": V, "top_k": K, "children": C, "depth": depth, "kept": m,
            "rows_read": rows, "algorithmic_bytes": alg, "per_build_us": round(us, 2),
            "valid": ok, "bound": "hbm", "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}


def time_layer_share(torch, lib, db, inp, reps: int, theta: float = 500000.0) -> dict:
    """sv_layer_share on the timed workload; reported against the bf16 MFMA
    peak with the algorithmic flops of its four projections and its tree
    attention. Repeated calls rewrite the same cache rows."""
    import numpy as np
    W = inp.workload
    t = db.t
    B, R, N, d = W.batch, W.rows, W.n_nodes, W.hidden
    Hq, Hkv, D = W.n_q_heads, W.n_kv_heads, W.head_dim
    M = B * R
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    mk = lambda n, k: (torch.randn((n, k), device="cuda", generator=gen) * 0.02).to(
        torch.bfloat16).view(torch.int16)
    wq, wk, wv, wo = mk(Hq * D, d), mk(Hkv * D, d), mk(Hkv * D, d), mk(d, Hq * D)
    out = torch.empty((M, d), dtype=torch.int16, device="cuda")
    st = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(lib.sv_layer_workspace_size(db.prob), dtype=torch.uint8, device="cuda")

    def call():
        lib.sv_layer_share(db.prob, t["node_hidden"], wq, wk, wv, wo, theta, t["kv"],
                           t["kv_offset"], t["parent"], out, st, workspace=ws)
    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    proj = 2.0 * M * d * (Hq + 2 * Hkv) * D + 2.0 * M * Hq * D * d
    depth_sum = 0
    for b in range(B):
        par = inp.parent[b * N:(b + 1) * N]
        dep = np.zeros(N, dtype=np.int64)
        for j in range(N):
            dep[j] = 1 if par[j] < 0 else dep[par[j]] + 1
        depth_sum += int(dep.sum())
    attn = 4.0 * D * Hq * (R * float(inp.prefix_len.sum()) + depth_sum)
    flops = proj + attn
    achieved = flops / (us * 1e-6) / 1e12
    ok = bool((st == 0).all().item())
    del ws
    return {"kernels": "bf16 GEMMs (Q, K, V, O), k_rope_scatter, k_attn_mfma + k_attn_merge "
                       "(bf16 output), k_residual",
            "rope_theta": theta, "algorithmic_flops": flops, "projection_flops": proj,
            "attention_flops": attn, "per_call_us": round(us, 1), "valid": ok, "bound": "mfma",
            "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}


def time_sampling_variants(torch, lib, synth, db, inp, steps: int, variants=None) -> dict:
    """The verification step with the sampling variants; per variant the step
    time, the sampling stage time and its rate over the algorithmic bytes of
    the rows the walk visited. variants: name -> workload (default: i.i.d.
    siblings, siblings without replacement, top-k 50 / top-p 0.9)."""
    import dataclasses

    import numpy as np
    from speculative_decoding_tree_amd.runner import DeviceBatch, problem_for
    W = inp.workload
    B, N, R, V = W.batch, W.n_nodes, W.rows, W.vocab
    if variants is None:
        variants = {"iid": W, "distinct": W.with_(children="distinct"),
                    "top_k50_top_p0.9": W.with_(top_k=50, top_p=0.9)}
    out = {}
    for name, wv in variants.items():
        if wv is W:
            tok = inp.node_token
        else:
            rng = np.random.default_rng(31)
            tok = np.concatenate([
                synth._draw_tokens(rng, inp.draft_logits[b * R:(b + 1) * R],
                                   inp.parent[b * N:(b + 1) * N], float(inp.temperature[b]),
                                   wv.children == "distinct", wv.top_k, wv.top_p)
                for b in range(B)]).astype(np.int32)
        vin = dataclasses.replace(inp, workload=wv, node_token=tok)
        prob = problem_for(vin)
        t = dict(db.t)
        t["node_token"] = torch.from_numpy(tok).cuda()
        ws = torch.empty(lib.sv_workspace_size(prob), dtype=torch.uint8, device="cuda")
        vdb = DeviceBatch(prob, vin, t, ws)
        for _ in range(3):
            vdb.verify()
        events = [lib.StageEvents() for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            vdb.verify(dbg={"stage_events": events[k]})
        torch.cuda.synchronize()
        step_ms = (time.perf_counter() - t0) * 1e3 / steps
        samp_ms = sum(ev.elapsed()["sampling"] for ev in events) / steps
        for ev in events:
            ev.destroy()
        alen = t["accept_len"].cpu().numpy()
        apath = t["accept_path"].cpu().numpy()
        ok = bool((t["seq_status"].cpu().numpy() & lib.SEQ_ERR_MASK == 0).all())
        rows = 0
        for b in range(B):
            if inp.temperature[b] == 0.0:
                continue
            par = inp.parent[b * N:(b + 1) * N]
            slots = [0] + [int(j) + 1 for j in apath[b * N:b * N + max(int(alen[b]), 0)]]
            rows += len(slots)                                   # target rows
            rows += sum(1 for s in slots if (par == s - 1).any())  # draft rows
        alg = 4.0 * V * rows
        achieved = alg / (samp_ms * 1e-3) / 1e9
        out[name] = {"step_ms": round(step_ms, 4), "sampling_ms": round(samp_ms, 4),
                     "rows_read": rows, "algorithmic_bytes": alg, "valid": ok,
                     "mean_accept_len_sampled": round(float(alen[inp.temperature > 0].mean()), 3),
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
        del ws
    return out


def stage_rooflines(inp, db, stages: dict, lm_flops: float, lm_bytes: float,
                    step_ms: float) -> dict:
    """Each stage of the timed step against the resource that bounds it, and
    the step against the sum of the stage floors."""
    import numpy as np
    W = inp.workload
    B, N, R, V = W.batch, W.n_nodes, W.rows, W.vocab
    Hq, Hkv, D = W.n_q_heads, W.n_kv_heads, W.head_dim
    s = 2 if W.dtype == "bf16" else 4
    L = inp.prefix_len.astype(np.int64)
    attn_bytes = float(s * 2 * (L + N).sum() * Hkv * D + s * B * R * Hq * D + 4 * B * R * Hq * D)
    alen = db.t["accept_len"].cpu().numpy()
    apath = db.t["accept_path"].cpu().numpy()
    rows = 0
    for b in range(B):
        if inp.temperature[b] == 0.0:
            continue
        par = inp.parent[b * N:(b + 1) * N]
        slots = [0] + [int(j) + 1 for j in apath[b * N:b * N + max(int(alen[b]), 0)]]
        rows += len(slots) + sum(1 for q in slots if (par == q - 1).any())
    samp_bytes = 4.0 * V * rows
    peak_mma = PEAK_BF16_TFLOPS if W.dtype == "bf16" else PEAK_F32_TFLOPS

    def hbm(bytes_, ms):
        gbs = bytes_ / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "algorithmic_bytes": bytes_, "ms": round(ms, 4),
                "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    lm_tf = lm_flops / (stages["lm_head"] * 1e-3) / 1e12
    # the LM head is a dense contraction above the ridge only when many rows
    # share W (the batched workload); at batch 1 it streams W from HBM
    lm_mma = lm_flops / lm_bytes >= peak_mma * 1e12 / (PEAK_HBM_GBS * 1e9)
    lm_floor = lm_flops / (peak_mma * 1e12) if lm_mma else lm_bytes / (PEAK_HBM_GBS * 1e9)
    floor_ms = (attn_bytes / (PEAK_HBM_GBS * 1e9) + lm_floor
                + samp_bytes / (PEAK_HBM_GBS * 1e9)) * 1e3
    lm = ({"bound": "mfma", "algorithmic_flops": lm_flops, "ms": round(stages["lm_head"], 4),
           "achieved": round(lm_tf, 1), "peak": peak_mma, "unit": "TFLOP/s",
           "frac": round(lm_tf / peak_mma, 4)} if lm_mma else hbm(lm_bytes, stages["lm_head"]))
    return {
        "attention": hbm(attn_bytes, stages["attention"]),
        "lm_head": lm,
        "sampling": dict(hbm(samp_bytes, stages["sampling"]), rows_read=rows),
        "step": {"floor_ms": round(floor_ms, 4), "ms": round(step_ms, 4),
                 "frac": round(floor_ms / step_ms, 4)},
    }


def time_vendor_gemm(torch, M: int, N: int, K: int, reps: int = 20) -> dict:
    """torch's bf16 GEMM (hipBLASLt) on the LM-head shape: x [M, K] times
    w [N, K] transposed, bf16 output and fp32 output."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    x = torch.randn((M, K), device="cuda", dtype=torch.bfloat16, generator=gen)
    w = torch.randn((N, K), device="cuda", dtype=torch.bfloat16, generator=gen)
    out = {}
    flops = 2.0 * M * N * K
    calls = {"bf16_out": lambda: torch.nn.functional.linear(x, w),
             "fp32_out": lambda: torch.mm(x, w.t(), out_dtype=torch.float32)}
    for name, f in calls.items():
        try:
            for _ in range(3):
                f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            out[name] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                         "frac": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
        except (RuntimeError, TypeError) as ex:      # an older torch without out_dtype
            out[name] = {"error": str(ex)[:120]}
    del x, w
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: as many as fill\n"
                         f"{WARMUP_SECONDS:g} s, at least {WARMUP_MIN})")
    ap.add_argument("--workload", default="batch32_8b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--no-next-rows", dest="next_rows", action="store_false",
                    help="skip the next-row timings (compaction, tree build, layer share, "
                         "sampling variants)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 device-to-device copies of MIB MiB (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a copy of known size)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the verification step runs on one GPU (asked for --gpus {args.gpus}); "
              "there is no multi-GPU path to time.", file=sys.stderr)
        sys.exit(2)

    import torch
    from speculative_decoding_tree_amd import lib, synth
    from speculative_decoding_tree_amd.runner import DeviceBatch

    ap_next = args.next_rows
    lib.load()     # raises when the HIP library is missing: nothing runs without it
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return
    wl = synth.WORKLOADS[args.workload]
    log(f"[bench] generating {wl.name} seed {args.seed} ...")
    t0 = time.perf_counter()
    inp = synth.generate(wl, seed=args.seed)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
    db = DeviceBatch.create(inp)
    # A workload whose inputs fit the 256 MB Infinity Cache (the batch-1
    # shapes) would be timed from cache on back-to-back steps, which a decode
    # loop never sees (the rest of the model runs in between). Such inputs are
    # uploaded several times and the steps rotate over the copies until they
    # span ROTATE_BYTES.
    per_copy = sum(v.numel() * v.element_size() for v in db.t.values())
    copies = 1
    if per_copy < ROTATE_BYTES:
        copies = min(16, -(-ROTATE_BYTES // per_copy))
    dbs = [db] + [DeviceBatch.create(inp) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    B, N, R, V, d = wl.batch, wl.n_nodes, wl.rows, wl.vocab, wl.hidden
    if copies > 1:
        log(f"[bench] {per_copy / 2**20:.1f} MiB of inputs per step: rotating over {copies} "
            f"copies ({copies * per_copy / 2**20:.0f} MiB)")

    # The vendor GEMM reference (untimed for value, ~40 launches of the LM-head
    # shape) runs first: it also brings the GPU from idle (input generation
    # leaves it idle for seconds) to the load the timed steps see in a
    # continuously busy serving loop.
    vendor = None
    if wl.dtype == synth.BF16:
        log("[bench] timing the vendor GEMM on the LM-head shape")
        vendor = time_vendor_gemm(torch, B * R, V, d)
        log(f"[bench] vendor GEMM: {vendor}")
    # The timed steps record a HIP event pair around the LM-head stage (the
    # dominant kernel's per-launch time for the roofline). The same steps then
    # run twice more, untimed: with an event pair around every stage (the
    # per-stage times and the step's device-side spread) and with no events at
    # all (what the timed steps' two events add). Events are recorded without
    # the system-scope fence, which otherwise writes back and invalidates the
    # caches at every event and slows the kernel after it. Every event set is
    # created and primed before the warmup, so the GPU does not sit idle
    # between the warmup and the timed steps.
    head_events = [lib.StageEvents(stages=("lm_head",)) for _ in range(args.steps)]
    events = [lib.StageEvents() for _ in range(args.steps)]
    for ev in head_events + events:
        ev.prime()
    # Warmup: by default steps until WARMUP_SECONDS have passed (at least
    # WARMUP_MIN), which brings the GPU's clocks to the level a continuously
    # busy serving loop runs at; after a few milliseconds of load the first
    # LM-head launches still run up to ~13% slower than later ones.
    torch.cuda.synchronize()
    tw = time.perf_counter()
    warmup = 0
    while (warmup < args.warmup) if args.warmup is not None else \
            (warmup < WARMUP_MIN or time.perf_counter() - tw < WARMUP_SECONDS):
        dbs[warmup % copies].verify()
        warmup += 1
        if args.warmup is None and warmup % 8 == 0:
            torch.cuda.synchronize()              # the clock measures GPU work, not queueing
    torch.cuda.synchronize()
    log(f"[bench] warmup {warmup} steps in {time.perf_counter() - tw:.2f} s; "
        f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.steps):
        dbs[k % copies].verify(dbg={"stage_events": head_events[k]})
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    lm_launch_ms = sum(ev.elapsed()["lm_head"] for ev in head_events) / args.steps
    for ev in head_events:
        ev.destroy()
    t2 = time.perf_counter()
    for k in range(args.steps):
        dbs[k % copies].verify(dbg={"stage_events": events[k]})
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    ms_per_step_staged = (t3 - t2) * 1e3 / args.steps
    t4 = time.perf_counter()
    for k in range(args.steps):
        dbs[k % copies].verify()
    torch.cuda.synchronize()
    t5 = time.perf_counter()
    ms_per_step_bare = (t5 - t4) * 1e3 / args.steps
    db = dbs[(args.steps - 1) % copies]          # the copy the last step used
    stages = {s: 0.0 for s in lib.STAGES}
    for ev in events:
        for s, ms in ev.elapsed().items():
            stages[s] += ms / args.steps
    step_dev = sorted(ev.step_ms() for ev in events)
    for ev in events:
        ev.destroy()

    def pct(q):
        return step_dev[min(len(step_dev) - 1, int(round(q * (len(step_dev) - 1))))]
    status = db.t["seq_status"].cpu().numpy()
    if (status & lib.SEQ_ERR_MASK).any():
        log(f"[bench] WARNING: sequence errors {status.tolist()}")
    log(f"[bench] {ms_per_step:.3f} ms/step ({ms_per_step_staged:.3f} with every stage timed, "
        f"{ms_per_step_bare:.3f} with no events); stages (ms): "
        + ", ".join(f"{k} {v:.3f}" for k, v in stages.items()))

    M = B * R
    lm_ms = lm_launch_ms
    flops = 2.0 * M * V * d
    elem = 2 if wl.dtype == synth.BF16 else 4
    # W and X once; logits stored for rows of sequences with T > 0 (the GEMM
    # reduces greedy rows to their argmax statistics); 8-byte statistics per
    # row and 256-token tile
    fused = wl.dtype == synth.BF16 and M >= 512
    if fused:
        m_sampled = R * int((inp.temperature > 0).sum())
        alg_bytes = elem * (V * d + M * d) + 4.0 * m_sampled * V + 8.0 * M * ((V + 255) // 256)
    else:
        # the plain GEMM stores every row's logits
        alg_bytes = elem * (V * d + M * d) + 4.0 * M * V
    intensity = flops / alg_bytes
    peak_flops = PEAK_BF16_TFLOPS if wl.dtype == synth.BF16 else PEAK_F32_TFLOPS
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    traffic = read_traffic(M, V)
    if intensity >= ridge:
        achieved = flops / (lm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(achieved / peak_flops, 4),
                "traffic": traffic, "kernel": lm_kernel_for(M, d, wl.dtype),
                "per_launch_ms": round(lm_ms, 4), "algorithmic_flops": flops}
    else:
        achieved = alg_bytes / (lm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic, "kernel": lm_kernel_for(M, d, wl.dtype),
                "per_launch_ms": round(lm_ms, 4), "algorithmic_bytes": alg_bytes}

    stage_roof = stage_rooflines(inp, db, stages, flops, alg_bytes, ms_per_step)

    next_rows = None
    if ap_next:
        next_rows = {}
        log("[bench] timing KV-cache compaction")
        compact = time_compaction(torch, lib, db, inp, layers=32, reps=20)
        next_rows["kv_compact"] = compact
        log(f"[bench] kv_compact: {compact['per_launch_us']} us, {compact['achieved']} GB/s")
        log("[bench] timing EAGLE-2 tree construction")
        tree = time_tree_build(torch, lib, B, V, reps=20)
        next_rows["tree_build"] = tree
        log(f"[bench] tree_build: {tree['per_build_us']} us, {tree['achieved']} GB/s")
        if wl.dtype == synth.BF16 and wl.head_dim == 128:
            log("[bench] timing the full verify-layer share")
            layer = time_layer_share(torch, lib, db, inp, reps=10)
            next_rows["layer_share"] = layer
            log(f"[bench] layer_share: {layer['per_call_us']} us, {layer['achieved']} TFLOP/s")
        if (inp.temperature > 0).any():
            log("[bench] timing the sampling variants")
            variants = time_sampling_variants(torch, lib, synth, db, inp, steps=10)
            next_rows["sampling_variants"] = variants
            for k, v in variants.items():
                log(f"[bench] sampling {k}: step {v['step_ms']} ms, "
                    f"sampling {v['sampling_ms']} ms")

    cpu = None
    if args.cpu_budget > 0:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_budget:.0f} s")
        cpu = cpu_baseline(inp, args.cpu_budget)

    out = {
        "metric": METRIC,
        "value": B * N / (ms_per_step * 1e-3),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_all_stages_timed": round(ms_per_step_staged, 4),
        "ms_per_step_no_events": round(ms_per_step_bare, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == synth.BF16 else "f32",
        "data": f"synthetic (seeded; shapes of the {wl.name} workload)",
        "config": {"workload": wl.name, "batch": B, "nodes_per_seq": N, "vocab": V, "hidden": d,
                   "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
                   "prefix": list(wl.prefix), "temperatures": sorted(set(map(float,
                                                                             inp.temperature))),
                   "sum_prefix": int(inp.prefix_len.sum()), "seed": args.seed},
        "step_ms_p10": round(pct(0.1), 4),
        "step_ms_p50": round(pct(0.5), 4),
        "step_ms_p90": round(pct(0.9), 4),
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "stage_roofline": stage_roof,
        "roofline": roof,
        "cpu_baseline": cpu,
        "lm_head_vendor_reference": vendor,
        "input_copies": copies,
        "next_rows": next_rows,
    }
    print(json.dumps(out), flush=True)
    # release device memory and drain the stream while the runtime is whole,
    # so nothing of ours touches HIP during interpreter shutdown
    del db, dbs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
