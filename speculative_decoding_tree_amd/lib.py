"""Thin Python binding of include/specverify.h (argument marshalling only).

Each function has the C entry point's name and argument order; tensors are
torch tensors on the GPU and are passed by device pointer. Every step of the
verification runs in the HIP library: if libspecverify.so is missing the
binding raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "specverify.h")

SV_BF16, SV_F32 = 0, 1
SV_OK = 0
STATUS_NAMES = {0: "SV_OK", 1: "SV_ERR_NULL", 2: "SV_ERR_SHAPE", 3: "SV_ERR_DTYPE",
                4: "SV_ERR_WORKSPACE", 5: "SV_ERR_HIP", 6: "SV_ERR_ALIGN", 7: "SV_ERR_SCRATCH"}
SEQ_ERR_TREE = 1 << 0
SEQ_ERR_TOKEN = 1 << 1
SEQ_ERR_TEMPERATURE = 1 << 2
SEQ_ERR_PREFIX = 1 << 3
SEQ_ERR_NONFINITE = 1 << 4
SEQ_ERR_INTERNAL = 1 << 5
SEQ_ERR_PATH = 1 << 6
SEQ_ERR_POOL = 1 << 7
SEQ_WARN_UNIFORM = 1 << 8
SEQ_WARN_RESIDUAL = 1 << 9
SEQ_WARN_CDF_CLAMP = 1 << 10
SEQ_ERR_MASK = 0xFF


class SVError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS_NAMES.get(code, code)} ({_status_text(code)})")
        self.code = code


SV_SAMPLE_IID, SV_SAMPLE_DISTINCT = 0, 1


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_nodes", "n_q_heads", "n_kv_heads", "head_dim", "hidden", "vocab", "dtype",
        "max_prefix", "max_children", "sampling", "top_k")] + [("top_p", ctypes.c_float)]


class Debug(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("slot_stats", ctypes.c_void_p),
                ("slot_argmax", ctypes.c_void_p), ("node_ratio", ctypes.c_void_p),
                ("residual_mass", ctypes.c_void_p), ("stage_events", ctypes.c_void_p)]


STAGES = ("prep", "attention", "lm_head", "sampling")


# hipEventDisableSystemFence: recording the event does no system-scope release
# (no cache writeback and invalidation). The events only time work the caller
# has already waited for (elapsed() after a stream or device synchronisation),
# and without the fence they no longer slow the steps they time.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class StageEvents:
    """hipEvents for sv_debug.stage_events, created with the HIP runtime
    without the system-scope fence at record time: a pair per stage in
    `stages` (default: all), NULL entries for the others (the library does not
    record those). elapsed() gives each timed stage's device milliseconds once
    the stream has passed its last event."""

    def __init__(self, stages=None):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                      ctypes.c_uint]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                  ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.stages = list(STAGES) if stages is None else [s for s in STAGES if s in stages]
        self.arr = (ctypes.c_void_p * (2 * len(STAGES)))()
        for i, name in enumerate(STAGES):
            if name not in self.stages:
                continue
            for k in (2 * i, 2 * i + 1):
                ev = ctypes.c_void_p()
                rc = self._hip.hipEventCreateWithFlags(ctypes.byref(ev),
                                                       HIP_EVENT_DISABLE_SYSTEM_FENCE)
                if rc != 0:
                    raise RuntimeError(f"hipEventCreate failed ({rc})")
                self.arr[k] = ev.value

    def prime(self) -> None:
        """Record every event once on the null stream and wait for it, so that
        whatever the runtime sets up at an event's first record happens here
        and not inside a timed region."""
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        for i in range(2 * len(STAGES)):
            if self.arr[i]:
                self._hip.hipEventRecord(self.arr[i], None)
        self._hip.hipEventSynchronize(self._last())

    def _last(self):
        i = STAGES.index(self.stages[-1])
        return self.arr[2 * i + 1]

    def elapsed(self) -> dict:
        out = {}
        for i, name in enumerate(STAGES):
            if name not in self.stages:
                continue
            # stages on different streams end in any order
            self._hip.hipEventSynchronize(self.arr[2 * i + 1])
            ms = ctypes.c_float()
            rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[2 * i],
                                               self.arr[2 * i + 1])
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            out[name] = ms.value
        return out

    def step_ms(self) -> float:
        """Device milliseconds from the first stage's start to the latest stage
        end (events for every stage only; attention and sampling run side by
        side, so either may end last)."""
        if self.stages != list(STAGES):
            raise ValueError("step_ms needs events for every stage")
        last = 0.0
        for i in range(len(STAGES)):
            end = self.arr[2 * i + 1]
            self._hip.hipEventSynchronize(end)
            ms = ctypes.c_float()
            rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[0], end)
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            last = max(last, ms.value)
        return last

    def destroy(self) -> None:
        """Destroy the events (idempotent). Call it explicitly once the events
        are no longer needed: there is no finaliser, because a HIP call made
        while the interpreter shuts down can run after the HIP runtime (or a
        profiler attached to it) has already been torn down. Events never
        destroyed are released with the process."""
        if self.arr is None:
            return
        for i in range(2 * len(STAGES)):
            if self.arr[i]:
                self._hip.hipEventDestroy(self.arr[i])
        self.arr = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()
        return False


_lib = None
ABI_VERSION = 200          # sv_version() of the library whose struct layouts these are


def load():
    """Load libspecverify.so (built by speculative_decoding_tree_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m speculative_decoding_tree_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp = ctypes.c_void_p
    lib.sv_version.restype = ctypes.c_int
    if lib.sv_version() != ABI_VERSION:
        # the structs below mirror one layout of include/specverify.h
        raise RuntimeError(f"{LIB_PATH} reports version {lib.sv_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild it")
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_status_string.argtypes = [ctypes.c_int]
    lib.sv_seq_status_string.restype = ctypes.c_char_p
    lib.sv_seq_status_string.argtypes = [ctypes.c_int]
    lib.sv_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.sv_verify_tree.argtypes = [P] + [vp] * 14 + [ctypes.POINTER(Debug), vp, ctypes.c_size_t, vp]
    lib.sv_tree_attention.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sv_lm_head.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp]
    lib.sv_sample.argtypes = [P] + [vp] * 10 + [ctypes.POINTER(Debug), vp, ctypes.c_size_t, vp]
    lib.sv_sample_noalloc.argtypes = [P] + [vp] * 10 + [ctypes.POINTER(Debug), vp]
    lib.sv_compact_cache.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32] + [vp] * 7
    i32 = ctypes.c_int32
    lib.sv_layer_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.sv_layer_share.argtypes = [P] + [vp] * 5 + [ctypes.c_float] + [vp] * 7 + [
        ctypes.c_size_t, vp]
    lib.sv_tree_init.argtypes = [i32, i32] + [vp] * 5
    lib.sv_tree_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.sv_tree_expand.argtypes = [i32] * 5 + [vp] * 10 + [ctypes.c_size_t, vp]
    lib.sv_tree_finalize.argtypes = [i32] * 3 + [vp] * 10
    for f in ("sv_workspace_size", "sv_verify_tree", "sv_tree_attention", "sv_lm_head",
              "sv_sample", "sv_sample_noalloc", "sv_compact_cache", "sv_tree_init",
              "sv_tree_workspace_size",
              "sv_tree_expand", "sv_tree_finalize", "sv_layer_workspace_size",
              "sv_layer_share"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def header_symbols() -> list:
    """Names of the functions include/specverify.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(sv_\w+)\s*\(", text, re.M)))


def _status_text(code: int) -> str:
    try:
        return load().sv_status_string(code).decode()
    except Exception:  # the library may be the thing that is missing
        return "?"


def sv_version() -> int:
    return load().sv_version()


def sv_status_string(code: int) -> str:
    return load().sv_status_string(code).decode()


def sv_seq_status_string(bit: int) -> str:
    return load().sv_seq_status_string(bit).decode()


def make_problem(batch, n_nodes, n_q_heads, n_kv_heads, head_dim, vocab, dtype, max_prefix,
                 max_children, hidden=None, sampling=SV_SAMPLE_IID, top_k=0,
                 top_p=1.0) -> Problem:
    return Problem(batch, n_nodes, n_q_heads, n_kv_heads, head_dim,
                   n_q_heads * head_dim if hidden is None else hidden, vocab, dtype, max_prefix,
                   max_children, sampling, top_k, top_p)


def sv_workspace_size(prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    rc = load().sv_workspace_size(ctypes.byref(prob), ctypes.byref(n))
    if rc != SV_OK:
        raise SVError(rc, "sv_workspace_size")
    return n.value


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _debug(dbg: dict | None):
    if not dbg:
        return None
    d = Debug()
    for k in ("logits", "slot_stats", "slot_argmax", "node_ratio", "residual_mass"):
        setattr(d, k, _ptr(dbg.get(k)))
    ev = dbg.get("stage_events")
    if ev is not None:
        d.stage_events = ctypes.cast(ev.arr, ctypes.c_void_p).value
    return ctypes.byref(d)


def _check_dtypes(**kw):
    for name, (t, dt) in kw.items():
        if t is not None and t.dtype != dt:
            raise TypeError(f"{name}: expected {dt}, got {t.dtype}")


def sv_verify_tree(prob: Problem, kv, kv_offset, node_hidden, parent, node_token, lm_head,
                   draft_logits, uniforms, temperature, attn_out, accept_len, accept_path,
                   out_tokens, seq_status, dbg=None, workspace=None, stream=None) -> None:
    _check_dtypes(kv_offset=(kv_offset, torch.int32), parent=(parent, torch.int32),
                  node_token=(node_token, torch.int32), draft_logits=(draft_logits, torch.float32),
                  uniforms=(uniforms, torch.float32), temperature=(temperature, torch.float32),
                  attn_out=(attn_out, torch.float32), accept_len=(accept_len, torch.int32),
                  accept_path=(accept_path, torch.int32), out_tokens=(out_tokens, torch.int32),
                  seq_status=(seq_status, torch.int32))
    rc = load().sv_verify_tree(
        ctypes.byref(prob), _ptr(kv), _ptr(kv_offset), _ptr(node_hidden), _ptr(parent),
        _ptr(node_token), _ptr(lm_head), _ptr(draft_logits), _ptr(uniforms), _ptr(temperature),
        _ptr(attn_out), _ptr(accept_len), _ptr(accept_path), _ptr(out_tokens), _ptr(seq_status),
        _debug(dbg), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    if rc != SV_OK:
        raise SVError(rc, "sv_verify_tree")


def sv_tree_attention(prob: Problem, kv, kv_offset, node_hidden, parent, attn_out, seq_status,
                      workspace, stream=None) -> None:
    rc = load().sv_tree_attention(
        ctypes.byref(prob), _ptr(kv), _ptr(kv_offset), _ptr(node_hidden), _ptr(parent),
        _ptr(attn_out), _ptr(seq_status), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != SV_OK:
        raise SVError(rc, "sv_tree_attention")


def sv_lm_head(prob: Problem, rows: int, hidden, lm_head, logits, stream=None) -> None:
    _check_dtypes(logits=(logits, torch.float32))
    rc = load().sv_lm_head(ctypes.byref(prob), rows, _ptr(hidden), _ptr(lm_head), _ptr(logits),
                           _stream(stream))
    if rc != SV_OK:
        raise SVError(rc, "sv_lm_head")


def sv_sample(prob: Problem, parent, node_token, logits, draft_logits, uniforms, temperature,
              accept_len, accept_path, out_tokens, seq_status, dbg=None, workspace=None,
              stream=None) -> None:
    _check_dtypes(logits=(logits, torch.float32), draft_logits=(draft_logits, torch.float32))
    rc = load().sv_sample(
        ctypes.byref(prob), _ptr(parent), _ptr(node_token), _ptr(logits), _ptr(draft_logits),
        _ptr(uniforms), _ptr(temperature), _ptr(accept_len), _ptr(accept_path), _ptr(out_tokens),
        _ptr(seq_status), _debug(dbg), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != SV_OK:
        raise SVError(rc, "sv_sample")


def sv_sample_noalloc(prob: Problem, parent, node_token, logits, draft_logits, uniforms,
                      temperature, accept_len, accept_path, out_tokens, seq_status, dbg=None,
                      stream=None) -> None:
    """sv_sample on the library's static scratch: no workspace, nothing
    allocated (raises SVError with SV_ERR_SCRATCH when the problem needs more
    than SV_NOALLOC_SCRATCH_BYTES)."""
    _check_dtypes(logits=(logits, torch.float32), draft_logits=(draft_logits, torch.float32))
    rc = load().sv_sample_noalloc(
        ctypes.byref(prob), _ptr(parent), _ptr(node_token), _ptr(logits), _ptr(draft_logits),
        _ptr(uniforms), _ptr(temperature), _ptr(accept_len), _ptr(accept_path), _ptr(out_tokens),
        _ptr(seq_status), _debug(dbg), _stream(stream))
    if rc != SV_OK:
        raise SVError(rc, "sv_sample_noalloc")


def sv_compact_cache(cache, layer_stride: int, n_layers: int, row_bytes: int, batch: int,
                     n_nodes: int, kv_offset, prefix_len, accept_len, accept_path,
                     new_prefix_len, status=None, stream=None) -> None:
    """Compact the cache in place (layer_stride and row_bytes in bytes)."""
    _check_dtypes(kv_offset=(kv_offset, torch.int32), prefix_len=(prefix_len, torch.int32),
                  accept_len=(accept_len, torch.int32),
                  new_prefix_len=(new_prefix_len, torch.int32))
    rc = load().sv_compact_cache(
        _ptr(cache), layer_stride, n_layers, row_bytes, batch, n_nodes, _ptr(kv_offset),
        _ptr(prefix_len), _ptr(accept_len), _ptr(accept_path), _ptr(new_prefix_len),
        _ptr(status), _stream(stream))
    if rc != SV_OK:
        raise SVError(rc, "sv_compact_cache")


def sv_tree_workspace_size(batch: int, n_expand: int, vocab: int) -> int:
    n = ctypes.c_size_t(0)
    rc = load().sv_tree_workspace_size(batch, n_expand, vocab, ctypes.byref(n))
    if rc != SV_OK:
        raise SVError(rc, "sv_tree_workspace_size")
    return n.value


class TreePool:
    """Device state of an EAGLE-2 draft-tree build (the arrays sv_tree_*
    read and write, and the expansion workspace for `vocab`), allocated with
    torch."""

    def __init__(self, batch: int, n_expand: int, capacity: int, vocab: int, device="cuda"):
        i32 = dict(dtype=torch.int32, device=device)
        self.batch, self.n_expand, self.capacity, self.vocab = batch, n_expand, capacity, vocab
        self.workspace = torch.empty(sv_tree_workspace_size(batch, n_expand, vocab),
                                     dtype=torch.uint8, device=device)
        self.frontier = torch.empty(batch * n_expand, **i32)
        self.frontier_count = torch.empty(batch, **i32)
        self.token = torch.empty(batch * capacity, **i32)
        self.parent = torch.empty(batch * capacity, **i32)
        self.value = torch.empty(batch * capacity, dtype=torch.float32, device=device)
        self.depth = torch.empty(batch * capacity, **i32)
        self.count = torch.empty(batch, **i32)
        self.status = torch.empty(batch, **i32)


def sv_tree_init(pool: TreePool, stream=None) -> None:
    rc = load().sv_tree_init(pool.batch, pool.n_expand, _ptr(pool.frontier),
                             _ptr(pool.frontier_count), _ptr(pool.count), _ptr(pool.status),
                             _stream(stream))
    if rc != SV_OK:
        raise SVError(rc, "sv_tree_init")


def sv_tree_expand(pool: TreePool, vocab: int, n_children: int, draft_logits,
                   stream=None) -> None:
    _check_dtypes(draft_logits=(draft_logits, torch.float32))
    rc = load().sv_tree_expand(
        pool.batch, vocab, pool.n_expand, n_children, pool.capacity, _ptr(draft_logits),
        _ptr(pool.frontier), _ptr(pool.frontier_count), _ptr(pool.token), _ptr(pool.parent),
        _ptr(pool.value), _ptr(pool.depth), _ptr(pool.count), _ptr(pool.status),
        _ptr(pool.workspace), pool.workspace.numel(), _stream(stream))
    if rc != SV_OK:
        raise SVError(rc, "sv_tree_expand")


def sv_tree_finalize(pool: TreePool, m: int, parent, node_token, node_pool_id, n_kept,
                     stream=None) -> None:
    rc = load().sv_tree_finalize(
        pool.batch, pool.capacity, m, _ptr(pool.token), _ptr(pool.parent), _ptr(pool.value),
        _ptr(pool.depth), _ptr(pool.count), _ptr(parent), _ptr(node_token), _ptr(node_pool_id),
        _ptr(n_kept), _stream(stream))
    if rc != SV_OK:
        raise SVError(rc, "sv_tree_finalize")


def sv_layer_workspace_size(prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    rc = load().sv_layer_workspace_size(ctypes.byref(prob), ctypes.byref(n))
    if rc != SV_OK:
        raise SVError(rc, "sv_layer_workspace_size")
    return n.value


def sv_layer_share(prob: Problem, hidden, wq, wk, wv, wo, rope_theta: float, kv, kv_offset,
                   parent, out_hidden, seq_status, attn_out=None, workspace=None,
                   stream=None) -> None:
    rc = load().sv_layer_share(
        ctypes.byref(prob), _ptr(hidden), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo),
        float(rope_theta), _ptr(kv), _ptr(kv_offset), _ptr(parent), _ptr(out_hidden),
        _ptr(attn_out), _ptr(seq_status), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != SV_OK:
        raise SVError(rc, "sv_layer_share")

