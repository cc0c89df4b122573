"""Device-side batch: uploads a synthetic batch, owns the outputs and the
workspace, and calls the C ABI through the binding. Plumbing only."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import lib
from .synth import BF16, Inputs


def problem_for(inp: Inputs, max_prefix: int | None = None) -> lib.Problem:
    wl = inp.workload
    return lib.make_problem(
        batch=wl.batch, n_nodes=wl.n_nodes, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
        head_dim=wl.head_dim, vocab=wl.vocab, dtype=lib.SV_BF16 if wl.dtype == BF16 else lib.SV_F32,
        max_prefix=int(inp.prefix_len.max()) if max_prefix is None else max_prefix,
        max_children=inp.max_children,
        sampling=lib.SV_SAMPLE_DISTINCT if wl.children == "distinct" else lib.SV_SAMPLE_IID,
        top_k=wl.top_k, top_p=wl.top_p)


def _dev(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class DeviceBatch:
    prob: lib.Problem
    inp: Inputs
    t: dict
    workspace: torch.Tensor

    @classmethod
    def create(cls, inp: Inputs, device="cuda", max_prefix: int | None = None):
        prob = problem_for(inp, max_prefix)
        wl = inp.workload
        B, N, R = wl.batch, wl.n_nodes, wl.rows
        t = {
            "kv": _dev(inp.kv, device),
            "kv_offset": _dev(inp.kv_offset, device),
            "node_hidden": _dev(inp.node_hidden, device),
            "parent": _dev(inp.parent, device),
            "node_token": _dev(inp.node_token, device),
            "lm_head": _dev(inp.lm_head, device),
            "draft_logits": _dev(inp.draft_logits, device),
            "uniforms": _dev(inp.uniforms, device),
            "temperature": _dev(inp.temperature, device),
            "attn_out": torch.empty((B * R, wl.n_q_heads, wl.head_dim), dtype=torch.float32,
                                    device=device),
            "accept_len": torch.empty(B, dtype=torch.int32, device=device),
            "accept_path": torch.empty(max(B * N, 1), dtype=torch.int32, device=device),
            "out_tokens": torch.empty(B * R, dtype=torch.int32, device=device),
            "seq_status": torch.empty(B, dtype=torch.int32, device=device),
        }
        ws = torch.empty(lib.sv_workspace_size(prob), dtype=torch.uint8, device=device)
        return cls(prob, inp, t, ws)

    def debug_buffers(self) -> dict:
        wl = self.inp.workload
        B, N, R, V = wl.batch, wl.n_nodes, wl.rows, wl.vocab
        dev = self.workspace.device
        return {
            "logits": torch.empty((B * R, V), dtype=torch.float32, device=dev),
            "slot_stats": torch.full((B * R, 4), float("nan"), dtype=torch.float32, device=dev),
            "slot_argmax": torch.empty(B * R, dtype=torch.int32, device=dev),
            "node_ratio": torch.full((max(B * N, 1),), float("nan"), dtype=torch.float32,
                                     device=dev),
            "residual_mass": torch.full((B * R, self.prob.max_children), float("nan"),
                                        dtype=torch.float32, device=dev),
        }

    def verify(self, dbg: dict | None = None, stream=None) -> None:
        t = self.t
        lib.sv_verify_tree(self.prob, t["kv"], t["kv_offset"], t["node_hidden"], t["parent"],
                           t["node_token"], t["lm_head"], t["draft_logits"], t["uniforms"],
                           t["temperature"], t["attn_out"], t["accept_len"], t["accept_path"],
                           t["out_tokens"], t["seq_status"], dbg=dbg, workspace=self.workspace,
                           stream=stream)

    def results(self) -> dict:
        return {k: self.t[k].cpu().numpy() for k in
                ("attn_out", "accept_len", "accept_path", "out_tokens", "seq_status")}
