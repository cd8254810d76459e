"""Chunked driver of a whole workload through run_layer_group.

Holds a workload's device-resident inputs (indexer inputs of the F layers,
attention inputs and outputs of every layer, the index cache) and issues one
run_layer_group call per query chunk, exactly as a prefill engine would:
chunk c covers query rows q0 .. q0+tq-1 against the tq+q0 keys present
(decode: one row per sequence against the whole cache).  Descriptors are
views into the resident tensors; no data moves between chunks.
"""
from __future__ import annotations

import time

import torch

from . import inputs, lcsi


def pairs_in_chunk(q0: int, tq: int) -> int:
    """Causal (query, key) pairs of rows q0 .. q0+tq-1 (row p sees p+1 keys)."""
    return tq * (q0 + 1) + tq * (tq - 1) // 2


class Workload:
    def __init__(self, wl: inputs.Workload, f_layers=None, n_slots: int = 1, device="cuda", log=None):
        """f_layers: layers whose indexer inputs to draw (default: the F
        layers of the workload's pattern).  n_slots: index-cache slots."""
        self.wl = wl
        L = wl.n_layers
        self.pattern_f = [l for l in range(L) if wl.pattern[l]]
        need_f = self.pattern_f if f_layers is None else list(f_layers)
        t0 = time.time()
        self.idx_in = {l: inputs.indexer_inputs(wl, l, device) for l in need_f}
        self.attn_in = [inputs.attn_inputs(wl, l, device) for l in range(L)]
        self.outs = [torch.empty((wl.B, wl.n_q, wl.H_q, wl.D_v), dtype=torch.bfloat16, device=device)
                     for _ in range(L)]
        self.n_slots = n_slots
        self.cache = torch.empty((n_slots, wl.B, wl.n_q, wl.top_k), dtype=torch.int32, device=device)
        torch.cuda.synchronize()
        if log:
            log(f"[runner] inputs for {wl.name} ready in {time.time() - t0:.1f}s")
        self.tau = inputs.sm_scale(wl)
        self.ws = None
        self.ws_bytes = 0

    # strides of the index cache (elements)
    @property
    def slot_stride(self):
        return self.wl.B * self.wl.n_q * self.wl.top_k

    @property
    def idx_sb(self):
        return self.wl.n_q * self.wl.top_k

    @property
    def idx_st(self):
        return self.wl.top_k

    def chunk_descs(self, q0, tq, T_kv, pattern):
        wl = self.wl
        r0 = q0 - wl.q_pos0
        ids = []
        for l in range(len(pattern)):
            if not pattern[l]:
                continue
            x = self.idx_in[l]
            qs = x["q_scale"][:, r0:r0 + tq] if x["q_scale"] is not None else None
            ids.append(lcsi.indexer_desc(x["q"][:, r0:r0 + tq], x["k"], x["w"][:, r0:r0 + tq], wl.top_k, q0,
                                         k_scale=x["k_scale"], T_kv=T_kv, q_scale=qs))
        ads = []
        for l in range(len(pattern)):
            x = self.attn_in[l]
            ads.append(lcsi.attn_desc(x["q"][:, r0:r0 + tq], x["k"], x["v"], self.outs[l][:, r0:r0 + tq],
                                      wl.top_k, q0, self.tau, T_kv=T_kv))
        return ids, ads

    def plan(self, pattern=None):
        """Per-chunk descriptors; grows the shared workspace as needed."""
        wl = self.wl
        pattern = wl.pattern if pattern is None else pattern
        plans = []
        need = 0
        for (q0, tq, T_kv) in wl.chunks():
            ids, ads = self.chunk_descs(q0, tq, T_kv, pattern)
            cache = self.cache[:, :, q0 - wl.q_pos0:]
            n = lcsi.layer_group_ws_bytes(pattern, ids, ads, cache, self.n_slots, self.slot_stride,
                                          self.idx_sb, self.idx_st)
            need = max(need, n)
            plans.append((q0, tq, T_kv, ids, ads, cache))
        if need > self.ws_bytes:
            self.ws = None
            self.ws = torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda")
            self.ws_bytes = need
        return pattern, plans

    def step(self, plan, events=None):
        """One pass of the whole path: every chunk through run_layer_group.
        events: optional per-chunk lists of 4*L torch.cuda.Event."""
        pattern, plans = plan
        for c, (q0, tq, T_kv, ids, ads, cache) in enumerate(plans):
            lcsi.run_layer_group(pattern, ids, ads, cache, self.n_slots, self.slot_stride, self.idx_sb,
                                 self.idx_st, ws=self.ws, events=events[c] if events is not None else None)

    def capture(self, plan):
        """One step recorded as a HIP graph (torch.cuda.CUDAGraph): replaying
        it re-issues every launch of the step with one host call.  The step
        must have run eagerly once before (workspace, kernel loading).  Only
        kernels are captured (the library issues no memset or copy)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(plan)
        return g
