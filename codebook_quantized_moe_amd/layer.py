"""Buffers and call sequence of one routed-MoE layer forward over libmoeq's calls.

Plumbing only: torch allocates the device buffers once; ``forward`` enqueues
route -> permute -> gate|up+SwiGLU -> down -> unpermute/combine on one stream with no
host synchronisation in between; ``forward_routed`` puts the bf16 router in front.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (MOEQ_GATING_SOFTMAX_TOPK, moeq_down, moeq_gateup_swiglu, moeq_moe_decode,
               moeq_moe_decode_workspace_bytes, moeq_permute_by_expert, moeq_route_permute,
               moeq_route_topk, moeq_router_logits, moeq_shared_expert,
               moeq_shared_workspace_bytes, moeq_unpermute_combine,
               moeq_unpermute_combine_shared, moeq_workspace_bytes)


@dataclass
class DeviceWeights:
    """One layer's encoded experts on the device. Codes [E, N, K/2] u8, scales [E, N, K/32] u8."""
    gate_codes: torch.Tensor
    gate_scales: torch.Tensor
    up_codes: torch.Tensor
    up_scales: torch.Tensor
    down_codes: torch.Tensor
    down_scales: torch.Tensor
    tables: np.ndarray          # host fp32 [n_tables, 8]
    table_id: torch.Tensor      # device u8 [E]

    @classmethod
    def from_host(cls, lw, device="cuda"):
        def d(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return cls(d(lw.gate_codes), d(lw.gate_scales), d(lw.up_codes), d(lw.up_scales),
                   d(lw.down_codes), d(lw.down_scales),
                   np.ascontiguousarray(lw.tables, dtype=np.float32), d(lw.table_id))

    @property
    def E(self):
        return self.gate_codes.shape[0]

    @property
    def I(self):
        return self.gate_codes.shape[1]

    @property
    def H(self):
        return self.gate_codes.shape[2] * 2


class MoeLayer:
    """Preallocated buffers for T tokens of a layer with E experts, top-k (and, with
    shared_I, a shared expert of intermediate size shared_I)."""

    def __init__(self, T: int, H: int, I: int, E: int, k: int, device="cuda",
                 gating: int = MOEQ_GATING_SOFTMAX_TOPK, shared_I: int | None = None):
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.gating = gating
        self.shared_I = shared_I
        if shared_I is not None:
            self.s_inter = torch.empty((T, shared_I), dtype=torch.int16, device=device)
            self.s_z = torch.empty((T, H), dtype=torch.float32, device=device)
            self.s_ws_bytes = moeq_shared_workspace_bytes(T, H, shared_I)
            self.s_ws = torch.empty(max(self.s_ws_bytes, 1), dtype=torch.uint8, device=device)
            self.side = torch.cuda.Stream(device=device)      # default priority
            self.fork = torch.cuda.Event()
            self.join = torch.cuda.Event()
        P = T * k
        i32 = dict(dtype=torch.int32, device=device)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device)
        self.topk_ids = torch.empty(P, **i32)
        self.topk_w = torch.empty(P, dtype=torch.float32, device=device)
        self.offsets = torch.empty(E + 1, **i32)
        self.sorted_pair = torch.empty(P, **i32)
        self.pair_pos = torch.empty(P, **i32)
        self.inter = torch.empty((P, I), dtype=torch.int16, device=device)
        self.yp = torch.empty((P, H), dtype=torch.float32, device=device)
        self.y = torch.empty((T, H), dtype=torch.int16, device=device)
        self.ws_bytes = moeq_workspace_bytes(T, k, E, H, I)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device)

    def router(self, x, router_w, stream=None):
        """x: bf16 bits [T, H]; router_w: bf16 bits [E, H]. Writes and returns self.logits."""
        moeq_router_logits(x, self.T, self.H, router_w, self.E, self.logits, stream=stream)
        return self.logits

    def route(self, logits, stream=None):
        moeq_route_topk(logits, self.T, self.E, self.k, self.topk_ids, self.topk_w,
                        gating=self.gating, stream=stream)

    def route_permute(self, logits, stream=None):
        """route then permute (one launch for few tokens)."""
        moeq_route_permute(logits, self.T, self.E, self.k, self.topk_ids, self.topk_w,
                           self.offsets, self.sorted_pair, self.pair_pos, gating=self.gating,
                           stream=stream)

    def permute(self, stream=None):
        moeq_permute_by_expert(self.topk_ids, self.T, self.k, self.E, self.offsets,
                               self.sorted_pair, self.pair_pos, stream=stream)

    def gateup(self, x, w: DeviceWeights, stream=None):
        moeq_gateup_swiglu(x, self.T, self.H, self.I, self.E, self.k, self.offsets,
                           self.sorted_pair, w.gate_codes, w.gate_scales, w.up_codes,
                           w.up_scales, w.tables, w.table_id, self.inter, self.ws, self.ws_bytes,
                           stream=stream)

    def down(self, w: DeviceWeights, stream=None):
        moeq_down(self.inter, self.T, self.H, self.I, self.E, self.k, self.offsets,
                  self.sorted_pair, self.topk_w, w.down_codes, w.down_scales, w.tables,
                  w.table_id, self.yp, self.ws, self.ws_bytes, stream=stream)

    def shared_expert(self, x, sw: DeviceWeights, stream=None):
        """The shared expert (E = 1 weights) on every token into self.s_z."""
        moeq_shared_expert(x, self.T, self.H, self.shared_I, sw.gate_codes, sw.gate_scales,
                           sw.up_codes, sw.up_scales, sw.down_codes, sw.down_scales, sw.tables,
                           sw.table_id, self.s_inter, self.s_z, self.s_ws, self.s_ws_bytes,
                           stream=stream)

    def combine(self, residual=None, out=None, stream=None, shared=False):
        out = self.y if out is None else out
        if shared:
            moeq_unpermute_combine_shared(self.yp, self.pair_pos, self.offsets, self.T, self.k,
                                          self.E, self.H, self.s_z, residual, out, stream=stream)
        else:
            moeq_unpermute_combine(self.yp, self.pair_pos, self.offsets, self.T, self.k, self.E,
                                   self.H, residual, out, stream=stream)
        return out

    def _fork_shared(self, x, sw, stream):
        """Start the shared expert on the side stream once x is ready on the main stream."""
        main = stream if stream is not None else torch.cuda.current_stream()
        self.fork.record(main)
        self.side.wait_event(self.fork)
        self.shared_expert(x, sw, stream=self.side)
        self.join.record(self.side)
        return main

    def forward(self, x, logits, w: DeviceWeights, residual=None, out=None, stream=None,
                shared: DeviceWeights | None = None):
        """x: int16 (bf16 bits) [T, H] cuda; logits fp32 [T, E] cuda. Returns y (bf16 bits).
        With shared weights, the shared expert runs on a side stream beside the routed path
        and is added in the combine."""
        if shared is not None:
            stream = self._fork_shared(x, shared, stream)
        self.route_permute(logits, stream)
        self.gateup(x, w, stream)
        self.down(w, stream)
        if shared is not None:
            stream.wait_event(self.join)
        return self.combine(residual, out, stream, shared=shared is not None)

    def forward_fused(self, x, logits, w: DeviceWeights, residual=None, out=None, stream=None):
        """The decode layer as one cooperative launch (moeq_moe_decode); T * k <= 4096."""
        if not hasattr(self, "f_ws"):
            self.f_ws_bytes = moeq_moe_decode_workspace_bytes(self.T, self.k, self.E, self.H,
                                                              self.I)
            self.f_ws = torch.empty(self.f_ws_bytes, dtype=torch.uint8, device=self.y.device)
        out = self.y if out is None else out
        moeq_moe_decode(x, logits, self.T, self.H, self.I, self.E, self.k, w.gate_codes,
                        w.gate_scales, w.up_codes, w.up_scales, w.down_codes, w.down_scales,
                        w.tables, w.table_id, residual, out, self.f_ws, self.f_ws_bytes,
                        gating=self.gating, stream=stream)
        return out

    def forward_routed(self, x, router_w, w: DeviceWeights, residual=None, out=None,
                       stream=None, shared: DeviceWeights | None = None):
        """As forward, with the logits computed from x by the bf16 router router_w [E, H]."""
        if shared is not None:
            stream = self._fork_shared(x, shared, stream)
        self.router(x, router_w, stream)
        self.route_permute(self.logits, stream)
        self.gateup(x, w, stream)
        self.down(w, stream)
        if shared is not None:
            stream.wait_event(self.join)
        return self.combine(residual, out, stream, shared=shared is not None)
