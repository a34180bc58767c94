"""One MoE expert layer step on the GPU through the C ABI.

This module owns device buffers and issues the ABI calls in order; it does no
arithmetic of its own.  Forward:

  moe_router_logits -> moe_route -> moe_permute -> moe_grouped_gemm_fwd
  -> moe_combine

Backward:

  moe_combine_bwd -> moe_grouped_gemm_bwd -> moe_unpermute_sum -> moe_router_bwd

Every call is enqueued on torch's current stream; nothing is copied to the
host in between (routing metadata stays on the GPU: Olmo-core 3 overview,
"Routing and compute optimisation").
"""

from __future__ import annotations

import torch

from . import _abi


class MoELayerGPU:
    """Buffers for one layer shape.  Weights are the caller's tensors."""

    def __init__(self, T: int, d: int, E: int, k: int, h: int, dtype: torch.dtype, device="cuda"):
        self.T, self.d, self.E, self.k, self.h = T, d, E, k, h
        self.R = R = T * k
        self.dtype = dtype
        dev = torch.device(device)
        f32, i32 = torch.float32, torch.int32
        e = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=dev)
        self.logits = e(T, E, dt=f32)
        self.probs = e(T, E, dt=f32)
        self.topk_idx = e(T, k, dt=i32)
        self.topk_w = e(T, k, dt=f32)
        self.counts = e(E, dt=i32)
        self.offsets = e(E + 1, dt=i32)
        self.off32 = e(E + 1, dt=i32)
        self.pos = e(T, k, dt=i32)
        self.src = e(R, dt=i32)
        self.err_flag = torch.zeros(1, dtype=i32, device=dev)
        self.xp = e(R, d)
        self.g = e(R, h)
        self.u = e(R, h)
        self.hb = e(R, h)
        self.yp = e(R, d)
        self.y = e(T, d)
        self.dyp = e(R, d)
        self.dgate = e(T, k, dt=f32)
        self.dgu = e(R, 2 * h)
        self.dxp = e(R, d)
        self.dx = e(T, d)
        self.dwr = e(E, d)
        self.dw1 = e(E, h, d)
        self.dw3 = e(E, h, d)
        self.dw2 = e(E, d, h)
        self.ws_route = _abi.workspace(_abi.moe_route_workspace_size(T, E, k), dev)
        self.ws_gemm = _abi.workspace(_abi.moe_grouped_gemm_workspace_size(E, R, d, h), dev)
        self.ws_router = _abi.workspace(_abi.moe_router_bwd_workspace_size(T, d, E), dev)

    # ------------------------------------------------------------------
    def forward(self, x, wr, w1, w3, w2, forced_idx=None):
        _abi.moe_router_logits(x, wr, self.logits)
        _abi.moe_route(self.logits, self.k, self.probs, self.topk_idx, self.topk_w, self.counts, self.offsets,
                       self.pos, self.src, self.ws_route, off32=self.off32, forced_idx=forced_idx,
                       err_flag=self.err_flag)
        _abi.moe_permute(x, self.pos, self.xp)
        _abi.moe_grouped_gemm_fwd(self.xp, w1, w3, w2, self.offsets, self.g, self.u, self.hb, self.yp, self.ws_gemm)
        _abi.moe_combine(self.yp, self.topk_w, self.pos, self.y)
        return self.y

    def backward(self, dy, x, wr, w1, w3, w2):
        _abi.moe_combine_bwd(dy, self.yp, self.topk_w, self.pos, self.dyp, self.dgate)
        _abi.moe_grouped_gemm_bwd(self.dyp, self.xp, self.g, self.u, self.hb, w1, w3, w2, self.offsets, self.dgu,
                                  self.dxp, self.dw1, self.dw3, self.dw2, self.ws_gemm)
        _abi.moe_unpermute_sum(self.dxp, self.pos, self.dx)
        _abi.moe_router_bwd(self.probs, self.topk_idx, self.dgate, x, wr, self.dx, self.dwr, self.ws_router)
        return self.dx

    def step(self, x, wr, w1, w3, w2, dy, forced_idx=None):
        self.forward(x, wr, w1, w3, w2, forced_idx)
        self.backward(dy, x, wr, w1, w3, w2)
