"""One MoE expert layer step on the GPU through the C ABI.

This module owns device buffers and issues the ABI calls in order; it does no
arithmetic of its own.  Forward:

  moe_router_logits -> moe_route -> moe_permute -> moe_grouped_gemm_fwd
  -> moe_combine

Backward:

  moe_combine_bwd -> moe_grouped_gemm_bwd -> moe_router_bwd_unpermute

(the last one writes dx once: the unpermute-sum of dXp plus the router's term,
and dWr).  With overlap=True the weight-gradient GEMMs run on a second stream
(moe_grouped_gemm_bwd_parts / _mx_parts), and in MXFP8 also the router's dWr
part (moe_router_bwd_unpermute_parts).  With aux_alpha > 0 the router balance
step runs after routing (moe_balance) and its loss's gradient enters the
router backward (aux_g).
With lean=True the forward does not store G and U and the backward recomputes
them (moe_grouped_gemm_recompute_gu[_mx]) before moe_grouped_gemm_bwd[_mx].

Every call is enqueued on torch's current stream; nothing is copied to the
host in between (routing metadata stays on the GPU: Olmo-core 3 overview,
"Routing and compute optimisation").
"""

from __future__ import annotations

import torch

from . import _abi


class MoELayerGPU:
    """Buffers for one layer shape.  Weights are the caller's tensors.

    mx=True runs the six grouped GEMMs in MXFP8 (E4M3 + E8M0 per 32 values,
    each operand blocked along its own GEMM's K): the routed rows of x are
    quantised straight from x (dispatch and quantisation in one pass), the
    weights are quantised in both layouts every step, dYp's MX copies come
    straight from dy (gate-scaled gather; dYp itself is not stored), and H and
    dG|dU are quantised inside the grouped-GEMM calls.  Router, combine and
    all outputs stay bf16.
    """

    def __init__(self, T: int, d: int, E: int, k: int, h: int, dtype: torch.dtype, device="cuda", mx: bool = False,
                 aux_alpha: float = 0.0, lean: bool = False, overlap: bool = False, wq_overlap: bool = True):
        self.T, self.d, self.E, self.k, self.h = T, d, E, k, h
        self.aux_alpha = float(aux_alpha)
        # memory-lean: the forward does not store G and U; the backward
        # recomputes them (one more up projection) into g / u, which then act
        # as backward scratch
        self.lean = bool(lean)
        # overlap: the weight-gradient GEMMs run on a second stream (default
        # priority) next to the dgrad chain, joined by events
        self.overlap = bool(overlap)
        # with two streams: whether the dx pass (unpermute-sum + router
        # backward) runs before the main stream joins the side stream's weight
        # gradients, i.e. next to them
        self.dx_before_join = True
        # MXFP8 with two streams: wgrad-down starts as soon as dYp's MX copies
        # exist (next to dgrad-down) instead of after dgrad-down
        self.mx_early_wgrad_down = True
        # with two streams: the router's dWr part runs on the side stream
        # right after the combine backward (the dx part stays on the main one).
        # MXFP8 only: there the side stream idles while dYp's MX copies are
        # made (wide 3.44 -> 3.42 ms/step); in bf16 it would delay wgrad-down,
        # which starts right after the combine backward (small +1%).
        self.router_dwr_on_side = bool(mx)
        self.R = R = T * k
        self.dtype = dtype
        self.mx = mx
        dev = torch.device(device)
        f32, i32 = torch.float32, torch.int32
        e = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=dev)
        self.logits = e(T, E, dt=f32)
        self.probs = e(T, E, dt=f32)
        self.topk_idx = e(T, k, dt=i32)
        self.topk_w = e(T, k, dt=f32)
        self.counts = e(E, dt=i32)
        self.offsets = e(E + 1, dt=i32)
        self.off128 = e(E + 1, dt=i32)
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
        if self.overlap:
            self.side_stream = torch.cuda.Stream(device=dev)
            self.ws_gemm2 = _abi.workspace(_abi.moe_grouped_gemm_workspace_size(E, R, d, h), dev)
            self.ws_router2 = _abi.workspace(_abi.moe_router_bwd_workspace_size(T, d, E), dev)
        # router balance step: {score, aux loss, max/mean load, min/mean load},
        # the aux loss's per-expert probability gradient and mean probabilities
        self.balance_stats = e(4, dt=f32)
        self.aux_g = e(E, dt=f32)
        self.mean_probs = e(E, dt=f32)
        self.ws_balance = _abi.workspace(_abi.moe_balance_workspace_size(T, E), dev)
        self.wq_stream = None
        if mx:
            self._alloc_mx(dev)
            if wq_overlap:
                self.wq_stream = torch.cuda.Stream(device=dev)  # default priority

    def _alloc_mx(self, dev):
        T, d, E, k, h, R = self.T, self.d, self.E, self.k, self.h, self.R
        u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device=dev)
        self.rcap = rc = (R + 127 * E + 127) // 128 * 128  # columnwise row stride
        # routed x: rowwise (up) and columnwise per expert (wgrad up)
        self.xq, self.xs, self.xqT, self.xsT = u8(R, d), u8(R, d // 32), u8(d * rc), u8(d, rc // 32)
        # weights: rowwise (forward) and blocked along the other dim (dgrad)
        # columnwise (dgrad) copies expert-major: [E*d, h] for W1/W3 (blocked on h), [E*h, d] for W2
        self.w1q, self.w1s, self.w1tq, self.w1ts = u8(E, h, d), u8(E, h, d // 32), u8(E * d, h), u8(E * d, h // 32)
        self.w3q, self.w3s, self.w3tq, self.w3ts = u8(E, h, d), u8(E, h, d // 32), u8(E * d, h), u8(E * d, h // 32)
        self.w2q, self.w2s, self.w2tq, self.w2ts = u8(E, d, h), u8(E, d, h // 32), u8(E * h, d), u8(E * h, d // 32)
        self.hq, self.hs, self.hqT, self.hsT = u8(R, h), u8(R, h // 32), u8(h * rc), u8(h, rc // 32)
        self.dyq, self.dys, self.dyqT, self.dysT = u8(R, d), u8(R, d // 32), u8(d * rc), u8(d, rc // 32)
        self.dguq, self.dgus = u8(R, 2 * h), u8(R, 2 * h // 32)
        self.dguqT, self.dgusT = u8(2 * h * rc), u8(2 * h, rc // 32)

    def quantize_w13(self, w1, w3):
        """Both MX layouts of W1 and W3 (one pass per matrix)."""
        E, d, h = self.E, self.d, self.h
        _abi.mx_quantize(w1.view(E * h, d), E * h, self.w1q.view(E * h, d), self.w1s.view(E * h, d // 32), self.w1tq,
                         self.w1ts, seg_rows=h)
        _abi.mx_quantize(w3.view(E * h, d), E * h, self.w3q.view(E * h, d), self.w3s.view(E * h, d // 32), self.w3tq,
                         self.w3ts, seg_rows=h)

    def quantize_w2(self, w2):
        """Both MX layouts of W2."""
        E, d, h = self.E, self.d, self.h
        _abi.mx_quantize(w2.view(E * d, h), E * d, self.w2q.view(E * d, h), self.w2s.view(E * d, h // 32), self.w2tq,
                         self.w2ts, seg_rows=d)

    def quantize_weights(self, w1, w3, w2):
        """Both MX layouts of every expert weight."""
        self.quantize_w13(w1, w3)
        self.quantize_w2(w2)

    # ------------------------------------------------------------------
    def forward(self, x, wr, w1, w3, w2, forced_idx=None):
        if self.mx and self.wq_stream is not None:
            # the weights' MX copies do not depend on the routing: they are made
            # on a second stream while the router and the routing run (small,
            # latency-bound launches that leave most of the GPU idle)
            main = torch.cuda.current_stream()
            ev = torch.cuda.Event()
            ev.record(main)
            with torch.cuda.stream(self.wq_stream):
                self.wq_stream.wait_event(ev)
                self.quantize_w13(w1, w3)  # the up projection waits for these
                self._ev_w13 = torch.cuda.Event()
                self._ev_w13.record(self.wq_stream)
                self.quantize_w2(w2)  # the down projection waits for this one
                self._ev_w2 = torch.cuda.Event()
                self._ev_w2.record(self.wq_stream)
        _abi.moe_router_logits(x, wr, self.logits)
        _abi.moe_route(self.logits, self.k, self.probs, self.topk_idx, self.topk_w, self.counts, self.offsets,
                       self.pos, self.src, self.ws_route, off128=self.off128, forced_idx=forced_idx,
                       err_flag=self.err_flag)
        if self.aux_alpha > 0.0:
            self.balance()
        if self.mx:
            # routed rows of x straight into their experts' MX buffers
            _abi.mx_quantize(x, self.R, self.xq, self.xs, self.xqT, self.xsT, gather_src=self.src, gather_k=self.k,
                             seg_off=self.offsets, seg_off128=self.off128)
            fields = dict(E=self.E, R=self.R, d=self.d, h=self.h, rcap=self.rcap, offsets=self.offsets,
                          off128=self.off128, xq=self.xq, xs=self.xs, w1q=self.w1q, w1s=self.w1s, w3q=self.w3q,
                          w3s=self.w3s, w2q=self.w2q, w2s=self.w2s, g=None if self.lean else self.g,
                          u=None if self.lean else self.u, hbuf=self.hb, hq=self.hq, hs=self.hs, hqT=self.hqT,
                          hsT=self.hsT, yp=self.yp, ws=self.ws_gemm, ws_bytes=self.ws_gemm.numel())
            if self.wq_stream is not None:
                # the up projection starts once W1's and W3's copies exist;
                # W2's are made meanwhile and waited for before the down one
                main = torch.cuda.current_stream()
                main.wait_event(self._ev_w13)
                _abi.moe_grouped_gemm_fwd_mx_parts(_abi.FWD_UP, **fields)
                main.wait_event(self._ev_w2)
                _abi.moe_grouped_gemm_fwd_mx_parts(_abi.FWD_DOWN, **fields)
            else:
                self.quantize_weights(w1, w3, w2)
                _abi.moe_grouped_gemm_fwd_mx(**fields)
        else:
            _abi.moe_permute(x, self.pos, self.xp)
            _abi.moe_grouped_gemm_fwd(self.xp, w1, w3, w2, self.offsets, None if self.lean else self.g,
                                      None if self.lean else self.u, self.hb, self.yp, self.ws_gemm)
        _abi.moe_combine(self.yp, self.topk_w, self.pos, self.y)
        return self.y

    def recompute_gu(self, w1, w3):
        """G and U of the current routing, bit-identical to what the forward
        would have stored (memory-lean backward)."""
        if self.mx:
            _abi.moe_grouped_gemm_recompute_gu_mx(E=self.E, R=self.R, d=self.d, h=self.h, rcap=self.rcap,
                                                  offsets=self.offsets, off128=self.off128, xq=self.xq, xs=self.xs,
                                                  w1q=self.w1q, w1s=self.w1s, w3q=self.w3q, w3s=self.w3s, g=self.g,
                                                  u=self.u, ws=self.ws_gemm, ws_bytes=self.ws_gemm.numel())
        else:
            _abi.moe_grouped_gemm_recompute_gu(self.xp, w1, w3, self.offsets, self.g, self.u, self.ws_gemm)

    def backward(self, dy, x, wr, w1, w3, w2):
        # MXFP8: dYp is not stored; its MX copies come straight from dy (gate-scaled gather)
        self._dy = dy
        _abi.moe_combine_bwd(dy, self.yp, self.topk_w, self.pos, None if self.mx else self.dyp, self.dgate)
        aux_g = self.aux_g if self.aux_alpha > 0.0 else None
        split_router = self.overlap and self.router_dwr_on_side
        if split_router:
            # the router's dWr needs only dgate: it runs on the side stream
            # ahead of the weight gradients, the dx part stays on this one
            ev_dgate = torch.cuda.Event()
            ev_dgate.record(torch.cuda.current_stream())
            with torch.cuda.stream(self.side_stream):
                self.side_stream.wait_event(ev_dgate)
                _abi.moe_router_bwd_unpermute_parts(_abi.ROUTER_DWR, self.probs, self.topk_idx, self.dgate, x, wr,
                                                    None, None, None, self.dwr, self.ws_router2, aux_g=aux_g)
        if self.lean:
            self.recompute_gu(w1, w3)
        if self.mx and self.overlap:
            self._backward_gemms_two_streams_mx()
        elif self.mx:
            _abi.moe_grouped_gemm_bwd_mx(**self._mx_bwd_fields(self.ws_gemm))
        elif self.overlap:
            self._backward_gemms_two_streams(w1, w3, w2)
        else:
            _abi.moe_grouped_gemm_bwd(self.dyp, self.xp, self.g, self.u, self.hb, w1, w3, w2, self.offsets, self.dgu,
                                      self.dxp, self.dw1, self.dw3, self.dw2, self.ws_gemm)
        # dx in one pass: the unpermute-sum of dXp plus the router's term
        if self.overlap and not self.dx_before_join:
            torch.cuda.current_stream().wait_event(self._ev_side_done)
        if split_router:
            _abi.moe_router_bwd_unpermute_parts(_abi.ROUTER_DX, self.probs, self.topk_idx, self.dgate, x, wr, self.dxp,
                                                self.pos, self.dx, None, self.ws_router, aux_g=aux_g)
        else:
            _abi.moe_router_bwd_unpermute(self.probs, self.topk_idx, self.dgate, x, wr, self.dxp, self.pos, self.dx,
                                          self.dwr, self.ws_router, aux_g=aux_g)
        if self.overlap and self.dx_before_join:
            torch.cuda.current_stream().wait_event(self._ev_side_done)
        return self.dx

    def balance(self, alpha=None):
        """Router balance step on the current routing: balance score, aux loss,
        actual max/min load over the mean, and the aux loss's gradient (all on
        the device)."""
        _abi.moe_balance(self.probs, self.counts, self.k, self.aux_alpha if alpha is None else alpha,
                         self.balance_stats, self.ws_balance, aux_g=self.aux_g, mean_probs=self.mean_probs)
        return self.balance_stats

    def _mx_bwd_fields(self, ws):
        return dict(E=self.E, R=self.R, d=self.d, h=self.h, rcap=self.rcap, offsets=self.offsets, off128=self.off128,
                    dyp=None, dy=self._dy, topk_w=self.topk_w, src=self.src, k=self.k, dyq=self.dyq, dys=self.dys, dyqT=self.dyqT, dysT=self.dysT, g=self.g, u=self.u,
                    hqT=self.hqT, hsT=self.hsT, xqT=self.xqT, xsT=self.xsT, w1tq=self.w1tq, w1ts=self.w1ts,
                    w3tq=self.w3tq, w3ts=self.w3ts, w2tq=self.w2tq, w2ts=self.w2ts, dgu=self.dgu, dguq=self.dguq,
                    dgus=self.dgus, dguqT=self.dguqT, dgusT=self.dgusT, dxp=self.dxp, dw1=self.dw1, dw3=self.dw3,
                    dw2=self.dw2, ws=ws, ws_bytes=ws.numel())

    def _backward_gemms_two_streams_mx(self):
        """MXFP8: dYp's MX copies, then wgrad-down on the side stream next to
        dgrad-down (which also makes dG|dU's copies) on the current stream,
        then wgrad-up on the side stream while dgrad-up runs."""
        main, side = torch.cuda.current_stream(), self.side_stream
        if self.mx_early_wgrad_down:
            _abi.moe_grouped_gemm_bwd_mx_parts(_abi.BWD_MX_QUANT_DY, **self._mx_bwd_fields(self.ws_gemm))
            ev_dy = torch.cuda.Event()
            ev_dy.record(main)
            with torch.cuda.stream(side):
                side.wait_event(ev_dy)
                _abi.moe_grouped_gemm_bwd_mx_parts(_abi.BWD_WGRAD_DOWN, **self._mx_bwd_fields(self.ws_gemm2))
            _abi.moe_grouped_gemm_bwd_mx_parts(_abi.BWD_DGRAD_DOWN | _abi.BWD_MX_DY_READY,
                                               **self._mx_bwd_fields(self.ws_gemm))
            side_parts = _abi.BWD_WGRAD_UP
        else:
            _abi.moe_grouped_gemm_bwd_mx_parts(_abi.BWD_DGRAD_DOWN, **self._mx_bwd_fields(self.ws_gemm))
            side_parts = _abi.BWD_WGRAD_DOWN | _abi.BWD_WGRAD_UP
        ev = torch.cuda.Event()
        ev.record(main)
        with torch.cuda.stream(side):
            side.wait_event(ev)
            _abi.moe_grouped_gemm_bwd_mx_parts(side_parts, **self._mx_bwd_fields(self.ws_gemm2))
            self._ev_side_done = torch.cuda.Event()
            self._ev_side_done.record(side)
        _abi.moe_grouped_gemm_bwd_mx_parts(_abi.BWD_DGRAD_UP, **self._mx_bwd_fields(self.ws_gemm))

    def _backward_gemms_two_streams(self, w1, w3, w2):
        """dgrad chain on the current stream, weight gradients on the side
        stream: wgrad-down as soon as dYp exists, wgrad-up once dG|dU does."""
        main, side = torch.cuda.current_stream(), self.side_stream
        args = (self.dyp, self.xp, self.g, self.u, self.hb, w1, w3, w2, self.offsets, self.dgu, self.dxp, self.dw1,
                self.dw3, self.dw2)
        ev_dyp = torch.cuda.Event()
        ev_dyp.record(main)
        with torch.cuda.stream(side):
            side.wait_event(ev_dyp)
            _abi.moe_grouped_gemm_bwd_parts(*args, _abi.BWD_WGRAD_DOWN, self.ws_gemm2)
        _abi.moe_grouped_gemm_bwd_parts(*args, _abi.BWD_DGRAD_DOWN, self.ws_gemm)
        ev_dgu = torch.cuda.Event()
        ev_dgu.record(main)
        with torch.cuda.stream(side):
            side.wait_event(ev_dgu)
            _abi.moe_grouped_gemm_bwd_parts(*args, _abi.BWD_WGRAD_UP, self.ws_gemm2)
            self._ev_side_done = torch.cuda.Event()
            self._ev_side_done.record(side)
        _abi.moe_grouped_gemm_bwd_parts(*args, _abi.BWD_DGRAD_UP, self.ws_gemm)

    def saved_tensors(self):
        """The layer's own buffers that must live from the forward to the
        backward (routing metadata excluded: it is the same in every mode;
        the caller's inputs and weights excluded)."""
        keep = [self.yp]  # combine backward: dgate = <dy, Yp>
        if self.mx:
            keep += [self.xqT, self.xsT, self.hqT, self.hsT]  # weight gradients
            keep += [self.xq, self.xs] if self.lean else [self.g, self.u]
        else:
            keep += [self.xp, self.hb]  # weight gradients (and the recompute's input)
            if not self.lean:
                keep += [self.g, self.u]
        return keep

    def saved_bytes(self):
        return sum(t.numel() * t.element_size() for t in self.saved_tensors())

    def step(self, x, wr, w1, w3, w2, dy, forced_idx=None):
        self.forward(x, wr, w1, w3, w2, forced_idx)
        self.backward(dy, x, wr, w1, w3, w2)
