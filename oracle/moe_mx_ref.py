"""MXFP8 variant of the layer oracle: the float64 layer run on dequantised values.

Test infrastructure only (see the package header).

Every grouped-GEMM operand is quantised to MX (E4M3 + E8M0 per 32 values)
along its own GEMM's reduction dimension, then dequantised, and the product is
taken in float64 ("quantise-dequantise", QDQ).  Router, combine, unpermute and
the router backward stay unquantised.  Readings (the pages only name the
format and where its gain comes from [OC3 "Precision optimisation with
MXFP8"]):

  GEMM          A operand (blocked on K)          B operand (blocked on K)
  up   fwd      Xp rowwise (K = d)                W1, W3 rowwise (K = d)
  down fwd      H rowwise (K = h)                 W2 rowwise (K = h)
  dgrad down    dYp rowwise (K = d)               W2 along d (columns of [d, h])
  wgrad down    dYp column/segment (K = rows)     H column/segment
  dgrad up      dG, dU rowwise (K = h)            W1, W3 along h (columns of [h, d])
  wgrad up      dG, dU column/segment             Xp column/segment

Quantisation sources are bfloat16 values: tensors the layer stores in bf16
(H, dYp, dG, dU) are rounded to bf16 before they are quantised; inputs and
weights already are bf16.  Every MX copy is made from its bf16 source, never
from another MX copy.
"""

from __future__ import annotations

import numpy as np

from . import moe_ref as ref
from . import mx_ref as mx


def bf16_value(v):
    """Nearest bfloat16 value (8 significant bits, ties to even), as float64."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -126)
    spacing = np.ldexp(1.0, e - 7)
    return np.copysign(np.rint(a / spacing) * spacing, v)


def layer_forward_mx(x, wr, w1, w3, w2, k, forced_idx=None, logits=None):
    L = ref.router_logits(x, wr) if logits is None else np.asarray(logits)
    rt = ref.route(L, k, forced_idx)
    offsets = rt["offsets"]
    E = len(offsets) - 1
    xp = ref.permute(np.asarray(x, np.float64), rt["pos"])
    xq = mx.qdq_rows(xp)
    R, h, d = xp.shape[0], w1.shape[1], w1.shape[2]
    G = np.zeros((R, h))
    U = np.zeros((R, h))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a < b:
            G[a:b] = xq[a:b] @ mx.qdq_rows(w1[e]).T
            U[a:b] = xq[a:b] @ mx.qdq_rows(w3[e]).T
    H = bf16_value(ref.silu(G) * U)
    hq = mx.qdq_rows(H)
    yp = np.zeros((R, d))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a < b:
            yp[a:b] = hq[a:b] @ mx.qdq_rows(w2[e]).T
    y = ref.combine(yp, rt["w"], rt["pos"])
    return dict(logits=L, **rt, xp=xp, G=bf16_value(G), U=bf16_value(U), H=H, yp=yp, y=y)


def layer_backward_mx(fwd, dy, x, wr, w1, w3, w2):
    offsets, off128, pos = fwd["offsets"], fwd["off128"], fwd["pos"]
    E = len(offsets) - 1
    dyp, dgate = ref.combine_backward(dy, fwd["yp"], fwd["w"], pos)
    dyp = bf16_value(dyp)
    R, h, d = fwd["xp"].shape[0], w1.shape[1], w1.shape[2]
    dyq_r = mx.qdq_rows(dyp)
    dH = np.zeros((R, h))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a < b:
            dH[a:b] = dyq_r[a:b] @ mx.qdq_cols(w2[e])
    dG, dU = ref.swiglu_backward(dH, fwd["G"], fwd["U"])
    dG, dU = bf16_value(dG), bf16_value(dU)
    dyq_c = mx.qdq_cols_segmented(dyp, offsets, off128)
    hq_c = mx.qdq_cols_segmented(fwd["H"], offsets, off128)
    dgq_c = mx.qdq_cols_segmented(dG, offsets, off128)
    duq_c = mx.qdq_cols_segmented(dU, offsets, off128)
    xq_c = mx.qdq_cols_segmented(fwd["xp"], offsets, off128)
    dgq_r, duq_r = mx.qdq_rows(dG), mx.qdq_rows(dU)
    dxp = np.zeros((R, d))
    dw1 = np.zeros((E, h, d))
    dw3 = np.zeros((E, h, d))
    dw2 = np.zeros((E, d, h))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        dw2[e] = dyq_c[a:b].T @ hq_c[a:b]
        dw1[e] = dgq_c[a:b].T @ xq_c[a:b]
        dw3[e] = duq_c[a:b].T @ xq_c[a:b]
        dxp[a:b] = dgq_r[a:b] @ mx.qdq_cols(w1[e]) + duq_r[a:b] @ mx.qdq_cols(w3[e])
    dx_e = ref.unpermute_sum(dxp, pos)
    dL, dwr, dx_r = ref.router_backward(fwd["probs"], fwd["idx"], dgate, x, wr)
    return dict(dyp=dyp, dgate=dgate, dlogits=dL, dG=dG, dU=dU, dxp=dxp, dx_e=dx_e,
                dx=dx_e + dx_r, dwr=dwr, dw1=dw1, dw3=dw3, dw2=dw2)
