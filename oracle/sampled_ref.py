"""Sampled outputs of the layer at full workload size (float64 numpy).

Test infrastructure only (see the package header).

At the workloads' own sizes the whole-layer oracle (``moe_ref.layer_forward`` /
``layer_backward`` and their MXFP8 twins) would take minutes and, for the
trillion shape, hundreds of GB of float64 weight gradients.  Every output
checked here depends on a few rows only, so it is computed on its own, from
the same definitions and in the same order as the whole-layer oracle:

  token t      y[t] = sum_j w[t, j] FFN_{e_j}(x[t])                 (combine)
               dgate[t, j] = <dy[t], Yp of (t, j)>
               dx[t] = sum_j dXp of (t, j) + dL[t] Wr                 (unpermute-sum
                                                                      + router backward)
  expert e     rows i of dW1[e] = dG_e[:, i]^T Xp_e and dW3[e] = dU_e[:, i]^T Xp_e,
               column i of dW2[e] = dYp_e^T H_e[:, i], over the expert's routed
               rows in segment order (ascending token)

Each routed row's forward and data gradient involve only its token, its
expert's weights and its gate [OC3 "Routing and compute optimisation": one
FFN per expert over the rows routed to it]; a weight gradient's row or column
involves only its expert's rows.  The MXFP8 variant applies the quantise-
dequantise steps of ``moe_mx_ref`` at the same places: rowwise operands are
blocked along their own row, the weights along their GEMM's K, and the weight
gradients' operands in 32-row blocks along the expert's segment (one segment
here, which is how the full layer blocks it too).

``tests/test_oracle_sampled.py`` pins both functions to the whole-layer
oracles on small problems (the same values to 1e-12).
"""

from __future__ import annotations

import numpy as np

from . import moe_mx_ref as mxl
from . import moe_ref as ref
from . import mx_ref as mx


def _q_rows(a, on):
    return mx.qdq_rows(a) if on else a


def _bf(a, on):
    return mxl.bf16_value(a) if on else a


def tokens(x_s, dy_s, logits_s, idx_s, wr, experts, w1_e, w3_e, w2_e, mx_on=False):
    """y, dgate and dx of the sampled tokens.

    x_s, dy_s [S, d]; logits_s [S, E] (float32, as routed); idx_s [S, k] (the
    routing's expert choice); wr [E, d]; experts: sorted expert ids, with
    w1_e[i], w3_e[i] [h, d] and w2_e[i] [d, h] the weights of experts[i].
    """
    x_s = np.asarray(x_s, np.float64)
    dy_s = np.asarray(dy_s, np.float64)
    idx_s = np.asarray(idx_s)
    S, k = idx_s.shape
    d = x_s.shape[1]
    p = ref.softmax(logits_s)
    w = np.take_along_axis(p, idx_s, axis=1)
    where = {int(e): i for i, e in enumerate(experts)}
    # each expert's weights as its GEMMs see them
    W = {}
    for e, i in where.items():
        w1 = np.asarray(w1_e[i], np.float64)
        w3 = np.asarray(w3_e[i], np.float64)
        w2 = np.asarray(w2_e[i], np.float64)
        if mx_on:
            W[e] = dict(w1f=mx.qdq_rows(w1), w3f=mx.qdq_rows(w3), w2f=mx.qdq_rows(w2),
                        w2b=mx.qdq_cols(w2), w1b=mx.qdq_cols(w1), w3b=mx.qdq_cols(w3))
        else:
            W[e] = dict(w1f=w1, w3f=w3, w2f=w2, w2b=w2, w1b=w1, w3b=w3)
    y = np.zeros((S, d))
    dgate = np.zeros((S, k))
    dx_e = np.zeros((S, d))
    for s in range(S):
        xq = _q_rows(x_s[s:s + 1], mx_on)
        for j in range(k):
            m = W[int(idx_s[s, j])]
            G = xq @ m["w1f"].T
            U = xq @ m["w3f"].T
            H = _bf(ref.silu(G) * U, mx_on)
            yp = _q_rows(H, mx_on) @ m["w2f"].T
            y[s] += w[s, j] * yp[0]
            dgate[s, j] = float(np.sum(dy_s[s] * yp[0]))
            dyp = _bf(w[s, j] * dy_s[s:s + 1], mx_on)
            dH = _q_rows(dyp, mx_on) @ m["w2b"]
            dG, dU = ref.swiglu_backward(dH, _bf(G, mx_on), _bf(U, mx_on))
            dG, dU = _bf(dG, mx_on), _bf(dU, mx_on)
            dx_e[s] += (_q_rows(dG, mx_on) @ m["w1b"] + _q_rows(dU, mx_on) @ m["w3b"])[0]
    _, _, dx_r = ref.router_backward(p, idx_s, dgate, x_s, wr)
    return dict(y=y, dgate=dgate, dx=dx_e + dx_r, w=w, probs=p)


def expert_slices(x_e, dy_e, gate_e, w1, w3, w2, hid, mx_on=False):
    """Rows ``hid`` of dW1[e] and dW3[e] ([len(hid), d] each) and columns ``hid``
    of dW2[e] ([d, len(hid)]) for one expert.

    x_e, dy_e [n, d]: the tokens of the expert's routed rows, in segment order;
    gate_e [n]: their gates; w1, w3 [h, d], w2 [d, h]: the expert's weights.
    """
    x_e = np.asarray(x_e, np.float64)
    n = x_e.shape[0]
    hid = np.asarray(hid)
    w1 = np.asarray(w1, np.float64)
    w3 = np.asarray(w3, np.float64)
    w2 = np.asarray(w2, np.float64)
    dyp = _bf(np.asarray(gate_e, np.float64)[:, None] * np.asarray(dy_e, np.float64), mx_on)
    if mx_on:
        xq = mx.qdq_rows(x_e)
        G = xq @ mx.qdq_rows(w1)[hid].T
        U = xq @ mx.qdq_rows(w3)[hid].T
        dH = mx.qdq_rows(dyp) @ mx.qdq_cols(w2)[:, hid]
    else:
        G = x_e @ w1[hid].T
        U = x_e @ w3[hid].T
        dH = dyp @ w2[:, hid]
    H = _bf(ref.silu(G) * U, mx_on)
    dG, dU = ref.swiglu_backward(dH, _bf(G, mx_on), _bf(U, mx_on))
    dG, dU = _bf(dG, mx_on), _bf(dU, mx_on)
    if mx_on:
        # one segment of n rows, padded to whole 32-row blocks with zeros
        seg, pad = np.array([0, n]), np.array([0, (n + 127) // 128 * 128])
        col = lambda a: mx.qdq_cols_segmented(a, seg, pad)  # noqa: E731
        dG, dU, xs, H, dyp = col(dG), col(dU), col(x_e), col(H), col(dyp)
    else:
        xs = x_e
    return dict(dw1=dG.T @ xs, dw3=dU.T @ xs, dw2=dyp.T @ H)
