"""Plain CPU oracle of the MoE expert layer, forward and backward (float64 numpy).

Test infrastructure only (see the package header).  Nothing here is blocked,
fused or reordered: each step is the definition written out, one expert at a
time, with numpy's matmul as the only library primitive.

The layer (one GPU's share of an Olmo-core 3 style MoE block):
  route    -- softmax over the router logits, top-k experts per token, and the
              routing metadata (counts, offsets, positions) [OC3 "Routing and
              compute optimisation": routing metadata is kept on the GPU].
  permute  -- each routed (token, slot) row is written once, straight into its
              expert's contiguous input block [OC3 same section: routed tokens
              go directly into the experts' input buffers; AI2 "Trillion-
              parameter tests, open access" says the same].
  experts  -- every expert's FFN over its block; on the GPU this is one grouped
              GEMM over all experts [OC3 same section; TH "Scaling and
              optimising MoE training"].
  combine  -- each token's output is the gate-weighted sum of its k expert rows
              (the inverse of the dispatch).

Readings taken where the pages are silent (plainest reading):
  * router: logits = x Wr^T; probabilities = softmax over all E experts; the k
    experts with the largest logits are chosen, ties to the lower expert index;
    slot j holds the j-th largest.  Selection compares the float32 logits
    themselves (softmax is monotone, so this is the same order and avoids
    rounding-made ties); the gate of slot j is the softmax probability of that
    expert, not renormalised over the k chosen.
  * forced routing (random-routing stress modes): indices are given; gates are
    still the router softmax probabilities of the given experts.
  * dropless: every routed row is kept; sum(counts) = T*k.
  * offsets are the exclusive prefix sum of counts (length E+1, unpadded);
    within an expert, rows are in ascending token order (a stable counting
    sort; unique because a token never picks an expert twice).  ``off128`` is
    the same prefix sum over counts rounded up to 128 (starts of the MX
    column segments; a layout choice, the pages fix none).
  * expert FFN: SwiGLU without biases, silu on the W1 branch:
    G = Xp W1^T, U = Xp W3^T, H = silu(G) * U, Yp = H W2^T.
    Weight layouts: w1, w3 [E, h, d]; w2 [E, d, h] (output, input).
  * combine: y[t] = sum_j w[t, j] * Yp[pos[t, j]], gate applied here.
  * backward of the loss sum_t <dy[t], y[t]>; indices are not differentiated,
    the router gradient flows through the gates only.
"""

from __future__ import annotations

import numpy as np

F = np.float64


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

def router_logits(x, wr, dtype=F):
    """L[t, e] = <x[t], Wr[e]> (router of the MoE block)."""
    return np.asarray(x, dtype) @ np.asarray(wr, dtype).T


def softmax(logits, dtype=F):
    """Row softmax, max-subtracted."""
    L = np.asarray(logits, dtype)
    z = L - L.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def topk_experts(logits, k):
    """Indices of the k largest logits per row; ties go to the lower index.

    A stable sort of the negated logits orders experts by (-logit, index); the
    first k are the chosen ones, in slot order.  The comparison is done on the
    logits exactly as given (no conversion changes float32 ordering).
    """
    L = np.asarray(logits)
    order = np.argsort(-L, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :k].astype(np.int64))


def route(logits, k, forced_idx=None, dtype=F):
    """Routing step of the layer: gates and the GPU-resident metadata.

    Returns a dict with
      probs [T,E], idx [T,k], w [T,k]  -- softmax, chosen experts, gates
      counts [E], offsets [E+1]        -- histogram and its exclusive prefix sum
      pos [T,k]  -- row of (t, j) in the expert-contiguous buffer
      src [R]    -- inverse map: src[pos[t, j]] = t*k + j
      off128 [E+1] -- prefix sum of counts rounded up to multiples of 128
    """
    L = np.asarray(logits)
    T, E = L.shape
    probs = softmax(L, dtype)
    idx = topk_experts(L, k) if forced_idx is None else np.asarray(forced_idx, np.int64)
    w = np.take_along_axis(probs, idx, axis=1)
    flat = idx.reshape(-1)                     # entry t*k + j
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    # stable sort of the (t, j) entries by expert: rows of one expert keep
    # ascending token order
    src = np.argsort(flat, kind="stable").astype(np.int64)
    pos = np.empty(T * k, np.int64)
    pos[src] = np.arange(T * k)
    pos = pos.reshape(T, k)
    c128 = (counts + 127) // 128 * 128
    off128 = np.concatenate([[0], np.cumsum(c128)]).astype(np.int64)
    return dict(probs=probs, idx=idx, w=w, counts=counts, offsets=offsets, pos=pos,
                src=src, off128=off128)


# ----------------------------------------------------------------------------
# dispatch / combine
# ----------------------------------------------------------------------------

def permute(x, pos):
    """Xp[pos[t, j]] = x[t]: every routed row lands in its expert's block."""
    x = np.asarray(x)
    T, k = pos.shape
    xp = np.zeros((T * k, x.shape[1]), x.dtype)
    for j in range(k):
        xp[pos[:, j]] = x
    return xp


def combine(yp, w, pos, dtype=F):
    """y[t] = sum_j w[t, j] * Yp[pos[t, j]], summed in slot order."""
    T, k = pos.shape
    yp = np.asarray(yp, dtype)
    y = np.zeros((T, yp.shape[1]), dtype)
    for j in range(k):
        y += np.asarray(w, dtype)[:, j:j + 1] * yp[pos[:, j]]
    return y


def unpermute_sum(dxp, pos, dtype=F):
    """dx[t] = sum_j dXp[pos[t, j]] (adjoint of ``permute``)."""
    T, k = pos.shape
    dxp = np.asarray(dxp, dtype)
    dx = np.zeros((T, dxp.shape[1]), dtype)
    for j in range(k):
        dx += dxp[pos[:, j]]
    return dx


# ----------------------------------------------------------------------------
# experts (SwiGLU FFN), one expert at a time
# ----------------------------------------------------------------------------

def silu(z):
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def experts_forward(xp, offsets, w1, w3, w2, dtype=F):
    """Per expert e over rows [off_e, off_{e+1}): G, U, H = silu(G)*U, Yp = H W2^T."""
    xp = np.asarray(xp, dtype)
    R = xp.shape[0]
    E = len(offsets) - 1
    h = w1.shape[1]
    d = w2.shape[1]
    G = np.zeros((R, h), dtype)
    U = np.zeros((R, h), dtype)
    yp = np.zeros((R, d), dtype)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        G[a:b] = xp[a:b] @ np.asarray(w1[e], dtype).T
        U[a:b] = xp[a:b] @ np.asarray(w3[e], dtype).T
    H = silu(G) * U
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        yp[a:b] = H[a:b] @ np.asarray(w2[e], dtype).T
    return G, U, H, yp


def swiglu_backward(dH, G, U):
    """Chain rule of H = silu(G) * U with s = sigmoid(G):
    dU = dH * silu(G);  dG = dH * U * s * (1 + G (1 - s))."""
    s = sigmoid(G)
    dU = dH * G * s
    dG = dH * U * s * (1.0 + G * (1.0 - s))
    return dG, dU


def experts_backward(dyp, xp, G, U, H, offsets, w1, w3, w2, dtype=F):
    """Backward of ``experts_forward`` given dYp.

    dH = dYp W2[e];  (dG, dU) from the SwiGLU chain rule;
    dW2[e] = dYp_e^T H_e;  dW1[e] = dG_e^T Xp_e;  dW3[e] = dU_e^T Xp_e;
    dXp = dG W1[e] + dU W3[e].
    """
    dyp = np.asarray(dyp, dtype)
    xp = np.asarray(xp, dtype)
    R = xp.shape[0]
    E = len(offsets) - 1
    h, d = w1.shape[1], w1.shape[2]
    dH = np.zeros((R, h), dtype)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a < b:
            dH[a:b] = dyp[a:b] @ np.asarray(w2[e], dtype)
    dG, dU = swiglu_backward(dH, np.asarray(G, dtype), np.asarray(U, dtype))
    dxp = np.zeros((R, d), dtype)
    dw1 = np.zeros((E, h, d), dtype)
    dw3 = np.zeros((E, h, d), dtype)
    dw2 = np.zeros((E, d, h), dtype)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        dw2[e] = dyp[a:b].T @ np.asarray(H[a:b], dtype)
        dw1[e] = dG[a:b].T @ xp[a:b]
        dw3[e] = dU[a:b].T @ xp[a:b]
        dxp[a:b] = dG[a:b] @ np.asarray(w1[e], dtype) + dU[a:b] @ np.asarray(w3[e], dtype)
    return dict(dH=dH, dG=dG, dU=dU, dxp=dxp, dw1=dw1, dw3=dw3, dw2=dw2)


# ----------------------------------------------------------------------------
# combine backward and router backward
# ----------------------------------------------------------------------------

def combine_backward(dy, yp, w, pos, dtype=F):
    """dYp[pos[t, j]] = w[t, j] dy[t];  dgate[t, j] = <dy[t], Yp[pos[t, j]]>."""
    dy = np.asarray(dy, dtype)
    yp = np.asarray(yp, dtype)
    T, k = pos.shape
    dyp = np.zeros_like(yp)
    dgate = np.zeros((T, k), dtype)
    for j in range(k):
        dyp[pos[:, j]] = np.asarray(w, dtype)[:, j:j + 1] * dy
        dgate[:, j] = np.sum(dy * yp[pos[:, j]], axis=1)
    return dyp, dgate


def router_backward(probs, idx, dgate, x, wr, dtype=F, aux_g=None):
    """Gradient through gates w = probs[idx] into the logits, Wr and x.

    g[t, e] = dgate[t, j] where e = idx[t, j], else 0;  plus aux_g[e] for every
    t when the balance loss is on (see oracle/balance_ref.py);
    dL = p * (g - sum_e p g)  (softmax Jacobian);  dWr = dL^T x;  dx_r = dL Wr.
    """
    p = np.asarray(probs, dtype)
    T, E = p.shape
    g = np.zeros((T, E), dtype)
    np.put_along_axis(g, np.asarray(idx), np.asarray(dgate, dtype), axis=1)
    if aux_g is not None:
        g = g + np.asarray(aux_g, dtype)[None, :]
    dL = p * (g - np.sum(p * g, axis=1, keepdims=True))
    dwr = dL.T @ np.asarray(x, dtype)
    dx_r = dL @ np.asarray(wr, dtype)
    return dL, dwr, dx_r


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def layer_forward(x, wr, w1, w3, w2, k, forced_idx=None, logits=None, dtype=F):
    """Forward of the layer.  ``logits`` may be supplied (routing is then
    decided on exactly those float32 values); otherwise they are x Wr^T."""
    L = router_logits(x, wr, dtype) if logits is None else np.asarray(logits)
    rt = route(L, k, forced_idx, dtype)
    xp = permute(np.asarray(x, dtype), rt["pos"])
    G, U, H, yp = experts_forward(xp, rt["offsets"], w1, w3, w2, dtype)
    y = combine(yp, rt["w"], rt["pos"], dtype)
    return dict(logits=L, **rt, xp=xp, G=G, U=U, H=H, yp=yp, y=y)


def layer_backward(fwd, dy, x, wr, w1, w3, w2, dtype=F, aux_alpha=0.0):
    """Backward of ``layer_forward`` for upstream gradient dy.  With aux_alpha
    > 0 the loss also holds the balance term alpha * score
    (oracle/balance_ref.py), whose gradient enters the router backward."""
    dyp, dgate = combine_backward(dy, fwd["yp"], fwd["w"], fwd["pos"], dtype)
    eb = experts_backward(dyp, fwd["xp"], fwd["G"], fwd["U"], fwd["H"], fwd["offsets"],
                          w1, w3, w2, dtype)
    dx_e = unpermute_sum(eb["dxp"], fwd["pos"], dtype)
    aux_g = None
    if aux_alpha:
        from oracle import balance_ref
        aux_g = balance_ref.balance(fwd["probs"], fwd["counts"], fwd["idx"].shape[1], aux_alpha, dtype)["g"]
    dL, dwr, dx_r = router_backward(fwd["probs"], fwd["idx"], dgate, x, wr, dtype, aux_g=aux_g)
    return dict(dyp=dyp, dgate=dgate, dlogits=dL, dx_e=dx_e, dx=dx_e + dx_r, dwr=dwr, **eb)
