"""Pins of the oracle's layer forward/backward: dense brute force, special
cases, permutation identities and float64 finite differences."""

import math

import numpy as np
import pytest

from oracle import moe_ref as ref


def _params(T, d, E, h, seed, std=0.3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) * std
    w1 = rng.standard_normal((E, h, d)) * std
    w3 = rng.standard_normal((E, h, d)) * std
    w2 = rng.standard_normal((E, d, h)) * std
    return x, wr, w1, w3, w2


def _swiglu_textbook(xt, w1e, w3e, w2e):
    """One token through one expert with Python scalars only."""
    h = len(w1e)
    hid = []
    for i in range(h):
        g = sum(a * b for a, b in zip(xt, w1e[i]))
        u = sum(a * b for a, b in zip(xt, w3e[i]))
        hid.append(g / (1.0 + math.exp(-g)) * u)
    return [sum(w2e[c][i] * hid[i] for i in range(h)) for c in range(len(w2e))]


@pytest.mark.parametrize("T,d,E,k,h,seed", [(12, 6, 4, 2, 5, 0), (9, 4, 5, 3, 3, 1), (6, 5, 3, 3, 4, 2)])
def test_sparse_equals_dense_masked_mixture(T, d, E, k, h, seed):
    """Every expert on every token, masked by the top-k set and weighted by the
    softmax probability, equals the routed (sparse) computation."""
    x, wr, w1, w3, w2 = _params(T, d, E, h, seed)
    out = ref.layer_forward(x, wr, w1, w3, w2, k)
    xl, wrl, w1l, w3l, w2l = x.tolist(), wr.tolist(), w1.tolist(), w3.tolist(), w2.tolist()
    for t in range(T):
        logits = [sum(a * b for a, b in zip(xl[t], wrl[e])) for e in range(E)]
        m = max(logits)
        den = sum(math.exp(v - m) for v in logits)
        p = [math.exp(v - m) / den for v in logits]
        chosen = sorted(range(E), key=lambda e: (-logits[e], e))[:k]
        y = [0.0] * d
        for e in range(E):
            ye = _swiglu_textbook(xl[t], w1l[e], w3l[e], w2l[e])
            mask = 1.0 if e in chosen else 0.0
            y = [a + mask * p[e] * b for a, b in zip(y, ye)]
        assert np.allclose(out["y"][t], y, rtol=1e-12, atol=1e-12)


def test_single_expert_is_plain_swiglu():
    """E = 1, k = 1: the gate is softmax over one logit = 1, so y = FFN(x)."""
    x, wr, w1, w3, w2 = _params(7, 5, 1, 6, 3)
    out = ref.layer_forward(x, wr, w1, w3, w2, 1)
    for t in range(7):
        assert np.allclose(out["y"][t], _swiglu_textbook(x[t].tolist(), w1[0].tolist(), w3[0].tolist(),
                                                          w2[0].tolist()), rtol=1e-12, atol=1e-13)


def test_k_equals_E_is_full_softmax_mixture():
    T, d, E, h = 6, 4, 3, 5
    x, wr, w1, w3, w2 = _params(T, d, E, h, 4)
    out = ref.layer_forward(x, wr, w1, w3, w2, E)
    L = x @ wr.T
    p = np.exp(L - L.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    y = np.zeros((T, d))
    for e in range(E):
        for t in range(T):
            y[t] += p[t, e] * np.array(_swiglu_textbook(x[t].tolist(), w1[e].tolist(), w3[e].tolist(),
                                                        w2[e].tolist()))
    assert np.allclose(out["y"], y, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("k", [2, 4, 8])
def test_permute_unpermute_identities(k):
    T, d, E = 37, 16, 12
    rng = np.random.default_rng(k)
    x = rng.standard_normal((T, d)).astype(np.float32)
    rt = ref.route(rng.standard_normal((T, E)).astype(np.float32), k)
    xp = ref.permute(x, rt["pos"])
    for j in range(k):
        assert (xp[rt["pos"][:, j]] == x).all()
    assert (xp == x[rt["src"] // k]).all()
    # adjoint: a sum of k equal values is k*x exactly (k a power of two)
    assert (ref.unpermute_sum(xp, rt["pos"]) == k * x.astype(np.float64)).all()
    # one-hot gates make combine a gather of slot 0
    onehot = np.zeros((T, k))
    onehot[:, 0] = 1
    assert (ref.combine(xp, onehot, rt["pos"]) == x[:, :].astype(np.float64)).all()


def _loss(x, wr, w1, w3, w2, k, dy):
    return float(np.sum(ref.layer_forward(x, wr, w1, w3, w2, k)["y"] * dy))


@pytest.mark.parametrize("T,d,E,k,h,seed", [(10, 6, 5, 2, 4, 0), (8, 4, 4, 3, 6, 1)])
def test_backward_matches_finite_differences(T, d, E, k, h, seed):
    x, wr, w1, w3, w2 = _params(T, d, E, h, seed)
    dy = np.random.default_rng(seed + 100).standard_normal((T, d))
    fwd = ref.layer_forward(x, wr, w1, w3, w2, k)
    g = ref.layer_backward(fwd, dy, x, wr, w1, w3, w2)
    params = {"x": x, "wr": wr, "w1": w1, "w3": w3, "w2": w2}
    grads = {"x": g["dx"], "wr": g["dwr"], "w1": g["dw1"], "w3": g["dw3"], "w2": g["dw2"]}
    rng = np.random.default_rng(seed + 7)
    eps = 1e-6
    for name, arr in params.items():
        checked = 0
        tries = 0
        while checked < 6 and tries < 60:
            tries += 1
            i = tuple(int(rng.integers(s)) for s in arr.shape)
            old = arr[i]
            arr[i] = old + eps
            fp = ref.layer_forward(x, wr, w1, w3, w2, k)
            lp = float(np.sum(fp["y"] * dy))
            arr[i] = old - eps
            fm = ref.layer_forward(x, wr, w1, w3, w2, k)
            lm = float(np.sum(fm["y"] * dy))
            arr[i] = old
            if not ((fp["idx"] == fwd["idx"]).all() and (fm["idx"] == fwd["idx"]).all()):
                continue            # routing changed at +-eps: resample the coordinate
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grads[name][i]) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, grads[name][i])
            checked += 1
        assert checked >= 3, name


def test_gate_gradient_and_softmax_backward():
    T, d, E, k, h = 9, 5, 6, 3, 4
    x, wr, w1, w3, w2 = _params(T, d, E, h, 11)
    dy = np.random.default_rng(5).standard_normal((T, d))
    fwd = ref.layer_forward(x, wr, w1, w3, w2, k)
    g = ref.layer_backward(fwd, dy, x, wr, w1, w3, w2)
    # dgate[t, j] = <dy[t], Yp[pos[t, j]]> and the loss is linear in each gate
    for t in range(T):
        for j in range(k):
            assert abs(g["dgate"][t, j] - float(dy[t] @ fwd["yp"][fwd["pos"][t, j]])) < 1e-12
            w = fwd["w"].copy()
            w[t, j] += 1.0
            dl = float(np.sum((ref.combine(fwd["yp"], w, fwd["pos"]) - fwd["y"]) * dy))
            assert abs(dl - g["dgate"][t, j]) < 1e-11
    # softmax backward rows sum to zero (probabilities sum to one)
    assert np.allclose(g["dlogits"].sum(1), 0, atol=1e-13)


def test_swiglu_backward_finite_difference():
    rng = np.random.default_rng(2)
    G = rng.standard_normal(50) * 3
    U = rng.standard_normal(50)
    dH = rng.standard_normal(50)
    dG, dU = ref.swiglu_backward(dH, G, U)
    eps = 1e-6
    f = lambda g, u: np.sum(dH * ref.silu(g) * u)
    for i in range(50):
        e = np.zeros(50)
        e[i] = eps
        assert abs((f(G + e, U) - f(G - e, U)) / (2 * eps) - dG[i]) < 1e-7
        assert abs((f(G, U + e) - f(G, U - e)) / (2 * eps) - dU[i]) < 1e-7


def test_forced_routing_keeps_softmax_gates():
    T, d, E, k, h = 8, 4, 6, 2, 3
    x, wr, w1, w3, w2 = _params(T, d, E, h, 9)
    idx = np.stack([np.arange(T) % E, (np.arange(T) + 3) % E], 1)
    out = ref.layer_forward(x, wr, w1, w3, w2, k, forced_idx=idx)
    p = ref.softmax(x @ wr.T)
    assert np.allclose(out["w"], np.take_along_axis(p, idx, 1), atol=1e-15)
    assert (out["idx"] == idx).all()
