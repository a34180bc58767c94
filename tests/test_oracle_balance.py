"""Pins of the router balance oracle (oracle/balance_ref.py).

- closed form: balanced routing with uniform probabilities gives score 1,
  loss alpha, actual balance 1 and a zero logit gradient;
- the hand-worked gerrymandering case of tests/golden/ (score improves while
  the actual load balance gets worse);
- central finite differences of sum <dy, y> + alpha * score with respect to
  Wr and x against layer_backward(..., aux_alpha) (routing unchanged at +-eps).
"""

import os

import numpy as np
import pytest

from oracle import balance_ref as bal
from oracle import moe_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_uniform_closed_form():
    T, E, k, alpha = 8, 4, 2, 0.01
    idx = np.array([[(t + j) % E for j in range(k)] for t in range(T)])
    rt = ref.route(np.zeros((T, E), np.float32), k, forced_idx=idx)
    assert (rt["counts"] == T * k // E).all()
    b = bal.balance(rt["probs"], rt["counts"], k, alpha)
    assert b["score"] == pytest.approx(1.0, abs=1e-15)
    assert b["loss"] == pytest.approx(alpha, abs=1e-15)
    assert b["max_over_mean"] == 1.0
    assert np.allclose(b["g"], alpha / T)
    # a gradient that is the same for every expert vanishes through the softmax
    dL, _, _ = ref.router_backward(rt["probs"], rt["idx"], np.zeros((T, k)), np.ones((T, 3)), np.ones((E, 3)),
                                   aux_g=b["g"])
    assert np.abs(dL).max() < 1e-18


def _golden():
    cases = []
    with open(os.path.join(GOLDEN, "balance_gerrymander_hand.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, k, alpha, probs, counts, score, actual, loss, g = [p.strip() for p in line.split("|")]
                p = np.array([[float(v) for v in row.split()] for row in probs.split(";")])
                cases.append((name, int(k), float(alpha), p, np.array([int(v) for v in counts.split()]),
                              float(score), float(actual), float(loss), np.array([float(v) for v in g.split()])))
    return cases


def test_gerrymandering_hand_case():
    res = {}
    for name, k, alpha, p, counts, score, actual, loss, g in _golden():
        # the counts are the top-k choice of these probabilities
        idx = ref.topk_experts(p, k)
        assert (np.bincount(idx.ravel(), minlength=p.shape[1]) == counts).all(), name
        b = bal.balance(p, counts, k, alpha)
        assert b["score"] == pytest.approx(score, abs=1e-12), name
        assert b["max_over_mean"] == pytest.approx(actual, abs=1e-12), name
        assert b["loss"] == pytest.approx(loss, abs=1e-12), name
        assert np.allclose(b["g"], g, atol=1e-15), name
        res[name] = b
    # the pitfall: the score says "better", the actual balance says "worse"
    assert res["gerrymandered"]["score"] < res["balanced"]["score"]
    assert res["gerrymandered"]["max_over_mean"] > res["balanced"]["max_over_mean"]


def _params(T, d, E, h, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, d)), rng.standard_normal((E, d)) * 0.5,
            rng.standard_normal((E, h, d)) * 0.3, rng.standard_normal((E, h, d)) * 0.3,
            rng.standard_normal((E, d, h)) * 0.3)


@pytest.mark.parametrize("T,d,E,k,h,seed,alpha", [(10, 6, 5, 2, 4, 0, 0.3), (12, 4, 4, 1, 3, 2, 1.0)])
def test_aux_gradient_matches_finite_differences(T, d, E, k, h, seed, alpha):
    x, wr, w1, w3, w2 = _params(T, d, E, h, seed)
    dy = np.random.default_rng(seed + 100).standard_normal((T, d))

    def loss(f):
        return float(np.sum(f["y"] * dy)) + bal.balance(f["probs"], f["counts"], k, alpha)["loss"]

    fwd = ref.layer_forward(x, wr, w1, w3, w2, k)
    g = ref.layer_backward(fwd, dy, x, wr, w1, w3, w2, aux_alpha=alpha)
    g0 = ref.layer_backward(fwd, dy, x, wr, w1, w3, w2)
    assert not np.allclose(g["dwr"], g0["dwr"])  # the balance term does reach the router
    rng = np.random.default_rng(seed + 7)
    eps = 1e-6
    for name, arr, grad in (("wr", wr, g["dwr"]), ("x", x, g["dx"])):
        checked = tries = 0
        while checked < 6 and tries < 60:
            tries += 1
            i = tuple(int(rng.integers(s)) for s in arr.shape)
            old = arr[i]
            arr[i] = old + eps
            fp = ref.layer_forward(x, wr, w1, w3, w2, k)
            arr[i] = old - eps
            fm = ref.layer_forward(x, wr, w1, w3, w2, k)
            arr[i] = old
            if not ((fp["idx"] == fwd["idx"]).all() and (fm["idx"] == fwd["idx"]).all()):
                continue  # routing changed at +-eps: resample the coordinate
            fd = (loss(fp) - loss(fm)) / (2 * eps)
            assert abs(fd - grad[i]) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, grad[i])
            checked += 1
        assert checked >= 3, name
