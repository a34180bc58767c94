"""GPU parity of the router balance step (moe_balance, moe_router_bwd_aux)
against oracle/balance_ref.py and the oracle layer with the balance loss on.

Inputs: routing probabilities and counts from the oracle's routing of seeded
logits (router, uniform or Zipf choice), in float32 as moe_route writes them.
"""

import numpy as np
import pytest
import torch

from oracle import balance_ref as bal
from oracle import moe_ref as ref
from token_routing_grouped_amd import configs, inputs

from helpers import assert_close, say, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _routing(T, E, k, mode, seed):
    L = (np.random.default_rng(seed).standard_normal((T, E)) * 0.9).astype(np.float32)
    forced = None if mode == "router" else inputs.forced_routing(mode, T, E, k, seed)
    rt = ref.route(L, k, forced_idx=forced)
    return rt["probs"].astype(np.float32), rt["counts"].astype(np.int32)


def _gpu_balance(probs, counts, k, alpha):
    from token_routing_grouped_amd import _abi

    T, E = probs.shape
    p = torch.from_numpy(np.ascontiguousarray(probs)).to(DEV)
    c = torch.from_numpy(counts).to(DEV)
    stats = torch.full((4,), float("nan"), device=DEV)
    g = torch.full((E,), float("nan"), device=DEV)
    P = torch.full((E,), float("nan"), device=DEV)
    ws = _abi.workspace(_abi.moe_balance_workspace_size(T, E), DEV)
    _abi.moe_balance(p, c, k, alpha, stats, ws, aux_g=g, mean_probs=P)
    torch.cuda.synchronize()
    return to_np(stats), to_np(g), to_np(P)


CASES = [(1, 8, 2, "router"), (256, 8, 2, "router"), (8192, 8, 4, "router"), (16384, 128, 4, "zipf"),
         (4096, 384, 8, "uniform"), (300, 1024, 8, "router"), (513, 5, 5, "router")]


@pytest.mark.parametrize("T,E,k,mode", CASES)
def test_balance_matches_oracle(T, E, k, mode):
    say(f"balance T={T} E={E} k={k} {mode}")
    probs, counts = _routing(T, E, k, mode, T + E + k)
    alpha = 0.01
    stats, g, P = _gpu_balance(probs, counts, k, alpha)
    b = bal.balance(probs, counts, k, alpha)
    assert stats[0] == pytest.approx(b["score"], rel=1e-5)
    assert stats[1] == pytest.approx(b["loss"], rel=1e-5)
    assert stats[2] == pytest.approx(b["max_over_mean"], rel=1e-6)
    assert stats[3] == pytest.approx(float(counts.min()) / (T * k / E), rel=1e-6)
    assert np.allclose(g, b["g"], rtol=1e-5, atol=0)
    assert np.allclose(P, b["P"], rtol=1e-5, atol=1e-9)


def test_balance_gerrymandering_case_on_gpu():
    """The hand-worked golden case: the score ranks the two states the other way
    round from the actual load balance."""
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "balance_gerrymander_hand.txt")
    got = {}
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            name, k, alpha, probs, counts, score, actual, loss, g = [p.strip() for p in line.split("|")]
            p = np.array([[float(v) for v in row.split()] for row in probs.split(";")], np.float32)
            c = np.array([int(v) for v in counts.split()], np.int32)
            stats, gg, _ = _gpu_balance(p, c, int(k), float(alpha))
            assert stats[0] == pytest.approx(float(score), rel=1e-6), name
            assert stats[2] == pytest.approx(float(actual), rel=1e-6), name
            assert stats[1] == pytest.approx(float(loss), rel=1e-6), name
            assert np.allclose(gg, [float(v) for v in g.split()], rtol=1e-6, atol=1e-9), name
            got[name] = stats
    assert got["gerrymandered"][0] < got["balanced"][0] and got["gerrymandered"][2] > got["balanced"][2]


def test_balance_empty_and_deterministic():
    stats, g, _ = _gpu_balance(np.zeros((0, 8), np.float32), np.zeros(8, np.int32), 2, 0.01)
    assert (stats == 0).all() and (g == 0).all()
    probs, counts = _routing(5000, 128, 4, "zipf", 3)
    a = _gpu_balance(probs, counts, 4, 0.01)
    b = _gpu_balance(probs, counts, 4, 0.01)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


LAYER_CASES = [("tiny", "tiny", {}, "router"), ("wide_T512_zipf", "wide", dict(T=512, d=512, h=256), "zipf"),
               ("small_T384", "small", dict(T=384, d=512, h=256), "router")]


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_with_balance_loss(case):
    from token_routing_grouped_amd.layer import MoELayerGPU

    name, base, over, mode = case
    cfg = configs.get(base).with_(**over)
    alpha = 1.0
    say(f"layer+balance {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h} {cfg.dtype} {mode}")
    inp = inputs.layer_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(v).to(DEV).to(dt) for n, v in inp.items()}
    x, wr, w1, w3, w2, dy = (inp[n] for n in ("x", "wr", "w1", "w3", "w2", "dy"))
    if mode == "router":
        forced = ref.topk_experts(ref.router_logits(x, wr).astype(np.float32), cfg.k).astype(np.int32)
    else:
        forced = inputs.forced_routing(mode, cfg.T, cfg.E, cfg.k, cfg.seed)
    fi = torch.from_numpy(forced).to(DEV)
    grads = {}
    for a in (0.0, alpha):
        layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dt, DEV, aux_alpha=a)
        layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"], forced_idx=fi)
        torch.cuda.synchronize()
        grads[a] = (to_np(layer.dwr), to_np(layer.dx), to_np(layer.balance_stats))
    f = ref.layer_forward(x, wr, w1, w3, w2, cfg.k, forced_idx=forced)
    b = ref.layer_backward(f, dy, x, wr, w1, w3, w2, aux_alpha=alpha)
    b0 = ref.layer_backward(f, dy, x, wr, w1, w3, w2)
    rel = 1e-4 if cfg.dtype == "f32" else 1e-2
    frac = 1e-3 if cfg.dtype == "f32" else 2e-2
    assert_close("dWr", grads[alpha][0], b["dwr"], rel=rel, max_frac=frac)
    assert_close("dx", grads[alpha][1], b["dx"], rel=rel, max_frac=frac)
    st = grads[alpha][2]
    ref_b = bal.balance(f["probs"], f["counts"], cfg.k, alpha)
    assert st[0] == pytest.approx(ref_b["score"], rel=1e-4)
    assert st[2] == pytest.approx(ref_b["max_over_mean"], rel=1e-6)
    if cfg.dtype == "f32":  # the balance term's own contribution to dWr
        assert_close("dWr_aux", grads[alpha][0] - grads[0.0][0], b["dwr"] - b0["dwr"], rel=1e-3, max_frac=1e-2)
