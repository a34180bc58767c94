"""Whole-layer GPU parity (forward + backward through the C ABI) against the
float64 oracle at sizes the oracle finishes in seconds.

Routing: the GPU computes its logits, which are checked against the oracle's
to tolerance.  Top-k decided on two differently rounded sets of logits can
legitimately differ where two logits nearly tie, so the layer itself is run
with the expert choice fixed to the oracle's (forced indices; gates still come
from the GPU's softmax), and the GPU's own unforced choice is checked to agree
everywhere except at near-ties.  moe_route's bit-exactness on identical logits
is covered in test_gpu_route.py.
"""

import numpy as np
import pytest
import torch

from oracle import moe_ref as ref
from token_routing_grouped_amd import configs, inputs

from helpers import assert_close, holes_routing, say, tail_routing, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CASES = [
    # id, base config, overrides, routing mode, layer flags
    ("tiny", "tiny", {}, "router", {}),
    ("small_T384", "small", dict(T=384), "router", {}),
    ("wide_T512_router", "wide", dict(T=512, d=512, h=256), "router", {}),
    ("wide_T512_zipf", "wide", dict(T=512, d=512, h=256), "zipf", {}),
    ("wide_T640_uniform", "wide", dict(T=640, d=512, h=256), "uniform", {}),
    ("trillion_shape_E8", "trillion", dict(T=32, E=8), "uniform", {}),
    ("glu_mask_h192", "small", dict(T=100, d=256, h=192), "router", {}),
    ("one_expert", "small", dict(T=200, E=1, k=1, d=256, h=256), "router", {}),
    ("k_eq_E", "small", dict(T=130, E=4, k=4, d=256, h=128), "router", {}),
    ("T1", "small", dict(T=1, d=256, h=128), "router", {}),
    ("E384_k8_sparse", "trillion", dict(T=24, d=256, h=128), "uniform", {}),
    # experts of >= 2048 rows on average: light tails (50 and 2 rows past whole
    # 256-row tiles) are scheduled apart from the full-cost tiles
    ("tail_split_E4", "small", dict(T=4096, E=4, k=2, d=256, h=128), "tails", {}),
    # experts 3, 7 and 15 of 16 get no rows: empty segments inside and at the
    # end of the expert list
    ("holes_E16", "wide", dict(T=400, E=16, d=256, h=128), "holes", {}),
    # the same tails over longer K loops (16 steps in the up projection and
    # dgrad down, 8 in dgrad up, 4 in down): the light tails' three-stage
    # pipeline in its steady state
    ("tail_split_E4_K1024", "small", dict(T=4096, E=4, k=2, d=1024, h=256), "tails", {}),
    # d not a multiple of the 256-wide tiles: partial N tiles of the down and
    # dgrad-up GEMMs, partial M tiles of wgrad-down and partial N tiles of
    # wgrad-up (256-row tiles at d = 320, 128-row tiles at d = 192)
    ("d320_router", "small", dict(T=600, d=320, h=256), "router", {}),
    ("d192_uniform_E16", "wide", dict(T=500, E=16, d=192, h=128), "uniform", {}),
    # memory-lean backward: G and U recomputed in the backward, checked against
    # the oracle like the stored ones
    ("small_T384_lean", "small", dict(T=384), "router", dict(lean=True)),
    ("wide_T512_zipf_lean", "wide", dict(T=512, d=512, h=256), "zipf", dict(lean=True)),
    ("trillion_shape_lean", "trillion", dict(T=48, d=256, h=256), "uniform", dict(lean=True)),
]


def _near_tie_tokens(L32, k, tol):
    s = np.sort(L32, axis=1)[:, ::-1]
    if k >= L32.shape[1]:
        return np.zeros(L32.shape[0], bool)
    return (s[:, k - 1] - s[:, k]) <= tol


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_parity(case):
    from token_routing_grouped_amd import _abi
    from token_routing_grouped_amd.layer import MoELayerGPU

    name, base, over, mode, flags = case
    cfg = configs.get(base).with_(**over)
    say(f"layer {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h} {cfg.dtype} {mode} {flags}")
    inp = inputs.layer_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(v).to(DEV).to(dt) for n, v in inp.items()}
    x, wr, w1, w3, w2, dy = (inp[n] for n in ("x", "wr", "w1", "w3", "w2", "dy"))
    layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dt, DEV, **flags)

    # --- logits and the unforced routing
    L_ref = ref.router_logits(x, wr)
    layer.forward(t["x"], t["wr"], t["w1"], t["w3"], t["w2"])
    torch.cuda.synchronize()
    assert_close("logits", to_np(layer.logits), L_ref, rel=1e-5, max_frac=1e-4)
    L32 = L_ref.astype(np.float32)
    if mode == "router":
        forced = ref.topk_experts(L32, cfg.k).astype(np.int32)
        differ = (to_np(layer.topk_idx) != forced).any(axis=1)
        ties = _near_tie_tokens(L32, cfg.k, 1e-4 * max(1.0, float(np.abs(L32).max())))
        assert not (differ & ~ties).any(), f"routing differs on {int((differ & ~ties).sum())} non-tied tokens"
    elif mode == "tails":
        forced = tail_routing(cfg.T, [2098, 1998, 2050, 2046])
    elif mode == "holes":
        forced = holes_routing(cfg.T, cfg.E, cfg.k, cfg.seed)
    else:
        forced = inputs.forced_routing(mode, cfg.T, cfg.E, cfg.k, cfg.seed)

    # --- the layer with the oracle's expert choice
    fi = torch.from_numpy(forced).to(DEV)
    layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"], forced_idx=fi)
    torch.cuda.synchronize()
    assert int(layer.err_flag.item()) == 0
    f = ref.layer_forward(x, wr, w1, w3, w2, cfg.k, forced_idx=forced)
    b = ref.layer_backward(f, dy, x, wr, w1, w3, w2)

    for n, g in (("counts", layer.counts), ("offsets", layer.offsets), ("pos", layer.pos), ("src", layer.src),
                 ("off128", layer.off128)):
        assert (to_np(g) == f[n]).all(), n
    assert (to_np(layer.topk_idx) == f["idx"]).all()
    assert np.allclose(to_np(layer.topk_w), f["w"], rtol=1e-4, atol=1e-7)
    assert (to_np(layer.xp) == f["xp"]).all(), "xp (a copy) must be bit-exact"

    rel = 1e-4 if cfg.dtype == "f32" else 1e-2
    frac = 1e-3 if cfg.dtype == "f32" else 2e-2
    R, h = cfg.R, cfg.h
    dgu = to_np(layer.dgu)
    checks = [("G", layer.g, f["G"]), ("U", layer.u, f["U"]), ("H", layer.hb, f["H"]), ("Yp", layer.yp, f["yp"]),
              ("y", layer.y, f["y"]), ("dYp", layer.dyp, b["dyp"]), ("dgate", layer.dgate, b["dgate"]),
              ("dG", dgu[:, :h], b["dG"]), ("dU", dgu[:, h:], b["dU"]), ("dXp", layer.dxp, b["dxp"]),
              ("dx", layer.dx, b["dx"]), ("dW1", layer.dw1, b["dw1"]), ("dW3", layer.dw3, b["dw3"]),
              ("dW2", layer.dw2, b["dw2"]), ("dWr", layer.dwr, b["dwr"])]
    report = {}
    for n, g, r in checks:
        gv = g if isinstance(g, np.ndarray) else to_np(g)
        report[n] = assert_close(n, gv, r, rel=rel, max_frac=frac)[0]
    say("  rel-L2: " + " ".join(f"{n}={v:.1e}" for n, v in report.items()))


def test_layer_deterministic():
    from token_routing_grouped_amd.layer import MoELayerGPU

    cfg = configs.get("wide").with_(T=700, d=512, h=256)
    inp = inputs.layer_inputs(cfg)
    t = {n: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for n, v in inp.items()}
    outs = []
    for _ in range(2):
        layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, torch.bfloat16, DEV)
        layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"])
        torch.cuda.synchronize()
        outs.append([a.clone() for a in (layer.y, layer.dx, layer.dw1, layer.dw3, layer.dw2, layer.dwr, layer.pos)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
