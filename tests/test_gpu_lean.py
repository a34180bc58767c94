"""Memory-lean backward on the GPU: the forward stores neither G nor U, the
backward recomputes them.  The recompute runs the forward's own kernel on the
same inputs, so the whole step must be bit-identical to the normal one (which
the layer parity tests pin to the oracle)."""

import numpy as np
import pytest
import torch

from token_routing_grouped_amd import configs, inputs

from helpers import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CASES = [("small_T384", "small", dict(T=384, d=512, h=256), False),
         ("wide_T700_zipf", "wide", dict(T=700, d=512, h=256), False),
         ("trillion_shape", "trillion", dict(T=48, d=256, h=256), False),
         ("mx_small_T384", "small", dict(T=384, d=512, h=256), True),
         ("mx_wide_T512", "wide", dict(T=512, d=256, h=128), True)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_lean_step_is_bit_identical(case):
    from token_routing_grouped_amd.layer import MoELayerGPU

    name, base, over, mx = case
    cfg = configs.get(base).with_(**over)
    say(f"lean {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h} mx={mx}")
    inp = inputs.layer_inputs(cfg)
    t = {n: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for n, v in inp.items()}
    forced = None
    if "zipf" in name or "trillion" in name:
        mode = "zipf" if "zipf" in name else "uniform"
        forced = torch.from_numpy(inputs.forced_routing(mode, cfg.T, cfg.E, cfg.k, cfg.seed)).to(DEV)
    out = {}
    for lean in (False, True):
        layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, torch.bfloat16, DEV, mx=mx, lean=lean)
        if lean:  # G / U are scratch in lean mode: poison them so nothing stale can pass
            layer.g.fill_(float("nan"))
            layer.u.fill_(float("nan"))
        layer.forward(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], forced)
        torch.cuda.synchronize()
        if lean:
            assert torch.isnan(layer.g.float()).all(), "the lean forward must not write G"
        layer.backward(t["dy"], t["x"], t["wr"], t["w1"], t["w3"], t["w2"])
        torch.cuda.synchronize()
        out[lean] = {n: getattr(layer, n).clone() for n in ("y", "hb", "g", "u", "dx", "dw1", "dw3", "dw2", "dwr")}
        out[lean]["saved"] = layer.saved_bytes()
    for n in ("y", "hb", "g", "u", "dx", "dw1", "dw3", "dw2", "dwr"):
        assert torch.equal(out[False][n], out[True][n]), n
    R, h = cfg.R, cfg.h
    assert out[False]["saved"] - out[True]["saved"] == (2 * R * h * 2 if not mx else
                                                        2 * R * h * 2 - (R * cfg.d + R * cfg.d // 32))
