"""Weight-gradient GEMMs on a second stream next to the dgrad chain
(moe_grouped_gemm_bwd_parts, and moe_grouped_gemm_bwd_mx_parts for MXFP8):
every GEMM computes exactly what it computes on one stream, so the whole step
must be bit-identical to the serial one."""

import pytest
import torch

from token_routing_grouped_amd import configs, inputs

from helpers import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

# id, base config, overrides, forced routing, layer attributes of the two-stream run
# (the router's dWr part on the side stream is the MXFP8 default; both ways are covered)
CASES = [("small_T1024", "small", dict(T=1024, d=512, h=256), None, {}),
         ("small_T1024_router_dwr_on_side", "small", dict(T=1024, d=512, h=256), None,
          dict(router_dwr_on_side=True)),
         ("wide_T700_zipf", "wide", dict(T=700, d=512, h=256), "zipf", {}),
         ("lean_small_T384", "small", dict(T=384, d=512, h=256), None, {}),
         ("mx_small_T1024", "small", dict(T=1024, d=512, h=256), None, {}),
         ("mx_small_T1024_router_dwr_on_main", "small", dict(T=1024, d=512, h=256), None,
          dict(router_dwr_on_side=False)),
         ("mx_wide_T700_zipf", "wide", dict(T=700, d=512, h=256), "zipf", {}),
         ("mx_lean_small_T384", "small", dict(T=384, d=512, h=256), None, {})]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_two_stream_backward_is_bit_identical(case):
    from token_routing_grouped_amd.layer import MoELayerGPU

    name, base, over, mode, attrs = case
    cfg = configs.get(base).with_(**over)
    say(f"overlap {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h}")
    inp = inputs.layer_inputs(cfg)
    t = {n: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for n, v in inp.items()}
    forced = None
    if mode:
        forced = torch.from_numpy(inputs.forced_routing(mode, cfg.T, cfg.E, cfg.k, cfg.seed)).to(DEV)
    lean = "lean" in name
    mx = name.startswith("mx_")
    out = {}
    for ov in (False, True):
        layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, torch.bfloat16, DEV, mx=mx, lean=lean, overlap=ov)
        assert layer.overlap == ov
        if ov:
            for a, v in attrs.items():
                setattr(layer, a, v)
        for _ in range(2):  # the second step reuses the side stream and its events
            layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"], forced_idx=forced)
        torch.cuda.synchronize()
        out[ov] = {n: getattr(layer, n).clone() for n in ("y", "dx", "dw1", "dw3", "dw2", "dwr")}
    for n in out[False]:
        assert torch.equal(out[False][n], out[True][n]), n
