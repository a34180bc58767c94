"""Guard bands and poisoned outputs around every buffer one layer step writes.

Each buffer of the layer (routing metadata, activations, gradients, MX copies,
workspaces) is replaced by a view into a larger allocation with a 4 KiB guard
band on each side, filled with a byte pattern.  Float buffers are prefilled
with NaN, integer ones with -1, MX byte buffers with 0xEE.  After one full
forward + backward:

  * every guard band still holds its pattern (no kernel wrote outside its
    buffer, e.g. a row past an expert's last row or past R);
  * no NaN survives in a float output that the step must write in full (so
    every row, ragged tails included, was written);
  * the MX column copies are untouched past the last padded segment
    (off128[E]) up to their row stride.

Cases cover ragged tails (T and d not tile multiples), empty experts, the
light-tail schedule, the two-stream backward, the memory-lean backward and the
MXFP8 path.  Values are checked elsewhere; this file checks where the kernels
write.
"""

import pytest
import torch

from token_routing_grouped_amd import configs, inputs

from helpers import holes_routing, say, tail_routing

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GUARD = 4096

ROUTING = ["logits", "probs", "topk_idx", "topk_w", "counts", "offsets", "off128", "pos", "src"]
FLOAT_OUT = ["g", "u", "hb", "yp", "y", "dyp", "dgate", "dgu", "dxp", "dx", "dwr", "dw1", "dw3", "dw2"]
MX_BUFS = ["xq", "xs", "xqT", "xsT", "w1q", "w1s", "w1tq", "w1ts", "w3q", "w3s", "w3tq", "w3ts", "w2q", "w2s",
           "w2tq", "w2ts", "hq", "hs", "hqT", "hsT", "dyq", "dys", "dyqT", "dysT", "dguq", "dgus", "dguqT", "dgusT"]
WORKSPACES = ["ws_route", "ws_gemm", "ws_router", "ws_balance"]


def _pattern(n):
    return (torch.arange(n, dtype=torch.int32, device=DEV) * 37 % 251).to(torch.uint8)


def _install_guards(layer, names):
    guards = {}
    for name in names:
        buf = getattr(layer, name)
        es = buf.element_size()
        g = GUARD // es
        big = torch.empty(buf.numel() + 2 * g, dtype=buf.dtype, device=DEV)
        raw = big.view(torch.uint8)
        raw[:GUARD] = _pattern(GUARD)
        raw[GUARD + buf.numel() * es:] = _pattern(GUARD)
        body = big[g:g + buf.numel()]
        if buf.dtype.is_floating_point:
            body.fill_(float("nan"))
        elif buf.dtype == torch.uint8:
            body.fill_(0xEE)
        else:
            body.fill_(-1)
        setattr(layer, name, body.view(buf.shape))
        guards[name] = (big, buf.numel() * es)
    return guards


def _check_guards(guards):
    want = _pattern(GUARD)
    for name, (big, nbytes) in guards.items():
        raw = big.view(torch.uint8)
        assert torch.equal(raw[:GUARD], want), f"{name}: guard band before the buffer was written"
        assert torch.equal(raw[GUARD + nbytes:], want), f"{name}: guard band after the buffer was written"


CASES = [
    # id, base config, overrides, routing, layer flags
    ("ragged_T300_d320_h192", "small", dict(T=300, d=320, h=192), "router", {}),
    ("empty_experts_E16", "wide", dict(T=400, E=16, d=256, h=128), "holes", {}),
    ("light_tails_E4", "small", dict(T=4096, E=4, k=2, d=256, h=128), "tails", {}),
    ("two_stream_ragged", "small", dict(T=300, d=320, h=192), "router", dict(overlap=True)),
    ("lean_ragged", "small", dict(T=300, d=320, h=192), "router", dict(lean=True)),
    ("mx_ragged_T300_d384", "small", dict(T=300, d=384, h=256), "router", dict(mx=True)),
    ("mx_empty_experts_E16", "wide", dict(T=400, E=16, d=256, h=128), "holes", dict(mx=True)),
    ("mx_light_tails_E4", "small", dict(T=4096, E=4, k=2, d=256, h=128), "tails", dict(mx=True)),
    ("mx_two_stream", "wide", dict(T=400, E=16, d=256, h=128), "uniform", dict(mx=True, overlap=True)),
]


def _routing(cfg, mode):
    if mode == "router":
        return None
    if mode == "tails":
        return tail_routing(cfg.T, [2098, 1998, 2050, 2046])
    if mode == "holes":  # experts 3, 7 and 15 get no rows
        return holes_routing(cfg.T, cfg.E, cfg.k, cfg.seed)
    return inputs.forced_routing(mode, cfg.T, cfg.E, cfg.k, cfg.seed)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_step_writes_only_its_buffers(case):
    from token_routing_grouped_amd.layer import MoELayerGPU

    name, base, over, mode, flags = case
    cfg = configs.get(base).with_(**over)
    say(f"guards {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h} {mode} {flags}")
    inp = inputs.layer_inputs(cfg)
    t = {n: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for n, v in inp.items()}
    forced = _routing(cfg, mode)
    fi = None if forced is None else torch.from_numpy(forced).to(DEV)
    layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, torch.bfloat16, DEV, **flags)
    names = ROUTING + FLOAT_OUT + WORKSPACES + (["xp"] if not flags.get("mx") else MX_BUFS)
    if flags.get("overlap"):
        names += ["ws_gemm2", "ws_router2"]
    guards = _install_guards(layer, names)
    layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"], forced_idx=fi)
    torch.cuda.synchronize()
    assert int(layer.err_flag.item()) == 0
    _check_guards(guards)
    counts = layer.counts.cpu().numpy()
    if mode == "holes":
        assert (counts[[3, 7, 15]] == 0).all()
    written = [n for n in FLOAT_OUT if not (flags.get("mx") and n == "dyp")]  # MXFP8 does not store dYp
    for n in written + ["logits", "probs", "topk_w"] + (["xp"] if not flags.get("mx") else []):
        assert not torch.isnan(getattr(layer, n).float()).any(), f"{n}: rows left unwritten"
    for n in ("topk_idx", "counts", "offsets", "off128", "pos", "src"):
        assert (getattr(layer, n) >= 0).all(), f"{n}: entries left unwritten"
    if flags.get("mx"):
        end = int(layer.off128[-1].item())
        for n in ("xqT", "hqT", "dyqT", "dguqT"):  # payload: segment e at byte off128[e] * cols, flat
            buf = getattr(layer, n)
            cols = buf.numel() // layer.rcap
            assert (buf.reshape(-1)[end * cols:] == 0xEE).all(), f"{n}: written past the last padded segment"
        for n in ("xsT", "hsT", "dysT", "dgusT"):  # scales, K-chunk major: [rcap/128][cols][4]
            buf = getattr(layer, n)
            cols = buf.shape[0]
            assert (buf.reshape(-1)[end // 128 * cols * 4:] == 0xEE).all(), f"{n}: written past the last segment"
    say(f"  {len(guards)} buffers guarded, expert rows {counts.tolist()[:16]}")
