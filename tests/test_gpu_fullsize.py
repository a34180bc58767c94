"""Parity at the workloads' full sizes, in the configuration bench.py times.

Each case runs one step of the layer exactly as bench.py does (the same
inputs from ``inputs.device_inputs``, the same layer flags, including the
workload's two-stream backward where its config sets it, so the same kernels
and tile shapes) and checks against the float64 oracle.

Whole tensors (small, wide with router / uniform / Zipf routing, MXFP8 at the
small shape): the whole-layer oracle runs on the host in seconds to a minute
at these sizes, so every element of y, Yp, dgate, dx, dW1, dW3, dW2 and dWr is
compared, and routing (indices, counts, offsets, positions, src, off128) is
bit-exact over all tokens.  The oracle routes from the GPU's float32 logits
(bit-exact routing is defined on identical logits), and those logits are
themselves checked against the oracle's on every token; nothing else the
oracle uses comes from the GPU.

Sampled (MXFP8 at the wide shape, trillion shape): the whole-layer oracle would
take minutes (MX quantisation of 0.8 G weight values) or hundreds of GB, so
y, dgate and dx of sampled tokens (oracle/sampled_ref.tokens) and whole dW1 /
dW3 rows and dW2 columns of two experts (oracle/sampled_ref.expert_slices) are
checked, with routing still bit-exact over all tokens.

Tolerances: bf16 rel-L2 <= 1e-2 and max-abs <= 2e-2 max|ref| per tensor;
MXFP8 rel-L2 <= 3e-2 against the quantise-dequantise oracle.
"""

import numpy as np
import pytest
import torch

from oracle import moe_mx_ref as mxl
from oracle import moe_ref as ref
from oracle import sampled_ref as sref
from token_routing_grouped_amd import configs, inputs

from helpers import assert_close, rel_l2, say, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MX_REL = 3e-2

WHOLE = [  # workload slug, routing mode (ordered so that cases of one input set run together)
    ("small", "router"),
    ("mxfp8_small", "router"),
    ("wide", "router"),
    ("wide", "uniform"),
    ("wide", "zipf"),
]
SAMPLED = [  # workload slug, routing mode, sampled tokens
    ("mxfp8", "router", 3),
    ("mxfp8", "uniform", 3),
    ("trillion", "uniform", 2),
]

_cache = {}


def _inputs(cfg):
    """Device inputs of the workload (as bench.py draws them) and their float64
    host copies; kept for the next case of the same shape and seed."""
    key = (cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, cfg.seed, cfg.dtype)
    if key not in _cache:
        _cache.clear()
        t, where = inputs.device_inputs(cfg, DEV)
        host = None
        if where == "host":
            host = {n: to_np(v).astype(np.float64) for n, v in t.items()}
        _cache[key] = (t, host)
    return _cache[key]


def _check(name, got, want, mx_on):
    """MXFP8 tensors against the QDQ oracle: rel-L2 only; bf16: rel-L2 and max-abs."""
    if mx_on:
        r = rel_l2(got, want)
        assert np.isfinite(np.asarray(got)).all(), f"{name}: non-finite values"
        assert r <= MX_REL, f"{name}: rel-L2 {r:.3e} > {MX_REL:.0e}"
        return r
    return assert_close(name, got, want)[0]


def _step(cfg, mode, t):
    from token_routing_grouped_amd.layer import MoELayerGPU

    forced_np = None if mode == "router" else inputs.forced_routing(mode, cfg.T, cfg.E, cfg.k, cfg.seed)
    forced = None if forced_np is None else torch.from_numpy(forced_np).to(DEV)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dt, DEV, mx=cfg.mx, overlap=cfg.overlap)
    layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"], forced_idx=forced)
    torch.cuda.synchronize()
    assert int(layer.err_flag.item()) == 0
    return layer, forced_np


def _routing_bit_exact(layer, L, k, forced_np):
    r = ref.route(L, k, forced_idx=forced_np)
    for n, g in (("idx", layer.topk_idx), ("counts", layer.counts), ("offsets", layer.offsets), ("pos", layer.pos),
                 ("src", layer.src), ("off128", layer.off128)):
        assert (to_np(g) == r[n]).all(), n
    assert np.allclose(to_np(layer.topk_w), r["w"], rtol=1e-5, atol=1e-9), "gates"
    return r


@pytest.mark.parametrize("case", WHOLE, ids=[f"{c[0]}_{c[1]}" for c in WHOLE])
def test_full_size_whole_tensor_parity(case):
    slug, mode = case
    cfg = configs.get(slug)
    say(f"full size, whole tensors {slug}/{mode}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h} mx={cfg.mx}")
    t, host = _inputs(cfg)
    layer, forced_np = _step(cfg, mode, t)
    x, wr, w1, w3, w2, dy = (host[n] for n in ("x", "wr", "w1", "w3", "w2", "dy"))

    L = to_np(layer.logits).astype(np.float32)
    assert_close("logits", L, ref.router_logits(x, wr), rel=1e-5, max_frac=1e-4)
    _routing_bit_exact(layer, L, cfg.k, forced_np)

    fwd, bwd = (mxl.layer_forward_mx, mxl.layer_backward_mx) if cfg.mx else (ref.layer_forward, ref.layer_backward)
    f = fwd(x, wr, w1, w3, w2, cfg.k, forced_idx=forced_np, logits=L)
    b = bwd(f, dy, x, wr, w1, w3, w2)
    report = {}
    for n, g, r in (("Yp", layer.yp, f["yp"]), ("y", layer.y, f["y"]), ("dgate", layer.dgate, b["dgate"]),
                    ("dx", layer.dx, b["dx"]), ("dW1", layer.dw1, b["dw1"]), ("dW3", layer.dw3, b["dw3"]),
                    ("dW2", layer.dw2, b["dw2"]), ("dWr", layer.dwr, b["dwr"])):
        report[n] = _check(n, to_np(g), r, cfg.mx)
    say("  rel-L2: " + " ".join(f"{n}={v:.1e}" for n, v in report.items()))


@pytest.mark.parametrize("case", SAMPLED, ids=[f"{c[0]}_{c[1]}" for c in SAMPLED])
def test_full_size_sampled_parity(case):
    slug, mode, ns = case
    cfg = configs.get(slug)
    say(f"full size, sampled {slug}/{mode}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h} mx={cfg.mx}")
    t, _ = _inputs(cfg)
    layer, forced_np = _step(cfg, mode, t)
    k, h = cfg.k, cfg.h

    L = to_np(layer.logits).astype(np.float32)
    r = _routing_bit_exact(layer, L, k, forced_np)
    idx = to_np(layer.topk_idx)

    x, wr, dy = (to_np(t[n]).astype(np.float64) for n in ("x", "wr", "dy"))
    rng = np.random.default_rng(cfg.seed + 17)
    S = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, ns - 2, replace=False)]))
    assert_close("logits[S]", L[S], ref.router_logits(x[S], wr), rel=1e-5, max_frac=1e-4)

    # --- sampled tokens
    experts = np.unique(idx[S])
    w1_e, w3_e, w2_e = (to_np(t[n][torch.from_numpy(experts).to(DEV)]) for n in ("w1", "w3", "w2"))
    o = sref.tokens(x[S], dy[S], L[S], idx[S], wr, experts, w1_e, w3_e, w2_e, mx_on=cfg.mx)
    report = {}
    report["y"] = _check("y[S]", to_np(layer.y)[S], o["y"], cfg.mx)
    report["dgate"] = _check("dgate[S]", to_np(layer.dgate)[S], o["dgate"], cfg.mx)
    report["dx"] = _check("dx[S]", to_np(layer.dx)[S], o["dx"], cfg.mx)
    del w1_e, w3_e, w2_e

    # --- weight-gradient slices of two experts
    counts = r["counts"]
    busy = int(np.argmax(counts))
    other = int(rng.choice(np.flatnonzero((counts > 0) & (np.arange(cfg.E) != busy))))
    hid = np.unique(np.concatenate([[0, h - 1], rng.choice(h, 2, replace=False)]))
    p = ref.softmax(L)
    for e in (busy, other):
        rows = np.arange(r["offsets"][e], r["offsets"][e + 1])
        tok, slot = r["src"][rows] // k, r["src"][rows] % k
        gate = p[tok, idx[tok, slot]]
        w1, w3, w2 = (to_np(t[n][e]) for n in ("w1", "w3", "w2"))
        s = sref.expert_slices(x[tok], dy[tok], gate, w1, w3, w2, hid, mx_on=cfg.mx)
        hid_t = torch.from_numpy(hid).to(DEV)
        report[f"dW1[{e}]"] = _check(f"dW1[{e}][hid]", to_np(layer.dw1[e][hid_t]), s["dw1"], cfg.mx)
        report[f"dW3[{e}]"] = _check(f"dW3[{e}][hid]", to_np(layer.dw3[e][hid_t]), s["dw3"], cfg.mx)
        report[f"dW2[{e}]"] = _check(f"dW2[{e}][:,hid]", to_np(layer.dw2[e][:, hid_t]), s["dw2"], cfg.mx)
    say(f"  {len(S)} tokens, experts {busy} ({counts[busy]} rows) and {other} ({counts[other]} rows); rel-L2: "
        + " ".join(f"{n}={v:.1e}" for n, v in report.items()))


@pytest.mark.parametrize("slug", ["small", "mxfp8"])
def test_full_size_step_is_bitwise_reproducible(slug):
    """Two steps of the timed configuration (two streams where the workload's
    config sets them; light-tail tile order at the small shape) give the same
    bits in every output and gradient."""
    from token_routing_grouped_amd.layer import MoELayerGPU

    cfg = configs.get(slug)
    say(f"full size determinism {slug}: overlap={cfg.overlap} mx={cfg.mx}")
    t, _ = _inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dt, DEV, mx=cfg.mx, overlap=cfg.overlap)
    outs = []
    for _ in range(2):
        layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"])
        torch.cuda.synchronize()
        outs.append({n: getattr(layer, n).clone() for n in ("y", "dx", "dw1", "dw3", "dw2", "dwr", "dgate")})
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), n
