"""GPU parity of the MXFP8 path against the oracle.

mx_quantize: payload and scale bytes bit-exact against oracle/mx_ref.py
(rowwise, column-per-segment, gathered rows, fixed weight segments, the hand
vectors of tests/golden/).  MXFP8 layer: forward + backward within rel-L2 3e-2
of the oracle run on the same quantise-dequantised operands
(oracle/moe_mx_ref.py), routing fixed to the oracle's choice.
"""

import os

import numpy as np
import pytest
import torch

from oracle import moe_mx_ref as mxl
from oracle import moe_ref as ref
from oracle import mx_ref as mx
from token_routing_grouped_amd import configs, inputs

from helpers import holes_routing, mx_scale_bytes, mx_cols_side_by_side, mx_scales_to_rows, rel_l2, say, tail_routing, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MX_REL = 3e-2


def _u8(*shape):
    return torch.full(shape, 0xEE, dtype=torch.uint8, device=DEV)  # poison: every used byte must be written


def _dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dt)


def _rowwise(a_f32, dt=torch.bfloat16):
    from token_routing_grouped_amd import _abi

    rows, cols = a_f32.shape
    q, s = _u8(rows, cols), _u8(mx_scale_bytes(rows, cols))
    _abi.mx_quantize(_dev(a_f32, dt), rows, q, s, seg_rows=rows)
    torch.cuda.synchronize()
    return q.cpu().numpy(), mx_scales_to_rows(s.cpu().numpy(), rows, cols)


def _hand_cases():
    def expand(tokens, conv):
        out = []
        for tok in tokens.split():
            v, n = (tok.split("*") + ["1"])[:2] if "*" in tok else (tok, "1")
            out += [conv(v)] * int(n)
        return out

    cases = []
    with open(os.path.join(GOLDEN, "mx_e4m3_hand_vectors.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                name, vals, scale, elems = [p.strip() for p in line.split("|")]
                cases.append((name, expand(vals, float), int(scale, 16), expand(elems, lambda s: int(s, 16))))
    return cases


def test_mx_quantize_hand_vectors():
    cases = _hand_cases()
    block = np.array([c[1] for c in cases], np.float32)
    for dt in (torch.float32, torch.bfloat16):
        say(f"mx hand vectors {dt}")
        q, s = _rowwise(block, dt)
        for i, (name, _, scale, elems) in enumerate(cases):
            assert int(s[i, 0]) == scale, (name, dt)
            assert q[i].tolist() == elems, (name, dt)


def _special_matrix(rows, cols, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (rows, 1)))
    a = inputs.bf16_round(a)
    a[0, :32] = 0.0                        # all-zero block
    if rows > 2:
        a[1, :32] = -0.0
        a[2, 32:64] = 1e-39                # float subnormal amax (bf16 keeps it)
    a[-1, -32:] = inputs.bf16_round(np.full(32, 3.0e38, np.float32))  # near the top of the range
    return a


@pytest.mark.parametrize("rows,cols", [(1, 32), (77, 96), (256, 2048), (1000, 288)])
def test_mx_quantize_rowwise_bit_exact(rows, cols):
    say(f"mx rowwise {rows}x{cols}")
    a = _special_matrix(rows, cols, rows + cols)
    q, s = _rowwise(a)
    rq, rs = mx.quantize_rows(a)
    assert (s == rs).all()
    assert (q == rq).all()


def _routing(T, E, k, seed, mode="uniform"):
    idx = inputs.forced_routing(mode, T, E, k, seed)
    L = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    return ref.route(L, k, forced_idx=idx)


@pytest.mark.parametrize("T,E,k,cols,mode", [(300, 8, 2, 64, "uniform"), (129, 40, 4, 256, "zipf"),
                                             (64, 384, 8, 96, "uniform"), (5, 8, 1, 32, "uniform")])
def test_mx_quantize_gather_both_layouts(T, E, k, cols, mode):
    """Routed rows of x quantised straight from x: rowwise = quantise(permute(x));
    columnwise = blocks of 32 routed rows per expert, zero-padded."""
    from token_routing_grouped_amd import _abi

    say(f"mx gather T={T} E={E} k={k} cols={cols} {mode}")
    rt = _routing(T, E, k, T + E, mode)
    x = _special_matrix(T, cols, 3 * T)
    R = T * k
    rc = (R + 127 * E + 127) // 128 * 128
    q, s, qT, sT = _u8(R, cols), _u8(mx_scale_bytes(R, cols)), _u8(cols, rc), _u8(mx_scale_bytes(cols, rc))
    i32 = lambda a: _dev(np.asarray(a, np.int32), torch.int32)
    _abi.mx_quantize(_dev(x, torch.bfloat16), R, q, s, qT, sT, gather_src=i32(rt["src"]), gather_k=k,
                     seg_off=i32(rt["offsets"]), seg_off128=i32(rt["off128"]))
    torch.cuda.synchronize()
    xp = ref.permute(x, rt["pos"])
    rq, rs = mx.quantize_rows(xp)
    assert (q.cpu().numpy() == rq).all() and (mx_scales_to_rows(s.cpu().numpy(), R, cols) == rs).all()
    cq, cs = mx.quantize_cols_segmented(xp, rt["offsets"], rt["off128"])
    R32 = int(rt["off128"][-1])
    assert (mx_cols_side_by_side(qT.cpu().numpy(), cols, rt["off128"]) == cq).all()  # segment e at byte off128[e]*cols
    assert (mx_scales_to_rows(sT.cpu().numpy(), cols, rc)[:, :R32 // 32] == cs).all()


@pytest.mark.parametrize("E,h,d", [(3, 96, 160), (4, 256, 128)], ids=["h96", "h256"])
def test_mx_quantize_fixed_segments(E, h, d):
    """Weights: E segments of h rows each, both layouts in one pass.  The
    columnwise copy is expert-major: row e*d + c holds column c of segment e
    (h96: segments not a multiple of 128 rows, scale bytes written one by
    one; h256: whole scale dwords)."""
    from token_routing_grouped_amd import _abi

    w = _special_matrix(E * h, d, 5)
    q, s, qT, sT = _u8(E * h, d), _u8(mx_scale_bytes(E * h, d)), _u8(E * d, h), _u8(mx_scale_bytes(E * d, h))
    _abi.mx_quantize(_dev(w, torch.bfloat16), E * h, q, s, qT, sT, seg_rows=h)
    torch.cuda.synchronize()
    rq, rs = mx.quantize_rows(w)
    assert (q.cpu().numpy() == rq).all() and (mx_scales_to_rows(s.cpu().numpy(), E * h, d) == rs).all()
    off = np.arange(E + 1) * h
    cq, cs = mx.quantize_cols_segmented(w, off, off)  # the oracle's [d, E*h], [d, E*h/32]; restacked per segment
    want_q = np.concatenate([cq[:, e * h:(e + 1) * h] for e in range(E)], axis=0)
    want_s = np.concatenate([cs[:, e * h // 32:(e + 1) * h // 32] for e in range(E)], axis=0)
    assert (qT.cpu().numpy() == want_q).all()
    assert (mx_scales_to_rows(sT.cpu().numpy(), E * d, h) == want_s).all()


def test_mx_quantize_deterministic():
    a = _special_matrix(513, 256, 9)
    q1, s1 = _rowwise(a)
    q2, s2 = _rowwise(a)
    assert (q1 == q2).all() and (s1 == s2).all()


LAYER_CASES = [
    # id, base config, overrides, routing mode, layer flags
    ("small_T384", "small", dict(T=384, d=512, h=256), "router", {}),
    ("wide_T512_uniform", "wide", dict(T=512, d=256, h=128), "uniform", {}),
    ("wide_T512_zipf", "wide", dict(T=512, d=256, h=128), "zipf", {}),
    ("trillion_shape", "trillion", dict(T=48, d=256, h=256), "uniform", {}),
    ("k_eq_E", "small", dict(T=130, E=4, k=4, d=256, h=128), "router", {}),
    ("one_expert", "small", dict(T=200, E=1, k=1, d=128, h=256), "router", {}),
    ("T1", "small", dict(T=1, d=128, h=128), "router", {}),
    ("tail_split_E4", "small", dict(T=4096, E=4, k=2, d=256, h=128), "tails", {}),
    # experts 3, 7 and 15 of 16 get no rows: zero-length column segments inside
    # and at the end of the expert-major copies
    ("holes_E16", "wide", dict(T=400, E=16, d=256, h=128), "holes", {}),
    # d not a multiple of the 256-wide tiles (partial N / M tiles)
    ("d384_router", "small", dict(T=600, d=384, h=256), "router", {}),
    # memory-lean backward (G and U recomputed from the fp8 copies)
    ("small_T384_lean", "small", dict(T=384, d=512, h=256), "router", dict(lean=True)),
    ("wide_T512_zipf_lean", "wide", dict(T=512, d=256, h=128), "zipf", dict(lean=True)),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_mx_layer_parity(case):
    from token_routing_grouped_amd.layer import MoELayerGPU

    name, base, over, mode, flags = case
    cfg = configs.get(base).with_(**over)
    say(f"mx layer {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h} {mode} {flags}")
    inp = inputs.layer_inputs(cfg)
    t = {n: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for n, v in inp.items()}
    x, wr, w1, w3, w2, dy = (inp[n] for n in ("x", "wr", "w1", "w3", "w2", "dy"))
    if mode == "router":
        forced = ref.topk_experts(ref.router_logits(x, wr).astype(np.float32), cfg.k).astype(np.int32)
    elif mode == "tails":
        forced = tail_routing(cfg.T, [2098, 1998, 2050, 2046])
    elif mode == "holes":
        forced = holes_routing(cfg.T, cfg.E, cfg.k, cfg.seed)
    else:
        forced = inputs.forced_routing(mode, cfg.T, cfg.E, cfg.k, cfg.seed)
    layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, torch.bfloat16, DEV, mx=True, **flags)
    layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"], forced_idx=torch.from_numpy(forced).to(DEV))
    torch.cuda.synchronize()
    f = mxl.layer_forward_mx(x, wr, w1, w3, w2, cfg.k, forced_idx=forced)
    b = mxl.layer_backward_mx(f, dy, x, wr, w1, w3, w2)
    assert (to_np(layer.pos) == f["pos"]).all()
    h, d, R = cfg.h, cfg.d, cfg.R
    dgu = to_np(layer.dgu)
    # dYp is not stored on the MXFP8 path: its two MX copies are checked
    off, off128 = f["offsets"], f["off128"]
    R32 = int(off128[-1])
    dyq = mx.dequantize_rows(to_np(layer.dyq), mx_scales_to_rows(to_np(layer.dys), R, d))
    dyqT = mx.dequantize_cols_segmented(mx_cols_side_by_side(to_np(layer.dyqT), d, off128),
                                        mx_scales_to_rows(to_np(layer.dysT), d, layer.rcap)[:, :R32 // 32], off, off128)
    checks = [("G", layer.g, f["G"]), ("U", layer.u, f["U"]), ("H", layer.hb, f["H"]), ("Yp", layer.yp, f["yp"]),
              ("y", layer.y, f["y"]), ("dYp (MX rows)", dyq, mx.qdq_rows(b["dyp"])),
              ("dYp (MX cols)", dyqT, mx.qdq_cols_segmented(b["dyp"], off, off128)), ("dG", dgu[:, :h], b["dG"]),
              ("dU", dgu[:, h:], b["dU"]), ("dXp", layer.dxp, b["dxp"]), ("dx", layer.dx, b["dx"]),
              ("dW1", layer.dw1, b["dw1"]), ("dW3", layer.dw3, b["dw3"]), ("dW2", layer.dw2, b["dw2"]),
              ("dWr", layer.dwr, b["dwr"])]
    report = {}
    for n, g, r in checks:
        gv = g if isinstance(g, np.ndarray) else to_np(g)
        assert np.isfinite(gv).all(), n
        report[n] = rel_l2(gv, r)
    say("  rel-L2: " + " ".join(f"{n}={v:.1e}" for n, v in report.items()))
    bad = {n: v for n, v in report.items() if not v <= MX_REL}
    assert not bad, bad


@pytest.mark.parametrize("base,over", [("small", dict(T=384, d=512, h=256)), ("wide", dict(T=512, d=256, h=128))])
def test_mx_forward_halves_equal_the_single_call(base, over):
    """Weights quantised on a second stream with the forward in two halves
    (moe_grouped_gemm_fwd_mx_parts: up, then down after W2's copies) give the
    same step, bit for bit, as the weights quantised in line and one
    moe_grouped_gemm_fwd_mx call."""
    from token_routing_grouped_amd.layer import MoELayerGPU

    cfg = configs.get(base).with_(**over)
    say(f"mx forward halves {base}: T={cfg.T} d={cfg.d} E={cfg.E} h={cfg.h}")
    inp = inputs.layer_inputs(cfg)
    t = {n: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for n, v in inp.items()}
    outs = []
    for wq in (False, True):
        layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, torch.bfloat16, DEV, mx=True, wq_overlap=wq)
        assert (layer.wq_stream is not None) == wq
        for _ in range(2):
            layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"])
        torch.cuda.synchronize()
        outs.append([a.clone() for a in (layer.y, layer.yp, layer.hb, layer.dx, layer.dw1, layer.dw3, layer.dw2)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_mx_layer_deterministic():
    from token_routing_grouped_amd.layer import MoELayerGPU

    cfg = configs.get("wide").with_(T=300, d=256, h=128)
    inp = inputs.layer_inputs(cfg)
    t = {n: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for n, v in inp.items()}
    outs = []
    for _ in range(2):
        layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, torch.bfloat16, DEV, mx=True)
        layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"])
        torch.cuda.synchronize()
        R32 = int(layer.off128[-1].item())  # columnwise copies: off128[-1] * cols bytes written
        outs.append([a.clone() for a in (layer.y, layer.dx, layer.dw1, layer.dw2, layer.xq, layer.hqT[:R32 * cfg.h],
                                         layer.dguqT[:R32 * 2 * cfg.h])])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("T,E,mode", [(512, 16, "uniform"), (300, 8, "router")])
def test_mx_dy_copies_from_dy_equal_the_quantised_stored_dyp(T, E, mode):
    """The MXFP8 backward builds dYp's MX copies straight from dy (row r =
    bf16(topk_w[src[r]] * dy[src[r] / k])); they must equal, byte for byte,
    mx_quantize of the dYp that moe_combine_bwd stores (the reading that every
    MX copy is made from its bf16 value)."""
    from token_routing_grouped_amd import _abi
    from token_routing_grouped_amd.layer import MoELayerGPU

    cfg = configs.get("wide").with_(T=T, E=E, d=256, h=128)
    say(f"mx dY copies T={T} E={E} {mode}")
    inp = inputs.layer_inputs(cfg)
    t = {n: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for n, v in inp.items()}
    forced = None if mode == "router" else torch.from_numpy(
        inputs.forced_routing(mode, cfg.T, cfg.E, cfg.k, cfg.seed)).to(DEV)
    layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, torch.bfloat16, DEV, mx=True)
    layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"], forced_idx=forced)
    R, d, rc = cfg.R, cfg.d, layer.rcap
    dyp = torch.empty(R, d, dtype=torch.bfloat16, device=DEV)
    dgate = torch.empty_like(layer.dgate)
    _abi.moe_combine_bwd(t["dy"], layer.yp, layer.topk_w, layer.pos, dyp, dgate)
    q, s, qT, sT = _u8(R, d), _u8(mx_scale_bytes(R, d)), _u8(d, rc), _u8(mx_scale_bytes(d, rc))
    _abi.mx_quantize(dyp, R, q, s, qT, sT, seg_off=layer.offsets, seg_off128=layer.off128)
    torch.cuda.synchronize()
    end = int(layer.off128[-1].item())
    assert torch.equal(dgate, layer.dgate)
    assert torch.equal(q, layer.dyq) and torch.equal(s.view(-1), layer.dys.view(-1))
    assert torch.equal(qT.reshape(-1)[:end * d], layer.dyqT[:end * d])
    nb = end // 128 * d * 4  # scale chunks up to the last padded segment
    assert torch.equal(sT.view(-1)[:nb], layer.dysT.view(-1)[:nb])
