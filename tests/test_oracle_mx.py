"""Pins of the MXFP8 oracle: hand vectors (tests/golden/mx_e4m3_hand_vectors.txt),
the exhaustive E4M3FN grid, torch's independent float8_e4m3fn cast, the
rounding error bound, and layout invariants."""

import os

import numpy as np
import pytest
import torch

from oracle import moe_ref as ref
from oracle import moe_mx_ref as mxl
from oracle import mx_ref as mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _expand(tokens, conv):
    out = []
    for tok in tokens.split():
        if "*" in tok:
            v, n = tok.split("*")
            out += [conv(v)] * int(n)
        else:
            out.append(conv(tok))
    return out


def _hand_vectors():
    cases = []
    with open(os.path.join(GOLDEN, "mx_e4m3_hand_vectors.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, vals, scale, elems = [p.strip() for p in line.split("|")]
            cases.append((name, _expand(vals, float), int(scale, 16), _expand(elems, lambda s: int(s, 16))))
    return cases


@pytest.mark.parametrize("case", _hand_vectors(), ids=lambda c: c[0])
def test_hand_vectors(case):
    name, vals, scale, elems = case
    assert len(vals) == 32 and len(elems) == 32
    q, s = mx.quantize_rows(np.array([vals]))
    assert int(s[0, 0]) == scale, name
    assert q[0].tolist() == elems, name


def _finite_grid():
    bits = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    return bits, mx.e4m3_decode(bits)


def test_grid_round_trip_and_order():
    bits, vals = _finite_grid()
    assert (mx.e4m3_encode(vals) == bits).all()
    pos = np.sort(vals[~np.signbit(vals)])
    # 0, 7 subnormals (step 2^-9), then 15 binades of 8 values up to 448 minus the NaN slot
    assert pos[0] == 0 and pos[1] == 2.0 ** -9 and pos[-1] == 448.0 and len(pos) == 127


def test_midpoints_round_to_even():
    _, vals = _finite_grid()
    pos = np.unique(vals[~np.signbit(vals)])
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2
    got = mx.e4m3_round(mid)
    lo_bits = mx.e4m3_encode(lo)
    expect = np.where(lo_bits % 2 == 0, lo, hi)
    assert (got == expect).all()
    # just off the midpoint goes to the nearer neighbour
    assert (mx.e4m3_round(mid - (hi - lo) * 1e-3) == lo).all()
    assert (mx.e4m3_round(mid + (hi - lo) * 1e-3) == hi).all()


def test_matches_torch_float8_cast():
    """torch's float8_e4m3fn cast is an independent implementation of the same
    rounding; it turns values above the range into NaN, so clamp first."""
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 300)]).astype(np.float32)
    v = np.concatenate([v, np.array([448, 449, 463, 464, 465, 500, 511, -511, 2 ** -10, 2 ** -11], np.float32)])
    clamped = np.clip(v, -448, 448)
    t = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (mx.e4m3_encode(v.astype(np.float64)) == t).all()


def test_error_bound():
    """|v - deq(q(v))| <= 2^-4 * 2^floor(log2 |v|) for elements in the normal range."""
    rng = np.random.default_rng(1)
    a = rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)) * 3)
    deq = mx.qdq_rows(a)
    _, ex = np.frexp(np.abs(a))
    bound = np.ldexp(1.0, ex - 1 - 4)
    q, s = mx.quantize_rows(a)
    X = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)   # block scale 2^s
    err = np.abs(a - deq)
    in_range = (np.abs(a) >= X * 2.0 ** -6) & (np.abs(a) <= 448 * X)
    assert in_range.sum() > 0.9 * a.size
    assert (err[in_range] <= bound[in_range]).all()
    # saturated elements (scaled value in (448, 512)) come back as 448 * 2^s
    sat = np.abs(a) > 464 * X
    assert sat.any()
    assert (np.abs(deq[sat]) == 448 * X[sat]).all() and (err[sat] < 64 * X[sat]).all()
    # below the smallest normal the absolute error is at most half a subnormal step
    sub = np.abs(a) < X * 2.0 ** -6
    assert (err[sub] <= X[sub] * 2.0 ** -10).all()


def test_scale_is_floor_log2_amax_minus_8_brute_force():
    rng = np.random.default_rng(2)
    for _ in range(200):
        blk = rng.standard_normal(32) * 2.0 ** rng.integers(-20, 20)
        _, s = mx.quantize_rows(blk[None, :])
        amax = np.abs(blk).max()
        e = 0
        while 2.0 ** (e + 1) <= amax:
            e += 1
        while 2.0 ** e > amax:
            e -= 1
        assert int(s[0, 0]) == max(-127, min(127, e - 8)) + 127


def test_permute_commutes_with_rowwise_quantisation():
    rng = np.random.default_rng(3)
    T, d, E, k = 40, 64, 8, 2
    x = rng.standard_normal((T, d))
    rt = ref.route(rng.standard_normal((T, E)).astype(np.float32), k)
    q, s = mx.quantize_rows(x)
    qp, sp = mx.quantize_rows(ref.permute(x, rt["pos"]))
    assert (ref.permute(q, rt["pos"]) == qp).all()
    assert (ref.permute(s, rt["pos"]) == sp).all()


def test_column_segment_layout():
    rng = np.random.default_rng(4)
    T, E, k, K = 45, 6, 2, 64
    rt = ref.route(rng.standard_normal((T, E)).astype(np.float32), k)
    a = rng.standard_normal((T * k, K))
    qT, sT = mx.quantize_cols_segmented(a, rt["offsets"], rt["off128"])
    off, off128 = rt["offsets"], rt["off128"]
    for e in range(E):
        n = int(off[e + 1] - off[e])
        base = int(off128[e])
        # brute force per column and block
        for c in range(0, K, 7):
            for b0 in range(0, n, 32):
                blk = np.zeros(32)
                m = min(32, n - b0)
                blk[:m] = a[off[e] + b0: off[e] + b0 + m, c]
                qb, sb = mx.quantize_rows(blk[None, :])
                assert (qT[c, base + b0: base + b0 + 32] == qb[0]).all()
                assert sT[c, (base + b0) // 32] == sb[0, 0]
        # padding is zero
        assert (qT[:, base + n: int(off128[e + 1])] == 0).all()
    back = mx.dequantize_cols_segmented(qT, sT, off, off128)
    assert back.shape == a.shape
    assert np.max(np.abs(back - a)) <= np.max(np.abs(a)) * 2 ** -3


def test_bf16_value_matches_torch():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-30, 30, 10000),
                        np.array([2.0 ** -130, -2.0 ** -133, 1 + 2 ** -8, 1 + 3 * 2 ** -8])])
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert (mxl.bf16_value(v.astype(np.float32).astype(np.float64)) == t).all()


def test_mx_layer_close_to_float_layer():
    """QDQ changes each operand by at most 2^-4 relative; the MX layer output stays
    within a few percent of the unquantised oracle (sanity bound, not a pin of
    the exact value)."""
    rng = np.random.default_rng(6)
    T, d, E, k, h = 64, 64, 4, 2, 96
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) * 0.1
    w1, w3 = rng.standard_normal((2, E, h, d)) * 0.1
    w2 = rng.standard_normal((E, d, h)) * 0.1
    dy = rng.standard_normal((T, d))
    f = ref.layer_forward(x, wr, w1, w3, w2, k)
    fm = mxl.layer_forward_mx(x, wr, w1, w3, w2, k)
    rel = np.linalg.norm(fm["y"] - f["y"]) / np.linalg.norm(f["y"])
    assert 1e-4 < rel < 0.1
    b = ref.layer_backward(f, dy, x, wr, w1, w3, w2)
    bm = mxl.layer_backward_mx(fm, dy, x, wr, w1, w3, w2)
    for key in ("dx", "dw1", "dw3", "dw2", "dwr"):
        rel = np.linalg.norm(bm[key] - b[key]) / np.linalg.norm(b[key])
        assert rel < 0.1, key


def test_mx_layer_exact_when_operands_are_representable():
    """If every GEMM operand is already on the MX grid, QDQ is the identity and the
    MX oracle's GEMM results equal the float oracle's."""
    rng = np.random.default_rng(7)
    T, d, E, k, h = 32, 32, 2, 1, 32
    # small integers times a shared power of two are exact in E4M3 with any
    # block scale that covers them
    x = rng.integers(-3, 4, (T, d)) * 0.25
    w1, w3 = rng.integers(-3, 4, (2, E, h, d)) * 0.125
    w2 = rng.integers(-3, 4, (E, d, h)) * 0.125
    wr = rng.standard_normal((E, d))
    for arr in (x, w1, w3):
        assert (mx.qdq_rows(arr.reshape(-1, d)) == arr.reshape(-1, d)).all()
    f = ref.layer_forward(x, wr, w1, w3, w2, k)
    fm = mxl.layer_forward_mx(x, wr, w1, w3, w2, k)
    assert np.allclose(fm["G"], mxl.bf16_value(f["G"]), rtol=0, atol=0)
    assert np.allclose(fm["U"], mxl.bf16_value(f["U"]), rtol=0, atol=0)
