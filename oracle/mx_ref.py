"""MXFP8 quantisation oracle (OCP microscaling: E4M3FN elements, E8M0 block scale).

Test infrastructure only (see the package header).

The pages name MXFP8 as the low-precision format that cuts both compute and
the traffic between experts, with most of the gain in the feed-forward
compute [OC3 "Precision optimisation with MXFP8"].  They do not define the
encoding; the reading taken is the OCP MX v1.0 one:

  * a block is 32 consecutive values along the GEMM reduction (K) dimension;
  * shared scale X = 2^s with s = floor(log2(amax)) - emax_elem, emax_elem = 8
    for E4M3, clamped to [-127, 127]; stored as the E8M0 byte s + 127
    (255 = NaN is never produced).  An all-zero block gets s = -127;
  * elements are v / X, rounded to E4M3FN (1 sign, 4 exponent bits with bias
    7, 3 mantissa bits; subnormals down to 2^-9; no infinities; S.1111.111 is
    NaN; largest finite 448) with round-to-nearest-even, saturating to +-448
    (v / X can reach [448, 512)); the sign of zero is kept.

floor(log2(amax)) is taken exactly from the binary exponent (frexp), never
from a rounded logarithm.

Layouts:
  rowwise      -- blocks along the columns of a row-major [M, K] matrix:
                  q [M, K] uint8, scales [M, K/32] uint8.
  column/segment -- blocks of 32 consecutive rows inside each expert segment
                  [off_e, off_{e+1}) of an [R, K] matrix; a partial last block
                  is zero-padded; blocks never straddle experts.  Stored as the
                  rowwise form of the transpose: qT [K, R32], sT [K, R32/32]
                  with segment e starting at column off128[e].
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
EMAX_E4M3 = 8
BLOCK = 32


def e4m3_round(v):
    """Nearest E4M3FN value (ties to even), saturated to +-448, as float64."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                    # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)             # binade exponent; subnormals share 2^-6's spacing
    spacing = np.ldexp(1.0, e - 3)         # 3 mantissa bits
    q = np.rint(a / spacing) * spacing     # a / spacing is exact; rint ties to even
    q = np.minimum(q, E4M3_MAX)
    return np.copysign(q, v)


def e4m3_encode(v):
    """Bit pattern (uint8) of ``e4m3_round(v)``; -0 keeps its sign bit."""
    q = e4m3_round(v)
    sign = np.signbit(q).astype(np.int64) << 7
    a = np.abs(q)
    _, ex = np.frexp(a)
    e = ex - 1
    normal = a >= 2.0 ** -6
    field = np.where(normal, e + 7, 0)
    mant = np.where(normal, np.ldexp(a, -e) * 8 - 8, a * 2.0 ** 9)
    mant = np.where(a == 0, 0, mant)
    bits = sign | (field.astype(np.int64) << 3) | mant.astype(np.int64)
    return bits.astype(np.uint8)


def e4m3_decode(b):
    """Float64 value of E4M3FN bit patterns (NaN for S.1111.111)."""
    b = np.asarray(b, np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    field = (b >> 3) & 0xF
    mant = b & 0x7
    val = np.where(field == 0, mant * 2.0 ** -9, (8 + mant) * np.ldexp(1.0, field - 10))
    val = np.where((field == 15) & (mant == 7), np.nan, val)
    return sign * val


def block_scale_exp(amax):
    """s = clamp(floor(log2 amax) - 8, -127, 127); s = -127 for amax == 0."""
    amax = np.asarray(amax, np.float64)
    _, ex = np.frexp(amax)
    s = np.clip(ex - 1 - EMAX_E4M3, -127, 127)
    return np.where(amax == 0, -127, s).astype(np.int64)


def quantize_rows(a):
    """Rowwise MX quantisation of [M, K] (K a multiple of 32) -> (q, scales)."""
    a = np.asarray(a, np.float64)
    M, K = a.shape
    assert K % BLOCK == 0
    blocks = a.reshape(M, K // BLOCK, BLOCK)
    s = block_scale_exp(np.max(np.abs(blocks), axis=2))
    scaled = blocks * np.ldexp(1.0, -s)[:, :, None]     # exact power-of-two scaling
    q = e4m3_encode(scaled).reshape(M, K)
    return q, (s + 127).astype(np.uint8)


def dequantize_rows(q, scales):
    M, K = q.shape
    s = scales.astype(np.int64) - 127
    v = e4m3_decode(q).reshape(M, K // BLOCK, BLOCK) * np.ldexp(1.0, s)[:, :, None]
    return v.reshape(M, K)


def quantize_cols_segmented(a, offsets, off128):
    """Column-per-segment MX quantisation of [R, K] -> (qT [K, R32], sT [K, R32/32])."""
    a = np.asarray(a, np.float64)
    R, K = a.shape
    E = len(offsets) - 1
    R32 = int(off128[E])
    qT = np.zeros((K, R32), np.uint8)
    sT = np.zeros((K, R32 // BLOCK), np.uint8)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        base = int(off128[e])
        n32 = int(off128[e + 1]) - base
        if n32 == 0:
            continue
        seg = np.zeros((n32, K))
        seg[:hi - lo] = a[lo:hi]
        q, s = quantize_rows(seg.T)                 # blocks along the rows of the segment
        qT[:, base:base + n32] = q
        sT[:, base // BLOCK:(base + n32) // BLOCK] = s
    return qT, sT


def dequantize_cols_segmented(qT, sT, offsets, off128):
    """Inverse layout of ``quantize_cols_segmented`` back to [R, K]."""
    K = qT.shape[0]
    E = len(offsets) - 1
    R = int(offsets[E])
    out = np.zeros((R, K))
    full = dequantize_rows(qT, sT)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        base = int(off128[e])
        out[lo:hi] = full[:, base:base + hi - lo].T
    return out


def qdq_rows(a):
    return dequantize_rows(*quantize_rows(a))


def qdq_cols_segmented(a, offsets, off128):
    return dequantize_cols_segmented(*quantize_cols_segmented(a, offsets, off128), offsets, off128)


def qdq_cols(a):
    """Blocks of 32 along the rows of [K, N] (no segments): MX operand blocked on K = rows."""
    return qdq_rows(np.asarray(a).T).T
