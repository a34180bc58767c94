"""Shared helpers for the GPU parity tests (no arithmetic of the method here)."""

from __future__ import annotations

import numpy as np

# Float tolerances for bf16 storage (and reused for fp32 layers): per tensor,
# rel-L2 <= 1e-2 and max-abs <= 2e-2 * max|ref|.
REL_L2 = 1e-2
MAX_ABS_FRAC = 2e-2


def rel_l2(a, r) -> float:
    a = np.asarray(a, np.float64)
    r = np.asarray(r, np.float64)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(a - r) / den) if den > 0 else float(np.linalg.norm(a))


def assert_close(name, got, ref, rel=REL_L2, max_frac=MAX_ABS_FRAC):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref))) if got.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    assert r <= rel, f"{name}: rel-L2 {r:.3e} > {rel:.1e}"
    assert m <= max_frac * scale + 1e-30, f"{name}: max-abs {m:.3e} > {max_frac:.0e} * {scale:.3e}"
    return r, m


def tail_routing(T, counts):
    """Forced top-2 routing with the given per-expert row counts (sum 2T): the
    first T entries of the expert list fill slot 0, the rest slot 1, so a
    token's two experts differ as long as no count exceeds T.  Used to give
    experts tails of chosen lengths past their whole 256-row tiles."""
    lst = np.repeat(np.arange(len(counts)), counts)
    assert lst.size == 2 * T and max(counts) <= T
    return np.stack([lst[:T], lst[T:]], axis=1).astype(np.int32)


def holes_routing(T, E, k, seed, empty=(3, 7, 15)):
    """Forced uniform routing over the experts not in `empty`, which get no
    rows (zero-length segments in the middle and, with E = 16, at the end of
    the expert list)."""
    from token_routing_grouped_amd import inputs

    keep = np.array([e for e in range(E) if e not in empty])
    idx = inputs.forced_routing("uniform", T, len(keep), k, seed)
    return keep[idx].astype(np.int32)


def to_np(t):
    return t.detach().float().cpu().numpy() if t.dtype.is_floating_point else t.detach().cpu().numpy()


def say(*a):
    print(*a, flush=True)


def mx_scale_bytes(rows, K):
    """Bytes of an MX scale array in the library's K-chunk-major layout."""
    return -(-K // 128) * rows * 4


def mx_cols_side_by_side(buf, cols, off128):
    """The library's columnwise MX copy of segmented rows (segment e's copy a
    [cols, len_e] block at byte off128[e] * cols, len_e = off128[e+1] -
    off128[e]) as the [cols, off128[-1]] array with the segments side by side,
    the layout the oracle uses.  A pure re-indexing."""
    flat = np.asarray(buf).reshape(-1)
    off = np.asarray(off128).astype(np.int64)
    out = np.zeros((cols, int(off[-1])), dtype=flat.dtype)
    for e in range(len(off) - 1):
        ps, pe = int(off[e]), int(off[e + 1])
        if pe > ps:
            out[:, ps:pe] = flat[ps * cols:pe * cols].reshape(cols, pe - ps)
    return out


def mx_scales_to_rows(buf, rows, K):
    """The library's K-chunk-major scale bytes (block b of row r at byte
    (b // 4 * rows + r) * 4 + b % 4) as a [rows, K/32] array, the layout the
    oracle uses.  A pure re-indexing."""
    a = np.asarray(buf).reshape(-1)[:mx_scale_bytes(rows, K)].reshape(-(-K // 128), rows, 4)
    return np.ascontiguousarray(a.transpose(1, 0, 2).reshape(rows, -1)[:, :K // 32])
