"""Pins of the oracle's routing step against brute force, closed forms and a
hand-derived case (tests/golden/route_hand_T3E4k2.txt)."""

import math
import os

import numpy as np
import pytest

from oracle import moe_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            rows = [[float(v) for v in part.split()] for part in rest.split("|")]
            out[key] = rows
    return out


def _brute_topk(L, k):
    """Python sort per row by (-logit, index)."""
    return [sorted(range(len(row)), key=lambda e: (-row[e], e))[:k] for row in L.tolist()]


@pytest.mark.parametrize("T,E,k,seed", [(64, 8, 2, 0), (50, 16, 4, 1), (33, 128, 4, 2), (17, 384, 8, 3),
                                        (9, 5, 5, 4), (7, 1, 1, 5)])
def test_topk_matches_brute_force(T, E, k, seed):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    assert ref.topk_experts(L, k).tolist() == _brute_topk(L, k)
    # heavy ties: logits on a coarse grid
    Lt = (np.rint(L * 2) / 2).astype(np.float32)
    assert ref.topk_experts(Lt, k).tolist() == _brute_topk(Lt, k)


def test_topk_signed_zero_is_a_tie():
    L = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert ref.topk_experts(L, 2).tolist() == [[0, 1]]


def test_hand_case_golden():
    g = _parse_golden("route_hand_T3E4k2.txt")
    L = np.array(g["logits"], np.float32)
    k = int(g["k"][0][0])
    rt = ref.route(L, k)
    assert rt["idx"].tolist() == [[int(v) for v in r] for r in g["idx"]]
    assert rt["counts"].tolist() == [int(v) for v in g["counts"][0]]
    assert rt["offsets"].tolist() == [int(v) for v in g["offsets"][0]]
    assert rt["pos"].tolist() == [[int(v) for v in r] for r in g["pos"]]
    assert rt["src"].tolist() == [int(v) for v in g["src"][0]]
    assert rt["off128"].tolist() == [int(v) for v in g["off128"][0]]
    assert np.allclose(rt["w"][1], g["w_t1"][0], rtol=0, atol=1e-15)
    # gates of t0 from the definition of softmax, by hand
    den = math.exp(1) + 2 * math.exp(2) + math.exp(0.5)
    assert np.allclose(rt["w"][0], [math.exp(2) / den, math.exp(2) / den], rtol=1e-14)


@pytest.mark.parametrize("T,E,k", [(40, 8, 2), (64, 16, 4), (12, 6, 6)])
def test_zero_router_closed_form(T, E, k):
    """Wr = 0: every logit ties, so every token picks experts 0..k-1 and
    pos[t, j] = j*T + t; all probabilities are 1/E."""
    x = np.random.default_rng(0).standard_normal((T, 32))
    L = ref.router_logits(x, np.zeros((E, 32))).astype(np.float32)
    rt = ref.route(L, k)
    assert (rt["idx"] == np.arange(k)[None, :]).all()
    assert rt["counts"].tolist() == [T] * k + [0] * (E - k)
    assert (rt["pos"] == (np.arange(k)[None, :] * T + np.arange(T)[:, None])).all()
    assert np.allclose(rt["probs"], 1.0 / E, rtol=0, atol=1e-15)


@pytest.mark.parametrize("T,E,k", [(48, 8, 2), (50, 7, 3), (384, 384, 8)])
def test_forced_cyclic_routing_closed_form(T, E, k):
    """idx[t, j] = (t + j) mod E: expert e gets every (t, j) with t = e - j mod E."""
    t = np.arange(T)[:, None]
    idx = (t + np.arange(k)[None, :]) % E
    L = np.zeros((T, E), np.float32)
    rt = ref.route(L, k, forced_idx=idx)
    expect = [sum(1 for j in range(k) for tt in range(T) if (tt + j) % E == e) for e in range(E)]
    assert rt["counts"].tolist() == expect
    if T % E == 0:
        assert rt["counts"].tolist() == [T * k // E] * E


@pytest.mark.parametrize("T,E,k,seed", [(100, 8, 2, 0), (257, 128, 4, 1), (64, 384, 8, 2)])
def test_metadata_invariants(T, E, k, seed):
    L = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    rt = ref.route(L, k)
    R = T * k
    counts, off, pos, src, idx = rt["counts"], rt["offsets"], rt["pos"], rt["src"], rt["idx"]
    assert counts.sum() == R
    assert (counts == np.bincount(idx.ravel(), minlength=E)).all()
    assert off[0] == 0 and off[-1] == R and (np.diff(off) == counts).all()
    assert sorted(src.tolist()) == list(range(R))                 # bijection
    assert (src[pos.ravel()] == np.arange(R)).all()                # src[pos[t,j]] = t*k+j
    # every row of expert e's segment holds an (t, j) with idx == e, tokens ascending
    for e in range(E):
        seg = src[off[e]:off[e + 1]]
        assert (idx.ravel()[seg] == e).all()
        assert (np.diff(seg // k) > 0).all()
    c128 = rt["off128"]
    assert c128[0] == 0 and (np.diff(c128) % 128 == 0).all() and (np.diff(c128) >= counts).all()
    assert (np.diff(c128) - counts < 128).all()


def test_softmax_closed_forms():
    # two experts: p0 = sigmoid(L0 - L1)
    L = np.array([[0.3, -1.2], [5.0, 5.0], [-40.0, 40.0]])
    p = ref.softmax(L)
    for r in range(3):
        assert abs(p[r, 0] - 1 / (1 + math.exp(-(L[r, 0] - L[r, 1])))) < 1e-15
    # shift invariance, rows sum to one, Python math brute force
    rng = np.random.default_rng(3)
    L = rng.standard_normal((5, 9)) * 3
    p = ref.softmax(L)
    assert np.allclose(p, ref.softmax(L + 7.5), atol=1e-15)
    assert np.allclose(p.sum(1), 1, atol=1e-15)
    for r in range(5):
        den = sum(math.exp(v) for v in L[r])
        assert np.allclose(p[r], [math.exp(v) / den for v in L[r]], rtol=1e-13)


def test_gate_conservation_through_src():
    """The multiset of (token, gate) pairs is preserved by the permutation."""
    rng = np.random.default_rng(7)
    T, E, k = 40, 16, 4
    L = rng.standard_normal((T, E)).astype(np.float32)
    rt = ref.route(L, k)
    gates_by_row = rt["w"].ravel()[rt["src"]]
    tok_by_row = rt["src"] // k
    pairs_rows = sorted(zip(tok_by_row.tolist(), gates_by_row.tolist()))
    pairs_tok = sorted((t, rt["w"][t, j]) for t in range(T) for j in range(k))
    assert pairs_rows == pairs_tok
