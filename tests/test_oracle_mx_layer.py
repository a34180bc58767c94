"""Pins of the MXFP8 layer oracle (oracle/moe_mx_ref.py) and of mx_ref.qdq_cols.

The MX layer oracle runs the float layer on quantise-dequantised (QDQ)
operands, each grouped-GEMM operand blocked along its own GEMM's reduction
dimension ([OC3] "Precision optimisation with MXFP8" names the format; the
blocking axes are the reading c18).  What fixes it from outside:

  QDQ is the identity on an operand whose every 32-block along the blocking
  axis is already on the E4M3 grid of that block's scale.

So each case below builds an operand that is exact along the axis its GEMM
must block it on, and NOT exact along the other axis (values 2^-20 times
smaller share the other axis' blocks, so they underflow there).  Then the MX
oracle's result of that GEMM must equal the float oracle's exactly (the float
oracle is pinned by dense brute force and finite differences), and a
quantisation along the wrong axis -- rows for columns, a whole-R column block
instead of a per-expert segment block, or a copy made from another MX copy
instead of the bf16 value -- changes it.  ``test_each_mutation_is_caught``
applies exactly those mistakes to the oracle's source and checks that one of
the pins fails for each.

All values are small integers times powers of two, chosen so that every sum
the float oracle forms is exact in float64 and every bf16 rounding the MX
oracle applies (c19) is exact too; the gates are exactly 1 (one expert, or
logits +-1000 so that the softmax is exactly 0 / 1).
"""

from __future__ import annotations

import inspect
import types

import numpy as np
import pytest

from oracle import moe_mx_ref as mxl
from oracle import moe_ref as ref
from oracle import mx_ref as mx

BIG, SMALL = 0, -20  # exponents that can share a block only on the wrong axis


def _ints(rng, shape):
    """Nonzero small integers +-1, +-2, +-3 (products of two have <= 4 significant bits)."""
    return rng.integers(1, 4, shape) * rng.choice([-1, 1], shape)


def _alt(n, period=2):
    """Exponent per index: BIG and SMALL alternating, so every 32-block holds both."""
    return np.where(np.arange(n) % period == 0, BIG, SMALL)


def _one_hot_logits(expert):
    """Logits whose softmax is exactly one-hot on `expert` (gate 1.0)."""
    T = len(expert)
    E = int(expert.max()) + 1
    L = np.full((T, max(E, 2)), -1000.0, np.float32)
    L[np.arange(T), expert] = 1000.0
    return L


def _ragged_experts(T):
    """Two interleaved experts with 45 and 51 rows of 96 (segment ends off the 32-grid)."""
    assert T == 96
    return np.where((np.arange(T) * 7) % 96 < 45, 0, 1)


def _swiglu_weights(d, h, E, w1_extra=None, w3_extra=None, b=None):
    """W1 puts 64 on x's column 0 (G = 64 everywhere, so silu(G) = G and
    sigmoid(G) = 1 exactly in float64); W3 puts b_j on x's column 32
    (U[t, j] = x[t, 32] b_j).  Optional extra W1 / W3 columns (1 and 33) that x
    leaves at zero."""
    w1 = np.zeros((E, h, d))
    w3 = np.zeros((E, h, d))
    w1[:, :, 0] = 64.0
    w3[:, :, 32] = 1.0 if b is None else b
    if w1_extra is not None:
        w1[:, :, 1] = w1_extra
    if w3_extra is not None:
        w3[:, :, 33] = w3_extra
    return w1, w3


def _x(T, d, a=None):
    x = np.zeros((T, d))
    x[:, 0] = 1.0
    x[:, 32] = 1.0 if a is None else a
    return x


# ---------------------------------------------------------------------------
# the pins, each taking the MX layer module under test
# ---------------------------------------------------------------------------

def pin_up(m):
    """Up projection: Xp blocked along d, W1/W3 blocked along d (their rows)."""
    rng = np.random.default_rng(11)
    T, d, h = 96, 64, 64
    x = np.ldexp(_ints(rng, (T, d)), _alt(T)[:, None])          # rows exact, columns mixed
    w1 = np.ldexp(_ints(rng, (1, h, d)), _alt(h)[None, :, None])  # rows exact, columns mixed
    w3 = np.ldexp(_ints(rng, (1, h, d)), _alt(h, 3)[None, :, None])
    w2 = np.zeros((1, d, h))
    L = np.zeros((T, 1), np.float32)
    f = ref.layer_forward(x, None, w1, w3, w2, 1, logits=L)
    fm = m.layer_forward_mx(x, None, w1, w3, w2, 1, logits=L)
    assert np.array_equal(fm["G"], mxl.bf16_value(f["G"])), "G"
    assert np.array_equal(fm["U"], mxl.bf16_value(f["U"])), "U"


def pin_down(m):
    """Down projection: H blocked along h, W2 blocked along h (its rows)."""
    rng = np.random.default_rng(12)
    T, d, h = 96, 64, 64
    a = np.ldexp(1.0, _alt(T))                                   # H = 64 a_t b_j: rows exact, columns mixed
    b = _ints(rng, h)
    x = _x(T, d, a)
    w1, w3 = _swiglu_weights(d, h, 1, b=b)
    w2 = np.ldexp(_ints(rng, (1, d, h)), _alt(d)[None, :, None])  # rows (along h) exact, columns mixed
    L = np.zeros((T, 1), np.float32)
    f = ref.layer_forward(x, None, w1, w3, w2, 1, logits=L)
    fm = m.layer_forward_mx(x, None, w1, w3, w2, 1, logits=L)
    assert np.array_equal(f["H"], 64.0 * a[:, None] * b[None, :])
    assert np.array_equal(fm["H"], f["H"]), "H"
    assert np.array_equal(fm["yp"], f["yp"]), "Yp"
    assert np.array_equal(fm["y"], f["y"]), "y"


def pin_dgrad_down(m):
    """dgrad down: dYp blocked along d, W2 blocked along d (its columns)."""
    rng = np.random.default_rng(13)
    T, d, h = 96, 64, 64
    b = _ints(rng, h)
    x = _x(T, d)
    w1, w3 = _swiglu_weights(d, h, 1, b=b)                       # G = 64, U[t, j] = b_j
    w2 = np.ldexp(_ints(rng, (1, d, h)), _alt(h)[None, None, :])  # columns (along d) exact, rows mixed
    dy = np.zeros((T, d))
    dy[:, :4] = np.ldexp(_ints(rng, (T, 4)), _alt(T)[:, None])    # rows exact, columns mixed
    L = np.zeros((T, 1), np.float32)
    f = ref.layer_forward(x, None, w1, w3, w2, 1, logits=L)
    b_ = ref.layer_backward(f, dy, x, np.zeros((1, d)), w1, w3, w2)
    fm = m.layer_forward_mx(x, None, w1, w3, w2, 1, logits=L)
    bm = m.layer_backward_mx(fm, dy, x, np.zeros((1, d)), w1, w3, w2)
    assert np.array_equal(b_["dU"], 64.0 * b_["dH"]) and np.array_equal(b_["dG"], b_["dH"] * b[None, :])
    assert np.array_equal(bm["dU"], mxl.bf16_value(b_["dU"])), "dU"
    assert np.array_equal(bm["dG"], mxl.bf16_value(b_["dG"])), "dG"


def pin_wgrad_down(m):
    """wgrad down: dYp and H blocked along the routed rows of each expert segment."""
    rng = np.random.default_rng(14)
    T, d, h = 96, 64, 64
    ex = _ragged_experts(T)
    seg = np.where(ex == 0, BIG, SMALL)                           # exponent per token's expert
    a = np.ldexp(_ints(rng, T), seg)                              # H = 64 a_t b_j
    b = np.ldexp(_ints(rng, h), _alt(h))                          # ... columns exact in a segment, rows mixed
    x = _x(T, d, a)
    w1, w3 = _swiglu_weights(d, h, 2, b=b)
    w2 = np.zeros((2, d, h))
    dy = np.ldexp(_ints(rng, (T, d)), _alt(d)[None, :] + seg[:, None])  # same for dYp
    L = _one_hot_logits(ex)
    wr = np.zeros((2, d))
    f = ref.layer_forward(x, wr, w1, w3, w2, 1, logits=L)
    assert (f["w"] == 1.0).all() and list(f["counts"]) == [45, 51]
    b_ = ref.layer_backward(f, dy, x, wr, w1, w3, w2)
    fm = m.layer_forward_mx(x, wr, w1, w3, w2, 1, logits=L)
    bm = m.layer_backward_mx(fm, dy, x, wr, w1, w3, w2)
    assert np.array_equal(fm["H"], f["H"]), "H"
    assert np.array_equal(bm["dyp"], b_["dyp"]), "dYp"
    assert np.array_equal(bm["dw2"], b_["dw2"]), "dW2"


def pin_dgrad_up(m):
    """dgrad up: dG and dU blocked along h, W1 and W3 blocked along h (their columns)."""
    rng = np.random.default_rng(15)
    T, d, h = 96, 64, 64
    x = _x(T, d)
    # extra W1 / W3 columns 2^-20 below the 64 / 1 of their row block: exact
    # along h, underflowing along d; x is zero there, so the forward is untouched
    w1, w3 = _swiglu_weights(d, h, 1, w1_extra=np.ldexp(_ints(rng, h), SMALL),
                             w3_extra=np.ldexp(_ints(rng, h), SMALL))
    w2 = np.zeros((1, d, h))
    w2[0, 0, :] = _ints(rng, h)
    dy = np.zeros((T, d))
    dy[:, 0] = np.ldexp(_ints(rng, T), _alt(T))                   # dH[t, j] = dy[t, 0] w2[0, j]
    L = np.zeros((T, 1), np.float32)
    wr = np.zeros((1, d))
    f = ref.layer_forward(x, wr, w1, w3, w2, 1, logits=L)
    b_ = ref.layer_backward(f, dy, x, wr, w1, w3, w2)
    fm = m.layer_forward_mx(x, wr, w1, w3, w2, 1, logits=L)
    bm = m.layer_backward_mx(fm, dy, x, wr, w1, w3, w2)
    assert np.array_equal(bm["dG"], b_["dG"]) and np.array_equal(bm["dU"], b_["dU"])
    assert np.all(b_["dxp"][:, 1] != 0) and np.all(b_["dxp"][:, 33] != 0)
    assert np.array_equal(bm["dxp"], b_["dxp"]), "dXp"
    assert np.array_equal(bm["dx"], b_["dx"]), "dx"


def pin_wgrad_up(m):
    """wgrad up: dG, dU and Xp blocked along the routed rows of each expert
    segment, each from its bf16 value (not from the rowwise MX copy)."""
    rng = np.random.default_rng(16)
    T, d, h = 96, 64, 64
    ex = _ragged_experts(T)
    seg = np.where(ex == 0, BIG, SMALL)
    x = _x(T, d)
    # x columns other than 0 and 32 (W1 / W3 are zero there): exact along the
    # rows of a segment, mixed along d and across the two segments
    cols = [c for c in range(d) if c not in (0, 32)]
    x[:, cols] = np.ldexp(_ints(rng, (T, len(cols))), _alt(len(cols))[None, :] + seg[:, None])
    w1, w3 = _swiglu_weights(d, h, 2)                             # G = 64, U = 1
    w2 = np.zeros((2, d, h))
    w2[:, 0, :] = np.ldexp(_ints(rng, h), _alt(h))[None, :]      # dH[t, j] = dy[t, 0] w2[0, j]
    dy = np.zeros((T, d))
    dy[:, 0] = np.ldexp(_ints(rng, T), seg)
    L = _one_hot_logits(ex)
    wr = np.zeros((2, d))
    f = ref.layer_forward(x, wr, w1, w3, w2, 1, logits=L)
    assert (f["w"] == 1.0).all() and np.array_equal(f["G"], np.full((T, h), 64.0))
    b_ = ref.layer_backward(f, dy, x, wr, w1, w3, w2)
    fm = m.layer_forward_mx(x, wr, w1, w3, w2, 1, logits=L)
    bm = m.layer_backward_mx(fm, dy, x, wr, w1, w3, w2)
    assert np.array_equal(bm["dG"], b_["dG"]) and np.array_equal(bm["dU"], b_["dU"])
    assert np.array_equal(bm["dw1"], b_["dw1"]), "dW1"
    assert np.array_equal(bm["dw3"], b_["dw3"]), "dW3"


PINS = [pin_up, pin_down, pin_dgrad_down, pin_wgrad_down, pin_dgrad_up, pin_wgrad_up]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_mx_layer_pin(pin):
    pin(mxl)


def test_pins_discriminate_the_axes():
    """The constructions really are off the grid along the wrong axis."""
    rng = np.random.default_rng(0)
    a = np.ldexp(_ints(rng, (96, 64)), _alt(96)[:, None])
    assert np.array_equal(mx.qdq_rows(a), a)
    assert not np.array_equal(mx.qdq_cols(a), a)
    assert np.array_equal(mx.qdq_cols(a.T), a.T)
    ex = _ragged_experts(96)
    rt = ref.route(_one_hot_logits(ex), 1)
    seg = np.where(ex == 0, BIG, SMALL)
    s = np.ldexp(_ints(rng, (96, 64)), seg[:, None])
    assert np.array_equal(mx.qdq_cols_segmented(s[rt["src"]], rt["offsets"], rt["off128"]), s[rt["src"]])
    assert not np.array_equal(mx.qdq_cols(s[rt["src"]]), s[rt["src"]])


# ---------------------------------------------------------------------------
# qdq_cols: blocks of 32 along the rows of [K, N]
# ---------------------------------------------------------------------------

def test_qdq_cols_brute_force():
    """Every 32-row block of every column quantised on its own (rowwise
    quantiser, pinned by the hand vectors, on a single block)."""
    rng = np.random.default_rng(21)
    K, N = 96, 40
    a = rng.standard_normal((K, N)) * np.exp(rng.standard_normal((K, 1)) * 4)
    got = mx.qdq_cols(a)
    for c in range(N):
        for b0 in range(0, K, 32):
            blk = a[b0:b0 + 32, c][None, :]
            want = mx.dequantize_rows(*mx.quantize_rows(blk))[0]
            assert np.array_equal(got[b0:b0 + 32, c], want), (c, b0)


# ---------------------------------------------------------------------------
# mutations of the oracle's source: each must fail one of the pins
# ---------------------------------------------------------------------------

MUTATIONS = [  # (name, old, new)
    ("up: Xp along rows", "xq = mx.qdq_rows(xp)", "xq = mx.qdq_cols(xp)"),
    ("up: W1 along h", "mx.qdq_rows(w1[e]).T", "mx.qdq_cols(w1[e]).T"),
    ("up: W3 along h", "mx.qdq_rows(w3[e]).T", "mx.qdq_cols(w3[e]).T"),
    ("down: H along rows", "hq = mx.qdq_rows(H)", "hq = mx.qdq_cols(H)"),
    ("down: W2 along d", "mx.qdq_rows(w2[e]).T", "mx.qdq_cols(w2[e]).T"),
    ("dgrad down: dYp along rows", "dyq_r = mx.qdq_rows(dyp)", "dyq_r = mx.qdq_cols(dyp)"),
    ("dgrad down: W2 along h", "dyq_r[a:b] @ mx.qdq_cols(w2[e])", "dyq_r[a:b] @ mx.qdq_rows(w2[e])"),
    ("wgrad down: dYp rowwise", "dyq_c = mx.qdq_cols_segmented(dyp, offsets, off128)", "dyq_c = mx.qdq_rows(dyp)"),
    ("wgrad down: dYp whole-R blocks", "dyq_c = mx.qdq_cols_segmented(dyp, offsets, off128)",
     "dyq_c = mx.qdq_cols(dyp)"),
    ("wgrad down: H rowwise", 'hq_c = mx.qdq_cols_segmented(fwd["H"], offsets, off128)', 'hq_c = mx.qdq_rows(fwd["H"])'),
    ("wgrad down: H whole-R blocks", 'hq_c = mx.qdq_cols_segmented(fwd["H"], offsets, off128)',
     'hq_c = mx.qdq_cols(fwd["H"])'),
    ("wgrad up: dG rowwise", "dgq_c = mx.qdq_cols_segmented(dG, offsets, off128)", "dgq_c = mx.qdq_rows(dG)"),
    ("wgrad up: dG whole-R blocks", "dgq_c = mx.qdq_cols_segmented(dG, offsets, off128)", "dgq_c = mx.qdq_cols(dG)"),
    ("wgrad up: dG from its MX row copy", "dgq_c = mx.qdq_cols_segmented(dG, offsets, off128)",
     "dgq_c = mx.qdq_cols_segmented(mx.qdq_rows(dG), offsets, off128)"),
    ("wgrad up: dU rowwise", "duq_c = mx.qdq_cols_segmented(dU, offsets, off128)", "duq_c = mx.qdq_rows(dU)"),
    ("wgrad up: dU whole-R blocks", "duq_c = mx.qdq_cols_segmented(dU, offsets, off128)", "duq_c = mx.qdq_cols(dU)"),
    ("wgrad up: dU from its MX row copy", "duq_c = mx.qdq_cols_segmented(dU, offsets, off128)",
     "duq_c = mx.qdq_cols_segmented(mx.qdq_rows(dU), offsets, off128)"),
    ("wgrad up: Xp rowwise", 'xq_c = mx.qdq_cols_segmented(fwd["xp"], offsets, off128)', 'xq_c = mx.qdq_rows(fwd["xp"])'),
    ("wgrad up: Xp whole-R blocks", 'xq_c = mx.qdq_cols_segmented(fwd["xp"], offsets, off128)',
     'xq_c = mx.qdq_cols(fwd["xp"])'),
    ("dgrad up: dG, dU along rows", "dgq_r, duq_r = mx.qdq_rows(dG), mx.qdq_rows(dU)",
     "dgq_r, duq_r = mx.qdq_cols(dG), mx.qdq_cols(dU)"),
    ("dgrad up: W1 along d", "dgq_r[a:b] @ mx.qdq_cols(w1[e])", "dgq_r[a:b] @ mx.qdq_rows(w1[e])"),
    ("dgrad up: W3 along d", "duq_r[a:b] @ mx.qdq_cols(w3[e])", "duq_r[a:b] @ mx.qdq_rows(w3[e])"),
]


def _mutant(old, new):
    src = inspect.getsource(mxl)
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    src = src.replace(old, new).replace("from . import moe_ref as ref", "from oracle import moe_ref as ref")
    src = src.replace("from . import mx_ref as mx", "from oracle import mx_ref as mx")
    mod = types.ModuleType("moe_mx_ref_mutant")
    exec(compile(src, "moe_mx_ref_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mut", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_each_mutation_is_caught(mut):
    name, old, new = mut
    mod = _mutant(old, new)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutation {name!r} passes every pin"


def test_qdq_cols_mutation_is_caught():
    """qdq_cols written as a plain rowwise QDQ (no transpose) fails the brute force."""
    rng = np.random.default_rng(22)
    a = rng.standard_normal((64, 64)) * np.exp(rng.standard_normal((64, 1)) * 4)
    wrong = mx.qdq_rows(a)
    right = mx.qdq_cols(a)
    assert not np.array_equal(wrong, right)
