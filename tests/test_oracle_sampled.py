"""Pins of the sampled oracle (oracle/sampled_ref.py) to the whole-layer oracles.

The sampled functions restate the layer's definitions for a few tokens or one
expert at a time; on problems small enough for the whole-layer oracle they must
give the same values (float64, to 1e-12), in bf16 and in MXFP8 (QDQ) form.
"""

import numpy as np
import pytest

from oracle import moe_mx_ref as mxl
from oracle import moe_ref as ref
from oracle import sampled_ref as sref
from token_routing_grouped_amd import inputs


def _problem(T, d, h, E, k, seed):
    rng = np.random.default_rng(seed)
    b = lambda *s, std=1.0: inputs.bf16_round((rng.standard_normal(s) * std).astype(np.float32))  # noqa: E731
    x, dy = b(T, d), b(T, d)
    wr = b(E, d, std=0.3)
    w1, w3, w2 = b(E, h, d, std=0.1), b(E, h, d, std=0.1), b(E, d, h, std=0.1)
    L32 = ref.router_logits(x, wr).astype(np.float32)
    return x, dy, wr, w1, w3, w2, L32


def _close(got, want, name):
    scale = max(float(np.max(np.abs(want))), 1e-300)
    err = float(np.max(np.abs(np.asarray(got) - np.asarray(want))))
    assert err <= 1e-12 * scale, f"{name}: {err:.3e} vs scale {scale:.3e}"


@pytest.mark.parametrize("mx_on", [False, True])
@pytest.mark.parametrize("T,d,h,E,k", [(40, 64, 64, 6, 2), (33, 96, 64, 5, 3)])
def test_sampled_equals_whole_layer(mx_on, T, d, h, E, k):
    x, dy, wr, w1, w3, w2, L32 = _problem(T, d, h, E, k, seed=T * 7 + k)
    fwd_f, bwd_f = (mxl.layer_forward_mx, mxl.layer_backward_mx) if mx_on else (ref.layer_forward, ref.layer_backward)
    f = fwd_f(x, wr, w1, w3, w2, k, logits=L32)
    b = bwd_f(f, dy, x, wr, w1, w3, w2)

    S = np.array([0, 5, T // 2, T - 1])
    idx_s = f["idx"][S]
    experts = np.unique(idx_s)
    t = sref.tokens(x[S], dy[S], L32[S], idx_s, wr, experts, w1[experts], w3[experts], w2[experts], mx_on=mx_on)
    _close(t["y"], f["y"][S], "y")
    _close(t["dgate"], b["dgate"][S], "dgate")
    _close(t["dx"], b["dx"][S], "dx")

    off, src = f["offsets"], f["src"]
    hid = np.array([0, 7, h - 1])
    checked = 0
    for e in range(E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size == 0:
            continue
        tok, slot = src[rows] // k, src[rows] % k
        s = sref.expert_slices(x[tok], dy[tok], f["w"][tok, slot], w1[e], w3[e], w2[e], hid, mx_on=mx_on)
        _close(s["dw1"], b["dw1"][e][hid], f"dW1[{e}]")
        _close(s["dw3"], b["dw3"][e][hid], f"dW3[{e}]")
        _close(s["dw2"], b["dw2"][e][:, hid], f"dW2[{e}]")
        checked += 1
    assert checked >= 3
