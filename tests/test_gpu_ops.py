"""GPU parity of the row-move steps (permute, combine, combine backward,
unpermute-sum) and the router GEMMs against the oracle."""

import numpy as np
import pytest
import torch

from oracle import moe_ref as ref
from token_routing_grouped_amd import inputs

from helpers import assert_close, say, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dt)


def _routing(T, E, k, seed):
    L = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    return ref.route(L, k)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,d,E,k", [(257, 2048, 8, 4), (100, 128, 8, 2), (64, 6144, 384, 8), (33, 64, 5, 5)])
def test_permute_bit_exact_and_unpermute(dt, T, d, E, k):
    from token_routing_grouped_amd import _abi

    say(f"permute {dt} T={T} d={d} E={E} k={k}")
    rt = _routing(T, E, k, T + d)
    x = inputs.bf16_round(np.random.default_rng(1).standard_normal((T, d)).astype(np.float32))
    xt = _dev(x, DT[dt])
    pos = _dev(rt["pos"].astype(np.int32), torch.int32)
    xp = torch.empty(T * k, d, dtype=DT[dt], device=DEV)
    _abi.moe_permute(xt, pos, xp)
    dx = torch.empty(T, d, dtype=DT[dt], device=DEV)
    _abi.moe_unpermute_sum(xp, pos, dx)
    torch.cuda.synchronize()
    assert (to_np(xp) == ref.permute(x, rt["pos"])).all()
    # a sum of k equal values is exact when k is a power of two
    got = to_np(dx)
    if k & (k - 1) == 0:
        assert (got == k * x.astype(np.float64)).all()
    else:
        assert_close("unpermute", got, k * x.astype(np.float64), rel=1e-2)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,d,E,k", [(257, 2048, 8, 4), (65, 6144, 384, 8), (40, 128, 8, 2)])
def test_combine_and_backward(dt, T, d, E, k):
    from token_routing_grouped_amd import _abi

    say(f"combine {dt} T={T} d={d} E={E} k={k}")
    rt = _routing(T, E, k, 7 * T)
    rng = np.random.default_rng(2)
    yp = inputs.bf16_round(rng.standard_normal((T * k, d)).astype(np.float32))
    dy = inputs.bf16_round(rng.standard_normal((T, d)).astype(np.float32))
    w = rt["w"].astype(np.float32)
    ypt, dyt = _dev(yp, DT[dt]), _dev(dy, DT[dt])
    wt, pos = _dev(w, torch.float32), _dev(rt["pos"].astype(np.int32), torch.int32)
    y = torch.empty(T, d, dtype=DT[dt], device=DEV)
    dyp = torch.empty(T * k, d, dtype=DT[dt], device=DEV)
    dgate = torch.empty(T, k, dtype=torch.float32, device=DEV)
    _abi.moe_combine(ypt, wt, pos, y)
    _abi.moe_combine_bwd(dyt, ypt, wt, pos, dyp, dgate)
    torch.cuda.synchronize()
    tol = 1e-2 if dt == "bf16" else 1e-5
    assert_close("y", to_np(y), ref.combine(yp, w, rt["pos"]), rel=tol)
    rdyp, rdgate = ref.combine_backward(dy, yp, w, rt["pos"])
    assert_close("dyp", to_np(dyp), rdyp, rel=tol)
    assert_close("dgate", to_np(dgate), rdgate, rel=1e-5)


@pytest.mark.parametrize("dt,T,d,E", [("bf16", 1000, 2048, 8), ("f32", 256, 128, 8), ("bf16", 700, 2048, 128),
                                      ("bf16", 300, 6144, 384), ("bf16", 129, 512, 40), ("f32", 77, 96, 64)])
def test_router_logits(dt, T, d, E):
    from token_routing_grouped_amd import _abi

    say(f"router logits {dt} T={T} d={d} E={E}")
    rng = np.random.default_rng(T + E)
    x = inputs.bf16_round(rng.standard_normal((T, d)).astype(np.float32))
    wr = inputs.bf16_round((rng.standard_normal((E, d)) * 0.02).astype(np.float32))
    L = torch.empty(T, E, dtype=torch.float32, device=DEV)
    _abi.moe_router_logits(_dev(x, DT[dt]), _dev(wr, DT[dt]), L)
    torch.cuda.synchronize()
    assert_close("logits", to_np(L), ref.router_logits(x, wr), rel=1e-5, max_frac=1e-4)


@pytest.mark.parametrize("acc", [False, True])
@pytest.mark.parametrize("dt,T,d,E,k", [("bf16", 1000, 2048, 8, 4), ("f32", 256, 128, 8, 2),
                                        ("bf16", 700, 2048, 128, 4), ("bf16", 300, 6144, 384, 8),
                                        ("bf16", 129, 512, 40, 3)])
def test_router_backward(dt, T, d, E, k, acc):
    """dx starts at zero (the router term alone) or at a random expert-path
    gradient (accumulation)."""
    from token_routing_grouped_amd import _abi

    say(f"router bwd {dt} T={T} d={d} E={E} k={k} acc={acc}")
    rng = np.random.default_rng(5 * T + E)
    x = inputs.bf16_round(rng.standard_normal((T, d)).astype(np.float32))
    wr = inputs.bf16_round((rng.standard_normal((E, d)) * 0.02).astype(np.float32))
    dx0 = inputs.bf16_round((rng.standard_normal((T, d)) * 0.01).astype(np.float32))
    if not acc:
        dx0[:] = 0
    L = ref.router_logits(x, wr).astype(np.float32)
    rt = ref.route(L, k)
    probs = rt["probs"].astype(np.float32)
    dgate = rng.standard_normal((T, k)).astype(np.float32)
    dx = _dev(dx0, DT[dt])
    dwr = torch.empty(E, d, dtype=DT[dt], device=DEV)
    ws = _abi.workspace(_abi.moe_router_bwd_workspace_size(T, d, E), DEV)
    _abi.moe_router_bwd(_dev(probs, torch.float32), _dev(rt["idx"].astype(np.int32), torch.int32),
                        _dev(dgate, torch.float32), _dev(x, DT[dt]), _dev(wr, DT[dt]), dx, dwr, ws)
    torch.cuda.synchronize()
    dL, rdwr, rdx = ref.router_backward(probs, rt["idx"], dgate, x, wr)
    assert_close("dwr", to_np(dwr), rdwr)
    assert_close("dx", to_np(dx), dx0.astype(np.float64) + rdx)


@pytest.mark.parametrize("aux", [False, True])
@pytest.mark.parametrize("dt,T,d,E,k", [("bf16", 1000, 2048, 8, 4), ("f32", 256, 128, 8, 2),
                                        ("bf16", 700, 2048, 128, 4), ("bf16", 300, 6144, 384, 8),
                                        ("bf16", 129, 512, 40, 3), ("bf16", 131, 320, 64, 1),
                                        ("f32", 77, 96, 64, 5)])
def test_router_backward_unpermute(dt, T, d, E, k, aux):
    """moe_router_bwd_unpermute: dx = unpermute-sum of dXp + the router term in
    one pass (one rounding) against the oracle; dWr identical to
    moe_router_bwd's; dx within a rounding of the two-call path."""
    from token_routing_grouped_amd import _abi

    say(f"router bwd + unpermute {dt} T={T} d={d} E={E} k={k} aux={aux}")
    rng = np.random.default_rng(11 * T + E + k)
    x = inputs.bf16_round(rng.standard_normal((T, d)).astype(np.float32))
    wr = inputs.bf16_round((rng.standard_normal((E, d)) * 0.02).astype(np.float32))
    dxp = inputs.bf16_round((rng.standard_normal((T * k, d)) * 0.01).astype(np.float32))
    L = ref.router_logits(x, wr).astype(np.float32)
    rt = ref.route(L, k)
    probs = rt["probs"].astype(np.float32)
    dgate = rng.standard_normal((T, k)).astype(np.float32)
    aux_g = (np.abs(rng.standard_normal(E)) * 0.1).astype(np.float32) if aux else None
    args = dict(probs=_dev(probs, torch.float32), topk_idx=_dev(rt["idx"].astype(np.int32), torch.int32),
                dgate=_dev(dgate, torch.float32), x=_dev(x, DT[dt]), wr=_dev(wr, DT[dt]))
    pos = _dev(rt["pos"].astype(np.int32), torch.int32)
    dxp_t = _dev(dxp, DT[dt])
    ag = None if aux_g is None else _dev(aux_g, torch.float32)
    ws = _abi.workspace(_abi.moe_router_bwd_workspace_size(T, d, E), DEV)
    dx = torch.full((T, d), float("nan"), dtype=DT[dt], device=DEV)  # written, not read
    dwr = torch.empty(E, d, dtype=DT[dt], device=DEV)
    _abi.moe_router_bwd_unpermute(args["probs"], args["topk_idx"], args["dgate"], args["x"], args["wr"], dxp_t, pos,
                                  dx, dwr, ws, aux_g=ag)
    # the two-call path on the same inputs
    dx2 = torch.empty(T, d, dtype=DT[dt], device=DEV)
    dwr2 = torch.empty(E, d, dtype=DT[dt], device=DEV)
    _abi.moe_unpermute_sum(dxp_t, pos, dx2)
    if ag is None:
        _abi.moe_router_bwd(args["probs"], args["topk_idx"], args["dgate"], args["x"], args["wr"], dx2, dwr2, ws)
    else:
        _abi.moe_router_bwd_aux(args["probs"], args["topk_idx"], args["dgate"], ag, args["x"], args["wr"], dx2, dwr2,
                                ws)
    torch.cuda.synchronize()
    dL, rdwr, rdx = ref.router_backward(probs, rt["idx"], dgate, x, wr, aux_g=aux_g)
    rdx_all = ref.unpermute_sum(dxp, rt["pos"]) + rdx
    tol = 1e-2 if dt == "bf16" else 1e-5
    assert_close("dx", to_np(dx), rdx_all, rel=tol, max_frac=2e-2 if dt == "bf16" else 1e-4)
    assert_close("dwr", to_np(dwr), rdwr, rel=tol, max_frac=2e-2 if dt == "bf16" else 1e-4)
    assert torch.equal(dwr, dwr2), "dwr differs from moe_router_bwd's"
    # one rounding instead of two: apart by at most the two paths' rounding
    # errors, a few units in the last place of the two terms' magnitudes
    d1, d2 = to_np(dx).astype(np.float64), to_np(dx2).astype(np.float64)
    ulp = 2.0 ** -7 if dt == "bf16" else 2.0 ** -22
    mag = np.abs(ref.unpermute_sum(dxp, rt["pos"])) + np.abs(rdx)
    assert np.all(np.abs(d1 - d2) <= 3 * ulp * mag + 1e-30)


@pytest.mark.parametrize("dt,T,d,E,k", [("bf16", 1000, 2048, 8, 4), ("bf16", 700, 2048, 128, 4), ("f32", 77, 96, 64, 5)])
def test_router_backward_parts_equal_the_whole_call(dt, T, d, E, k):
    """moe_router_bwd_unpermute_parts: the dWr part and the dx part, each with
    its own workspace, give the one-call result bit for bit."""
    from token_routing_grouped_amd import _abi

    say(f"router bwd parts {dt} T={T} d={d} E={E} k={k}")
    rng = np.random.default_rng(17 * T + E)
    x = _dev(inputs.bf16_round(rng.standard_normal((T, d)).astype(np.float32)), DT[dt])
    wr = _dev(inputs.bf16_round((rng.standard_normal((E, d)) * 0.02).astype(np.float32)), DT[dt])
    dxp = _dev(inputs.bf16_round((rng.standard_normal((T * k, d)) * 0.01).astype(np.float32)), DT[dt])
    rt = ref.route(ref.router_logits(to_np(x), to_np(wr)).astype(np.float32), k)
    probs = _dev(rt["probs"].astype(np.float32), torch.float32)
    idx = _dev(rt["idx"].astype(np.int32), torch.int32)
    pos = _dev(rt["pos"].astype(np.int32), torch.int32)
    dgate = _dev(rng.standard_normal((T, k)).astype(np.float32), torch.float32)
    ws1 = _abi.workspace(_abi.moe_router_bwd_workspace_size(T, d, E), DEV)
    ws2 = _abi.workspace(_abi.moe_router_bwd_workspace_size(T, d, E), DEV)
    dx, dwr = torch.empty(T, d, dtype=DT[dt], device=DEV), torch.empty(E, d, dtype=DT[dt], device=DEV)
    _abi.moe_router_bwd_unpermute(probs, idx, dgate, x, wr, dxp, pos, dx, dwr, ws1)
    dx2 = torch.full((T, d), float("nan"), dtype=DT[dt], device=DEV)
    dwr2 = torch.full((E, d), float("nan"), dtype=DT[dt], device=DEV)
    _abi.moe_router_bwd_unpermute_parts(_abi.ROUTER_DWR, probs, idx, dgate, x, wr, None, None, None, dwr2, ws2)
    _abi.moe_router_bwd_unpermute_parts(_abi.ROUTER_DX, probs, idx, dgate, x, wr, dxp, pos, dx2, None, ws1)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2) and torch.equal(dwr, dwr2)
