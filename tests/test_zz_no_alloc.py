"""moe_route_noalloc (routing with the library's static scratch, no workspace)
against moe_route with a caller workspace, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input, so the second
runs on the scratch the first left behind; every output must equal moe_route's
bit for bit (and the integer outputs the oracle's routing of the same logits).
A routing larger than the scratch is refused before anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

from oracle import moe_ref as ref
from token_routing_grouped_amd import inputs

from helpers import say, to_np

DEV = torch.device("cuda:0")
OUTS = ("probs", "topk_idx", "topk_w", "counts", "offsets", "pos", "src", "off128")


def _bufs(T, E, k):
    f32, i32 = torch.float32, torch.int32
    e = lambda *s, dt: torch.full(s, -7, dtype=dt, device=DEV)
    return dict(probs=e(T, E, dt=f32), topk_idx=e(T, k, dt=i32), topk_w=e(T, k, dt=f32), counts=e(E, dt=i32),
                offsets=e(E + 1, dt=i32), pos=e(T, k, dt=i32), src=e(T * k, dt=i32), off128=e(E + 1, dt=i32),
                err_flag=torch.zeros(1, dtype=i32, device=DEV))


def _route_both(L, k, forced=None):
    from token_routing_grouped_amd import _abi

    T, E = L.shape
    lg = torch.from_numpy(L).to(DEV)
    fi = None if forced is None else torch.from_numpy(forced).to(DEV)
    a, b = _bufs(T, E, k), _bufs(T, E, k)
    ws = _abi.workspace(_abi.moe_route_workspace_size(T, E, k), DEV)
    _abi.moe_route(lg, k, a["probs"], a["topk_idx"], a["topk_w"], a["counts"], a["offsets"], a["pos"], a["src"], ws,
                   off128=a["off128"], forced_idx=fi, err_flag=a["err_flag"])
    _abi.moe_route_noalloc(lg, k, b["probs"], b["topk_idx"], b["topk_w"], b["counts"], b["offsets"], b["pos"],
                           b["src"], off128=b["off128"], forced_idx=fi, err_flag=b["err_flag"])
    torch.cuda.synchronize()
    return a, b


@pytest.mark.gpu
def test_noalloc_route_matches_workspace_route_twice():
    cases = [  # T, E, k, forced routing: the second call is the smaller one
        (16384, 128, 4, None),
        (300, 16, 2, "zipf"),
    ]
    for T, E, k, mode in cases:
        say(f"route_noalloc T={T} E={E} k={k} forced={mode}")
        L = np.random.default_rng(T + E).standard_normal((T, E)).astype(np.float32)
        L[::7, :] = np.round(L[::7, :])  # ties on some rows
        forced = None if mode is None else inputs.forced_routing(mode, T, E, k, 3)
        a, b = _route_both(L, k, forced)
        for n in OUTS + ("err_flag",):
            assert torch.equal(a[n], b[n]), f"T={T}: {n} differs from moe_route"
        r = ref.route(L, k, forced_idx=forced)
        for n, rn in (("topk_idx", "idx"), ("counts", "counts"), ("offsets", "offsets"), ("pos", "pos"),
                      ("src", "src"), ("off128", "off128")):
            assert (to_np(b[n]) == r[rn]).all(), f"T={T}: {n} differs from the oracle"
        assert int(b["err_flag"].item()) == 0


def test_noalloc_route_refuses_routings_larger_than_its_scratch():
    """Host-side size check (no GPU needed): 300000 rows at E = 1024 need
    1172 chunks x 1024 x 4 bytes, more than the 4 MiB scratch."""
    from token_routing_grouped_amd import _abi

    lib = _abi.lib()
    c = ctypes.c_void_p(16)
    st = lib.moe_route_noalloc(c, 300000, 1024, 1, None, c, c, c, c, c, c, c, None, None, None)
    assert st == 4 and b"scratch" in lib.moe_last_error_string()
    st = lib.moe_route_noalloc(c, 8, 4, 5, None, c, c, c, c, c, c, c, None, None, None)
    assert st == 1
