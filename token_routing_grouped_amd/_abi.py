"""ctypes binding of the C ABI in include/moe.h (argument marshalling only).

Every function takes torch tensors that live on the current HIP device, checks
device, dtype and contiguity, and passes raw pointers plus torch's current
stream.  All arithmetic happens in the HIP library; if the library is missing
the first call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtrg_moe.so")

MOE_F32, MOE_BF16 = 0, 1
FLAG_INDEX_RANGE, FLAG_DUPLICATE = 1, 2
_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t

_SIGS = {
    "moe_version": ([], ctypes.c_char_p),
    "moe_last_error_string": ([], ctypes.c_char_p),
    "moe_prof_enable": ([_I], _I),
    "moe_prof_reset": ([], _I),
    "moe_prof_only": ([ctypes.c_char_p], _I),
    "moe_prof_query": ([ctypes.c_char_p, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float)], _I),
    "moe_prof_names": ([ctypes.c_char_p, _Z], _Z),
    "moe_router_logits": ([_P, _I, _P, _I, _I, _I, _P, _P], _I),
    "moe_route_workspace_size": ([_I, _I, _I], _Z),
    "moe_route": ([_P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P], _I),
    "moe_route_noalloc": ([_P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P], _I),
    "moe_permute": ([_P, _I, _I, _I, _I, _P, _P, _P], _I),
    "moe_combine": ([_P, _P, _P, _I, _I, _I, _I, _P, _P], _I),
    "moe_combine_bwd": ([_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P], _I),
    "moe_unpermute_sum": ([_P, _P, _I, _I, _I, _I, _P, _P], _I),
    "moe_grouped_gemm_workspace_size": ([_I, _I, _I, _I], _Z),
    "moe_grouped_gemm_fwd": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P], _I),
    "moe_grouped_gemm_bwd_parts": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P,
                                    ctypes.c_uint, _P, _Z, _P], _I),
    "moe_grouped_gemm_recompute_gu": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _Z, _P], _I),
    "moe_grouped_gemm_recompute_gu_mx": ([_P, _P], _I),
    "moe_grouped_gemm_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _Z,
                              _P], _I),
    "moe_router_bwd_workspace_size": ([_I, _I, _I], _Z),
    "moe_router_bwd": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _Z, _P], _I),
    "moe_router_bwd_aux": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _Z, _P], _I),
    "moe_router_bwd_unpermute": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _Z, _P], _I),
    "moe_router_bwd_unpermute_parts": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _Z,
                                        ctypes.c_uint, _P], _I),
    "moe_balance_workspace_size": ([_I, _I], _Z),
    "moe_balance": ([_P, _P, _I, _I, _I, ctypes.c_float, _P, _P, _P, _P, _Z, _P], _I),
    "mx_quantize": ([_P, _I, _I, _I, _P, _I, _P, _P, _I, _I, _P, _P, _P, _P, _I, _P], _I),
    "moe_grouped_gemm_fwd_mx": ([_P, _P], _I),
    "moe_grouped_gemm_bwd_mx": ([_P, _P], _I),
    "moe_grouped_gemm_bwd_mx_parts": ([_P, ctypes.c_uint, _P], _I),
    "moe_grouped_gemm_fwd_mx_parts": ([_P, ctypes.c_uint, _P], _I),
}


class MxFwdArgs(ctypes.Structure):
    """moe_mx_fwd_args (include/moe.h)."""
    _fields_ = [(n, ctypes.c_int) for n in ("E", "R", "d", "h", "rcap")] + \
        [(n, ctypes.c_void_p) for n in ("offsets", "off128", "xq", "xs", "w1q", "w1s", "w3q", "w3s", "w2q", "w2s", "g",
                                        "u", "hbuf", "hq", "hs", "hqT", "hsT", "yp", "ws")] + \
        [("ws_bytes", ctypes.c_size_t)]


class MxBwdArgs(ctypes.Structure):
    """moe_mx_bwd_args (include/moe.h)."""
    _fields_ = [(n, ctypes.c_int) for n in ("E", "R", "d", "h", "rcap")] + \
        [(n, ctypes.c_void_p) for n in ("offsets", "off128", "dyp", "dyq", "dys", "dyqT", "dysT", "g", "u", "hqT", "hsT",
                                        "xqT", "xsT", "w1tq", "w1ts", "w3tq", "w3ts", "w2tq", "w2ts", "dgu", "dguq",
                                        "dgus", "dguqT", "dgusT", "dxp", "dw1", "dw3", "dw2", "ws")] + \
        [("ws_bytes", ctypes.c_size_t)] + [(n, ctypes.c_void_p) for n in ("dy", "topk_w", "src")] + [("k", ctypes.c_int)]

EXPORTED = tuple(_SIGS)


class MoeError(RuntimeError):
    pass


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(f"HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = res
        _lib = h
    return _lib


def version() -> str:
    return lib().moe_version().decode()


def _check(status: int, fn: str):
    if status != 0:
        msg = lib().moe_last_error_string().decode()
        raise MoeError(f"{fn} failed (status {status}): {msg}")


def _p(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise MoeError(f"tensor on {t.device}, expected the GPU")
    if not t.is_contiguous():
        raise MoeError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dt(t) -> int:
    if t.dtype not in _DT:
        raise MoeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _expect(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------------------
# optional per-kernel event timing (benchmarks)
# ---------------------------------------------------------------------------

def prof_enable(on: bool = True):
    _check(lib().moe_prof_enable(1 if on else 0), "moe_prof_enable")


def prof_only(name=None):
    """Bracket only launches called `name` with events (None: every launch)."""
    _check(lib().moe_prof_only(name.encode() if name else None), "moe_prof_only")


def prof_reset():
    _check(lib().moe_prof_reset(), "moe_prof_reset")


def prof_names():
    n = lib().moe_prof_names(None, 0)
    buf = ctypes.create_string_buffer(int(n))
    lib().moe_prof_names(buf, n)
    return [s for s in buf.value.decode().split("\n") if s]


def prof_query(name: str):
    """(launch count, total milliseconds) of the recorded launches called name."""
    c = ctypes.c_int(0)
    ms = ctypes.c_float(0.0)
    _check(lib().moe_prof_query(name.encode(), ctypes.byref(c), ctypes.byref(ms)), "moe_prof_query")
    return c.value, ms.value


# ---------------------------------------------------------------------------
# workspace sizes
# ---------------------------------------------------------------------------

def moe_route_workspace_size(T: int, E: int, k: int) -> int:
    return int(lib().moe_route_workspace_size(T, E, k))


def moe_grouped_gemm_workspace_size(E: int, R: int, d: int, h: int) -> int:
    return int(lib().moe_grouped_gemm_workspace_size(E, R, d, h))


def moe_router_bwd_workspace_size(T: int, d: int, E: int) -> int:
    return int(lib().moe_router_bwd_workspace_size(T, d, E))


def moe_balance_workspace_size(T: int, E: int) -> int:
    return int(lib().moe_balance_workspace_size(T, E))


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# calls
# ---------------------------------------------------------------------------

def moe_router_logits(x, wr, logits):
    T, d = x.shape
    E = wr.shape[0]
    _expect(wr, x.dtype, "wr")
    _expect(logits, torch.float32, "logits")
    _check(lib().moe_router_logits(_p(x), _dt(x), _p(wr), T, d, E, _p(logits), _stream()), "moe_router_logits")


def moe_route(logits, k, probs, topk_idx, topk_w, counts, offsets, pos, src, ws, off128=None, forced_idx=None,
              err_flag=None):
    T, E = logits.shape
    for t, n, dt in ((logits, "logits", torch.float32), (probs, "probs", torch.float32),
                     (topk_w, "topk_w", torch.float32), (topk_idx, "topk_idx", torch.int32),
                     (counts, "counts", torch.int32), (offsets, "offsets", torch.int32), (pos, "pos", torch.int32),
                     (src, "src", torch.int32), (off128, "off128", torch.int32), (forced_idx, "forced_idx", torch.int32),
                     (err_flag, "err_flag", torch.int32)):
        _expect(t, dt, n)
    _check(lib().moe_route(_p(logits), T, E, k, _p(forced_idx), _p(probs), _p(topk_idx), _p(topk_w), _p(counts),
                           _p(offsets), _p(pos), _p(src), _p(off128), _p(err_flag), _p(ws), ws.numel(), _stream()),
           "moe_route")


def moe_route_noalloc(logits, k, probs, topk_idx, topk_w, counts, offsets, pos, src, off128=None, forced_idx=None,
                      err_flag=None):
    """moe_route with the library's own static scratch instead of a workspace
    (allocates nothing; calls that overlap on one GPU race)."""
    T, E = logits.shape
    for t, n, dt in ((logits, "logits", torch.float32), (probs, "probs", torch.float32),
                     (topk_w, "topk_w", torch.float32), (topk_idx, "topk_idx", torch.int32),
                     (counts, "counts", torch.int32), (offsets, "offsets", torch.int32), (pos, "pos", torch.int32),
                     (src, "src", torch.int32), (off128, "off128", torch.int32), (forced_idx, "forced_idx", torch.int32),
                     (err_flag, "err_flag", torch.int32)):
        _expect(t, dt, n)
    _check(lib().moe_route_noalloc(_p(logits), T, E, k, _p(forced_idx), _p(probs), _p(topk_idx), _p(topk_w),
                                   _p(counts), _p(offsets), _p(pos), _p(src), _p(off128), _p(err_flag), _stream()),
           "moe_route_noalloc")


def moe_permute(x, pos, xp):
    T, d = x.shape
    k = pos.shape[1]
    _expect(xp, x.dtype, "xp")
    _check(lib().moe_permute(_p(x), _dt(x), T, d, k, _p(pos), _p(xp), _stream()), "moe_permute")


def moe_combine(yp, topk_w, pos, y):
    T, k = pos.shape
    d = yp.shape[1]
    _expect(y, yp.dtype, "y")
    _check(lib().moe_combine(_p(yp), _p(topk_w), _p(pos), T, d, k, _dt(yp), _p(y), _stream()), "moe_combine")


def moe_combine_bwd(dy, yp, topk_w, pos, dyp, dgate):
    """dyp may be None: then only dgate is written."""
    T, k = pos.shape
    d = yp.shape[1]
    _expect(dy, yp.dtype, "dy")
    _expect(dyp, yp.dtype, "dyp")
    _expect(dgate, torch.float32, "dgate")
    _check(lib().moe_combine_bwd(_p(dy), _p(yp), _p(topk_w), _p(pos), T, d, k, _dt(yp), _p(dyp), _p(dgate),
                                 _stream()), "moe_combine_bwd")


def moe_unpermute_sum(dxp, pos, dx):
    T, k = pos.shape
    d = dxp.shape[1]
    _expect(dx, dxp.dtype, "dx")
    _check(lib().moe_unpermute_sum(_p(dxp), _p(pos), T, d, k, _dt(dxp), _p(dx), _stream()), "moe_unpermute_sum")


def moe_grouped_gemm_fwd(xp, w1, w3, w2, offsets, g, u, hbuf, yp, ws):
    R, d = xp.shape
    E, h, _ = w1.shape
    for t, n in ((w1, "w1"), (w3, "w3"), (w2, "w2"), (g, "g"), (u, "u"), (hbuf, "hbuf"), (yp, "yp")):
        _expect(t, xp.dtype, n)
    _check(lib().moe_grouped_gemm_fwd(_p(xp), _p(w1), _p(w3), _p(w2), _p(offsets), E, R, d, h, _dt(xp), _p(g), _p(u),
                                      _p(hbuf), _p(yp), _p(ws), ws.numel(), _stream()), "moe_grouped_gemm_fwd")


BWD_DGRAD_DOWN, BWD_WGRAD_DOWN, BWD_DGRAD_UP, BWD_WGRAD_UP, BWD_ALL = 1, 2, 4, 8, 15
BWD_MX_QUANT_DY, BWD_MX_DY_READY = 16, 32  # MXFP8 parts only


def moe_grouped_gemm_bwd_parts(dyp, xp, g, u, hbuf, w1, w3, w2, offsets, dgu, dxp, dw1, dw3, dw2, parts, ws):
    """A subset (MOE_BWD_* mask) of moe_grouped_gemm_bwd's four GEMMs."""
    R, d = xp.shape
    E, h, _ = w1.shape
    for t, n in ((dyp, "dyp"), (g, "g"), (u, "u"), (hbuf, "hbuf"), (w1, "w1"), (w3, "w3"), (w2, "w2"), (dgu, "dgu"),
                 (dxp, "dxp"), (dw1, "dw1"), (dw3, "dw3"), (dw2, "dw2")):
        _expect(t, xp.dtype, n)
    _check(lib().moe_grouped_gemm_bwd_parts(_p(dyp), _p(xp), _p(g), _p(u), _p(hbuf), _p(w1), _p(w3), _p(w2),
                                            _p(offsets), E, R, d, h, _dt(xp), _p(dgu), _p(dxp), _p(dw1), _p(dw3),
                                            _p(dw2), parts, _p(ws), ws.numel(), _stream()), "moe_grouped_gemm_bwd_parts")


def moe_grouped_gemm_recompute_gu(xp, w1, w3, offsets, g, u, ws):
    """The up projection alone, writing G and U (memory-lean backward)."""
    R, d = xp.shape
    E, h, _ = w1.shape
    for t, n in ((w1, "w1"), (w3, "w3"), (g, "g"), (u, "u")):
        _expect(t, xp.dtype, n)
    _check(lib().moe_grouped_gemm_recompute_gu(_p(xp), _p(w1), _p(w3), _p(offsets), E, R, d, h, _dt(xp), _p(g), _p(u),
                                               _p(ws), ws.numel(), _stream()), "moe_grouped_gemm_recompute_gu")


def moe_grouped_gemm_bwd(dyp, xp, g, u, hbuf, w1, w3, w2, offsets, dgu, dxp, dw1, dw3, dw2, ws):
    R, d = xp.shape
    E, h, _ = w1.shape
    for t, n in ((dyp, "dyp"), (g, "g"), (u, "u"), (hbuf, "hbuf"), (w1, "w1"), (w3, "w3"), (w2, "w2"), (dgu, "dgu"),
                 (dxp, "dxp"), (dw1, "dw1"), (dw3, "dw3"), (dw2, "dw2")):
        _expect(t, xp.dtype, n)
    _check(lib().moe_grouped_gemm_bwd(_p(dyp), _p(xp), _p(g), _p(u), _p(hbuf), _p(w1), _p(w3), _p(w2), _p(offsets), E,
                                      R, d, h, _dt(xp), _p(dgu), _p(dxp), _p(dw1), _p(dw3), _p(dw2), _p(ws), ws.numel(),
                                      _stream()), "moe_grouped_gemm_bwd")


def moe_router_bwd(probs, topk_idx, dgate, x, wr, dx, dwr, ws):
    T, d = x.shape
    E = wr.shape[0]
    k = topk_idx.shape[1]
    _expect(dx, x.dtype, "dx")
    _expect(dwr, x.dtype, "dwr")
    _check(lib().moe_router_bwd(_p(probs), _p(topk_idx), _p(dgate), _p(x), _p(wr), T, d, E, k, _dt(x), _p(dx), _p(dwr),
                                _p(ws), ws.numel(), _stream()), "moe_router_bwd")


def moe_router_bwd_unpermute(probs, topk_idx, dgate, x, wr, dxp, pos, dx, dwr, ws, aux_g=None):
    """dx = unpermute-sum of dxp + the router's input gradient (one pass,
    one rounding); dwr as moe_router_bwd; aux_g adds the balance loss."""
    T, d = x.shape
    E = wr.shape[0]
    k = topk_idx.shape[1]
    _expect(dx, x.dtype, "dx")
    _expect(dwr, x.dtype, "dwr")
    _expect(dxp, x.dtype, "dxp")
    if aux_g is not None:
        _expect(aux_g, torch.float32, "aux_g")
    _check(lib().moe_router_bwd_unpermute(_p(probs), _p(topk_idx), _p(dgate), _p(aux_g), _p(x), _p(wr), _p(dxp),
                                          _p(pos), T, d, E, k, _dt(x), _p(dx), _p(dwr), _p(ws), ws.numel(),
                                          _stream()), "moe_router_bwd_unpermute")


ROUTER_DWR, ROUTER_DX = 1, 2


def moe_router_bwd_unpermute_parts(parts, probs, topk_idx, dgate, x, wr, dxp, pos, dx, dwr, ws, aux_g=None):
    """moe_router_bwd_unpermute restricted to ROUTER_DWR and / or ROUTER_DX."""
    T, d = x.shape
    E = wr.shape[0]
    k = topk_idx.shape[1]
    if parts & ROUTER_DX:
        _expect(dx, x.dtype, "dx")
        _expect(dxp, x.dtype, "dxp")
    if parts & ROUTER_DWR:
        _expect(dwr, x.dtype, "dwr")
    if aux_g is not None:
        _expect(aux_g, torch.float32, "aux_g")
    _check(lib().moe_router_bwd_unpermute_parts(_p(probs), _p(topk_idx), _p(dgate), _p(aux_g), _p(x), _p(wr), _p(dxp),
                                                _p(pos), T, d, E, k, _dt(x), _p(dx), _p(dwr), _p(ws), ws.numel(),
                                                parts, _stream()), "moe_router_bwd_unpermute_parts")


def moe_router_bwd_aux(probs, topk_idx, dgate, aux_g, x, wr, dx, dwr, ws):
    """moe_router_bwd plus the balance loss's per-expert gradient aux_g [E] f32."""
    T, d = x.shape
    E = wr.shape[0]
    k = topk_idx.shape[1]
    _expect(dx, x.dtype, "dx")
    _expect(dwr, x.dtype, "dwr")
    _expect(aux_g, torch.float32, "aux_g")
    _check(lib().moe_router_bwd_aux(_p(probs), _p(topk_idx), _p(dgate), _p(aux_g), _p(x), _p(wr), T, d, E, k, _dt(x),
                                    _p(dx), _p(dwr), _p(ws), ws.numel(), _stream()), "moe_router_bwd_aux")


def moe_balance(probs, counts, k, alpha, stats, ws, aux_g=None, mean_probs=None):
    """Balance score, aux loss, max/min load over mean into stats [4] f32; the
    loss's probability gradient into aux_g [E] and P into mean_probs [E]."""
    T, E = probs.shape
    _expect(probs, torch.float32, "probs")
    _expect(counts, torch.int32, "counts")
    _expect(stats, torch.float32, "stats")
    for t, n in ((aux_g, "aux_g"), (mean_probs, "mean_probs")):
        if t is not None:
            _expect(t, torch.float32, n)
    _check(lib().moe_balance(_p(probs), _p(counts), T, E, k, float(alpha), _p(stats), _p(aux_g), _p(mean_probs), _p(ws),
                             ws.numel(), _stream()), "moe_balance")


# ---------------------------------------------------------------------------
# MXFP8
# ---------------------------------------------------------------------------

def mx_quantize(x, rows, q_row=None, s_row=None, q_col=None, s_col=None, gather_src=None, gather_k=1, seg_off=None,
                seg_off128=None, seg_rows=0):
    """Quantise `rows` rows of x (bf16/f32, [*, cols]) to rowwise and/or
    columnwise MX (E4M3 + E8M0); see mx_quantize in include/moe.h."""
    cols = x.shape[1]
    nseg = 0 if seg_off is None else seg_off.numel() - 1
    for t, n in ((q_row, "q_row"), (s_row, "s_row"), (q_col, "q_col"), (s_col, "s_col")):
        _expect(t, torch.uint8, n)
    for t, n in ((gather_src, "gather_src"), (seg_off, "seg_off"), (seg_off128, "seg_off128")):
        _expect(t, torch.int32, n)
    # columnwise row capacity: [rows, ldc] (fixed segments), or a flat buffer of cols * ldc bytes
    ldc = 0 if q_col is None else (q_col.shape[1] if q_col.dim() == 2 else q_col.numel() // cols)
    _check(lib().mx_quantize(_p(x), _dt(x), rows, cols, _p(gather_src), gather_k, _p(seg_off), _p(seg_off128), nseg,
                             seg_rows, _p(q_row), _p(s_row), _p(q_col), _p(s_col), ldc, _stream()), "mx_quantize")


def _fill(st, **kw):
    for k, v in kw.items():
        if isinstance(v, torch.Tensor):
            _p(v)
            setattr(st, k, v.data_ptr())
        else:
            setattr(st, k, v)
    return st


def moe_grouped_gemm_fwd_mx(**kw):
    """Keyword arguments are the fields of moe_mx_fwd_args (tensors or ints)."""
    a = _fill(MxFwdArgs(), **kw)
    _check(lib().moe_grouped_gemm_fwd_mx(ctypes.byref(a), _stream()), "moe_grouped_gemm_fwd_mx")


FWD_UP, FWD_DOWN, FWD_ALL = 1, 2, 3


def moe_grouped_gemm_fwd_mx_parts(parts, **kw):
    """moe_grouped_gemm_fwd_mx's up half (MOE_FWD_UP) and/or down half (MOE_FWD_DOWN)."""
    a = _fill(MxFwdArgs(), **kw)
    _check(lib().moe_grouped_gemm_fwd_mx_parts(ctypes.byref(a), parts, _stream()), "moe_grouped_gemm_fwd_mx_parts")


def moe_grouped_gemm_recompute_gu_mx(**kw):
    """The MX up projection alone, writing g and u (fields of moe_mx_fwd_args)."""
    a = _fill(MxFwdArgs(), **kw)
    _check(lib().moe_grouped_gemm_recompute_gu_mx(ctypes.byref(a), _stream()), "moe_grouped_gemm_recompute_gu_mx")


def moe_grouped_gemm_bwd_mx(**kw):
    """Keyword arguments are the fields of moe_mx_bwd_args (tensors or ints)."""
    a = _fill(MxBwdArgs(), **kw)
    _check(lib().moe_grouped_gemm_bwd_mx(ctypes.byref(a), _stream()), "moe_grouped_gemm_bwd_mx")


def moe_grouped_gemm_bwd_mx_parts(parts, **kw):
    """A subset (MOE_BWD_* mask) of moe_grouped_gemm_bwd_mx's four GEMMs."""
    a = _fill(MxBwdArgs(), **kw)
    _check(lib().moe_grouped_gemm_bwd_mx_parts(ctypes.byref(a), parts, _stream()), "moe_grouped_gemm_bwd_mx_parts")
