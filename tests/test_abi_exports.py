"""CPU checks of the boundary: the built library loads and exports every
function declared in include/moe.h, and the binding covers all of them."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "token_routing_grouped_amd", "libtrg_moe.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:moe|mx)_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for must in ("moe_route", "moe_permute", "moe_grouped_gemm_fwd", "moe_grouped_gemm_bwd", "moe_combine",
                 "moe_combine_bwd", "moe_unpermute_sum", "moe_router_logits", "moe_router_bwd"):
        assert must in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built (run __graft_entry__.build())")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    from token_routing_grouped_amd import _abi

    assert sorted(_abi.EXPORTED) == _declared()


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_host_side_validation_without_gpu():
    """Argument checks run before any device call, so they work without a GPU."""
    from token_routing_grouped_amd import _abi

    lib = _abi.lib()
    assert lib.moe_version().decode().startswith("trg-moe")
    # k > E
    st = lib.moe_route(None, 4, 2, 3, None, None, None, None, None, None, None, None, None, None, None, 0, None)
    assert st == 1 and b"k (3) > E (2)" in lib.moe_last_error_string()
    # bad dtype
    st = lib.moe_permute(None, 7, 4, 64, 2, None, None, None)
    assert st == 2
    # row width not a multiple of 16 bytes
    st = lib.moe_permute(None, 1, 4, 12, 2, None, None, None)
    assert st == 3
    # workspace too small
    st = lib.moe_route(ctypes.c_void_p(16), 8, 4, 2, None, ctypes.c_void_p(16), ctypes.c_void_p(16),
                       ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                       ctypes.c_void_p(16), None, None, None, 0, None)
    assert st == 4
    # unaligned pointer
    st = lib.moe_permute(ctypes.c_void_p(8), 1, 4, 64, 2, ctypes.c_void_p(16), ctypes.c_void_p(16), None)
    assert st == 3
    # bf16 grouped GEMM needs h % 64 == 0
    st = lib.moe_grouped_gemm_fwd(None, None, None, None, None, 4, 8, 64, 40, 1, None, None, None, None, None, 0,
                                  None)
    assert st == 1
    # k out of range
    st = lib.moe_combine(None, None, None, 4, 64, 0, 1, None, None)
    assert st == 1
    # optional G / U outputs must be 16-byte aligned when given
    c = ctypes.c_void_p(16)
    st = lib.moe_grouped_gemm_fwd(c, c, c, c, c, 2, 8, 64, 64, 1, ctypes.c_void_p(24), None, c, c, c, 1 << 20, None)
    assert st == 3 and b"g is not 16-byte aligned" in lib.moe_last_error_string()
    st = lib.moe_grouped_gemm_fwd(c, c, c, c, c, 2, 8, 64, 64, 1, None, ctypes.c_void_p(40), c, c, c, 1 << 20, None)
    assert st == 3 and b"u is not 16-byte aligned" in lib.moe_last_error_string()
    # the fused dx pass needs dxp and pos (and 16-byte aligned dxp)
    big = 1 << 30
    st = lib.moe_router_bwd_unpermute(c, c, c, None, c, c, None, c, 4, 64, 8, 2, 1, c, c, c, big, None)
    assert st == 1 and b"dxp is null" in lib.moe_last_error_string()
    st = lib.moe_router_bwd_unpermute(c, c, c, None, c, c, ctypes.c_void_p(24), c, 4, 64, 8, 2, 1, c, c, c, big,
                                      None)
    assert st == 3 and b"dxp is not 16-byte aligned" in lib.moe_last_error_string()
    st = lib.moe_router_bwd_unpermute(c, c, c, None, c, c, c, None, 4, 64, 8, 2, 1, c, c, c, big, None)
    assert st == 1 and b"pos is null" in lib.moe_last_error_string()


def test_mx_arg_structs_match_the_header(tmp_path):
    """The ctypes mirrors of moe_mx_fwd_args / moe_mx_bwd_args have the C
    layout: every field offset and the size, as gcc lays out include/moe.h."""
    import ctypes
    import shutil
    import subprocess

    from token_routing_grouped_amd import _abi

    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe.h"', "int main(void) {"]
    for cname, py in (("moe_mx_fwd_args", _abi.MxFwdArgs), ("moe_mx_bwd_args", _abi.MxBwdArgs)):
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in (("moe_mx_fwd_args", _abi.MxFwdArgs), ("moe_mx_bwd_args", _abi.MxBwdArgs)):
        assert got[(cname, "size")] == ctypes.sizeof(py)
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_mx_host_side_validation_without_gpu():
    from token_routing_grouped_amd import _abi

    lib = _abi.lib()
    # cols not a multiple of 32
    st = lib.mx_quantize(None, 1, 4, 48, None, 1, None, None, 0, 4, None, None, None, None, 0, None)
    assert st == 1
    # nothing to write
    st = lib.mx_quantize(None, 1, 4, 64, None, 1, None, None, 0, 4, None, None, None, None, 0, None)
    assert st == 1 and b"nothing to write" in lib.moe_last_error_string()
    # MX grouped GEMM needs d, h multiples of 128
    a = _abi.MxFwdArgs(E=2, R=8, d=192, h=128, rcap=128)
    assert lib.moe_grouped_gemm_fwd_mx(ctypes.byref(a), None) == 1
    # rcap below R + 127*E
    a = _abi.MxFwdArgs(E=4, R=8, d=128, h=128, rcap=128)
    assert lib.moe_grouped_gemm_fwd_mx(ctypes.byref(a), None) == 1
    # rcap not a multiple of 128
    a = _abi.MxFwdArgs(E=2, R=8, d=128, h=128, rcap=96)
    assert lib.moe_grouped_gemm_fwd_mx(ctypes.byref(a), None) == 1
    assert b"multiple of 128" in lib.moe_last_error_string()
    # optional G / U outputs must be 16-byte aligned when given
    p = {n: 16 for n in ("offsets", "off128", "xq", "xs", "w1q", "w1s", "w3q", "w3s", "w2q", "w2s", "hbuf", "hq", "hs",
                         "hqT", "hsT", "yp", "ws")}
    a = _abi.MxFwdArgs(E=2, R=8, d=128, h=128, rcap=384, ws_bytes=1 << 20, g=24, **p)
    assert lib.moe_grouped_gemm_fwd_mx(ctypes.byref(a), None) == 3
    assert b"g is not 16-byte aligned" in lib.moe_last_error_string()


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_host_validation_of_the_next_rows():
    """Argument checks of the balance, lean and two-stream entry points (no GPU)."""
    from token_routing_grouped_amd import _abi

    lib = _abi.lib()
    c = ctypes.c_void_p(16)
    # balance: negative alpha, k > E
    assert lib.moe_balance(c, c, 8, 4, 2, -1.0, c, None, None, c, 1 << 20, None) == 1
    assert b"alpha" in lib.moe_last_error_string()
    assert lib.moe_balance(c, c, 8, 4, 5, 0.01, c, None, None, c, 1 << 20, None) == 1
    # lean forward (g, u null) is bf16 only
    st = lib.moe_grouped_gemm_fwd(c, c, c, c, c, 2, 8, 64, 64, 0, None, None, c, c, c, 1 << 20, None)
    assert st == 2 and b"memory-lean" in lib.moe_last_error_string()
    # recompute needs bf16
    assert lib.moe_grouped_gemm_recompute_gu(c, c, c, c, 2, 8, 64, 64, 0, c, c, c, 1 << 20, None) == 2
    # backward parts: empty and out-of-range masks
    args = [c] * 9 + [2, 8, 64, 64, 1] + [c] * 5
    assert lib.moe_grouped_gemm_bwd_parts(*args, 0, c, 1 << 20, None) == 1
    assert lib.moe_grouped_gemm_bwd_parts(*args, 16, c, 1 << 20, None) == 1
    assert b"parts" in lib.moe_last_error_string()
    # MXFP8 backward parts: empty and out-of-range masks are refused before anything else
    a = _abi.MxBwdArgs(E=2, R=8, d=128, h=128, rcap=512)
    assert lib.moe_grouped_gemm_bwd_mx_parts(ctypes.byref(a), 0, None) == 1
    assert lib.moe_grouped_gemm_bwd_mx_parts(ctypes.byref(a), 64, None) == 1
    assert b"parts" in lib.moe_last_error_string()
    # MOE_BWD_MX_DY_READY only beside MOE_BWD_DGRAD_DOWN, never with MOE_BWD_MX_QUANT_DY
    for bad in (_abi.BWD_MX_DY_READY, _abi.BWD_MX_DY_READY | _abi.BWD_WGRAD_DOWN,
                _abi.BWD_MX_DY_READY | _abi.BWD_DGRAD_DOWN | _abi.BWD_MX_QUANT_DY):
        assert lib.moe_grouped_gemm_bwd_mx_parts(ctypes.byref(a), bad, None) == 1
        assert b"MOE_BWD_MX_DY_READY" in lib.moe_last_error_string()
    # a valid mask gets past the mask check (and then stops at the null buffers)
    assert lib.moe_grouped_gemm_bwd_mx_parts(ctypes.byref(a), _abi.BWD_MX_QUANT_DY, None) != 0
    assert b"is null" in lib.moe_last_error_string()
    # MXFP8 forward halves: empty and out-of-range masks refused, valid ones reach the buffer checks
    f = _abi.MxFwdArgs(E=2, R=8, d=128, h=128, rcap=512)
    for bad in (0, 4, _abi.FWD_ALL | 8):
        assert lib.moe_grouped_gemm_fwd_mx_parts(ctypes.byref(f), bad, None) == 1
        assert b"parts" in lib.moe_last_error_string()
    for ok in (_abi.FWD_UP, _abi.FWD_DOWN, _abi.FWD_ALL):
        assert lib.moe_grouped_gemm_fwd_mx_parts(ctypes.byref(f), ok, None) != 0
        assert b"is null" in lib.moe_last_error_string()
