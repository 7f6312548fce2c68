"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/moe.h, and rejects bad arguments on the host before any
HIP call (so these run on a machine without a GPU)."""
import ctypes
import importlib.util
import os
import re
import threading

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "moe_expert_layer_router_amd", "libmoe.so")


def _ensure_built():
    if not os.path.exists(LIB):
        spec = importlib.util.spec_from_file_location(
            "_moe_build", os.path.join(ROOT, "moe_expert_layer_router_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build_library()


_ensure_built()
import moe_expert_layer_router_amd as moe  # noqa: E402

L = moe.lib
OK, EINVAL, EUNSUP, EWS = 0, -1, -2, -3
BF16, F32, FP8 = moe.MOE_BF16, moe.MOE_F32, moe.MOE_FP8
A = ctypes.c_void_p(0x100000)   # fake, 256-byte aligned; never dereferenced by a failing call
U = ctypes.c_void_p(0x100002)   # misaligned fake pointer
N = None
S = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), f"libmoe.so does not export {n}"


def test_abi_version_and_single_hip_runtime():
    assert L.moe_abi_version() == moe.ABI_VERSION == 10
    libs = moe.hip_runtimes_mapped()
    assert len(libs) <= 1, libs


def _err():
    return L.moe_last_error().decode()


def test_workspace_bytes_and_errors():
    ws = lambda *a: L.moe_workspace_bytes(*a)
    assert ws(moe.MOE_OP_ROUTE, 16384, 2048, 768, 128, 8, 0, 128, F32) == 0
    # bf16 router, E % 8 == 0 and E <= 128: one launch, no workspace
    assert ws(moe.MOE_OP_ROUTE, 16384, 2048, 768, 128, 8, 0, 128, BF16) == 0
    assert ws(moe.MOE_OP_ROUTE, 16384, 2048, 768, 40, 8, 0, 40, BF16) == 0
    # other bf16 shapes: fp32 partial logits of S slices of H (E=256: the slice
    # copy fits 128 KB of LDS at 256 rows, so S = 8; E=20: S = 4, 512-row slices)
    assert ws(moe.MOE_OP_ROUTE, 16384, 2048, 768, 256, 8, 0, 256, BF16) == 8 * 16384 * 256 * 4
    assert ws(moe.MOE_OP_ROUTE, 16384, 2048, 768, 20, 8, 0, 20, BF16) == 4 * 16384 * 20 * 4
    assert ws(moe.MOE_OP_PERMUTE, 16384, 2048, 768, 128, 8, 0, 128, BF16) > 16384 * 8 * 4
    assert ws(moe.MOE_OP_FFN_BWD, 8192, 2048, 768, 128, 8, 0, 16, BF16) >= 8192 * 8 * 2 * 768 * 2
    assert ws(moe.MOE_OP_PERMUTE, 0, 2048, 768, 128, 8, 0, 16, BF16) == 0
    assert ws(10, 16, 64, 32, 8, 2, 0, 8, F32) == EINVAL and "unknown op" in _err()
    assert ws(moe.MOE_OP_ROUTE, 16, 64, 32, 8, 9, 0, 8, F32) == EINVAL and "k=9" in _err()
    assert ws(moe.MOE_OP_ROUTE, 16, 64, 32, 300, 2, 0, 8, F32) == EINVAL
    assert ws(moe.MOE_OP_ROUTE, 16, 62, 32, 8, 2, 0, 8, BF16) == EINVAL and "multiple of 8" in _err()
    assert ws(moe.MOE_OP_PERMUTE, 16, 64, 32, 8, 2, 5, 5, F32) == EINVAL
    assert ws(moe.MOE_OP_PERMUTE, 16, 64, 32, 8, 2, 0, 9, F32) == EINVAL
    assert ws(moe.MOE_OP_ROUTE, 16, 64, 32, 8, 2, 0, 8, 7) == EINVAL and "dtype" in _err()


def test_route_errors():
    r = lambda *a: L.moe_route(*a)
    assert r(A, A, N, 32, 128, 8, 9, F32, N, A, A, N, 0, S) == EINVAL and "k=9" in _err()
    assert r(A, A, N, 32, 128, 8, 0, F32, N, A, A, N, 0, S) == EINVAL
    assert r(A, A, N, 32, 128, 0, 1, F32, N, A, A, N, 0, S) == EINVAL
    assert r(A, A, N, 32, 128, 257, 8, F32, N, A, A, N, 0, S) == EINVAL
    assert r(A, A, N, 32, 128, 64, 33, F32, N, A, A, N, 0, S) == EINVAL
    assert r(A, A, N, -1, 128, 8, 2, F32, N, A, A, N, 0, S) == EINVAL
    assert r(N, A, N, 32, 128, 8, 2, F32, N, A, A, N, 0, S) == EINVAL and "x must not be NULL" in _err()
    assert r(U, A, N, 32, 128, 8, 2, F32, N, A, A, N, 0, S) == EINVAL and "aligned" in _err()
    assert r(A, A, N, 32, 128, 8, 2, F32, N, N, A, N, 0, S) == EINVAL and "topk_idx" in _err()
    assert r(A, A, N, 32, 100, 8, 2, BF16, N, A, A, A, 1 << 20, S) == EINVAL       # H % 8
    assert r(A, A, N, 32, 96, 8, 2, BF16, N, A, A, A, 1 << 20, S) == EUNSUP        # H % 64
    # E % 8 != 0: the sliced bf16 router, which needs a workspace
    assert r(A, A, N, 32, 128, 20, 2, BF16, N, A, A, A, 100, S) == EWS and "workspace" in _err()
    assert r(A, A, N, 32, 128, 20, 2, BF16, N, A, A, N, 0, S) == EWS
    assert r(A, A, N, 32, 128, 8, 2, 5, N, A, A, N, 0, S) == EINVAL
    # valid arguments with T == 0: nothing to enqueue, no HIP call
    assert r(A, A, N, 0, 128, 8, 2, F32, N, A, A, N, 0, S) == OK


def test_route_from_logits_errors():
    f = L.moe_route_from_logits
    assert f(A, 10, 8, 9, A, A, S) == EINVAL
    assert f(N, 10, 8, 2, A, A, S) == EINVAL
    assert f(A, 0, 8, 2, A, A, S) == OK


def test_permute_errors():
    p = lambda *a: L.moe_permute(*a)
    big = 1 << 30
    assert p(A, A, 64, 128, 16, 4, 4, 4, BF16, A, A, A, A, A, A, big, S) == EINVAL     # e_lo == e_hi
    assert p(A, A, 64, 128, 16, 4, 0, 17, BF16, A, A, A, A, A, A, big, S) == EINVAL    # e_hi > E
    assert p(A, A, 64, 128, 16, 4, -1, 8, BF16, A, A, A, A, A, A, big, S) == EINVAL
    assert p(A, A, 64, 128, 16, 4, 0, 16, BF16, N, A, A, A, A, A, big, S) == EINVAL and "counts" in _err()
    assert p(A, A, 64, 128, 16, 4, 0, 16, BF16, A, A, A, A, U, A, big, S) == EINVAL    # x_perm misaligned
    assert p(A, A, 64, 128, 16, 4, 0, 16, BF16, A, A, A, A, A, A, 8, S) == EWS
    assert p(A, A, 64, 128, 16, 4, 0, 16, BF16, A, A, A, A, A, U, big, S) == EINVAL    # ws misaligned
    assert p(A, A, 64, 129, 16, 4, 0, 16, BF16, A, A, A, A, A, A, big, S) == EINVAL    # H % 8


def test_ffn_fwd_errors():
    f = lambda *a: L.moe_grouped_ffn_fwd(*a)
    big = 1 << 30
    assert f(A, A, 16, 512, 128, 96, A, A, A, BF16, N, A, A, A, big, S) == EUNSUP     # I % 64
    assert f(A, A, 16, 512, 96, 64, A, A, A, BF16, N, A, A, A, big, S) == EUNSUP      # H % 64
    assert f(A, A, 0, 512, 128, 64, A, A, A, BF16, N, A, A, A, big, S) == EINVAL      # E_l
    assert f(A, A, 257, 512, 128, 64, A, A, A, BF16, N, A, A, A, big, S) == EINVAL
    assert f(A, A, 16, -1, 128, 64, A, A, A, BF16, N, A, A, A, big, S) == EINVAL
    assert f(A, A, 16, 512, 128, 64, N, A, A, BF16, N, A, A, A, big, S) == EINVAL and "w_gate" in _err()
    assert f(A, A, 16, 512, 128, 64, A, A, A, BF16, N, N, A, A, big, S) == EINVAL and "h_perm" in _err()
    assert f(A, A, 16, 512, 128, 64, A, A, A, BF16, N, A, A, A, 4, S) == EWS
    assert f(A, A, 16, 0, 128, 64, A, A, A, BF16, N, N, N, A, big, S) == OK            # nothing routed


def test_ffn_fwd_gather_errors():
    """The gathering forward: bf16 only, a src_row map when rows are routed, the
    token matrix below 2 GiB, and the forward's own shape and workspace checks."""
    g = lambda *a: L.moe_grouped_ffn_fwd_gather(*a)
    big = 1 << 30
    # (x, src_row, offsets, E_l, R_cap, T, H, I, w_gate, w_up, w_down, dtype, gu, h, y, ws, ws_bytes, s)
    assert g(A, A, A, 16, 512, 64, 128, 64, A, A, A, F32, N, A, A, A, big, S) == EUNSUP and "bf16" in _err()
    assert g(A, N, A, 16, 512, 64, 128, 64, A, A, A, BF16, N, A, A, A, big, S) == EINVAL and "src_row" in _err()
    assert g(N, A, A, 16, 512, 64, 128, 64, A, A, A, BF16, N, A, A, A, big, S) == EINVAL and "x" in _err()
    assert g(A, A, A, 16, 512, -1, 128, 64, A, A, A, BF16, N, A, A, A, big, S) == EINVAL
    assert g(A, A, A, 16, 512, 1 << 19, 2048, 64, A, A, A, BF16, N, A, A, A, big, S) == EUNSUP
    assert "x spans" in _err()
    assert g(A, A, A, 16, 512, 64, 128, 96, A, A, A, BF16, N, A, A, A, big, S) == EUNSUP     # I % 64
    assert g(A, A, A, 16, 512, 64, 128, 64, A, A, A, BF16, N, A, A, A, 4, S) == EWS
    assert g(N, N, A, 16, 0, 0, 128, 64, A, A, A, BF16, N, N, N, A, big, S) == OK            # nothing routed


def test_ffn_fwd_fp8_gather_errors():
    g = lambda *a: L.moe_grouped_ffn_fwd_fp8_gather(*a)
    big = 1 << 30
    # (x_q, x_scale, src_row, offsets, E_l, R_cap, T, H, I, wg, wgs, wu, wus, wd, wds, gu, h, y, ws, nb, s)
    assert g(A, A, N, A, 16, 512, 64, 256, 128, A, A, A, A, A, A, N, A, A, A, big, S) == EINVAL and "src_row" in _err()
    assert g(A, A, A, A, 16, 512, 64, 192, 128, A, A, A, A, A, A, N, A, A, A, big, S) == EUNSUP      # H % 128
    assert g(A, A, A, A, 16, 512, -1, 256, 128, A, A, A, A, A, A, N, A, A, A, big, S) == EINVAL
    assert g(A, A, A, A, 16, 512, 1 << 20, 2048, 128, A, A, A, A, A, A, N, A, A, A, big, S) == EUNSUP
    assert "x_q spans" in _err()
    assert g(A, A, A, A, 16, 512, 64, 256, 128, A, A, A, A, A, A, N, A, A, A, 4, S) == EWS
    assert g(N, N, N, A, 16, 0, 0, 256, 128, A, A, A, A, A, A, N, N, N, A, big, S) == OK    # nothing routed


def test_operand_ranges_below_2gib():
    """The matrix-core kernels address operands with 32-bit byte ranges: shapes whose
    grouped-row buffers, expert weights or router input reach 2 GiB are refused on
    the host (MOE_EUNSUPPORTED) instead of wrapping on the device."""
    f = lambda *a: L.moe_grouped_ffn_fwd(*a)
    big = 1 << 40
    # R_cap * H * 2 = 2^19 * 2048 * 2 = 2^31 bytes: refused; one row fewer is accepted
    assert f(A, A, 16, 1 << 19, 2048, 768, A, A, A, BF16, N, A, A, A, big, S) == EUNSUP
    assert "2 GiB" in _err() and "grouped-row" in _err()
    assert f(A, A, 16, (1 << 19) - 1, 2048, 64, A, A, A, BF16, N, A, A, N, 0, S) == EWS
    # R_cap * 2I * 2 reaches 2^31 through I
    assert f(A, A, 16, 1 << 16, 128, 8192, A, A, A, BF16, N, A, A, A, big, S) == EUNSUP
    # one expert's gate + up weights: 2 * I * H * 2 = 2^31
    assert f(A, A, 1, 64, 16384, 32768, A, A, A, BF16, N, A, A, A, big, S) == EUNSUP
    assert "gate and up" in _err()
    # fp32 layers index with 64-bit offsets: no such limit (the call gets as far as
    # the NULL w_gate, so nothing is launched)
    assert f(A, A, 16, 1 << 19, 2048, 768, N, A, A, F32, N, A, A, N, 0, S) == EINVAL and "w_gate" in _err()
    b = lambda *a: L.moe_grouped_ffn_bwd(*a)
    assert b(A, A, A, A, A, 16, 1 << 19, 2048, 768, A, A, A, BF16, A, A, A, A, 0, A, big, S) == EUNSUP
    fp8 = L.moe_grouped_ffn_fwd_fp8
    assert fp8(A, A, A, A, 16, 1 << 20, 2048, 768, A, A, A, A, A, A, A, A, A, A, big, S) == EUNSUP
    rb = lambda *a: L.moe_route_bwd(*a)
    # x^T . dz with T * H * 2 = 2^31 bytes of x: refused only when dw_router is asked for
    assert rb(A, A, A, A, A, 1 << 19, 2048, 128, 8, BF16, A, N, A, A, big, S) == EUNSUP
    assert "x spans" in _err()


def test_fp8_entry_points_errors():
    q = lambda *a: L.moe_quantize_fp8(*a)
    assert q(A, 64, 2040, BF16, N, A, A, S) == EINVAL and "multiple of 16" in _err()
    assert q(A, -1, 2048, BF16, N, A, A, S) == EINVAL
    assert q(A, 64, 2048, FP8, N, A, A, S) == EINVAL and "dtype" in _err()     # source must be bf16/fp32
    assert q(U, 64, 2048, BF16, N, A, A, S) == EINVAL                          # src misaligned
    assert q(A, 64, 2048, BF16, N, N, A, S) == EINVAL and "q" in _err()
    assert q(N, 0, 2048, BF16, N, N, N, S) == OK                               # no rows
    f = lambda *a: L.moe_grouped_ffn_fwd_fp8(*a)
    big = 1 << 30
    args = lambda H=2048, I=768, El=16, R=512, ws=big, xq=A, wg=A, h=A: (
        xq, A, A, A, El, R, H, I, wg, A, A, A, A, A, N, h, A, A, ws, S)
    assert f(*args(I=704)) == EUNSUP and "128" in _err()                       # I % 128
    assert f(*args(H=1984)) == EUNSUP                                          # H % 128
    assert f(*args(H=2040)) == EINVAL                                          # H % 16 (row width)
    assert f(*args(El=0)) == EINVAL
    assert f(*args(wg=N)) == EINVAL and "wg_q" in _err()
    assert f(*args(h=N)) == EINVAL and "h_perm" in _err()
    assert f(*args(xq=U)) == EINVAL
    assert f(*args(ws=8)) == EWS
    assert f(*args(R=0, xq=N, h=N)) == OK                                      # nothing routed
    ws = lambda *a: L.moe_workspace_bytes(*a)
    n = ws(moe.MOE_OP_FFN_FWD_FP8, 8192, 2048, 768, 128, 8, 0, 16, BF16)
    assert n >= 8192 * 8 * (768 + 8)                                           # codes + scales of h
    assert ws(moe.MOE_OP_FFN_FWD_FP8, 8192, 2048, 768, 128, 8, 0, 16, FP8) == n
    assert ws(moe.MOE_OP_ROUTE, 16, 64, 32, 8, 2, 0, 8, FP8) == EINVAL and "MOE_FP8" in _err()
    p = lambda *a: L.moe_permute(*a)
    assert p(A, A, 64, 2040, 16, 4, 0, 16, FP8, A, A, A, A, A, A, big, S) == EINVAL   # H % 16 for codes


def test_fp8_dgrad_entry_points_errors():
    t = lambda *a: L.moe_quantize_fp8_t(*a)
    assert t(A, N, 16, 2048, 768, F32, A, A, S) == EUNSUP and "BF16" in _err()
    assert t(A, N, 16, 2048, 760, BF16, A, A, S) == EUNSUP and "64" in _err()    # K % 64
    assert t(A, A, 16, 2000, 768, BF16, A, A, S) == EUNSUP                       # N % 64
    assert t(A, N, -1, 2048, 768, BF16, A, A, S) == EINVAL
    assert t(A, U, 16, 2048, 768, BF16, A, A, S) == EINVAL and "src1" in _err()
    assert t(A, N, 16, 2048, 768, BF16, N, A, S) == EINVAL and "q" in _err()
    assert t(N, N, 0, 2048, 768, BF16, N, N, S) == OK                            # empty batch
    d = lambda *a: L.moe_grouped_ffn_dgrad_fp8(*a)
    big = 1 << 30
    args = lambda H=2048, I=768, El=16, R=512, ws=big, dq=A, wd=A, dx=A, gu=A: (
        dq, A, gu, A, El, R, H, I, wd, A, A, A, A, dx, A, ws, S)
    assert d(*args(I=704)) == EUNSUP and "128" in _err()
    assert d(*args(I=2176)) == EUNSUP and "2048" in _err()
    assert d(*args(H=1984)) == EUNSUP
    assert d(*args(El=0)) == EINVAL
    assert d(*args(wd=N)) == EINVAL and "wdt_q" in _err()
    assert d(*args(dx=N)) == EINVAL and "dx_perm" in _err()
    assert d(*args(gu=U)) == EINVAL and "gu_saved" in _err()
    assert d(*args(ws=8)) == EWS
    assert d(*args(R=0, dq=N, dx=N, gu=N)) == OK
    ws = lambda *a: L.moe_workspace_bytes(*a)
    n = ws(moe.MOE_OP_FFN_DGRAD_FP8, 8192, 2048, 768, 128, 8, 0, 16, BF16)
    assert n >= 8192 * 8 * (768 * 2 + 2 * 768 + 4)                            # dh, codes, scales
    assert ws(moe.MOE_OP_FFN_DGRAD_FP8, 8192, 2048, 768, 128, 8, 0, 16, FP8) == n



def test_fp8_wgrad_entry_points_errors():
    """Argument errors of the FP8 weight gradients and their column quantizer (every
    case fails on the host; none launches)."""
    q = lambda *a: L.moe_quantize_fp8_group_t(*a)
    pitch = moe.wgrad_fp8_pitch(4096, 16)
    qa = lambda C=2048, El=16, R=4096, p=pitch, src=A, off=A, qq=A, sc=A, po=A: (
        src, N, C, off, El, R, qq, p, sc, po, S)
    assert q(*qa(C=2000)) == EINVAL and "64" in _err()
    assert q(*qa(El=0)) == EINVAL
    assert q(*qa(El=300)) == EINVAL
    assert q(*qa(R=-1)) == EINVAL
    assert q(*qa(p=pitch - 64)) == EINVAL and "q_pitch" in _err()
    assert q(*qa(p=pitch + 1)) == EINVAL and "q_pitch" in _err()
    assert q(*qa(off=N)) == EINVAL and "offsets" in _err()
    assert q(*qa(qq=U)) == EINVAL and "q" in _err()
    assert q(*qa(po=N)) == EINVAL and "poff" in _err()
    assert q(*qa(src=U)) == EINVAL and "src" in _err()
    w = lambda *a: L.moe_grouped_ffn_wgrad_fp8(*a)
    big = 1 << 31
    wa = lambda H=2048, I=768, El=16, R=4096, ws=big, x=A, dgu=A, dwg=A, dwd=A, off=A: (
        x, A, dgu, A, A, off, El, R, H, I, dwg, A, dwd, 0, A, ws, S)
    assert w(*wa(I=704)) == EUNSUP and "128" in _err()
    assert w(*wa(H=1984)) == EUNSUP
    assert w(*wa(El=0)) == EINVAL
    assert w(*wa(off=N)) == EINVAL and "offsets" in _err()
    assert w(*wa(dwg=N)) == EINVAL and "dw_gate" in _err()
    assert w(*wa(dwd=U)) == EINVAL and "dw_down" in _err()
    assert w(*wa(x=N)) == EINVAL and "x" in _err()
    assert w(*wa(dgu=U)) == EINVAL and "dgu" in _err()
    assert w(*wa(ws=8)) == EWS
    # a transposed code matrix of 2 GiB or more is refused
    assert w(*wa(H=16384, R=131072)) == EUNSUP and "2 GiB" in _err()
    ws = lambda *a: L.moe_workspace_bytes(*a)
    n = ws(moe.MOE_OP_FFN_WGRAD_FP8, 4096, 2048, 768, 128, 4, 0, 16, BF16)
    assert n >= pitch * (2 * 768 + 2 * 2048 + 768) + 16 * (3 * 768 + 2 * 2048) * 4   # codes, scales
    assert ws(moe.MOE_OP_FFN_WGRAD_FP8, 4096, 2048, 768, 128, 4, 0, 16, FP8) == n


def test_fp8_weight_quantizer_errors():
    """Argument errors of moe_quantize_fp8_w (none launches)."""
    f = lambda *a: L.moe_quantize_fp8_w(*a)
    big = 1 << 28
    a = lambda w0=A, w1=A, B=16, N=768, K=2048, dt=BF16, q0=A, s0=A, q1=A, s1=A, qt=A, st=A, ws=big: (
        w0, w1, B, N, K, dt, q0, s0, q1, s1, qt, st, A, ws, S)
    assert f(*a(dt=F32)) == EUNSUP and "BF16" in _err()
    assert f(*a(N=704)) == EUNSUP and "128" in _err()
    assert f(*a(K=2000)) == EUNSUP
    assert f(*a(B=-1)) == EINVAL
    assert f(*a(w0=U)) == EINVAL and "w0" in _err()
    assert f(*a(q0=N)) == EINVAL and "q0" in _err()
    assert f(*a(s1=N)) == EINVAL and "s1" in _err()
    assert f(*a(qt=U)) == EINVAL and "qt" in _err()
    assert f(*a(st=N)) == EINVAL and "st" in _err()
    assert f(*a(ws=8)) == EWS
    assert f(*a(B=0)) == OK                                   # nothing to do, nothing launched
    n = L.moe_workspace_bytes(moe.MOE_OP_QUANTIZE_W_FP8, 4096, 2048, 768, 128, 8, 0, 16, BF16)
    assert n >= 2 * (2 * 16 * 768 * (2048 // 128) * 4) + 2 * 16 * 768 * 4 + 16 * 2048 * 4

def test_ffn_bwd_split_needs_a_second_stream():
    f = lambda *a: L.moe_grouped_ffn_bwd_split(*a)
    args = (A, A, A, A, A, 16, 512, 2048, 768, A, A, A, BF16, A, A, A, A, 0, A, 1 << 30)
    assert f(*args, S, S) == EINVAL and "second stream" in _err()
    assert f(*args, ctypes.c_void_p(0x1234), None) == EINVAL


def test_combine_errors():
    c = lambda *a: L.moe_combine(*a)
    assert c(A, A, A, N, 8, 128, 0, BF16, A, S) == EINVAL
    assert c(A, A, A, N, 8, 128, 33, BF16, A, S) == EINVAL
    assert c(A, A, A, N, 8, 100, 2, BF16, A, S) == EINVAL
    assert c(A, A, A, N, -3, 128, 2, BF16, A, S) == EINVAL
    assert c(N, A, A, N, 8, 128, 2, BF16, A, S) == EINVAL
    assert c(A, A, A, U, 8, 128, 2, BF16, A, S) == EINVAL and "addend" in _err()
    assert c(A, A, A, N, 0, 128, 2, BF16, A, S) == OK
    b = lambda *a: L.moe_combine_bwd(*a)
    assert b(A, A, N, A, 8, 128, 2, BF16, A, A, S) == EINVAL and "topk_w" in _err()
    assert b(A, A, A, A, 8, 128, 2, BF16, U, A, S) == EINVAL
    assert b(A, A, A, A, 0, 128, 2, BF16, A, A, S) == OK


def test_ffn_bwd_and_route_bwd_errors():
    f = lambda *a: L.moe_grouped_ffn_bwd(*a)
    big = 1 << 30
    args = [A, A, A, A, A, 16, 512, 128, 64, A, A, A, BF16, A, A, A, A, 0, A, big, S]
    bad = list(args); bad[17] = 2
    assert f(*bad) == EINVAL and "accumulate" in _err()
    bad = list(args); bad[2] = N
    assert f(*bad) == EINVAL and "gu_saved" in _err()
    bad = list(args); bad[19] = 16
    assert f(*bad) == EWS
    bad = list(args); bad[8] = 32
    assert f(*bad) == EUNSUP
    r = lambda *a: L.moe_route_bwd(*a)
    assert r(A, A, A, A, A, 64, 128, 8, 9, F32, A, A, A, A, big, S) == EINVAL
    assert r(A, A, A, A, A, 64, 128, 8, 2, F32, N, A, A, A, big, S) == EINVAL and "d_logits" in _err()
    assert r(A, A, A, A, A, 64, 128, 8, 2, F32, A, U, A, A, big, S) == EINVAL
    assert r(A, A, A, A, A, 64, 96, 8, 2, BF16, A, A, A, A, big, S) == EUNSUP
    assert r(A, A, A, A, A, 64, 128, 8, 2, BF16, A, A, A, A, 8, S) == EWS


def test_last_error_is_per_thread():
    L.moe_route(N, A, N, 32, 128, 8, 2, F32, N, A, A, N, 0, S)
    assert "x must not be NULL" in _err()
    seen = []
    th = threading.Thread(target=lambda: seen.append(L.moe_last_error().decode()))
    th.start()
    th.join()
    assert seen == [""]


def test_combine_dx_errors():
    f = lambda *a: L.moe_combine_dx(*a)
    big = 1 << 30
    args = [A, A, A, A, A, A, 64, 128, 8, 2, BF16, A, A, big, S]
    bad = list(args); bad[9] = 9        # k > E
    assert f(*bad) == EINVAL
    bad = list(args); bad[0] = N        # dx_perm
    assert f(*bad) == EINVAL and "dx_perm" in _err()
    bad = list(args); bad[13] = 16      # workspace too small
    assert f(*bad) == EWS
    bad = list(args); bad[6] = 0        # T = 0: nothing to do
    assert f(*bad) == OK


def test_combine_dx_t_and_router_weight_t_errors():
    f = lambda *a: L.moe_combine_dx_t(*a)
    args = [A, A, A, A, A, A, 64, 128, 8, 2, BF16, A, S]
    bad = list(args); bad[9] = 9        # k > E
    assert f(*bad) == EINVAL
    bad = list(args); bad[5] = N        # transposed router weight
    assert f(*bad) == EINVAL and "w_router_t" in _err()
    bad = list(args); bad[7] = 100      # H not a multiple of 8 (bf16 rows of 16 bytes)
    assert f(*bad) == EINVAL
    bad = list(args); bad[6] = 0        # T = 0: nothing to do
    assert f(*bad) == OK
    g = lambda *a: L.moe_router_weight_t(*a)
    assert g(A, 128, 8, 7, A, S) == EINVAL                     # dtype
    assert g(A, -1, 8, BF16, A, S) == EINVAL
    assert g(A, 128, (1 << 20) + 1, BF16, A, S) == EINVAL
    assert g(N, 128, 8, BF16, A, S) == EINVAL and "w_router" in _err()
    assert g(A, 128, 8, BF16, N, S) == EINVAL and "w_router_t" in _err()
    assert g(N, 0, 8, BF16, N, S) == OK                        # empty: nothing to do


def test_layer_buffers_and_workspace_on_host():
    """The layer's set-up (buffers, one workspace for every call) needs no GPU."""
    import torch
    import moe_expert_layer_router_amd as moe
    for train in (False, True):
        layer = moe.MoELayer(64, 128, 64, 8, 2, 0, 8, torch.bfloat16, device="cpu", train=train)
        need = max(moe.workspace_bytes(op, 64, 128, 64, 8, 2, 0, 8, moe.MOE_BF16)
                   for op in range(5 if train else 3))
        assert layer.ws_bytes >= need
        assert ("dx" in layer.buf) == train
