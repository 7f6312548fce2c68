"""Python binding of the gfx950 MoE expert layer library (libmoe.so).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in include/moe.h.  PyTorch provides device memory
(outputs and workspaces are torch tensors) and the stream (the current torch
stream).  There is no fallback: importing this package fails when the built
library is missing, and every call raises MoEError when the library reports
an error.

Functions keep the C names (moe_route, moe_permute, moe_grouped_ffn_fwd and its
gathering form moe_grouped_ffn_fwd_gather, moe_combine, moe_combine_bwd, moe_grouped_ffn_bwd, moe_route_bwd, and the FP8
forward: moe_quantize_fp8, moe_grouped_ffn_fwd_fp8; data gradients:
moe_quantize_fp8_t, moe_grouped_ffn_dgrad_fp8; both weight layouts at once:
moe_quantize_fp8_w; weight gradients:
moe_quantize_fp8_group_t, moe_grouped_ffn_wgrad_fp8, and its two halves
moe_grouped_ffn_wgrad_fp8_begin / _end) and return
freshly allocated torch tensors; each also accepts preallocated outputs via
``out=`` dictionaries so that steady-state loops allocate nothing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch  # loads torch's HIP runtime first, so libmoe binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_FP8 = 0, 1, 2
(MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_FFN_FWD, MOE_OP_FFN_BWD, MOE_OP_ROUTE_BWD,
 MOE_OP_COMBINE_DX, MOE_OP_FFN_FWD_FP8, MOE_OP_FFN_DGRAD_FP8, MOE_OP_FFN_WGRAD_FP8,
 MOE_OP_QUANTIZE_W_FP8) = range(10)
ABI_VERSION = 10


class MoEError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "moe_abi_version": ([], I32),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_workspace_bytes": ([I32] * 9, I64),
        "moe_route": ([P, P, P, I32, I32, I32, I32, I32, P, P, P, P, SZ, P], I32),
        "moe_route_from_logits": ([P, I32, I32, I32, P, P, P], I32),
        "moe_permute": ([P, P, I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, SZ, P], I32),
        "moe_grouped_ffn_fwd": ([P, P, I32, I32, I32, I32, P, P, P, I32, P, P, P, P, SZ, P], I32),
        "moe_grouped_ffn_fwd_noalloc": ([P, P, I32, I32, I32, I32, P, P, P, I32, P, P, P, P], I32),
        "moe_grouped_ffn_fwd_gather": ([P, P, P, I32, I32, I32, I32, I32, P, P, P, I32, P, P, P, P, SZ,
                                        P], I32),
        "moe_combine": ([P, P, P, P, I32, I32, I32, I32, P, P], I32),
        "moe_combine_bwd": ([P, P, P, P, I32, I32, I32, I32, P, P, P], I32),
        "moe_combine_dx": ([P, P, P, P, P, P, I32, I32, I32, I32, I32, P, P, SZ, P], I32),
        "moe_combine_dx_t": ([P, P, P, P, P, P, I32, I32, I32, I32, I32, P, P], I32),
        "moe_router_weight_t": ([P, I32, I32, I32, P, P], I32),
        "moe_grouped_ffn_bwd": ([P, P, P, P, P, I32, I32, I32, I32, P, P, P, I32, P, P, P, P, I32,
                                 P, SZ, P], I32),
        "moe_grouped_ffn_bwd_split": ([P, P, P, P, P, I32, I32, I32, I32, P, P, P, I32, P, P, P, P,
                                       I32, P, SZ, P, P], I32),
        "moe_route_bwd": ([P, P, P, P, P, I32, I32, I32, I32, I32, P, P, P, P, SZ, P], I32),
        "moe_quantize_fp8": ([P, I32, I32, I32, P, P, P, P], I32),
        "moe_quantize_fp8_t": ([P, P, I32, I32, I32, I32, P, P, P], I32),
        "moe_grouped_ffn_dgrad_fp8": ([P, P, P, P, I32, I32, I32, I32, P, P, P, P, P, P, P, SZ, P], I32),
        "moe_grouped_ffn_fwd_fp8_gather": ([P, P, P, P, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P,
                                            P, P, SZ, P], I32),
        "moe_grouped_ffn_fwd_fp8": ([P, P, P, P, I32, I32, I32, I32, P, P, P, P, P, P, P, P, P, P,
                                     SZ, P], I32),
        "moe_quantize_fp8_group_t": ([P, P, I32, P, I32, I32, P, I32, P, P, P], I32),
        "moe_quantize_fp8_w": ([P, P, I32, I32, I32, I32, P, P, P, P, P, P, P, SZ, P], I32),
        "moe_grouped_ffn_wgrad_fp8": ([P, P, P, P, P, P, I32, I32, I32, I32, P, P, P, I32, P, SZ, P],
                                      I32),
        "moe_grouped_ffn_wgrad_fp8_begin": ([P, P, P, P, P, I32, I32, I32, I32, P, I32, P, SZ, P], I32),
        "moe_grouped_ffn_wgrad_fp8_end": ([P, P, I32, I32, I32, I32, P, P, P, I32, P, SZ, P], I32),
        "moe_profile_kernel": ([I32, ctypes.POINTER(P), ctypes.POINTER(P), I32], I32),
        "moe_profile_recorded": ([], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"libmoe ABI {lib.moe_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


lib = _load()


def hip_runtimes_mapped():
    """Paths of every libamdhip64 mapped into this process (should be one)."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _check(rc: int, what: str):
    if rc != 0:
        raise MoEError(f"{what} failed ({rc}): {lib.moe_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.uint8:  # E4M3 codes
        return MOE_FP8
    raise ValueError(f"unsupported dtype {t.dtype}")


def workspace_bytes(op: int, T: int, H: int, I: int, E: int, k: int, e_lo: int, e_hi: int,
                    dtype: int) -> int:
    n = lib.moe_workspace_bytes(op, T, H, I, E, k, e_lo, e_hi, dtype)
    if n < 0:
        _check(int(n), "moe_workspace_bytes")
    return int(n)


def _ws(nbytes: int, device, ws: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: {nbytes} bytes needed")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


# ---------------------------------------------------------------------------
# ABI wrappers
# ---------------------------------------------------------------------------

def moe_route(x: torch.Tensor, w_router: torch.Tensor, k: int, bias: Optional[torch.Tensor] = None,
              want_logits: bool = False, ws: Optional[torch.Tensor] = None,
              out: Optional[Dict[str, torch.Tensor]] = None):
    """Router GEMM + top-k gating.  Returns (topk_idx int32 [T,k], topk_w fp32 [T,k], logits|None)."""
    T, H = x.shape
    E = w_router.shape[1]
    dt = _dtype_code(x)
    out = out or {}
    idx = out.get("topk_idx")
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = out.get("topk_w")
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = out.get("logits")
    if want_logits and logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    ws = _ws(workspace_bytes(MOE_OP_ROUTE, T, H, 1, E, k, 0, E, dt), x.device, ws)
    _check(lib.moe_route(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, dt, _ptr(logits),
                         _ptr(idx), _ptr(w), _ptr(ws), _nbytes(ws), _stream()), "moe_route")
    return idx, w, logits


def moe_route_from_logits(logits: torch.Tensor, k: int):
    T, E = logits.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib.moe_route_from_logits(_ptr(logits), T, E, k, _ptr(idx), _ptr(w), _stream()),
           "moe_route_from_logits")
    return idx, w


def moe_permute(x: torch.Tensor, topk_idx: torch.Tensor, E: int, e_lo: int, e_hi: int,
                ws: Optional[torch.Tensor] = None, out: Optional[Dict[str, torch.Tensor]] = None,
                copy_rows: bool = True):
    """Group routed rows by expert.  Returns dict counts, offsets, dest_row, src_row, x_perm
    (x_perm None with copy_rows=False: the maps alone, for moe_grouped_ffn_fwd_gather)."""
    T, H = x.shape
    k = topk_idx.shape[1]
    dt = _dtype_code(x)
    E_l = e_hi - e_lo
    dev = x.device
    o = dict(out or {})
    o.setdefault("counts", torch.empty(E_l, dtype=torch.int32, device=dev))
    o.setdefault("offsets", torch.empty(E_l + 1, dtype=torch.int32, device=dev))
    o.setdefault("dest_row", torch.empty(T * k, dtype=torch.int32, device=dev))
    o.setdefault("src_row", torch.empty(T * k, dtype=torch.int32, device=dev))
    if copy_rows:
        o.setdefault("x_perm", torch.empty((T * k, H), dtype=x.dtype, device=dev))
    else:
        o["x_perm"] = None
    ws = _ws(workspace_bytes(MOE_OP_PERMUTE, T, H, 1, E, k, e_lo, e_hi, dt), dev, ws)
    _check(lib.moe_permute(_ptr(x), _ptr(topk_idx), T, H, E, k, e_lo, e_hi, dt, _ptr(o["counts"]),
                           _ptr(o["offsets"]), _ptr(o["dest_row"]), _ptr(o["src_row"]),
                           _ptr(o["x_perm"]), _ptr(ws), _nbytes(ws), _stream()), "moe_permute")
    return o


def moe_grouped_ffn_fwd(x_perm: torch.Tensor, offsets: torch.Tensor, w_gate: torch.Tensor,
                        w_up: torch.Tensor, w_down: torch.Tensor, save_gu: bool = True,
                        ws: Optional[torch.Tensor] = None,
                        out: Optional[Dict[str, torch.Tensor]] = None):
    """Grouped SwiGLU FFN forward.  Returns dict h_perm, y_perm, gu (or None)."""
    R_cap, H = x_perm.shape
    E_l, I, _ = w_gate.shape
    dt = _dtype_code(x_perm)
    dev = x_perm.device
    o = dict(out or {})
    o.setdefault("h_perm", torch.empty((R_cap, I), dtype=x_perm.dtype, device=dev))
    o.setdefault("y_perm", torch.empty((R_cap, H), dtype=x_perm.dtype, device=dev))
    if save_gu:
        o.setdefault("gu", torch.empty((R_cap, 2 * I), dtype=x_perm.dtype, device=dev))
    else:
        o["gu"] = None
    nb = lib.moe_workspace_bytes(MOE_OP_FFN_FWD, max(R_cap, 0), H, I, max(E_l, 1), 1, 0, E_l, dt)
    if nb < 0:
        _check(int(nb), "moe_workspace_bytes")
    ws = _ws(int(nb), dev, ws)
    _check(lib.moe_grouped_ffn_fwd(_ptr(x_perm), _ptr(offsets), E_l, R_cap, H, I, _ptr(w_gate),
                                   _ptr(w_up), _ptr(w_down), dt, _ptr(o["gu"]), _ptr(o["h_perm"]),
                                   _ptr(o["y_perm"]), _ptr(ws), _nbytes(ws), _stream()),
           "moe_grouped_ffn_fwd")
    return o


def moe_grouped_ffn_fwd_gather(x: torch.Tensor, src_row: torch.Tensor, offsets: torch.Tensor,
                               w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                               R_cap: int, save_gu: bool = True, ws: Optional[torch.Tensor] = None,
                               out: Optional[Dict[str, torch.Tensor]] = None):
    """moe_grouped_ffn_fwd on the token rows x [T,H], grouped row r = x[src_row[r]]
    (moe_permute's src_row).  Returns dict h_perm, y_perm, gu (or None)."""
    T, H = x.shape
    E_l, I, _ = w_gate.shape
    dt = _dtype_code(x)
    dev = x.device
    o = dict(out or {})
    o.setdefault("h_perm", torch.empty((R_cap, I), dtype=x.dtype, device=dev))
    o.setdefault("y_perm", torch.empty((R_cap, H), dtype=x.dtype, device=dev))
    if save_gu:
        o.setdefault("gu", torch.empty((R_cap, 2 * I), dtype=x.dtype, device=dev))
    else:
        o["gu"] = None
    ws = _ws(workspace_bytes(MOE_OP_FFN_FWD, max(R_cap, 0), H, I, max(E_l, 1), 1, 0, E_l, dt), dev, ws)
    _check(lib.moe_grouped_ffn_fwd_gather(_ptr(x), _ptr(src_row), _ptr(offsets), E_l, R_cap, T, H, I,
                                          _ptr(w_gate), _ptr(w_up), _ptr(w_down), dt, _ptr(o["gu"]),
                                          _ptr(o["h_perm"]), _ptr(o["y_perm"]), _ptr(ws), _nbytes(ws),
                                          _stream()), "moe_grouped_ffn_fwd_gather")
    return o


def moe_combine(y_perm: torch.Tensor, topk_w: Optional[torch.Tensor], dest_row: torch.Tensor, T: int,
                addend: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """Weighted (or, with topk_w None, unweighted) unpermute-reduce.  Returns y [T,H]."""
    H = y_perm.shape[1]
    k = dest_row.numel() // max(T, 1)
    y = out if out is not None else torch.empty((T, H), dtype=y_perm.dtype, device=y_perm.device)
    _check(lib.moe_combine(_ptr(y_perm), _ptr(topk_w), _ptr(dest_row), _ptr(addend), T, H, k,
                           _dtype_code(y_perm), _ptr(y), _stream()), "moe_combine")
    return y


def moe_combine_bwd(dy: torch.Tensor, y_perm: torch.Tensor, topk_w: torch.Tensor,
                    dest_row: torch.Tensor, out: Optional[Dict[str, torch.Tensor]] = None):
    """Returns dict dy_perm [R_cap,H], d_topk_w [T,k]."""
    T, H = dy.shape
    k = topk_w.shape[1]
    o = dict(out or {})
    o.setdefault("dy_perm", torch.empty_like(y_perm))
    o.setdefault("d_topk_w", torch.empty((T, k), dtype=torch.float32, device=dy.device))
    _check(lib.moe_combine_bwd(_ptr(dy), _ptr(y_perm), _ptr(topk_w), _ptr(dest_row), T, H, k,
                               _dtype_code(dy), _ptr(o["dy_perm"]), _ptr(o["d_topk_w"]), _stream()),
           "moe_combine_bwd")
    return o


def moe_combine_dx(dx_perm: torch.Tensor, dest_row: torch.Tensor, d_topk_w: torch.Tensor,
                   topk_w: torch.Tensor, topk_idx: torch.Tensor, w_router: torch.Tensor,
                   ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """The layer's input gradient in one pass.  Returns dx [T,H] (dtype of dx_perm)."""
    T, k = topk_w.shape
    H, E = w_router.shape
    dt = _dtype_code(dx_perm)
    dx = out if out is not None else torch.empty((T, H), dtype=dx_perm.dtype, device=dx_perm.device)
    ws = _ws(workspace_bytes(MOE_OP_COMBINE_DX, T, H, 1, E, k, 0, E, dt), dx_perm.device, ws)
    _check(lib.moe_combine_dx(_ptr(dx_perm), _ptr(dest_row), _ptr(d_topk_w), _ptr(topk_w),
                              _ptr(topk_idx), _ptr(w_router), T, H, E, k, dt, _ptr(dx), _ptr(ws),
                              _nbytes(ws), _stream()), "moe_combine_dx")
    return dx


def moe_router_weight_t(w_router: torch.Tensor, out: Optional[torch.Tensor] = None):
    """The router weight [H,E] transposed to [E,H] (operand of moe_combine_dx_t)."""
    H, E = w_router.shape
    wt = out if out is not None else torch.empty((E, H), dtype=w_router.dtype, device=w_router.device)
    _check(lib.moe_router_weight_t(_ptr(w_router), H, E, _dtype_code(w_router), _ptr(wt), _stream()),
           "moe_router_weight_t")
    return wt


def moe_combine_dx_t(dx_perm: torch.Tensor, dest_row: torch.Tensor, d_topk_w: torch.Tensor,
                     topk_w: torch.Tensor, topk_idx: torch.Tensor, w_router_t: torch.Tensor,
                     out: Optional[torch.Tensor] = None):
    """moe_combine_dx with the transposed router weight [E,H].  Returns dx [T,H]."""
    T, k = topk_w.shape
    E, H = w_router_t.shape
    dx = out if out is not None else torch.empty((T, H), dtype=dx_perm.dtype, device=dx_perm.device)
    _check(lib.moe_combine_dx_t(_ptr(dx_perm), _ptr(dest_row), _ptr(d_topk_w), _ptr(topk_w),
                                _ptr(topk_idx), _ptr(w_router_t), T, H, E, k, _dtype_code(dx_perm),
                                _ptr(dx), _stream()), "moe_combine_dx_t")
    return dx


def moe_grouped_ffn_bwd(dy_perm: torch.Tensor, x_perm: torch.Tensor, gu: torch.Tensor,
                        h_perm: torch.Tensor, offsets: torch.Tensor, w_gate: torch.Tensor,
                        w_up: torch.Tensor, w_down: torch.Tensor, accumulate: bool = False,
                        ws: Optional[torch.Tensor] = None,
                        out: Optional[Dict[str, torch.Tensor]] = None):
    """Returns dict dx_perm, dw_gate, dw_up, dw_down (fp32 weight gradients)."""
    R_cap, H = x_perm.shape
    E_l, I, _ = w_gate.shape
    dt = _dtype_code(x_perm)
    dev = x_perm.device
    o = dict(out or {})
    o.setdefault("dx_perm", torch.empty_like(x_perm))
    for n, shp in (("dw_gate", (E_l, I, H)), ("dw_up", (E_l, I, H)), ("dw_down", (E_l, H, I))):
        o.setdefault(n, torch.empty(shp, dtype=torch.float32, device=dev))
    nb = lib.moe_workspace_bytes(MOE_OP_FFN_BWD, R_cap, H, I, max(E_l, 1), 1, 0, E_l, dt)
    if nb < 0:
        _check(int(nb), "moe_workspace_bytes")
    ws = _ws(int(nb), dev, ws)
    _check(lib.moe_grouped_ffn_bwd(_ptr(dy_perm), _ptr(x_perm), _ptr(gu), _ptr(h_perm),
                                   _ptr(offsets), E_l, R_cap, H, I, _ptr(w_gate), _ptr(w_up),
                                   _ptr(w_down), dt, _ptr(o["dx_perm"]), _ptr(o["dw_gate"]),
                                   _ptr(o["dw_up"]), _ptr(o["dw_down"]), int(accumulate),
                                   _ptr(ws), _nbytes(ws), _stream()), "moe_grouped_ffn_bwd")
    return o


def moe_route_bwd(d_topk_w: torch.Tensor, topk_w: torch.Tensor, topk_idx: torch.Tensor,
                  x: torch.Tensor, w_router: torch.Tensor, want_dx: bool = True,
                  want_dw: bool = True, ws: Optional[torch.Tensor] = None,
                  out: Optional[Dict[str, torch.Tensor]] = None):
    """Returns dict d_logits [T,E], dx_router [T,H] fp32 (or None), dw_router [H,E] fp32 (or None)."""
    T, H = x.shape
    E = w_router.shape[1]
    k = topk_idx.shape[1]
    dt = _dtype_code(x)
    dev = x.device
    o = dict(out or {})
    o.setdefault("d_logits", torch.empty((T, E), dtype=torch.float32, device=dev))
    if want_dx:
        o.setdefault("dx_router", torch.empty((T, H), dtype=torch.float32, device=dev))
    else:
        o["dx_router"] = None
    if want_dw:
        o.setdefault("dw_router", torch.empty((H, E), dtype=torch.float32, device=dev))
    else:
        o["dw_router"] = None
    ws = _ws(workspace_bytes(MOE_OP_ROUTE_BWD, T, H, 1, E, k, 0, E, dt), dev, ws)
    _check(lib.moe_route_bwd(_ptr(d_topk_w), _ptr(topk_w), _ptr(topk_idx), _ptr(x),
                             _ptr(w_router), T, H, E, k, dt, _ptr(o["d_logits"]),
                             _ptr(o["dx_router"]), _ptr(o["dw_router"]), _ptr(ws), _nbytes(ws),
                             _stream()), "moe_route_bwd")
    return o


from .layer import MoELayer  # noqa: E402,F401


def moe_quantize_fp8(src: torch.Tensor, nrows: Optional[torch.Tensor] = None,
                     out: Optional[Dict[str, torch.Tensor]] = None):
    """E4M3 codes of the rows of src [rows, cols] (bf16 / fp32), one power-of-two scale
    per row.  nrows: optional int32 device tensor whose first element bounds the
    rows written.  Returns (q uint8 [rows, cols], scale fp32 [rows])."""
    rows, cols = src.shape
    o = dict(out or {})
    o.setdefault("q", torch.empty((rows, cols), dtype=torch.uint8, device=src.device))
    o.setdefault("scale", torch.empty(rows, dtype=torch.float32, device=src.device))
    _check(lib.moe_quantize_fp8(_ptr(src), rows, cols, _dtype_code(src), _ptr(nrows), _ptr(o["q"]),
                                _ptr(o["scale"]), _stream()), "moe_quantize_fp8")
    return o["q"], o["scale"]


def moe_grouped_ffn_fwd_fp8(x_q: torch.Tensor, x_scale: torch.Tensor, src_row: torch.Tensor,
                            offsets: torch.Tensor, wg: tuple, wu: tuple, wd: tuple,
                            save_gu: bool = False, ws: Optional[torch.Tensor] = None,
                            out: Optional[Dict[str, torch.Tensor]] = None, R_cap: Optional[int] = None):
    """Grouped SwiGLU FFN forward on E4M3 codes.  x_q [R_cap, H] uint8 (permuted
    rows), x_scale [T] per-token scales, src_row [R_cap]; wg / wu / wd = (codes
    uint8 [E_l, N, K], scales fp32 [E_l, N]).  Returns dict h_perm, y_perm (bf16)
    and gu (or None).  With R_cap given, x_q is the token code rows [T, H] read
    through src_row (moe_grouped_ffn_fwd_fp8_gather)."""
    gather = R_cap is not None
    T, H = x_q.shape
    R_cap = R_cap if gather else T
    E_l, I, _ = wg[0].shape
    dev = x_q.device
    o = dict(out or {})
    o.setdefault("h_perm", torch.empty((R_cap, I), dtype=torch.bfloat16, device=dev))
    o.setdefault("y_perm", torch.empty((R_cap, H), dtype=torch.bfloat16, device=dev))
    if save_gu:
        o.setdefault("gu", torch.empty((R_cap, 2 * I), dtype=torch.bfloat16, device=dev))
    else:
        o["gu"] = None
    nb = lib.moe_workspace_bytes(MOE_OP_FFN_FWD_FP8, max(R_cap, 0), H, I, max(E_l, 1), 1, 0, E_l,
                                 MOE_BF16)
    if nb < 0:
        _check(int(nb), "moe_workspace_bytes")
    ws = _ws(int(nb), dev, ws)
    if gather:
        _check(lib.moe_grouped_ffn_fwd_fp8_gather(
            _ptr(x_q), _ptr(x_scale), _ptr(src_row), _ptr(offsets), E_l, R_cap, T, H, I, _ptr(wg[0]),
            _ptr(wg[1]), _ptr(wu[0]), _ptr(wu[1]), _ptr(wd[0]), _ptr(wd[1]), _ptr(o["gu"]),
            _ptr(o["h_perm"]), _ptr(o["y_perm"]), _ptr(ws), _nbytes(ws), _stream()),
            "moe_grouped_ffn_fwd_fp8_gather")
        return o
    _check(lib.moe_grouped_ffn_fwd_fp8(_ptr(x_q), _ptr(x_scale), _ptr(src_row), _ptr(offsets), E_l,
                                       R_cap, H, I, _ptr(wg[0]), _ptr(wg[1]), _ptr(wu[0]),
                                       _ptr(wu[1]), _ptr(wd[0]), _ptr(wd[1]), _ptr(o["gu"]),
                                       _ptr(o["h_perm"]), _ptr(o["y_perm"]), _ptr(ws), _nbytes(ws),
                                       _stream()), "moe_grouped_ffn_fwd_fp8")
    return o


def moe_quantize_fp8_t(w0: torch.Tensor, w1: Optional[torch.Tensor] = None,
                       out: Optional[Dict[str, torch.Tensor]] = None):
    """Per-input-channel E4M3 codes of bf16 expert weights w0 (and w1) [E_l, N, K]:
    rows of [w0^T | w1^T].  Returns (q uint8 [E_l, K, n N], scale fp32 [E_l, K])."""
    B, N, K = w0.shape
    n = 1 if w1 is None else 2
    o = dict(out or {})
    o.setdefault("q", torch.empty((B, K, n * N), dtype=torch.uint8, device=w0.device))
    o.setdefault("scale", torch.empty((B, K), dtype=torch.float32, device=w0.device))
    _check(lib.moe_quantize_fp8_t(_ptr(w0), _ptr(w1), B, N, K, _dtype_code(w0), _ptr(o["q"]),
                                  _ptr(o["scale"]), _stream()), "moe_quantize_fp8_t")
    return o["q"], o["scale"]


def moe_grouped_ffn_dgrad_fp8(dy_q: torch.Tensor, dy_scale: torch.Tensor, gu: torch.Tensor,
                              offsets: torch.Tensor, wdt: tuple, wgut: tuple,
                              ws: Optional[torch.Tensor] = None,
                              out: Optional[Dict[str, torch.Tensor]] = None):
    """Data gradients of the grouped SwiGLU FFN on E4M3 codes.  dy_q [R_cap, H] uint8
    with per-row dy_scale [R_cap]; gu [R_cap, 2I] bf16 (saved g, u); wdt = (codes
    [E_l, I, H], scales [E_l, I]) of W_down^T; wgut = (codes [E_l, H, 2I], scales
    [E_l, H]) of [W_gate^T | W_up^T].  Returns dict dgu [R_cap, 2I] and dx_perm
    [R_cap, H] (bf16)."""
    R_cap, H = dy_q.shape
    E_l, I, _ = wdt[0].shape
    dev = dy_q.device
    o = dict(out or {})
    o.setdefault("dgu", torch.empty((R_cap, 2 * I), dtype=torch.bfloat16, device=dev))
    o.setdefault("dx_perm", torch.empty((R_cap, H), dtype=torch.bfloat16, device=dev))
    nb = lib.moe_workspace_bytes(MOE_OP_FFN_DGRAD_FP8, max(R_cap, 0), H, I, max(E_l, 1), 1, 0, E_l,
                                 MOE_BF16)
    if nb < 0:
        _check(int(nb), "moe_workspace_bytes")
    ws = _ws(int(nb), dev, ws)
    _check(lib.moe_grouped_ffn_dgrad_fp8(_ptr(dy_q), _ptr(dy_scale), _ptr(gu), _ptr(offsets), E_l,
                                         R_cap, H, I, _ptr(wdt[0]), _ptr(wdt[1]), _ptr(wgut[0]),
                                         _ptr(wgut[1]), _ptr(o["dgu"]), _ptr(o["dx_perm"]),
                                         _ptr(ws), _nbytes(ws), _stream()),
           "moe_grouped_ffn_dgrad_fp8")
    return o


def wgrad_fp8_pitch(R_cap: int, E_l: int) -> int:
    """Row pitch (codes) of the transposed code matrices: room for every group's
    rows rounded up to 64."""
    return ((R_cap + 63) // 64) * 64 + 64 * E_l


def moe_quantize_fp8_group_t(src: torch.Tensor, offsets: torch.Tensor, E_l: int,
                             src_row: Optional[torch.Tensor] = None, R_cap: Optional[int] = None,
                             out: Optional[Dict[str, torch.Tensor]] = None):
    """Per-(group, column) E4M3 codes of grouped bf16 rows (row r = src[src_row[r]] if
    src_row is given, else src[r]), transposed: returns dict q uint8 [C, pitch]
    (group g at columns poff[g] ..), scale fp32 [E_l, C], poff int32 [E_l + 1]."""
    C = src.shape[1]
    if R_cap is None:
        R_cap = src_row.numel() if src_row is not None else src.shape[0]
    pitch = wgrad_fp8_pitch(R_cap, E_l)
    dev = src.device
    o = dict(out or {})
    o.setdefault("q", torch.empty((C, pitch), dtype=torch.uint8, device=dev))
    o.setdefault("scale", torch.empty((E_l, C), dtype=torch.float32, device=dev))
    o.setdefault("poff", torch.empty(E_l + 1, dtype=torch.int32, device=dev))
    _check(lib.moe_quantize_fp8_group_t(_ptr(src), _ptr(src_row), C, _ptr(offsets), E_l, R_cap,
                                        _ptr(o["q"]), o["q"].shape[1], _ptr(o["scale"]),
                                        _ptr(o["poff"]), _stream()), "moe_quantize_fp8_group_t")
    return o


def moe_grouped_ffn_wgrad_fp8(x: torch.Tensor, src_row: Optional[torch.Tensor], dgu: torch.Tensor,
                              h_perm: torch.Tensor, dy_perm: torch.Tensor, offsets: torch.Tensor,
                              E_l: int, accumulate: bool = False, ws: Optional[torch.Tensor] = None,
                              out: Optional[Dict[str, torch.Tensor]] = None):
    """Weight gradients of the grouped SwiGLU FFN on E4M3 codes (operands quantized per
    (expert, column)).  x [T, H] with src_row [R_cap] (or the grouped rows [R_cap, H]
    with src_row None), dgu [R_cap, 2I], h_perm [R_cap, I], dy_perm [R_cap, H], all
    bf16.  Returns dict dw_gate, dw_up [E_l, I, H] and dw_down [E_l, H, I] (fp32)."""
    R_cap, H = dy_perm.shape
    I = h_perm.shape[1]
    dev = dy_perm.device
    o = dict(out or {})
    for n, sh in (("dw_gate", (E_l, I, H)), ("dw_up", (E_l, I, H)), ("dw_down", (E_l, H, I))):
        o.setdefault(n, torch.empty(sh, dtype=torch.float32, device=dev))
    nb = lib.moe_workspace_bytes(MOE_OP_FFN_WGRAD_FP8, max(R_cap, 0), H, I, max(E_l, 1), 1, 0, E_l,
                                 MOE_BF16)
    if nb < 0:
        _check(int(nb), "moe_workspace_bytes")
    ws = _ws(int(nb), dev, ws)
    _check(lib.moe_grouped_ffn_wgrad_fp8(_ptr(x), _ptr(src_row), _ptr(dgu), _ptr(h_perm),
                                         _ptr(dy_perm), _ptr(offsets), E_l, R_cap, H, I,
                                         _ptr(o["dw_gate"]), _ptr(o["dw_up"]), _ptr(o["dw_down"]),
                                         1 if accumulate else 0, _ptr(ws), _nbytes(ws), _stream()),
           "moe_grouped_ffn_wgrad_fp8")
    return o


def _wgrad_fp8_ws(R_cap, H, I, E_l, dev, ws):
    nb = lib.moe_workspace_bytes(MOE_OP_FFN_WGRAD_FP8, max(R_cap, 0), H, I, max(E_l, 1), 1, 0, E_l,
                                 MOE_BF16)
    if nb < 0:
        _check(int(nb), "moe_workspace_bytes")
    return _ws(int(nb), dev, ws)


def moe_grouped_ffn_wgrad_fp8_begin(x: torch.Tensor, src_row: Optional[torch.Tensor],
                                    h_perm: torch.Tensor, dy_perm: torch.Tensor,
                                    offsets: torch.Tensor, E_l: int, ws: torch.Tensor,
                                    dw_down: torch.Tensor, accumulate: bool = False, stream=None):
    """First half of moe_grouped_ffn_wgrad_fp8: the columns of x (through src_row),
    dy_perm and h_perm quantized into ws, the K-chunk plans, dW_down (complete only
    after moe_grouped_ffn_wgrad_fp8_end on the same ws).  stream: a torch stream
    (default: the current one)."""
    R_cap, H = dy_perm.shape
    I = h_perm.shape[1]
    ws = _wgrad_fp8_ws(R_cap, H, I, E_l, dy_perm.device, ws)
    st = (stream or torch.cuda.current_stream()).cuda_stream
    _check(lib.moe_grouped_ffn_wgrad_fp8_begin(_ptr(x), _ptr(src_row), _ptr(h_perm), _ptr(dy_perm),
                                               _ptr(offsets), E_l, R_cap, H, I, _ptr(dw_down),
                                               1 if accumulate else 0, _ptr(ws), _nbytes(ws),
                                               ctypes.c_void_p(st)),
           "moe_grouped_ffn_wgrad_fp8_begin")


def moe_grouped_ffn_wgrad_fp8_end(dgu: torch.Tensor, offsets: torch.Tensor, E_l: int, H: int,
                                  ws: torch.Tensor, out: Dict[str, torch.Tensor],
                                  accumulate: bool = False, stream=None):
    """Second half: the columns of dgu [R_cap, 2I] quantized, dW_gate and dW_up, and
    the split experts' partial sums of both products (out: dw_gate, dw_up, and the
    dw_down that begin wrote)."""
    R_cap, I2 = dgu.shape
    I = I2 // 2
    ws = _wgrad_fp8_ws(R_cap, H, I, E_l, dgu.device, ws)
    st = (stream or torch.cuda.current_stream()).cuda_stream
    _check(lib.moe_grouped_ffn_wgrad_fp8_end(_ptr(dgu), _ptr(offsets), E_l, R_cap, H, I,
                                             _ptr(out["dw_gate"]), _ptr(out["dw_up"]),
                                             _ptr(out["dw_down"]), 1 if accumulate else 0, _ptr(ws),
                                             _nbytes(ws), ctypes.c_void_p(st)),
           "moe_grouped_ffn_wgrad_fp8_end")


def moe_quantize_fp8_w(w0: torch.Tensor, w1: Optional[torch.Tensor] = None, transposed: bool = True,
                       ws: Optional[torch.Tensor] = None,
                       out: Optional[Dict[str, torch.Tensor]] = None):
    """Both E4M3 code layouts of bf16 expert weights w0 (and w1) [B, N, K]: the rows
    (q0/s0, q1/s1, as moe_quantize_fp8) and, unless transposed is False, the rows of
    [w0^T | w1^T] (qt [B, K, n N] / st [B, K], as moe_quantize_fp8_t)."""
    B, N, K = w0.shape
    n = 1 if w1 is None else 2
    dev = w0.device
    o = dict(out or {})
    o.setdefault("q0", torch.empty((B, N, K), dtype=torch.uint8, device=dev))
    o.setdefault("s0", torch.empty((B, N), dtype=torch.float32, device=dev))
    if w1 is not None:
        o.setdefault("q1", torch.empty((B, N, K), dtype=torch.uint8, device=dev))
        o.setdefault("s1", torch.empty((B, N), dtype=torch.float32, device=dev))
    else:
        o["q1"] = o["s1"] = None
    if transposed:
        o.setdefault("qt", torch.empty((B, K, n * N), dtype=torch.uint8, device=dev))
        o.setdefault("st", torch.empty((B, K), dtype=torch.float32, device=dev))
    else:
        o["qt"] = o["st"] = None
    al = lambda b: (b + 255) // 256 * 256
    nb = 2 * al(n * B * N * (K // 128) * 4) + al(n * B * N * 4) + al(B * K * 4)
    ws = _ws(nb, dev, ws)
    _check(lib.moe_quantize_fp8_w(_ptr(w0), _ptr(w1), B, N, K, _dtype_code(w0), _ptr(o["q0"]),
                                  _ptr(o["s0"]), _ptr(o["q1"]), _ptr(o["s1"]), _ptr(o["qt"]),
                                  _ptr(o["st"]), _ptr(ws), _nbytes(ws), _stream()),
           "moe_quantize_fp8_w")
    return o
