"""A whole MoE expert layer (forward and backward) over preallocated buffers.

Chains the C-ABI calls in the order of the layer: route -> permute ->
grouped FFN -> combine (a bf16 layer built for the forward alone permutes the
maps only and its FFN reads the token rows through src_row), and for the
backward the router weight's transpose ->
combine_bwd -> grouped FFN backward -> unweighted combine of dx_perm plus the
router's dx (on that transpose) -> route_bwd.
All buffers and workspaces are allocated once in the constructor, so
forward()/backward() only enqueue kernels (and can be captured into a HIP
graph).  In the backward, the grouped FFN's weight gradients and then the
router backward run on a second stream (default priority) beside the data
gradients and the input-gradient pass; each concurrent call has its own
workspace, and the current stream waits for the second one before
backward() returns.

With fp8=True the expert FFN runs the library's FP8 recipe (E4M3 codes with
power-of-two scales): tokens are quantized per row, the permute writes its maps
alone and the FP8 gate/up product reads the token code rows through src_row;
every forward quantizes the weights per output channel
and, for training, per input channel as well (both layouts in one pass pair,
on the second stream beside routing and permute; the backward uses these
codes, so it must be given the forward's weights); the
backward quantizes the rows of dy_perm, and the weight gradients quantize
their operands per (expert, column): x, dy_perm and h (with dW_down) on the
second stream from the start of the backward, [dg | du] (with dW_gate and
dW_up) once the data gradients have produced it.  Routing, combine and the
router backward stay as in the bf16 layer.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import torch

from . import (MOE_BF16, MOE_F32, MOE_FP8, MOE_OP_FFN_BWD, MOE_OP_FFN_DGRAD_FP8, MOE_OP_FFN_FWD,
               MOE_OP_FFN_FWD_FP8, MOE_OP_FFN_WGRAD_FP8, MOE_OP_PERMUTE, MOE_OP_QUANTIZE_W_FP8,
               MOE_OP_ROUTE, MOE_OP_ROUTE_BWD, _check, _stream, lib, workspace_bytes)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class MoELayer:
    def __init__(self, T: int, H: int, I: int, E: int, k: int, e_lo: int, e_hi: int,
                 dtype: torch.dtype, device="cuda", train: bool = True, fp8: bool = False,
                 gather: Optional[bool] = None):
        if fp8 and (dtype != torch.bfloat16 or H % 128 or I % 128 or I > 2048):
            raise ValueError("the FP8 layer needs bf16 tensors, H % 128 == 0, I % 128 == 0 "
                             "and I <= 2048")
        self.fp8 = fp8
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.e_lo, self.e_hi, self.E_l = e_lo, e_hi, e_hi - e_lo
        self.dtype = dtype
        self.dt = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
        self.R_cap = T * k
        self.train = train
        dev = torch.device(device)
        f32, i32 = torch.float32, torch.int32
        R, E_l = self.R_cap, self.E_l
        b = {}
        b["topk_idx"] = torch.empty((T, k), dtype=i32, device=dev)
        b["topk_w"] = torch.empty((T, k), dtype=f32, device=dev)
        b["logits"] = torch.empty((T, E), dtype=f32, device=dev)
        b["counts"] = torch.empty(E_l, dtype=i32, device=dev)
        b["offsets"] = torch.empty(E_l + 1, dtype=i32, device=dev)
        b["dest_row"] = torch.empty(T * k, dtype=i32, device=dev)
        b["src_row"] = torch.empty(T * k, dtype=i32, device=dev)
        # A bf16 layer built for the forward alone reads the token rows through
        # src_row in its first product (moe_grouped_ffn_fwd_gather): no grouped
        # copy.  (FP8: the permute writes maps only, its FFN gathers the token
        # code rows the same way; training keeps x_perm for
        # the weight gradients.)
        can_gather = not train and not fp8 and dtype == torch.bfloat16
        if gather and not can_gather:
            raise ValueError("gather=True needs a bf16 layer built for the forward alone (not fp8)")
        self.gather = can_gather if gather is None else bool(gather)
        b["x_perm"] = None if (fp8 or self.gather) else torch.empty((R, H), dtype=dtype, device=dev)
        b["h_perm"] = torch.empty((R, I), dtype=dtype, device=dev)
        b["y_perm"] = torch.empty((R, H), dtype=dtype, device=dev)
        b["gu"] = torch.empty((R, 2 * I), dtype=dtype, device=dev) if train else None
        b["y"] = torch.empty((T, H), dtype=dtype, device=dev)
        if train:
            b["dy_perm"] = torch.empty((R, H), dtype=dtype, device=dev)
            b["d_topk_w"] = torch.empty((T, k), dtype=f32, device=dev)
            b["d_logits"] = torch.empty((T, E), dtype=f32, device=dev)
            b["dw_router"] = torch.empty((H, E), dtype=f32, device=dev)
            b["dx_perm"] = torch.empty((R, H), dtype=dtype, device=dev)
            b["dw_gate"] = torch.empty((E_l, I, H), dtype=f32, device=dev)
            b["dw_up"] = torch.empty((E_l, I, H), dtype=f32, device=dev)
            b["dw_down"] = torch.empty((E_l, H, I), dtype=f32, device=dev)
            b["dx"] = torch.empty((T, H), dtype=dtype, device=dev)
            b["w_router_t"] = torch.empty((E, H), dtype=dtype, device=dev)
        if fp8:
            u8 = torch.uint8
            b["x_q"] = torch.empty((T, H), dtype=u8, device=dev)
            b["x_scale"] = torch.empty(T, dtype=f32, device=dev)
            b["wg_q"] = torch.empty((E_l, I, H), dtype=u8, device=dev)
            b["wu_q"] = torch.empty((E_l, I, H), dtype=u8, device=dev)
            b["wd_q"] = torch.empty((E_l, H, I), dtype=u8, device=dev)
            b["wg_s"] = torch.empty((E_l, I), dtype=f32, device=dev)
            b["wu_s"] = torch.empty((E_l, I), dtype=f32, device=dev)
            b["wd_s"] = torch.empty((E_l, H), dtype=f32, device=dev)
            if train:
                b["dy_q"] = torch.empty((R, H), dtype=u8, device=dev)
                b["dy_scale"] = torch.empty(R, dtype=f32, device=dev)
                b["wdt_q"] = torch.empty((E_l, I, H), dtype=u8, device=dev)
                b["wdt_s"] = torch.empty((E_l, I), dtype=f32, device=dev)
                b["wgut_q"] = torch.empty((E_l, H, 2 * I), dtype=u8, device=dev)
                b["wgut_s"] = torch.empty((E_l, H), dtype=f32, device=dev)
                b["dgu"] = torch.empty((R, 2 * I), dtype=dtype, device=dev)
        self.buf = b
        ops = [MOE_OP_ROUTE, MOE_OP_PERMUTE]
        ops += [MOE_OP_FFN_FWD_FP8, MOE_OP_QUANTIZE_W_FP8] if fp8 else [MOE_OP_FFN_FWD]
        if train:
            ops += [MOE_OP_FFN_DGRAD_FP8] if fp8 else [MOE_OP_FFN_BWD]
            ops += [MOE_OP_ROUTE_BWD]
        nb = max(workspace_bytes(op, T, H, I, E, k, e_lo, e_hi, self.dt) for op in ops)
        # one workspace for the calls that run one after another on the current
        # stream; the backward's concurrent calls get their own
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.ws_bytes = self.ws.numel()
        ws = lambda op: torch.empty(max(workspace_bytes(op, T, H, I, E, k, e_lo, e_hi, self.dt), 256),
                                    dtype=torch.uint8, device=dev)
        if train:
            self.ws_rb = ws(MOE_OP_ROUTE_BWD)
            self.ws_w8 = ws(MOE_OP_FFN_WGRAD_FP8) if fp8 else None
        # FP8: the weight quantization runs on the side stream beside routing
        # and permute, with a workspace of its own
        self.ws_qw = ws(MOE_OP_QUANTIZE_W_FP8) if fp8 else None
        if train or fp8:
            self.side = torch.cuda.Stream(device=dev) if dev.type == "cuda" else None

    def forward(self, x, w_router, w_gate, w_up, w_down, bias=None, save_logits=True):
        b, T, H, I, E, k = self.buf, self.T, self.H, self.I, self.E, self.k
        s = _stream()
        ws, wsb = _p(self.ws), self.ws_bytes
        if self.fp8:
            self._quantize_weights_fp8(w_gate, w_up, w_down)
        _check(lib.moe_route(_p(x), _p(w_router), _p(bias), T, H, E, k, self.dt,
                             _p(b["logits"]) if save_logits else None, _p(b["topk_idx"]),
                             _p(b["topk_w"]), ws, wsb, s), "moe_route")
        if self.fp8:
            self._forward_ffn_fp8(x, w_gate, w_up, w_down, ws, wsb, s)
        elif self.gather:
            # the maps alone, then the FFN reads x through src_row
            _check(lib.moe_permute(_p(x), _p(b["topk_idx"]), T, H, E, k, self.e_lo, self.e_hi,
                                   self.dt, _p(b["counts"]), _p(b["offsets"]), _p(b["dest_row"]),
                                   _p(b["src_row"]), None, ws, wsb, s), "moe_permute")
            _check(lib.moe_grouped_ffn_fwd_gather(_p(x), _p(b["src_row"]), _p(b["offsets"]), self.E_l,
                                                  self.R_cap, T, H, I, _p(w_gate), _p(w_up),
                                                  _p(w_down), self.dt, _p(b["gu"]), _p(b["h_perm"]),
                                                  _p(b["y_perm"]), ws, wsb, s),
                   "moe_grouped_ffn_fwd_gather")
        else:
            _check(lib.moe_permute(_p(x), _p(b["topk_idx"]), T, H, E, k, self.e_lo, self.e_hi,
                                   self.dt, _p(b["counts"]), _p(b["offsets"]), _p(b["dest_row"]),
                                   _p(b["src_row"]), _p(b["x_perm"]), ws, wsb, s), "moe_permute")
            _check(lib.moe_grouped_ffn_fwd(_p(b["x_perm"]), _p(b["offsets"]), self.E_l, self.R_cap,
                                           H, I, _p(w_gate), _p(w_up), _p(w_down), self.dt, _p(b["gu"]),
                                           _p(b["h_perm"]), _p(b["y_perm"]), ws, wsb, s),
                   "moe_grouped_ffn_fwd")
        _check(lib.moe_combine(_p(b["y_perm"]), _p(b["topk_w"]), _p(b["dest_row"]), None, T, H, k,
                               self.dt, _p(b["y"]), s), "moe_combine")
        return b["y"]

    def _quantize_rows(self, src, rows, cols, q, scale, s, nrows=None):
        _check(lib.moe_quantize_fp8(_p(src), rows, cols, self.dt, _p(nrows), _p(q), _p(scale), s),
               "moe_quantize_fp8")

    def _quantize_weights_fp8(self, w_gate, w_up, w_down):
        """Both code layouts of the expert weights (rows for the forward products
        and, when training, the input channels for the data gradients, from the
        same reads) on the side stream: they need only the weights, so they run
        beside routing and permute; the FP8 FFN waits for them."""
        b, H, I, E_l, tr = self.buf, self.H, self.I, self.E_l, self.train
        self._fp8_weights = (w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr())
        self.side.wait_stream(torch.cuda.current_stream())
        side = ctypes.c_void_p(self.side.cuda_stream)
        ws, wsb = _p(self.ws_qw), self.ws_qw.numel()
        _check(lib.moe_quantize_fp8_w(_p(w_gate), _p(w_up), E_l, I, H, self.dt, _p(b["wg_q"]),
                                      _p(b["wg_s"]), _p(b["wu_q"]), _p(b["wu_s"]),
                                      _p(b["wgut_q"]) if tr else None, _p(b["wgut_s"]) if tr else None,
                                      ws, wsb, side), "moe_quantize_fp8_w")
        _check(lib.moe_quantize_fp8_w(_p(w_down), None, E_l, H, I, self.dt, _p(b["wd_q"]), _p(b["wd_s"]),
                                      None, None, _p(b["wdt_q"]) if tr else None,
                                      _p(b["wdt_s"]) if tr else None, ws, wsb, side), "moe_quantize_fp8_w")

    def _forward_ffn_fp8(self, x, w_gate, w_up, w_down, ws, wsb, s):
        """Token rows quantized, the permutation's maps, then (once the side
        stream's weight codes are there) the FP8 grouped FFN reading the token
        code rows through src_row (h, g and u kept in bf16)."""
        b, T, H, I, E, k, E_l = self.buf, self.T, self.H, self.I, self.E, self.k, self.E_l
        self._quantize_rows(x, T, H, b["x_q"], b["x_scale"], s)
        _check(lib.moe_permute(None, _p(b["topk_idx"]), T, H, E, k, self.e_lo, self.e_hi,
                               MOE_FP8, _p(b["counts"]), _p(b["offsets"]), _p(b["dest_row"]),
                               _p(b["src_row"]), None, ws, wsb, s), "moe_permute")
        torch.cuda.current_stream().wait_stream(self.side)
        _check(lib.moe_grouped_ffn_fwd_fp8_gather(_p(b["x_q"]), _p(b["x_scale"]), _p(b["src_row"]),
                                                  _p(b["offsets"]), E_l, self.R_cap, T, H, I,
                                                  _p(b["wg_q"]), _p(b["wg_s"]), _p(b["wu_q"]),
                                                  _p(b["wu_s"]), _p(b["wd_q"]), _p(b["wd_s"]),
                                                  _p(b["gu"]), _p(b["h_perm"]), _p(b["y_perm"]), ws,
                                                  wsb, s), "moe_grouped_ffn_fwd_fp8_gather")

    def _route_bwd(self, x, w_router, stream):
        b, T, H, E, k = self.buf, self.T, self.H, self.E, self.k
        _check(lib.moe_route_bwd(_p(b["d_topk_w"]), _p(b["topk_w"]), _p(b["topk_idx"]), _p(x),
                                 _p(w_router), T, H, E, k, self.dt, _p(b["d_logits"]),
                                 None, _p(b["dw_router"]), _p(self.ws_rb), self.ws_rb.numel(), stream),
               "moe_route_bwd")

    def _backward_ffn_fp8(self, x, w_router, w_gate, w_up, w_down, ws, wsb, s, side):
        """The first half of the FP8 weight gradients (x, dy_perm and h quantized
        per (expert, column), dW_down) and then the router backward on the side
        stream from the start; dy_perm rows quantized and the FP8 data gradients
        on this stream (weight codes per input channel from the forward); then
        the second half ([dg | du] quantized, dW_gate and dW_up, the split
        experts' sums) on the side stream once the data gradients have written
        [dg | du].  (The router backward needs only d_topk_w and x: it fills the
        side stream's wait for [dg | du] instead of trailing the step.)"""
        b, H, I, E_l = self.buf, self.H, self.I, self.E_l
        if getattr(self, "_fp8_weights", None) != (w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr()):
            raise ValueError("the FP8 backward uses the weight codes of the forward: pass it the "
                             "forward's weight tensors")
        main = torch.cuda.current_stream()
        w8, w8b = _p(self.ws_w8), self.ws_w8.numel()
        # dy_perm (the combine backward's output) exists: the side stream starts
        self.side.wait_stream(main)
        _check(lib.moe_grouped_ffn_wgrad_fp8_begin(_p(x), _p(b["src_row"]), _p(b["h_perm"]),
                                                   _p(b["dy_perm"]), _p(b["offsets"]), E_l, self.R_cap,
                                                   H, I, _p(b["dw_down"]), 0, w8, w8b, side),
               "moe_grouped_ffn_wgrad_fp8_begin")
        self._route_bwd(x, w_router, side)
        self._quantize_rows(b["dy_perm"], self.R_cap, H, b["dy_q"], b["dy_scale"], s,
                            nrows=b["offsets"][E_l:])
        _check(lib.moe_grouped_ffn_dgrad_fp8(_p(b["dy_q"]), _p(b["dy_scale"]), _p(b["gu"]),
                                             _p(b["offsets"]), E_l, self.R_cap, H, I, _p(b["wdt_q"]),
                                             _p(b["wdt_s"]), _p(b["wgut_q"]), _p(b["wgut_s"]),
                                             _p(b["dgu"]), _p(b["dx_perm"]), ws, wsb, s),
               "moe_grouped_ffn_dgrad_fp8")
        # the second half needs dgu: the side stream waits for this stream
        self.side.wait_stream(main)
        _check(lib.moe_grouped_ffn_wgrad_fp8_end(_p(b["dgu"]), _p(b["offsets"]), E_l, self.R_cap, H, I,
                                                 _p(b["dw_gate"]), _p(b["dw_up"]), _p(b["dw_down"]), 0,
                                                 w8, w8b, side),
               "moe_grouped_ffn_wgrad_fp8_end")

    def backward(self, dy, x, w_router, w_gate, w_up, w_down) -> Dict[str, torch.Tensor]:
        if not self.train:
            raise RuntimeError("layer was built without training buffers")
        b, T, H, I, E, k = self.buf, self.T, self.H, self.I, self.E, self.k
        s = _stream()
        ws, wsb = _p(self.ws), self.ws_bytes
        # the router weight's transpose while nothing else runs: later, behind
        # the data gradients, its small grid would wait for CUs that the
        # concurrent weight-gradient product holds
        _check(lib.moe_router_weight_t(_p(w_router), H, E, self.dt, _p(b["w_router_t"]), s),
               "moe_router_weight_t")
        _check(lib.moe_combine_bwd(_p(dy), _p(b["y_perm"]), _p(b["topk_w"]), _p(b["dest_row"]), T, H,
                                   k, self.dt, _p(b["dy_perm"]), _p(b["d_topk_w"]), s),
               "moe_combine_bwd")
        main = torch.cuda.current_stream()
        side = ctypes.c_void_p(self.side.cuda_stream)
        if self.fp8:
            self._backward_ffn_fp8(x, w_router, w_gate, w_up, w_down, ws, wsb, s, side)
        else:
            # data gradients on this stream; the weight gradients continue on the side stream
            _check(lib.moe_grouped_ffn_bwd_split(_p(b["dy_perm"]), _p(b["x_perm"]), _p(b["gu"]),
                                                 _p(b["h_perm"]), _p(b["offsets"]), self.E_l,
                                                 self.R_cap, H, I, _p(w_gate), _p(w_up), _p(w_down),
                                                 self.dt, _p(b["dx_perm"]), _p(b["dw_gate"]),
                                                 _p(b["dw_up"]), _p(b["dw_down"]), 0, ws, wsb, s, side),
                   "moe_grouped_ffn_bwd_split")
        # input gradient: the experts' part and the router's part in one pass
        _check(lib.moe_combine_dx_t(_p(b["dx_perm"]), _p(b["dest_row"]), _p(b["d_topk_w"]),
                                    _p(b["topk_w"]), _p(b["topk_idx"]), _p(b["w_router_t"]), T, H,
                                    E, k, self.dt, _p(b["dx"]), s),
               "moe_combine_dx_t")
        if not self.fp8:
            # router backward behind the weight gradients (the side stream already
            # waits for d_topk_w: the FFN backward forked it after the combine backward)
            self._route_bwd(x, w_router, side)
        main.wait_stream(self.side)
        return {n: b[n] for n in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "d_logits",
                                  "d_topk_w")}
