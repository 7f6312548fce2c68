"""moe_grouped_ffn_fwd_noalloc (the grouped FFN forward with its tile table in
the library's static per-GPU scratch) against moe_grouped_ffn_fwd with a
workspace: the same kernels, so the same bits, on two calls in a row (the
second smaller, so it runs over the first call's table), with rows >= R left
untouched.  The size limit is refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import moe_expert_layer_router_amd as moe
from workloads import EP_SHARE, make_inputs

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _noalloc(x_perm, offsets, wg, wu, wd, out, stream):
    R_cap, H = x_perm.shape
    E_l, I, _ = wg.shape
    return moe.lib.moe_grouped_ffn_fwd_noalloc(P(x_perm), P(offsets), E_l, R_cap, H, I, P(wg), P(wu),
                                               P(wd), moe.MOE_BF16, P(out["gu"]), P(out["h_perm"]),
                                               P(out["y_perm"]), ctypes.c_void_p(stream))


def test_noalloc_refuses_oversize_on_host():
    A = ctypes.c_void_p(0x100000)
    rc = moe.lib.moe_grouped_ffn_fwd_noalloc(A, A, 16, (1 << 20) + 1, 64, 64, A, A, A, moe.MOE_BF16,
                                             None, A, A, ctypes.c_void_p(0))
    assert rc == -2 and b"static scratch" in moe.lib.moe_last_error()


@pytest.mark.gpu
def test_noalloc_forward_equals_workspace_forward():
    cases = [EP_SHARE.scaled(name="noalloc_t2048_e128_local0_32", T=2048, k=8, e_lo=0, e_hi=32),
             EP_SHARE.scaled(name="noalloc_t300_e128_local96_112", T=300, k=8, e_lo=96, e_hi=112)]
    bf = torch.bfloat16
    nan = float("nan")
    stream = torch.cuda.current_stream().cuda_stream
    for w in cases:
        inp = make_inputs(w)
        t = {n: torch.from_numpy(inp[n]).to(DEV).to(bf).contiguous()
             for n in ("x", "w_router", "w_gate", "w_up", "w_down")}
        idx, _, _ = moe.moe_route(t["x"], t["w_router"], w.k)
        p = moe.moe_permute(t["x"], idx, w.E, w.e_lo, w.e_hi)
        R_cap = w.T * w.k
        ref = moe.moe_grouped_ffn_fwd(p["x_perm"], p["offsets"], t["w_gate"], t["w_up"], t["w_down"],
                                      save_gu=True)
        out = {"h_perm": torch.full((R_cap, w.I), nan, dtype=bf, device=DEV),
               "y_perm": torch.full((R_cap, w.H), nan, dtype=bf, device=DEV),
               "gu": torch.full((R_cap, 2 * w.I), nan, dtype=bf, device=DEV)}
        print(f"  case {w.name}", flush=True)
        rc = _noalloc(p["x_perm"], p["offsets"], t["w_gate"], t["w_up"], t["w_down"], out, stream)
        assert rc == 0, moe.lib.moe_last_error()
        torch.cuda.synchronize()
        R = int(p["offsets"][-1].item())
        print(f"  R = {R} of {R_cap}", flush=True)
        assert R > 0
        for n in out:
            assert torch.equal(out[n][:R].view(torch.int16), ref[n][:R].view(torch.int16)), n
            assert torch.isnan(out[n][R:].float()).all(), f"{n}: rows >= R were written"
