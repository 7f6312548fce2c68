"""Elementwise error bounds for the bf16 layer against the float64 oracle.

The bf16 layer stores some intermediates in bf16 (reading A11: h, y_perm, the
saved g and u, dy_perm, [dg | du], dx_perm, and the outputs y and dx) and sums
in fp32.  Each bf16 store perturbs a value v by at most u |v| with the unit
roundoff u = 2^-8 (8 significant bits), and an fp32 sum of n terms errs by at
most n 2^-24 times the sum of the terms' magnitudes.  To first order, the error
of any output is bounded by u times its *magnitude*: the same computation run on
the magnitudes of every operand, where each rounding site adds the magnitude of
the value it rounds and each nonlinear step multiplies incoming magnitudes by a
bound of its derivative:

    |SiLU'(a)| <= 1.1,   |d/da [s(a) (1 + a (1 - s(a)))]| <= 0.5,
    s = sigmoid (both maxima over the reals, rounded up).

The tests accept an element when |gpu - oracle| <= max(2e-2, BETA * M) with
M this magnitude and BETA = 2^-7: u for the first-order terms plus the same
again for fp32 accumulation (n 2^-24 <= 2^-8 for every sum here, n <= 65536)
and second-order terms.  rel-L2 <= 5e-3 over the whole tensor is checked as
well.  The magnitudes are computed from the oracle's own float64 values (test
infrastructure: nothing here runs on the GPU).
"""
import numpy as np

import oracle as O

BETA = 2.0 ** -7
SILU_D1 = 1.1      # max |d SiLU(a) / da|
SILU_D2 = 0.5      # max |d/da [s (1 + a (1 - s))]|


def expert_forward_magnitudes(x, wg, wu, wd):
    """Oracle values and first-order magnitudes of one expert's forward on rows x.

    Rounding sites: g and u (saved in bf16), h (bf16), the expert output o
    (y_perm, bf16).  Returns a dict with g, u, h, o and Mg, Mu, Mh, Mo."""
    x = np.asarray(x, np.float64)
    wg, wu, wd = (np.asarray(a, np.float64) for a in (wg, wu, wd))
    p = O.expert_ffn_parts(x, wg, wu, wd)
    g, u, h, o = p["g"], p["u"], p["h"], p["y"]
    ax = np.abs(x)
    Mg = ax @ np.abs(wg).T + np.abs(g)
    Mu = ax @ np.abs(wu).T + np.abs(u)
    Mh = np.abs(h) + SILU_D1 * np.abs(u) * Mg + np.abs(O.silu(g)) * Mu
    Mo = Mh @ np.abs(wd).T + np.abs(o)
    return {"g": g, "u": u, "h": h, "o": o, "Mg": Mg, "Mu": Mu, "Mh": Mh, "Mo": Mo}


def layer_magnitudes(x, w_router, idx, w, w_gate, w_up, w_down, e_lo, e_hi, dy=None):
    """First-order magnitudes of the layer output y and, with dy, of every gradient
    moe_backward returns (same keys), for the routing idx and gate weights w.

    Forward: M(y[t]) = sum_j w_j M(o_j) + |y[t]|.
    Backward (delta = w dy[t], stored bf16; dh = W_down^T delta; dg, du from dh
    and the saved g, u, each stored bf16):
      M(dw_j)   = <|dy|, M(o_j)>
      M(dz_j)   = w_j (M(dw_j) + sum_l w_l M(dw_l))
      M(dh)     = |delta| |W_down|
      M(dg)     = M(dh) |u| SILU_D1 + |dh| (|u| SILU_D2 M(g) + SILU_D1 M(u)) + |dg|
      M(du)     = M(dh) |SiLU(g)| + |dh| SILU_D1 M(g) + |du|
      M(dW_down)= |delta|^T M(h) + |delta|^T |h|
      M(dW_gate)= M(dg)^T |x|,  M(dW_up) = M(du)^T |x|
      M(dx_p)   = M(dg) |W_gate| + M(du) |W_up| + |dx_p|
      M(dx[t])  = sum_j M(dx_p,j) + M(dz[t]) |W_r|^T + |dx[t]|
      M(dW_r)   = |x|^T M(dz)
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    idx = np.asarray(idx)
    T, H = x.shape
    k = idx.shape[1]
    E = np.asarray(w_router).shape[1]
    E_l = e_hi - e_lo
    I = np.asarray(w_gate).shape[1]
    train = dy is not None
    if train:
        dy = np.asarray(dy, np.float64)
        ady = np.abs(dy)
    My = np.zeros((T, H))
    Mdw = np.zeros((T, k))
    Mdx = np.zeros((T, H))
    MdWg = np.zeros((E_l, I, H))
    MdWu = np.zeros((E_l, I, H))
    MdWd = np.zeros((E_l, H, I))
    ax = np.abs(x)
    for e in range(e_lo, e_hi):
        tt, jj = np.nonzero(idx == e)
        if len(tt) == 0:
            continue
        i = e - e_lo
        wg, wu, wd = (np.asarray(a[i], np.float64) for a in (w_gate, w_up, w_down))
        f = expert_forward_magnitudes(x[tt], wg, wu, wd)
        wt = w[tt, jj][:, None]
        np.add.at(My, tt, wt * f["Mo"])
        if not train:
            continue
        Mdw[tt, jj] = np.sum(ady[tt] * f["Mo"], axis=1)
        delta = wt * dy[tt]
        ad = np.abs(delta)
        dh = delta @ wd
        Mdh = ad @ np.abs(wd)
        g, u = f["g"], f["u"]
        dg, du = O.swiglu_grad(dh, g, u)
        adh = np.abs(dh)
        Mdg = Mdh * np.abs(u) * SILU_D1 + adh * (np.abs(u) * SILU_D2 * f["Mg"] + SILU_D1 * f["Mu"]) + np.abs(dg)
        Mdu = Mdh * np.abs(O.silu(g)) + adh * SILU_D1 * f["Mg"] + np.abs(du)
        MdWd[i] = ad.T @ (f["Mh"] + np.abs(f["h"]))
        MdWg[i] = Mdg.T @ ax[tt]
        MdWu[i] = Mdu.T @ ax[tt]
        dxp = dg @ wg + du @ wu
        Mdxp = Mdg @ np.abs(wg) + Mdu @ np.abs(wu) + np.abs(dxp)
        np.add.at(Mdx, tt, Mdxp)
    out = {}
    if not train:
        return {"y": My}
    Mdz = np.zeros((T, E))
    inner = np.sum(w * Mdw, axis=1, keepdims=True)
    np.add.at(Mdz, (np.arange(T)[:, None].repeat(k, 1), idx.astype(np.int64)), w * (Mdw + inner))
    Mdx += Mdz @ np.abs(np.asarray(w_router, np.float64)).T
    out.update({"y": My, "dw": Mdw, "d_logits": Mdz, "dx": Mdx, "dw_router": ax.T @ Mdz,
                "dw_gate": MdWg, "dw_up": MdWu, "dw_down": MdWd})
    return out
