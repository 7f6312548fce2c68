"""CPU oracle for the per-GPU MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
load this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library (no
kernels, headers, helpers or tables) and imports nothing from it.

Everything here is plain float64 NumPy written for a reader to check by eye:
no blocking, no fusion, no reordering beyond what each definition states.

What the pages fix, and what is a reading
-----------------------------------------
* The local expert computation of an expert-parallel MoE layer is "permute,
  unpermute and grouped matmul" between the two all-to-alls; the plain
  PyTorch form of these ops is the reference implementation, and a fused
  form may be used only where it matches it.  (Page "FSDPTurbo EP/EFSDP and
  LlamaFactory FSDP2/CP Design", section 3, dispatcher table, rows "eager"
  and "fused".)  Empty experts are legal (same table, "fused" row).
* Expert tensor shapes for Qwen3-MoE-30B-A3B: 128 experts, hidden 2048,
  intermediate 768; gate and up projections [E, I, H], down [E, H, I]; one
  EP rank of eight holds a [16, ...] slice along dim 0.  (Page
  "Qwen3-MoE-30B-A3B模型EP+FSDP2并行方案", sections "Qwen3-MoE-30B-A3B模型"
  and "完整并行流程".)  The gate tensor is printed there as [128, 768, 768];
  a product with a hidden-size-2048 token forces [128, 768, 2048], so that
  printed shape is read as garbled.
* The pages never state the router math, the activation or the precision.
  Readings used throughout (each restated where it is used):
    - logits z = x . W_r (+ bias), W_r laid out [H, E];
    - softmax over all E experts, keep the k largest, renormalise over the
      kept k (identical to a softmax over the k kept logits);
    - selection is made on logits; equal logits go to the lower expert id;
      slot order j is (logit descending, expert id ascending);
    - rows of an expert's group are in ascending token order (the order a
      stable sort by expert gives), dropless (no capacity limit);
    - expert FFN(v) = W_down . (SiLU(W_gate . v) * (W_up . v)),
      SiLU(a) = a * sigmoid(a);
    - on an EP rank only slots whose expert lies in [e_lo, e_hi) are
      computed; the other slots keep their weight (no re-renormalisation)
      and contribute zero here.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """z[t, e] = sum_h x[t, h] * W_r[h, e] (+ bias[e]), in float64.

    Reading of the router GEMM: W_r is stored [H, E]; an optional per-expert
    bias is added to the logits (it then affects both selection and weights).
    """
    z = _f64(x) @ _f64(w_router)
    if bias is not None:
        z = z + _f64(bias)[None, :]
    return z


def topk_experts(z, k: int) -> np.ndarray:
    """The k experts of each token, slot j ordered by (logit desc, expert id asc).

    Reading: selection on logits (softmax is monotone, so the kept set is the
    one the probabilities would give); equal logits go to the lower expert id.
    Implemented as a full lexicographic sort of (-z, id) per token.
    """
    z = _f64(z)
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError(f"need 1 <= k <= E, got k={k}, E={E}")
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -z), axis=-1)   # last key (-z) is the primary key
    return order[:, :k].astype(np.int32)


def softmax(z) -> np.ndarray:
    """Row-wise softmax exp(z - max) / sum exp(z - max), float64."""
    z = _f64(z)
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def gate_weights(z, idx) -> np.ndarray:
    """w[t, j] = p[t, idx[t, j]] / sum_l p[t, idx[t, l]], p = softmax over all E.

    Reading: softmax over all experts, then top-k, then renormalise over the
    kept k (a plain top-k-then-renormalise router).
    """
    p = softmax(z)
    sel = np.take_along_axis(p, np.asarray(idx, dtype=np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(x, w_router, k: int, bias=None):
    """Logits, top-k expert ids and renormalised gate weights of every token."""
    z = router_logits(x, w_router, bias)
    idx = topk_experts(z, k)
    return z, idx, gate_weights(z, idx)


# --------------------------------------------------------------------------
# Grouping of routed rows by expert ("permute" / "unpermute")
# --------------------------------------------------------------------------

def expert_counts(idx, e_lo: int, e_hi: int) -> np.ndarray:
    """counts[e - e_lo] = number of (token, slot) pairs routed to expert e."""
    idx = np.asarray(idx)
    return np.array([np.count_nonzero(idx == e) for e in range(e_lo, e_hi)], dtype=np.int64)


def expert_offsets(counts) -> np.ndarray:
    """Exclusive prefix sum of the counts; offsets[E_l] = R, the routed rows."""
    counts = np.asarray(counts, dtype=np.int64)
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    for e in range(len(counts)):
        off[e + 1] = off[e] + counts[e]
    return off


def permutation_maps(idx, e_lo: int, e_hi: int):
    """Row maps of the expert-grouped buffer.

    dest_row[t*k + j] = offsets[e - e_lo] + #{t' < t : token t' also chose e},
    with e = idx[t, j] local; -1 for slots whose expert is not in [e_lo, e_hi).
    src_row[r] = token whose row lands in grouped row r (inverse of dest_row).

    Reading: rows of an expert group are in ascending token order, which is
    what a stable sort of the (token, slot) list by expert id produces.  A
    token's k experts are distinct, so this order is unique.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    E_l = e_hi - e_lo
    off = expert_offsets(expert_counts(idx, e_lo, e_hi))
    seen = np.zeros(E_l, dtype=np.int64)
    dest = np.full(T * k, -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e_lo <= e < e_hi:
                dest[t * k + j] = off[e - e_lo] + seen[e - e_lo]
                seen[e - e_lo] += 1
    R = int(off[E_l])
    src = np.full(R, -1, dtype=np.int64)
    for s in range(T * k):
        if dest[s] >= 0:
            src[dest[s]] = s // k
    return dest, src


def permute_rows(x, dest_row, R: int) -> np.ndarray:
    """x_perm[dest_row[t*k+j]] = x[t] for every local slot (the permute)."""
    x = _f64(x)
    T = x.shape[0]
    k = len(dest_row) // T
    out = np.full((R, x.shape[1]), np.nan)
    for s, r in enumerate(dest_row):
        if r >= 0:
            out[r] = x[s // k]
    return out


def unpermute_rows(y_perm, dest_row, T: int, weights=None) -> np.ndarray:
    """y[t] = sum_j weight[t, j] * y_perm[dest_row[t*k+j]] over local slots,
    j ascending (weight 1 when weights is None): the (weighted) unpermute."""
    y_perm = _f64(y_perm)
    k = len(dest_row) // T
    out = np.zeros((T, y_perm.shape[1]))
    for t in range(T):
        for j in range(k):
            r = dest_row[t * k + j]
            if r >= 0:
                c = 1.0 if weights is None else float(weights[t, j])
                out[t] += c * y_perm[r]
    return out


# --------------------------------------------------------------------------
# Expert FFN
# --------------------------------------------------------------------------

def sigmoid(a) -> np.ndarray:
    a = _f64(a)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def silu(a) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a) (reading: the SwiGLU expert activation)."""
    a = _f64(a)
    return a * sigmoid(a)


def swiglu_grad(dh, g, u):
    """Gradients of h = SiLU(g) * u for the upstream gradient dh:
    dg = dh * u * s * (1 + g (1 - s)) and du = dh * SiLU(g), s = sigmoid(g)."""
    dh, g, u = _f64(dh), _f64(g), _f64(u)
    s = sigmoid(g)
    return dh * u * s * (1.0 + g * (1.0 - s)), dh * (g * s)


def expert_ffn_parts(v, w_gate_e, w_up_e, w_down_e) -> Dict[str, np.ndarray]:
    """One expert on rows v [n, H]: g = v.W_gate^T, u = v.W_up^T,
    h = SiLU(g) * u, y = h.W_down^T  (W_gate/W_up [I, H], W_down [H, I])."""
    v = _f64(v)
    g = v @ _f64(w_gate_e).T
    u = v @ _f64(w_up_e).T
    h = silu(g) * u
    y = h @ _f64(w_down_e).T
    return {"g": g, "u": u, "h": h, "y": y}


def expert_ffn(v, w_gate_e, w_up_e, w_down_e) -> np.ndarray:
    return expert_ffn_parts(v, w_gate_e, w_up_e, w_down_e)["y"]


def _local_slots(idx, e_lo, e_hi, e):
    """(tokens, slots) of all pairs routed to expert e, tokens ascending."""
    tt, jj = np.nonzero(np.asarray(idx) == e)
    return tt, jj


def moe_forward(x, idx, w, w_gate, w_up, w_down, e_lo: int, e_hi: int) -> np.ndarray:
    """y[t] = sum over local slots j of w[t, j] * FFN_{idx[t,j]}(x[t]).

    Grouped by expert with a boolean selection of the routed tokens (no
    permutation buffer, no offsets); a token with no local slot gets zero.
    """
    x = _f64(x)
    y = np.zeros_like(x)
    for e in range(e_lo, e_hi):
        tt, jj = _local_slots(idx, e_lo, e_hi, e)
        if len(tt) == 0:
            continue
        ye = expert_ffn(x[tt], w_gate[e - e_lo], w_up[e - e_lo], w_down[e - e_lo])
        np.add.at(y, tt, _f64(w)[tt, jj][:, None] * ye)
    return y


def moe_forward_pairs(x, idx, w, w_gate, w_up, w_down, e_lo: int, e_hi: int) -> np.ndarray:
    """Literal per-(token, slot) loop of the same definition (small inputs only)."""
    x = _f64(x)
    T, k = np.asarray(idx).shape
    y = np.zeros_like(x)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e_lo <= e < e_hi:
                y[t] += float(w[t, j]) * expert_ffn(x[t:t + 1], w_gate[e - e_lo], w_up[e - e_lo],
                                                    w_down[e - e_lo])[0]
    return y


def pair_values(x, idx, w_gate, w_up, w_down, e_lo: int, e_hi: int,
                tokens: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Per (token, slot) intermediates of the expert FFN for the listed tokens
    (all when None): g, u, h [n, k, I] and the expert output y [n, k, H] of
    slot j of token t, i.e. expert_ffn_parts(x[t], expert idx[t, j]).  Slots
    whose expert is not in [e_lo, e_hi) stay NaN (nothing is computed for
    them on this rank).  Each local expert takes the rows of all listed
    tokens that chose it at once (boolean selection, as moe_forward does)."""
    x = _f64(x)
    idx = np.asarray(idx)
    toks = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    sub = idx[toks]
    k = idx.shape[1]
    I = np.asarray(w_gate).shape[1]
    H = x.shape[1]
    out = {n: np.full((len(toks), k, d), np.nan) for n, d in (("g", I), ("u", I), ("h", I), ("y", H))}
    for e in range(e_lo, e_hi):
        aa, jj = np.nonzero(sub == e)          # positions in the token list, slots
        if len(aa) == 0:
            continue
        p = expert_ffn_parts(x[toks[aa]], w_gate[e - e_lo], w_up[e - e_lo], w_down[e - e_lo])
        for n in out:
            out[n][aa, jj] = p[n]
    return out


# --------------------------------------------------------------------------
# FP8 variant of the expert FFN (forward)
# --------------------------------------------------------------------------
# The pages name FP8 as their only kernel-level speed lever (page
# "TorchTitan FSDP2 完全指南", section "性能表现", H100 benchmark table, row
# FSDP + compile + FP8) and fix no format or scaling.  Readings used here:
#   - format OCP FP8 E4M3 ("fn": no infinities, one NaN code per sign, largest
#     finite 448, smallest subnormal 2^-9);
#   - every row (a token of the activations, an output channel of a weight
#     matrix, a row of h) has its own power-of-two scale s = 2^e with e the
#     smallest integer such that max|row| <= 448 * 2^e (e = 0 for a zero row);
#     a value v is stored as the code of v / s rounded to nearest, ties to
#     even.  Dividing by a power of two is exact, so the codes do not depend
#     on the precision the division runs in;
#   - products accumulate the exact products of the codes' values, and the
#     row scale times the column scale multiplies the sum;
#   - h = SiLU(g) * u is rounded to bf16 (as the bf16 layer stores it) before
#     its rows are quantized for the down projection.

def fp8_e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code: sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent 0 is subnormal (m * 2^-9); 0x7f / 0xff NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(ex == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(ex.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def fp8_e4m3_encode(v) -> np.ndarray:
    """Code of the E4M3 value nearest to v (ties to the even mantissa), for
    finite |v| <= 448; -0.0 and negative values that round to zero keep the
    sign bit."""
    v = _f64(v)
    if not np.all(np.abs(v) <= 448.0):
        raise ValueError("fp8_e4m3_encode: |v| > 448 or NaN")
    neg = np.signbit(v)
    a = np.abs(v)
    # round the magnitude to 3 mantissa bits in its binade (binades below
    # 2^-6 share the subnormal spacing 2^-9); a / spacing is exact
    _, fe = np.frexp(a)                         # a = f * 2^fe, f in [0.5, 1)
    spacing = np.exp2(np.maximum(fe - 1, -6) - 3.0)
    mag = np.rint(a / spacing) * spacing        # ties to even; may carry into the next binade
    sub = mag < 2.0 ** -6
    _, fe2 = np.frexp(mag)
    mant = np.where(sub, mag * 2.0 ** 9, mag / np.exp2(fe2 - 4.0) - 8)
    bexp = np.where(sub, 0, fe2 - 1 + 7)
    code = (bexp.astype(np.int64) << 3) | mant.astype(np.int64)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def fp8_row_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e (0 where amax == 0).  With
    amax = f * 2^E (f in [0.5, 1)) and 448 = 0.875 * 2^9 this is
    E - 9, plus 1 when f > 0.875."""
    amax = _f64(amax)
    f, E = np.frexp(amax)
    e = E - 9 + (f > 0.875).astype(np.int64)
    return np.where(amax == 0, 0, e).astype(np.int64)


def quantize_rows_fp8(a):
    """Per-row power-of-two scaled E4M3 codes of a [rows, cols]:
    returns (codes uint8 [rows, cols], scale float64 [rows] = 2^e)."""
    a = _f64(a)
    e = fp8_row_exponent(np.max(np.abs(a), axis=1) if a.shape[1] else np.zeros(a.shape[0]))
    s = np.exp2(e.astype(np.float64))
    return fp8_e4m3_encode(a / s[:, None]), s


def fp8_matmul_rows(aq, sa, bq, sb) -> np.ndarray:
    """(sa_r * codes_a[r]) . (sb_n * codes_b[n])  for row-scaled operands
    a [M, K] and b [N, K]: the sum of the codes' exact products, times
    sa[r] * sb[n]."""
    acc = fp8_e4m3_decode(aq) @ fp8_e4m3_decode(bq).T
    return acc * _f64(sa)[:, None] * _f64(sb)[None, :]


def round_bf16(a) -> np.ndarray:
    """a rounded to the nearest bfloat16 value (ties to the even mantissa), as
    float64, rounded once and directly from the float64 input.

    bfloat16 keeps 8 significant bits (7 stored) over float32's exponent
    range: for |a| in [2^(E-1), 2^E) the spacing of representable values is
    2^(E-8), and below the smallest normal 2^-126 the subnormal spacing
    2^-133 applies.  a / spacing is exact (a power of two), np.rint rounds it
    to the nearest integer with ties to even, which is the even stored
    mantissa.  Magnitudes that round past the largest finite value
    (2 - 2^-7) * 2^127 become infinities; the sign of zero is kept.
    """
    a = _f64(a)
    mag = np.abs(a)
    _, fe = np.frexp(mag)                                  # mag = f * 2^fe, f in [0.5, 1)
    spacing = np.exp2(np.maximum(fe - 1, -126) - 7.0)
    with np.errstate(over="ignore"):
        r = np.rint(mag / spacing) * spacing
    r = np.where(r > (2.0 - 2.0 ** -7) * 2.0 ** 127, np.inf, r)
    r = np.where(np.isnan(a), np.nan, r)
    return np.copysign(r, a)


def expert_ffn_fp8_parts(vq, sv, wgq, sg, wuq, su, wdq, sd) -> Dict[str, np.ndarray]:
    """One expert on quantized rows (vq, sv): g, u from the row-scaled
    products with the quantized gate / up weights, h = bf16(SiLU(g) * u),
    its rows quantized (hq, sh), y = the down product with (wdq, sd)."""
    g = fp8_matmul_rows(vq, sv, wgq, sg)
    u = fp8_matmul_rows(vq, sv, wuq, su)
    h = round_bf16(silu(g) * u)
    hq, sh = quantize_rows_fp8(h)
    y = fp8_matmul_rows(hq, sh, wdq, sd)
    return {"g": g, "u": u, "h": h, "hq": hq, "sh": sh, "y": y}


def quantize_expert_weights_fp8(w):
    """Row-scaled codes of an expert weight stack [E_l, N, K]: codes [E_l, N, K]
    and scales [E_l, N] (each output channel its own scale)."""
    w = _f64(w)
    El, N, K = w.shape
    q, s = quantize_rows_fp8(w.reshape(El * N, K))
    return q.reshape(El, N, K), s.reshape(El, N)


def moe_forward_fp8(x, idx, w, w_gate, w_up, w_down, e_lo: int, e_hi: int) -> np.ndarray:
    """The forward of moe_forward with the FP8 recipe above: tokens quantized
    per row once, weights per output channel, h per row; the gate-weighted
    sum over local slots as in moe_forward."""
    xq, sx = quantize_rows_fp8(x)
    gq, gs = quantize_expert_weights_fp8(w_gate)
    uq, us = quantize_expert_weights_fp8(w_up)
    dq, ds = quantize_expert_weights_fp8(w_down)
    y = np.zeros(_f64(x).shape)
    for e in range(e_lo, e_hi):
        tt, jj = _local_slots(idx, e_lo, e_hi, e)
        if len(tt) == 0:
            continue
        i = e - e_lo
        ye = expert_ffn_fp8_parts(xq[tt], sx[tt], gq[i], gs[i], uq[i], us[i], dq[i], ds[i])["y"]
        np.add.at(y, tt, _f64(w)[tt, jj][:, None] * ye)
    return y


# --------------------------------------------------------------------------
# FP8 variant of the expert data gradients (backward)
# --------------------------------------------------------------------------
# The pages fix no FP8 backward either.  Readings, on top of the forward's:
#   - the two data-gradient products run on E4M3 codes with per-row
#     power-of-two scales: the rows of dy (grouped rows, over H); the down
#     weight per input channel (a row of W_down^T, over H); the gate and up
#     weights per input channel h, over their 2I concatenated columns (a row
#     of [W_gate^T | W_up^T]);
#   - dh is rounded to bf16; dg, du follow from dh and the saved g, u as in the
#     bf16 backward and are rounded to bf16 (the weight gradients, which stay
#     bf16, take them as they are); the rows of [dg | du] are quantized for
#     the gate / up data gradient.

def quantize_expert_weights_t_fp8(w0, w1=None):
    """Per-input-channel codes of expert weights w0 [E_l, N, K] (and w1 of the
    same shape): the rows of [w0^T | w1^T] quantized, codes [E_l, K, N] (or
    [E_l, K, 2N]) and scales [E_l, K]."""
    parts = [_f64(w0).transpose(0, 2, 1)]
    if w1 is not None:
        parts.append(_f64(w1).transpose(0, 2, 1))
    a = np.concatenate(parts, axis=2)
    El, K, N = a.shape
    q, s = quantize_rows_fp8(a.reshape(El * K, N))
    return q.reshape(El, K, N), s.reshape(El, K)


def expert_dgrad_fp8_parts(dyq, sdy, g, u, wdtq, sdt, wgutq, sgut) -> Dict[str, np.ndarray]:
    """Data gradients of one expert on quantized rows: dh = bf16 of the
    product of the dy rows (dyq, sdy) with the rows of W_down^T (wdtq, sdt);
    [dg | du] = bf16 of swiglu_grad(dh, g, u), its rows quantized (dguq,
    sdgu); dx = the product with the rows of [W_gate^T | W_up^T] (wgutq,
    sgut)."""
    dh = round_bf16(fp8_matmul_rows(dyq, sdy, wdtq, sdt))
    dg, du = swiglu_grad(dh, g, u)
    dgu = round_bf16(np.concatenate([dg, du], axis=1))
    dguq, sdgu = quantize_rows_fp8(dgu)
    dx = fp8_matmul_rows(dguq, sdgu, wgutq, sgut)
    return {"dh": dh, "dgu": dgu, "dguq": dguq, "sdgu": sdgu, "dx": dx}


# --------------------------------------------------------------------------
# FP8 variant of the expert weight gradients
# --------------------------------------------------------------------------
# Readings, on top of the data gradients': a weight gradient sums over one
# expert's rows (dW_down[e] = sum_r dy[r]^T h[r], dW_gate[e] = sum_r dg[r]^T
# x[r], dW_up[e] likewise with du), so a scale that is to multiply the whole
# sum must stay the same along those rows.  Each operand is therefore
# quantized per (expert, column): the column restricted to the expert's rows
# gets the row rule above (its transpose is a row).  The operands are the
# values the bf16 layer holds: the grouped token rows x, the bf16 [dg | du]
# of the FP8 data gradients, the bf16 h of the forward and the bf16 rows of
# dy_perm.  The codes' exact products are summed and the two scales multiply
# the sum; the result is an fp32 tensor like the bf16 weight gradients.

def quantize_group_cols_fp8(a, offsets):
    """Per-(group, column) codes of the grouped rows a [R, C], group e being
    rows offsets[e] .. offsets[e + 1] - 1: for every group, quantize_rows_fp8
    of the transpose of its rows.  Returns a list of code matrices [C, n_e]
    (one per group) and the scales [E_l, C]."""
    a = _f64(a)
    off = np.asarray(offsets, dtype=np.int64)
    codes, scales = [], []
    for e in range(len(off) - 1):
        q, s = quantize_rows_fp8(a[off[e]:off[e + 1]].T)
        codes.append(q)
        scales.append(s)
    return codes, (np.stack(scales) if scales else np.zeros((0, a.shape[1])))


def moe_wgrad_fp8(x_perm, dgu, h_perm, dy_perm, offsets) -> Dict[str, np.ndarray]:
    """FP8 weight gradients of the local experts from their grouped rows:
    dW_gate[e], dW_up[e] [I, H] = the row-scaled product of the columns of
    [dg | du] with the columns of x (first I rows of the [2I, H] result for
    the gate, the rest for up); dW_down[e] [H, I] = that of the columns of dy
    with the columns of h.  An expert without rows gets zeros."""
    I = _f64(dgu).shape[1] // 2
    xq, sx = quantize_group_cols_fp8(x_perm, offsets)
    gq, sg = quantize_group_cols_fp8(dgu, offsets)
    hq, sh = quantize_group_cols_fp8(h_perm, offsets)
    dq, sd = quantize_group_cols_fp8(dy_perm, offsets)
    E_l = len(xq)
    H = _f64(x_perm).shape[1]
    dWg, dWu, dWd = np.zeros((E_l, I, H)), np.zeros((E_l, I, H)), np.zeros((E_l, H, I))
    for e in range(E_l):
        gu_w = fp8_matmul_rows(gq[e], sg[e], xq[e], sx[e])     # [2I, H]
        dWg[e], dWu[e] = gu_w[:I], gu_w[I:]
        dWd[e] = fp8_matmul_rows(dq[e], sd[e], hq[e], sh[e])    # [H, I]
    return {"dw_gate": dWg, "dw_up": dWu, "dw_down": dWd}


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

def router_logit_grad(w, dw, idx, E: int) -> np.ndarray:
    """dz = dL/dz [T, E] from the gradient dw [T, k] of the kept gate weights.

    The gate weights are a softmax over the kept logits, so for slot j
    (expert idx[t, j]) the contribution is w_j (dw_j - sum_l w_l dw_l); every
    other logit gets 0.  Reading: an expert listed in several slots of one
    token (top-k never does this) receives the sum of its slots'
    contributions, as the chain rule gives for a logit read several times.
    """
    w = _f64(w)
    dw = _f64(dw)
    idx = np.asarray(idx).astype(np.int64)
    T = w.shape[0]
    inner = np.sum(w * dw, axis=1, keepdims=True)
    dz = np.zeros((T, E))
    np.add.at(dz, (np.arange(T)[:, None].repeat(idx.shape[1], 1), idx), w * (dw - inner))
    return dz


def router_input_grad(dz, w_router) -> np.ndarray:
    """dx_router[t] = W_r dz[t] = sum_e dz[t, e] W_r[:, e]  (logits z = x . W_r)."""
    return _f64(dz) @ _f64(w_router).T


def moe_backward(x, w_router, idx, w, w_gate, w_up, w_down, dy, e_lo: int, e_hi: int
                 ) -> Dict[str, np.ndarray]:
    """Gradients of L = sum(dy * y) for the layer above, hand-derived.

    With e = idx[t, j] local, g = W_gate[e] x, u = W_up[e] x, h = SiLU(g) u,
    o = W_down[e] h and delta = w[t, j] dy[t]:
      dw[t, j]       = <dy[t], o>           (0 for non-local slots)
      dW_down[e]    += delta h^T
      dh             = W_down[e]^T delta
      dg             = dh * u * s * (1 + g (1 - s)),  s = sigmoid(g)
      du             = dh * SiLU(g)
      dW_gate[e]    += dg x^T,  dW_up[e] += du x^T
      dx[t]         += W_gate[e]^T dg + W_up[e]^T du
    Router: w is a softmax over the kept logits, so
      dz[t, idx[t, j]] = w_j (dw_j - sum_l w_l dw_l), and dz = 0 elsewhere;
      dx[t] += W_r dz[t]  and  dW_r = x^T dz.
    Non-local slots keep dw = 0 but still enter the softmax Jacobian (the
    other EP ranks add their own terms; the sum over ranks is the full
    gradient because the Jacobian is linear in dw).
    """
    x = _f64(x)
    dy = _f64(dy)
    w = _f64(w)
    idx = np.asarray(idx)
    T, H = x.shape
    k = idx.shape[1]
    E = np.asarray(w_router).shape[1]
    E_l = e_hi - e_lo
    I = np.asarray(w_gate).shape[1]

    dw = np.zeros((T, k))
    dx = np.zeros((T, H))
    dWg = np.zeros((E_l, I, H))
    dWu = np.zeros((E_l, I, H))
    dWd = np.zeros((E_l, H, I))
    for e in range(e_lo, e_hi):
        tt, jj = _local_slots(idx, e_lo, e_hi, e)
        if len(tt) == 0:
            continue
        Wg, Wu, Wd = _f64(w_gate[e - e_lo]), _f64(w_up[e - e_lo]), _f64(w_down[e - e_lo])
        p = expert_ffn_parts(x[tt], Wg, Wu, Wd)
        g, u, h, o = p["g"], p["u"], p["h"], p["y"]
        dw[tt, jj] = np.sum(dy[tt] * o, axis=1)
        delta = w[tt, jj][:, None] * dy[tt]
        dWd[e - e_lo] = delta.T @ h
        dh = delta @ Wd
        dg, du = swiglu_grad(dh, g, u)
        dWg[e - e_lo] = dg.T @ x[tt]
        dWu[e - e_lo] = du.T @ x[tt]
        np.add.at(dx, tt, dg @ Wg + du @ Wu)

    dz = router_logit_grad(w, dw, idx, E)
    dx += router_input_grad(dz, w_router)
    dWr = x.T @ dz
    return {"dw": dw, "d_logits": dz, "dx": dx, "dw_router": dWr,
            "dw_gate": dWg, "dw_up": dWu, "dw_down": dWd}
