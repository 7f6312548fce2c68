"""Parity of the FP8 forward of the expert FFN (through the C ABI) against the oracle.

Row quantization (codes and power-of-two scales) and the FP8 permute must match
bit for bit: the codes come from exact roundings, so both sides take the same
decisions.  h and y of moe_grouped_ffn_fwd_fp8 are compared with the oracle's
FP8 recipe on the same codes:
  h: within one bf16 step plus the summation error carried through
     h = SiLU(g) u: |d| <= 2^-7 |h| + 2 (|u| dg + (|g| + 1) du) with
     dg = (F8_SUM_REL + K 2^-24) sum_c |code products| * scales (du likewise):
     the E4M3 instruction's own sum error (below) plus the standard bound for
     a K-term fp32 sum;
  y: the layer's bf16 bar, max|d| <= 2e-2 * max(1, max|ref|) and rel-L2 <=
     5e-3, plus, elementwise, what the h elements that rounded to the
     neighbouring bf16 (fp32 versus fp64 sums) can move: such an element may
     land on the other side of an E4M3 step, so its code may differ by one step
     (<= |h|/8 + the subnormal step 2^-9 of its row scale), times |W_down|.
     Both codes are correct for the recipe.  A row whose largest |h| differs
     could change its scale; such rows (expected none) are only checked against
     the exact forward;
and the recipe as a whole stays within its quantization error of the exact
forward (rel-L2 < 0.12, as the oracle's own pin).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from workloads import EP_SHARE, SKEWED, TRAIN, make_inputs

pytestmark = pytest.mark.gpu

import moe_expert_layer_router_amd as moe  # noqa: E402  (no skip: a missing library must fail)

DEV = torch.device("cuda:0")

# Summation error of the E4M3 matrix instruction.  It adds its 64 exact code
# products in one step in which terms far below the largest one lose their
# low bits: measured on gfx950 (one wave, chosen codes), a lone product under
# about 2^-13 of the largest product of its instruction drops out, and one
# instruction's error reached 2^-11.2 of the sum of its products' magnitudes
# with 62 products just under that threshold (2^-13.3 at worst over random
# codes).  An FP8 product of K terms is therefore held to
# (F8_SUM_REL + K 2^-24) times the sum of the magnitudes of its code products
# (the second term: the fp32 accumulation across instructions).
F8_SUM_REL = 2.0 ** -10


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype).contiguous()


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_fp8_bit_exact(dtype):
    rng = np.random.default_rng(31)
    rows, cols = 300, 2048 if dtype == "bf16" else 512
    a = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-40, 40, size=(rows, 1)))
    a[5] = 0.0                                           # zero row: scale 1, codes 0
    a[7] = -0.0
    a[9, :] = 1.0
    a[9, 3] = 448.0 * 2.0 ** 5                           # max exactly on a boundary
    a[11, 7] = -448.0 * 2.0 ** -3
    a[13, :] = rng.standard_normal(cols) * 2.0 ** -12    # many values in the subnormal codes
    a[13, 0] = 1.0
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    src = _dev(a.astype(np.float32), tdt)
    print(f"  quantize {dtype} rows={rows} cols={cols}", flush=True)
    q, s = moe.moe_quantize_fp8(src)
    torch.cuda.synchronize()
    ref_q, ref_s = O.quantize_rows_fp8(_np(src))
    got_q = q.cpu().numpy()
    bad = np.nonzero(got_q != ref_q)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}: " \
                             f"{got_q[bad][0]:#x} vs {ref_q[bad][0]:#x}"
    assert np.array_equal(s.cpu().numpy().astype(np.float64), ref_s)
    # a device row bound: rows at or past it are left as they were
    nrows = torch.tensor([150], dtype=torch.int32, device=DEV)
    q2 = torch.full_like(q, 0xAA)
    s2 = torch.full_like(s, -1.0)
    moe.moe_quantize_fp8(src, nrows=nrows, out={"q": q2, "scale": s2})
    torch.cuda.synchronize()
    assert torch.equal(q2[:150], q[:150]) and torch.equal(s2[:150], s[:150])
    assert (q2[150:] == 0xAA).all() and (s2[150:] == -1.0).all()


FP8_CASES = [
    EP_SHARE.scaled(name="fp8_t512_h256_i128_e32_k4_local4to20", T=512, H=256, I=128, E=32, k=4,
                    e_lo=4, e_hi=20),
    SKEWED.scaled(name="fp8_skewed_t1024_h256_i256_e32_k4", T=1024, H=256, I=256, E=32, k=4, e_lo=0,
                  e_hi=32),
    EP_SHARE.scaled(name="fp8_t2048_h2048_i768_e16_k4_all_local", T=2048, E=16, k=4, e_lo=0, e_hi=16),
    # more tiles than persistent workgroups: ~870 gate/up tiles (6 N tiles) and ~430
    # down tiles, so workgroups run later tiles (next-tile scale loads, prologue
    # during the epilogue)
    EP_SHARE.scaled(name="fp8_multitile_t8192_h2048_i768_e16_k4_all_local", T=8192, E=16, k=4,
                    e_lo=0, e_hi=16),
]


@pytest.mark.parametrize("w", FP8_CASES, ids=lambda w: w.name)
def test_ffn_fwd_fp8_matches_oracle(w):
    inp = make_inputs(w)
    _, idx, _ = O.route(inp["x"], inp["w_router"], w.k, inp.get("bias"))
    print(f"  case {w.name}", flush=True)
    bf = torch.bfloat16
    x = _dev(inp["x"], bf)
    wts = {n: _dev(inp[n], bf) for n in ("w_gate", "w_up", "w_down")}
    # quantize tokens and weights on the GPU; the codes must be the oracle's
    xq, sx = moe.moe_quantize_fp8(x)
    wq = {}
    for n, t in wts.items():
        El, N, K = t.shape
        q, s = moe.moe_quantize_fp8(t.view(El * N, K))
        wq[n] = (q.view(El, N, K), s.view(El, N))
    torch.cuda.synchronize()
    ref_xq, ref_sx = O.quantize_rows_fp8(inp["x"])
    assert np.array_equal(xq.cpu().numpy(), ref_xq) and np.array_equal(_np(sx), ref_sx)
    ref_w = {n: O.quantize_expert_weights_fp8(inp[n]) for n in wts}
    for n in wts:
        assert np.array_equal(wq[n][0].cpu().numpy(), ref_w[n][0]), n
        assert np.array_equal(_np(wq[n][1]), ref_w[n][1]), n
    # FP8 permute: rows of codes move bit for bit
    perm = moe.moe_permute(xq, torch.from_numpy(idx.astype(np.int32)).to(DEV), w.E, w.e_lo, w.e_hi)
    R_cap, nan = w.T * w.k, float("nan")
    guard = {"h_perm": torch.full((R_cap, w.I), nan, dtype=bf, device=DEV),
             "y_perm": torch.full((R_cap, w.H), nan, dtype=bf, device=DEV),
             "gu": torch.full((R_cap, 2 * w.I), nan, dtype=bf, device=DEV)}
    out = moe.moe_grouped_ffn_fwd_fp8(perm["x_perm"], sx, perm["src_row"], perm["offsets"],
                                      wq["w_gate"], wq["w_up"], wq["w_down"], save_gu=True, out=guard)
    # the same forward reading the token code rows through src_row (the permute's
    # maps alone): the same bits, rows >= R untouched
    maps = moe.moe_permute(xq, torch.from_numpy(idx.astype(np.int32)).to(DEV), w.E, w.e_lo, w.e_hi,
                           copy_rows=False)
    guard2 = {n: torch.full_like(v, nan) for n, v in guard.items()}
    out2 = moe.moe_grouped_ffn_fwd_fp8(xq, sx, maps["src_row"], maps["offsets"], wq["w_gate"],
                                       wq["w_up"], wq["w_down"], save_gu=True, out=guard2, R_cap=R_cap)
    torch.cuda.synchronize()
    offsets = perm["offsets"].cpu().numpy()
    R = int(offsets[-1])
    for n in guard:
        assert torch.isnan(out[n][R:].float()).all(), f"{n}: rows >= R were written"
        assert torch.isnan(out2[n][R:].float()).all(), f"{n} (gathering): rows >= R were written"
        assert torch.equal(out2[n][:R].view(torch.int16), out[n][:R].view(torch.int16)), n
    src_row = perm["src_row"].cpu().numpy()[:R]
    assert np.array_equal(perm["x_perm"][:R].cpu().numpy(), ref_xq[src_row])
    h_got, y_got = _np(out["h_perm"][:R]), _np(out["y_perm"][:R])
    h_ref, y_ref, y_exact = np.zeros_like(h_got), np.zeros_like(y_got), np.zeros_like(y_got)
    h_slack, y_flip = np.zeros_like(h_got), np.zeros_like(y_got)
    same_max = np.zeros(R, dtype=bool)
    empty = 0
    for e in range(w.e_lo, w.e_hi):
        i = e - w.e_lo
        tt, _ = np.nonzero(np.asarray(idx) == e)
        assert offsets[i + 1] - offsets[i] == len(tt)
        if len(tt) == 0:
            empty += 1
            continue
        p = O.expert_ffn_fp8_parts(ref_xq[tt], ref_sx[tt], ref_w["w_gate"][0][i], ref_w["w_gate"][1][i],
                                   ref_w["w_up"][0][i], ref_w["w_up"][1][i], ref_w["w_down"][0][i],
                                   ref_w["w_down"][1][i])
        sl = slice(offsets[i], offsets[i + 1])
        h_ref[sl], y_ref[sl] = p["h"], p["y"]
        # absolute sums of the code products: the fp32 accumulation error scale
        mag = lambda q: q & np.uint8(0x7F)
        ga = O.fp8_matmul_rows(mag(ref_xq[tt]), ref_sx[tt], mag(ref_w["w_gate"][0][i]), ref_w["w_gate"][1][i])
        ua = O.fp8_matmul_rows(mag(ref_xq[tt]), ref_sx[tt], mag(ref_w["w_up"][0][i]), ref_w["w_up"][1][i])
        gam = F8_SUM_REL + w.H * 2.0 ** -24
        h_slack[sl] = 2 * (np.abs(p["u"]) * gam * ga + (np.abs(p["g"]) + 1) * gam * ua)
        d = h_got[sl] != p["h"]
        step = np.abs(p["h"]) / 8 + p["sh"][:, None] * 2.0 ** -9
        wdq = np.abs(O.fp8_e4m3_decode(ref_w["w_down"][0][i])) * ref_w["w_down"][1][i][:, None]
        y_flip[sl] = (d * step) @ wdq.T
        same_max[sl] = np.abs(h_got[sl]).max(axis=1) == np.abs(p["h"]).max(axis=1)
        y_exact[sl] = O.expert_ffn(inp["x"][tt], inp["w_gate"][i], inp["w_up"][i], inp["w_down"][i])
    hb = 2.0 ** -7 * np.abs(h_ref) + h_slack
    hbad = int((np.abs(h_got - h_ref) > hb).sum())
    ok_rows = same_max
    bar = 2e-2 * max(1.0, np.abs(y_ref).max())
    over = np.abs(y_got - y_ref) - (bar + y_flip)
    rel = np.linalg.norm(y_got - y_ref) / np.linalg.norm(y_ref)
    rel_exact = np.linalg.norm(y_got - y_exact) / np.linalg.norm(y_exact)
    print(f"  R={R} empty experts={empty}: h beyond one bf16 step: {hbad}; y max-abs "
          f"{np.abs(y_got - y_ref).max():.3e} (bar {bar:.3e}, largest code-step allowance "
          f"{y_flip.max():.3e}) rel-L2 {rel:.3e}; rows with a different max|h|: "
          f"{int((~ok_rows).sum())}; vs exact forward rel-L2 {rel_exact:.3e}", flush=True)
    assert hbad == 0
    assert (over[ok_rows] <= 0).all() and rel <= 5e-3
    assert (~ok_rows).mean() < 0.01
    assert rel_exact < 0.12
    # the saved g / u are the scaled products
    gu = _np(out["gu"][:R])
    I = w.I
    g_ref = np.concatenate([O.fp8_matmul_rows(ref_xq[np.nonzero(np.asarray(idx) == e)[0]],
                                              ref_sx[np.nonzero(np.asarray(idx) == e)[0]],
                                              ref_w["w_gate"][0][e - w.e_lo], ref_w["w_gate"][1][e - w.e_lo])
                            for e in range(w.e_lo, w.e_hi)], axis=0)
    assert np.abs(gu[:, :I] - g_ref).max() <= 2.0 ** -7 * np.abs(g_ref).max()


# ----------------------------------------------------------------------------
# FP8 data gradients
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("pair,N", [(False, 192), (True, 192), (True, 1152)],
                         ids=["single_n192", "pair_n192", "pair_n1152"])
def test_quantize_fp8_t_bit_exact(pair, N):
    rng = np.random.default_rng(41)
    B, K = 2, 128
    w0 = rng.standard_normal((B, N, K)) * np.exp2(rng.integers(-20, 20, size=(B, 1, K)))
    w1 = rng.standard_normal((B, N, K)) * np.exp2(rng.integers(-20, 20, size=(B, 1, K)))
    w0[0, :, 5] = 0.0
    if pair:
        w1[0, :, 5] = 0.0                                   # zero input channel: scale 1, codes 0
    w0[1, 7, 9] = 448.0 * 2.0 ** 3                          # a maximum exactly on the boundary
    w1[1, :, 9] = 0.0
    t0, t1 = _dev(w0.astype(np.float32), torch.bfloat16), _dev(w1.astype(np.float32), torch.bfloat16)
    print(f"  quantize_t pair={pair} B={B} N={N} K={K}", flush=True)
    q, s = moe.moe_quantize_fp8_t(t0, t1 if pair else None)
    torch.cuda.synchronize()
    ref_q, ref_s = O.quantize_expert_weights_t_fp8(_np(t0), _np(t1) if pair else None)
    assert q.shape == ref_q.shape
    bad = np.nonzero(q.cpu().numpy() != ref_q)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {[b[0] for b in bad]}"
    assert np.array_equal(_np(s), ref_s)


@pytest.mark.parametrize("pair,N,K,transposed", [(True, 768, 2048, True), (False, 2048, 768, True),
                                                  (True, 384, 128, False), (False, 128, 128, True)],
                         ids=["gate_up_pair", "down", "pair_rows_only", "single_tile"])
def test_quantize_fp8_w_matches_both_quantizers(pair, N, K, transposed):
    """moe_quantize_fp8_w gives, bit for bit, the row codes of moe_quantize_fp8 and the
    per-input-channel codes of moe_quantize_fp8_t (both checked against the oracle
    above) on weights whose rows and columns span 2^-20 .. 2^20, with a zero row, a
    zero column and maxima exactly on a scale boundary."""
    rng = np.random.default_rng(43)
    B = 3
    w0 = rng.standard_normal((B, N, K)) * np.exp2(rng.integers(-20, 20, size=(B, N, 1))) \
        * np.exp2(rng.integers(-4, 4, size=(B, 1, K)))
    w1 = rng.standard_normal((B, N, K)) * np.exp2(rng.integers(-20, 20, size=(B, N, 1)))
    w0[0, 3, :] = 0.0
    w0[1, :, 5] = 0.0
    w1[1, :, 5] = 0.0
    w0[2, 7, 9] = 448.0 * 2.0 ** 6
    t0, t1 = _dev(w0.astype(np.float32), torch.bfloat16), _dev(w1.astype(np.float32), torch.bfloat16)
    print(f"  quantize_w pair={pair} B={B} N={N} K={K} transposed={transposed}", flush=True)
    o = moe.moe_quantize_fp8_w(t0, t1 if pair else None, transposed=transposed)
    r0 = moe.moe_quantize_fp8(t0.view(B * N, K))
    r1 = moe.moe_quantize_fp8(t1.view(B * N, K)) if pair else None
    rt = moe.moe_quantize_fp8_t(t0, t1 if pair else None) if transposed else None
    torch.cuda.synchronize()
    assert torch.equal(o["q0"].view(B * N, K), r0[0]) and torch.equal(o["s0"].view(-1), r0[1])
    if pair:
        assert torch.equal(o["q1"].view(B * N, K), r1[0]) and torch.equal(o["s1"].view(-1), r1[1])
    if transposed:
        assert torch.equal(o["qt"], rt[0]) and torch.equal(o["st"], rt[1])
    else:
        assert o["qt"] is None


DGRAD_CASES = [
    EP_SHARE.scaled(name="dgrad_fp8_t512_h256_i128_e32_k4_local4to20", T=512, H=256, I=128, E=32, k=4,
                    e_lo=4, e_hi=20),
    SKEWED.scaled(name="dgrad_fp8_skewed_t1024_h256_i256_e32_k4", T=1024, H=256, I=256, E=32, k=4,
                  e_lo=0, e_hi=32),
    EP_SHARE.scaled(name="dgrad_fp8_t2048_h2048_i768_e16_k4_all_local", T=2048, E=16, k=4, e_lo=0, e_hi=16),
    # ~430 dh tiles and ~1150 dx tiles for 256 persistent workgroups
    EP_SHARE.scaled(name="dgrad_fp8_multitile_t8192_h2048_i768_e16_k4_all_local", T=8192, E=16, k=4,
                    e_lo=0, e_hi=16),
]


@pytest.mark.parametrize("w", DGRAD_CASES, ids=lambda w: w.name)
def test_ffn_dgrad_fp8_matches_oracle(w):
    """Two stages against the oracle's FP8 data gradients:
      dgu: within one bf16 step, plus what a dh that rounded to the neighbouring
           bf16 (GPU versus fp64 sums, bound: one bf16 step of dh plus the
           summation error F8_SUM_REL + K 2^-24 of its code products) moves
           through the SiLU derivative: |d dg / d dh| = |u s (1 + g (1 - s))|,
           |d du / d dh| = |g s|;
      dx:  against the oracle's second product applied to the GPU's own dgu rows
           (their quantization must match bit for bit): the layer's bf16 bar,
           max|d| <= 2e-2 * max(1, max|ref|) and rel-L2 <= 5e-3;
    rows >= R are left as they were, and the result stays within the recipe's
    quantization error of the exact data gradient (rel-L2 < 0.12, the oracle's
    own pin)."""
    inp = make_inputs(w)
    _, idx, _ = O.route(inp["x"], inp["w_router"], w.k, inp.get("bias"))
    print(f"  case {w.name}", flush=True)
    bf = torch.bfloat16
    x = _dev(inp["x"], bf)
    perm = moe.moe_permute(x, torch.from_numpy(idx.astype(np.int32)).to(DEV), w.E, w.e_lo, w.e_hi)
    offsets = perm["offsets"]
    off = offsets.cpu().numpy()
    R, R_cap, E_l = int(off[-1]), w.T * w.k, w.e_hi - w.e_lo
    rng = np.random.default_rng(zlib.crc32(w.name.encode()))
    g = rng.standard_normal((R_cap, w.I)) * 2.0
    u = rng.standard_normal((R_cap, w.I))
    gu = _dev(np.concatenate([g, u], axis=1).astype(np.float32), bf)
    dy = _dev((rng.standard_normal((R_cap, w.H)) * 0.05).astype(np.float32), bf)
    wts = {n: _dev(inp[n], bf) for n in ("w_gate", "w_up", "w_down")}
    dyq, sdy = moe.moe_quantize_fp8(dy, nrows=offsets[E_l:])
    wdt = moe.moe_quantize_fp8_t(wts["w_down"])
    wgut = moe.moe_quantize_fp8_t(wts["w_gate"], wts["w_up"])
    nan = float("nan")
    out = {"dgu": torch.full((R_cap, 2 * w.I), nan, dtype=bf, device=DEV),
           "dx_perm": torch.full((R_cap, w.H), nan, dtype=bf, device=DEV)}
    moe.moe_grouped_ffn_dgrad_fp8(dyq, sdy, gu, offsets, wdt, wgut, out=out)
    torch.cuda.synchronize()
    gu_np, dy_np = _np(gu), _np(dy)
    ref_dyq, ref_sdy = O.quantize_rows_fp8(dy_np[:R])
    assert np.array_equal(dyq[:R].cpu().numpy(), ref_dyq) and np.array_equal(_np(sdy[:R]), ref_sdy)
    ref_wdt = O.quantize_expert_weights_t_fp8(_np(wts["w_down"]))
    ref_wgut = O.quantize_expert_weights_t_fp8(_np(wts["w_gate"]), _np(wts["w_up"]))
    assert np.array_equal(wdt[0].cpu().numpy(), ref_wdt[0]) and np.array_equal(_np(wdt[1]), ref_wdt[1])
    assert np.array_equal(wgut[0].cpu().numpy(), ref_wgut[0]) and np.array_equal(_np(wgut[1]), ref_wgut[1])
    dgu_got, dx_got = _np(out["dgu"]), _np(out["dx_perm"])
    assert np.isnan(dgu_got[R:]).all() and np.isnan(dx_got[R:]).all()
    dgu_got, dx_got = dgu_got[:R], dx_got[:R]
    dgu_ref, dgu_bound = np.zeros_like(dgu_got), np.zeros_like(dgu_got)
    dx_ref, dx_exact = np.zeros_like(dx_got), np.zeros_like(dx_got)
    mag = lambda q: q & np.uint8(0x7F)
    for i in range(E_l):
        sl = slice(off[i], off[i + 1])
        if off[i + 1] == off[i]:
            continue
        gg, uu = gu_np[sl, :w.I], gu_np[sl, w.I:]
        p = O.expert_dgrad_fp8_parts(ref_dyq[sl], ref_sdy[sl], gg, uu, ref_wdt[0][i], ref_wdt[1][i],
                                     ref_wgut[0][i], ref_wgut[1][i])
        dgu_ref[sl] = p["dgu"]
        dh_abs = O.fp8_matmul_rows(mag(ref_dyq[sl]), ref_sdy[sl], mag(ref_wdt[0][i]), ref_wdt[1][i])
        dh_slack = 2.0 ** -7 * np.abs(p["dh"]) + 2 * (F8_SUM_REL + w.H * 2.0 ** -24) * dh_abs
        s = O.sigmoid(gg)
        ddg, ddu = np.abs(uu * s * (1 + gg * (1 - s))), np.abs(gg * s)
        dgu_bound[sl] = 2.0 ** -7 * np.abs(p["dgu"]) + np.concatenate([ddg * dh_slack, ddu * dh_slack],
                                                                       axis=1) + 1e-30
        # second stage on the GPU's own dgu rows
        q2, s2 = O.quantize_rows_fp8(dgu_got[sl])
        dx_ref[sl] = O.fp8_matmul_rows(q2, s2, ref_wgut[0][i], ref_wgut[1][i])
        # exact data gradient of the same operands
        dg, du = O.swiglu_grad(dy_np[sl] @ _np(wts["w_down"][i]), gg, uu)
        dx_exact[sl] = dg @ _np(wts["w_gate"][i]) + du @ _np(wts["w_up"][i])
    over = np.abs(dgu_got - dgu_ref) > dgu_bound
    bar = 2e-2 * max(1.0, np.abs(dx_ref).max())
    rel = np.linalg.norm(dx_got - dx_ref) / max(np.linalg.norm(dx_ref), 1e-30)
    rel_exact = np.linalg.norm(dx_got - dx_exact) / max(np.linalg.norm(dx_exact), 1e-30)
    print(f"  R={R}: dgu beyond bound {int(over.sum())} of {over.size} (max |d| {np.abs(dgu_got - dgu_ref).max():.3e}); "
          f"dx max-abs {np.abs(dx_got - dx_ref).max():.3e} (bar {bar:.3e}) rel-L2 {rel:.3e}; "
          f"vs exact rel-L2 {rel_exact:.3e}", flush=True)
    assert over.sum() == 0
    assert np.abs(dx_got - dx_ref).max() <= bar and rel <= 5e-3
    assert rel_exact < 0.12


# ----------------------------------------------------------------------------
# weight gradients
# ----------------------------------------------------------------------------

def _round64(n):
    return (n + 63) // 64 * 64


@pytest.mark.parametrize("layout", ["small", "chunked"])
@pytest.mark.parametrize("mapped", [False, True], ids=["grouped_rows", "token_rows_via_src_row"])
def test_quantize_fp8_group_t_bit_exact(mapped, layout):
    """Per-(group, column) codes of grouped rows, transposed: codes, scales and padded
    offsets bit for bit against the oracle, zero codes in each group's padding, and
    nothing written past the last group.  small: groups of 37, 0, 1, exactly 64 and
    130 rows; columns with a zero group column, a maximum exactly on a scale boundary
    and values deep in the subnormal codes.  chunked: groups past the quantizer's
    256-row chunks (700 rows, exactly 256, 257 and 512) among 100 groups (0..40
    rows, some empty), so that a group's maxima come from several chunks and the
    chunk list is longer than the grid; in the 700-row group one column's maximum
    sits in its last chunk only, one column is zero except for tiny values in the
    first chunk, one is zero throughout, and one has a scale below the smallest
    normal float (2^-129)."""
    rng = np.random.default_rng(51)
    if layout == "small":
        counts = [37, 0, 1, 64, 130]
    else:
        counts = [700, 0, 256, 257, 512, 1] + [int(v) * (v % 5 != 0) for v in rng.integers(0, 41, 94)]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R, C, E_l = int(off[-1]), 192, len(counts)
    a = rng.standard_normal((R, C)) * np.exp2(rng.integers(-30, 30, size=(1, C)))
    if layout == "small":
        a[off[0]:off[1], 5] = 0.0
        a[off[3] + 7, 9] = 448.0 * 2.0 ** 4
        a[off[4]:off[5], 11] = rng.standard_normal(counts[4]) * 2.0 ** -30
        a[off[4], 11] = 1.0
    else:
        a[:, 3] = rng.standard_normal(R)
        a[690, 3] = 448.0 * 2.0 ** 6          # group 0's maximum in its third chunk
        a[:, 4] = 0.0
        a[:100, 4] = rng.standard_normal(100) * 2.0 ** -40
        a[:700, 5] = 0.0
        a[:700, 6] = rng.choice([-1.0, 1.0], 700) * rng.uniform(1.0, 6.0, 700) * 2.0 ** -124  # normal floats
        a[300, 6] = 448.0 * 2.0 ** -129       # scale 2^-129: a float subnormal
        a[off[2] + 255, 7] = 448.0 * 2.0 ** 3  # last row of a 256-row group
        a[off[3] + 256, 7] = -448.0 * 2.0 ** 5  # the one row of a 257-row group's second chunk
    a32 = a.astype(np.float32)
    if mapped:     # token rows in another order, gathered through src_row
        perm = rng.permutation(R)
        src_np = np.empty_like(a32)
        src_np[perm] = a32
        src_row = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    else:
        src_np, src_row = a32, None
    src = _dev(src_np, torch.bfloat16)
    offsets = torch.from_numpy(off).to(DEV)
    pitch = moe.wgrad_fp8_pitch(R, E_l)
    out = {"q": torch.full((C, pitch), 0xAA, dtype=torch.uint8, device=DEV),
           "scale": torch.full((E_l, C), -1.0, dtype=torch.float32, device=DEV),
           "poff": torch.full((E_l + 1,), -1, dtype=torch.int32, device=DEV)}
    print(f"  quantize_group_t mapped={mapped} R={R} C={C} groups={counts}", flush=True)
    moe.moe_quantize_fp8_group_t(src, offsets, E_l, src_row=src_row, R_cap=R, out=out)
    torch.cuda.synchronize()
    rows = _np(src)[perm] if mapped else _np(src)
    ref_codes, ref_s = O.quantize_group_cols_fp8(rows, off)
    want_poff = np.concatenate([[0], np.cumsum([_round64(n) for n in counts])])
    assert np.array_equal(out["poff"].cpu().numpy(), want_poff)
    assert np.array_equal(_np(out["scale"]), ref_s)
    q = out["q"].cpu().numpy()
    for g, n in enumerate(counts):
        p0 = want_poff[g]
        got = q[:, p0:p0 + n]
        bad = np.nonzero(got != ref_codes[g])
        assert bad[0].size == 0, f"group {g}: {bad[0].size} codes differ, first at {[b[0] for b in bad]}"
        assert (q[:, p0 + n:p0 + _round64(n)] == 0).all(), f"group {g}: padding not zero"
    assert (q[:, want_poff[-1]:] == 0xAA).all()


WGRAD_CASES = [
    EP_SHARE.scaled(name="wgrad_fp8_t512_h256_i128_e32_k4_local4to20", T=512, H=256, I=128, E=32, k=4,
                    e_lo=4, e_hi=20),
    SKEWED.scaled(name="wgrad_fp8_skewed_t1024_h256_i256_e32_k4", T=1024, H=256, I=256, E=32, k=4,
                  e_lo=0, e_hi=32),
    # partial tiles on both sides: dW_down has M = H = 384 (a 128-row second M
    # tile) and N = I = 128; the gate/up product has N = H = 384
    EP_SHARE.scaled(name="wgrad_fp8_t512_h384_i128_e8_k2_partial_tiles", T=512, H=384, I=128, E=8, k=2,
                    e_lo=0, e_hi=8),
    # the expert layer's shapes: 16 experts x (48 gate/up + 24 down) tiles for 256
    # persistent workgroups
    EP_SHARE.scaled(name="wgrad_fp8_multitile_t4096_h2048_i768_e16_k4_all_local", T=4096, E=16, k=4,
                    e_lo=0, e_hi=16),
    # skewed load on a narrow layer (one tile per expert and product): experts past
    # 1024 padded rows are cut into K chunks whose partial sums are added in order
    SKEWED.scaled(name="wgrad_fp8_skewed_t4096_h256_i128_e16_k4_split", T=4096, H=256, I=128, E=16, k=4,
                  e_lo=0, e_hi=16),
]


@pytest.mark.parametrize("w", WGRAD_CASES, ids=lambda w: w.name)
def test_ffn_wgrad_fp8_matches_oracle(w):
    """dW_gate, dW_up, dW_down of moe_grouped_ffn_wgrad_fp8 against the oracle's FP8
    weight gradients on the same bf16 operands (x gathered through src_row): the
    codes are exact on both sides, so the only difference is the sum of n_e
    exact code products, bounded elementwise by (F8_SUM_REL + (n_e + 2) 2^-24)
    times the sum of their magnitudes times the scales (the instruction's own
    sum error, the standard n-term fp32 bound, and the fp32 rounding of the
    output).  accumulate adds to the previous result (exactly twice it where
    an expert is one K chunk, else within the bound plus the chunk additions'
    roundings), an expert without rows gets zeros, and the recipe stays within its
    quantization error of the exact weight gradients (rel-L2 < 0.10)."""
    inp = make_inputs(w)
    _, idx, _ = O.route(inp["x"], inp["w_router"], w.k, inp.get("bias"))
    print(f"  case {w.name}", flush=True)
    bf = torch.bfloat16
    x = _dev(inp["x"], bf)
    perm = moe.moe_permute(x, torch.from_numpy(idx.astype(np.int32)).to(DEV), w.E, w.e_lo, w.e_hi)
    offsets, src_row = perm["offsets"], perm["src_row"]
    off = offsets.cpu().numpy()
    R, R_cap, E_l = int(off[-1]), w.T * w.k, w.e_hi - w.e_lo
    rng = np.random.default_rng(zlib.crc32(w.name.encode()))
    dgu = _dev((rng.standard_normal((R_cap, 2 * w.I)) * 0.3).astype(np.float32), bf)
    h = _dev(rng.standard_normal((R_cap, w.I)).astype(np.float32), bf)
    dy = _dev((rng.standard_normal((R_cap, w.H)) * 0.05).astype(np.float32), bf)
    nan = float("nan")
    out = {"dw_gate": torch.full((E_l, w.I, w.H), nan, device=DEV),
           "dw_up": torch.full((E_l, w.I, w.H), nan, device=DEV),
           "dw_down": torch.full((E_l, w.H, w.I), nan, device=DEV)}
    moe.moe_grouped_ffn_wgrad_fp8(x, src_row, dgu, h, dy, offsets, E_l, out=out)
    torch.cuda.synchronize()
    got = {n: _np(t) for n, t in out.items()}
    acc = {n: t.clone() for n, t in out.items()}
    moe.moe_grouped_ffn_wgrad_fp8(x, src_row, dgu, h, dy, offsets, E_l, accumulate=True, out=acc)
    torch.cuda.synchronize()
    acc = {n: _np(t) for n, t in acc.items()}
    rows = {"x": _np(x)[src_row[:R].cpu().numpy()], "dgu": _np(dgu)[:R], "h": _np(h)[:R],
            "dy": _np(dy)[:R]}
    ref = O.moe_wgrad_fp8(rows["x"], rows["dgu"], rows["h"], rows["dy"], off)
    # magnitude bound: the same recipe on the codes' magnitudes
    cq = {n: O.quantize_group_cols_fp8(v, off) for n, v in rows.items()}
    mag = lambda q: q & np.uint8(0x7F)
    worst = 0.0
    for i in range(E_l):
        n_e = int(off[i + 1] - off[i])
        if n_e == 0:
            for n in got:
                assert not got[n][i].any(), f"{n}: expert {i} without rows is not zero"
            continue
        gu_abs = O.fp8_matmul_rows(mag(cq["dgu"][0][i]), cq["dgu"][1][i], mag(cq["x"][0][i]), cq["x"][1][i])
        dn_abs = O.fp8_matmul_rows(mag(cq["dy"][0][i]), cq["dy"][1][i], mag(cq["h"][0][i]), cq["h"][1][i])
        for n, r, a in (("dw_gate", ref["dw_gate"][i], gu_abs[:w.I]), ("dw_up", ref["dw_up"][i], gu_abs[w.I:]),
                        ("dw_down", ref["dw_down"][i], dn_abs)):
            bound = (F8_SUM_REL + (n_e + 2) * 2.0 ** -24) * a + 2.0 ** -24 * np.abs(r) + 1e-38
            ratio = np.abs(got[n][i] - r) / bound
            worst = max(worst, float(ratio.max()))
            assert (ratio <= 1.0).all(), f"{n} expert {i}: {int((ratio > 1).sum())} beyond the bound"
            # accumulate adds to the previous result.  An expert of at most 1024
            # padded rows is never cut into K chunks: exactly twice it.  A larger
            # one may be (chunk 0 added to the old value, then each partial in
            # chunk order): acc - old is the oracle's sum within the same bound
            # plus one rounding of |acc| + a per addition (at most 8 chunks)
            old = got[n][i].astype(np.float64)
            if ((n_e + 63) // 64) * 64 <= 1024:
                assert (acc[n][i] == 2 * old).all(), f"{n} expert {i}: accumulate is not old + new"
            else:
                tol = bound + 9 * 2.0 ** -24 * (2 * np.abs(old) + a)
                assert (np.abs(acc[n][i] - old - r) <= tol).all(), \
                    f"{n} expert {i}: accumulated result beyond the bound"
    rel_exact = []
    for i in range(E_l):
        sl = slice(off[i], off[i + 1])
        if off[i + 1] == off[i]:
            continue
        ex_gu = rows["dgu"][sl].T @ rows["x"][sl]
        ex_dn = rows["dy"][sl].T @ rows["h"][sl]
        rel_exact.append(max(np.linalg.norm(got["dw_gate"][i] - ex_gu[:w.I]) / np.linalg.norm(ex_gu[:w.I]),
                             np.linalg.norm(got["dw_up"][i] - ex_gu[w.I:]) / np.linalg.norm(ex_gu[w.I:]),
                             np.linalg.norm(got["dw_down"][i] - ex_dn) / np.linalg.norm(ex_dn)))
    print(f"  R={R}: worst |d| / bound {worst:.3f}; vs exact rel-L2 max {max(rel_exact):.3e}", flush=True)
    assert max(rel_exact) < 0.10


@pytest.mark.parametrize("acc", [False, True], ids=["overwrite", "accumulate"])
@pytest.mark.parametrize("w", [WGRAD_CASES[3], WGRAD_CASES[4]], ids=lambda w: w.name)
def test_ffn_wgrad_fp8_halves_equal_the_whole(w, acc):
    """moe_grouped_ffn_wgrad_fp8_begin on one stream, then _end on another stream
    ordered after it by an event (begin started before dgu is written, as the layer
    runs it), equals moe_grouped_ffn_wgrad_fp8 bit for bit, overwriting and
    accumulating into the same prior values; one case splits hot experts into K
    chunks (dW_down is complete only after end)."""
    inp = make_inputs(w)
    _, idx, _ = O.route(inp["x"], inp["w_router"], w.k, inp.get("bias"))
    print(f"  case {w.name} accumulate={acc}", flush=True)
    bf = torch.bfloat16
    x = _dev(inp["x"], bf)
    perm = moe.moe_permute(x, torch.from_numpy(idx.astype(np.int32)).to(DEV), w.E, w.e_lo, w.e_hi)
    offsets, src_row = perm["offsets"], perm["src_row"]
    R_cap, E_l = w.T * w.k, w.e_hi - w.e_lo
    rng = np.random.default_rng(zlib.crc32(w.name.encode()) + 1)
    dgu_src = _dev((rng.standard_normal((R_cap, 2 * w.I)) * 0.3).astype(np.float32), bf)
    h = _dev(rng.standard_normal((R_cap, w.I)).astype(np.float32), bf)
    dy = _dev((rng.standard_normal((R_cap, w.H)) * 0.05).astype(np.float32), bf)
    prior = {"dw_gate": torch.randn((E_l, w.I, w.H), device=DEV),
             "dw_up": torch.randn((E_l, w.I, w.H), device=DEV),
             "dw_down": torch.randn((E_l, w.H, w.I), device=DEV)}
    whole = {n: t.clone() for n, t in prior.items()}
    moe.moe_grouped_ffn_wgrad_fp8(x, src_row, dgu_src, h, dy, offsets, E_l, accumulate=acc, out=whole)
    torch.cuda.synchronize()
    halves = {n: t.clone() for n, t in prior.items()}
    nb = moe.lib.moe_workspace_bytes(moe.MOE_OP_FFN_WGRAD_FP8, R_cap, w.H, w.I, E_l, 1, 0, E_l,
                                     moe.MOE_BF16)
    ws = torch.full((int(nb),), 0x5A, dtype=torch.uint8, device=DEV)  # stale bytes
    dgu = torch.full_like(dgu_src, float("nan"))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    moe.moe_grouped_ffn_wgrad_fp8_begin(x, src_row, h, dy, offsets, E_l, ws, halves["dw_down"],
                                        accumulate=acc, stream=s1)
    # dgu written on the current stream while begin runs on s1
    dgu.copy_(dgu_src)
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream())
    done = torch.cuda.Event()
    done.record(s1)
    s2.wait_event(ready)
    s2.wait_event(done)
    moe.moe_grouped_ffn_wgrad_fp8_end(dgu, offsets, E_l, w.H, ws, halves, accumulate=acc, stream=s2)
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    for n in whole:
        assert torch.equal(halves[n], whole[n]), f"{n}: halves differ from the whole call"


# ----------------------------------------------------------------------------
# the layer with fp8=True
# ----------------------------------------------------------------------------

LAYER_FP8_CASES = [
    TRAIN.scaled(name="layer_fp8_t512_h256_i128_e32_k4_local4to20", T=512, H=256, I=128, E=32, k=4,
                 e_lo=4, e_hi=20),
    TRAIN.scaled(name="layer_fp8_t2048_h2048_i768_e128_k8_local0to16", T=2048),
]


def test_layer_fp8_inference_equals_the_training_forward():
    """MoELayer(fp8=True, train=False) (no backward buffers; the weight codes of one
    layout, still quantized on the layer's second stream beside routing) gives the
    training layer's forward bit for bit, on two calls in a row with different
    weights (the second call must wait for its own weight codes)."""
    w = LAYER_FP8_CASES[0]
    inp = make_inputs(w)
    bf = torch.bfloat16
    t = {n: _dev(inp[n], bf) for n in ("x", "w_router", "w_gate", "w_up", "w_down")}
    inf = moe.MoELayer(w.T, w.H, w.I, w.E, w.k, w.e_lo, w.e_hi, bf, DEV, train=False, fp8=True)
    tr = moe.MoELayer(w.T, w.H, w.I, w.E, w.k, w.e_lo, w.e_hi, bf, DEV, train=True, fp8=True)
    for scale in (1.0, 0.5):
        ws = {n: (t[n] * scale).contiguous() for n in ("w_gate", "w_up", "w_down")}
        args = (t["x"], t["w_router"], ws["w_gate"], ws["w_up"], ws["w_down"])
        y_inf = inf.forward(*args).clone()
        y_tr = tr.forward(*args).clone()
        torch.cuda.synchronize()
        assert torch.equal(y_inf, y_tr), f"weights x{scale}: inference forward differs"


@pytest.mark.parametrize("w", LAYER_FP8_CASES, ids=lambda w: w.name)
def test_layer_fp8_is_the_call_chain_and_tracks_the_exact_layer(w):
    """MoELayer(fp8=True): forward and backward equal, bit for bit, the FP8 calls
    chained by hand (every call is checked against the oracle's FP8 recipe above),
    and stay within the recipe's quantization error of the exact layer (oracle,
    fp64): each quantized operand carries a relative rounding error of at most
    2^-4, so y stays under the forward pin's 0.12 rel-L2, and the gradients,
    which chain through more quantized operands (dy, dh, [dg | du] and the
    forward's g, u, h), under 0.2."""
    inp = make_inputs(w)
    bf = torch.bfloat16
    print(f"  case {w.name}", flush=True)
    t = {n: _dev(inp[n], bf) for n in ("x", "w_router", "w_gate", "w_up", "w_down", "dy")}
    layer = moe.MoELayer(w.T, w.H, w.I, w.E, w.k, w.e_lo, w.e_hi, bf, DEV, train=True, fp8=True)
    args = (t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"])
    y = layer.forward(*args).clone()
    g = {n: v.clone() for n, v in layer.backward(t["dy"], *args).items()}
    torch.cuda.synchronize()
    # the same chain, call by call
    E_l = w.E_l
    idx, tw, _ = moe.moe_route(t["x"], t["w_router"], w.k)
    xq, sx = moe.moe_quantize_fp8(t["x"])
    perm = moe.moe_permute(xq, idx, w.E, w.e_lo, w.e_hi)
    wq = {}
    for n in ("w_gate", "w_up", "w_down"):
        El, N, K = t[n].shape
        q, s = moe.moe_quantize_fp8(t[n].view(El * N, K))
        wq[n] = (q.view(El, N, K), s.view(El, N))
    f = moe.moe_grouped_ffn_fwd_fp8(perm["x_perm"], sx, perm["src_row"], perm["offsets"], wq["w_gate"],
                                    wq["w_up"], wq["w_down"], save_gu=True)
    y2 = moe.moe_combine(f["y_perm"], tw, perm["dest_row"], w.T)
    cb = moe.moe_combine_bwd(t["dy"], f["y_perm"], tw, perm["dest_row"])
    dyq, sdy = moe.moe_quantize_fp8(cb["dy_perm"], nrows=perm["offsets"][E_l:])
    d = moe.moe_grouped_ffn_dgrad_fp8(dyq, sdy, f["gu"], perm["offsets"], moe.moe_quantize_fp8_t(t["w_down"]),
                                      moe.moe_quantize_fp8_t(t["w_gate"], t["w_up"]))
    wgr = moe.moe_grouped_ffn_wgrad_fp8(t["x"], perm["src_row"], d["dgu"], f["h_perm"], cb["dy_perm"],
                                        perm["offsets"], E_l)
    dx2 = moe.moe_combine_dx_t(d["dx_perm"], perm["dest_row"], cb["d_topk_w"], tw, idx,
                               moe.moe_router_weight_t(t["w_router"]))
    rb = moe.moe_route_bwd(cb["d_topk_w"], tw, idx, t["x"], t["w_router"], want_dx=False)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.equal(g["dx"], dx2)
    assert torch.equal(g["d_topk_w"], cb["d_topk_w"])
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert torch.equal(g[n], wgr[n]), n
    assert torch.equal(g["d_logits"], rb["d_logits"]) and torch.equal(g["dw_router"], rb["dw_router"])
    # against the exact layer
    _, idx_o, gw = O.route(inp["x"], inp["w_router"], w.k)
    ref_y = O.moe_forward(inp["x"], idx_o, gw, inp["w_gate"], inp["w_up"], inp["w_down"], w.e_lo, w.e_hi)
    ref = O.moe_backward(inp["x"], inp["w_router"], idx_o, gw, inp["w_gate"], inp["w_up"], inp["w_down"],
                         inp["dy"], w.e_lo, w.e_hi)
    rel = lambda a, b: float(np.linalg.norm(_np(a) - b) / max(np.linalg.norm(b), 1e-30))
    r = {"y": rel(y, ref_y), "dx": rel(g["dx"], ref["dx"]), "dw_gate": rel(g["dw_gate"], ref["dw_gate"]),
         "dw_up": rel(g["dw_up"], ref["dw_up"]), "dw_down": rel(g["dw_down"], ref["dw_down"]),
         "d_logits": rel(g["d_logits"], ref["d_logits"]), "dw_router": rel(g["dw_router"], ref["dw_router"])}
    print("  rel-L2 vs the exact layer: " + ", ".join(f"{n} {v:.3e}" for n, v in r.items()), flush=True)
    assert r["y"] < 0.12
    assert all(v < 0.2 for n, v in r.items() if n != "y")
    # the forward-only FP8 layer (no per-input-channel weight codes) gives the same y
    inf = moe.MoELayer(w.T, w.H, w.I, w.E, w.k, w.e_lo, w.e_hi, bf, DEV, train=False, fp8=True)
    y_inf = inf.forward(*args)
    torch.cuda.synchronize()
    assert torch.equal(y_inf, y)
