"""Pins of the CPU oracle against things other than itself.

Each check compares the oracle with a closed form (hand-derived golden
fixtures), a brute force on tiny inputs, an invariant, a special case that
reduces to a textbook or library routine, or an independent float64 autograd
computation.  The mutation tests at the end plant plausible mistakes in the
oracle (on the CPU) and require at least one check to fail for each.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from oracle import moe_oracle as OM
from workloads import TINY, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def _tiny(**kw):
    w = TINY.scaled(**kw)
    return w, make_inputs(w)


def _eval_expr(s):
    """Evaluate a fixture expression over L = ln 3 (no names besides L)."""
    return float(eval(s, {"__builtins__": {}}, {"L": math.log(3.0)}))


def _read_gating_golden():
    cases = []
    with open(os.path.join(GOLDEN, "gating_closed_form.txt")) as f:
        for line in f:
            if not line.startswith("case "):
                continue
            name, k, cs, ids, ws = [p.strip() for p in line[5:].split("|")]
            cases.append((name, int(k), [int(c) for c in cs.split()], [int(i) for i in ids.split()],
                          [Fraction(w) for w in ws.split()]))
    return cases


def _read_scalar_golden():
    vals, expect = {}, {}
    with open(os.path.join(GOLDEN, "scalar_layer_closed_form.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = [p.strip() for p in line.split("=", 1)]
            nums = [_eval_expr(p) for p in rhs.split(",")]
            if lhs.startswith("expect "):
                expect[lhs[7:].strip()] = np.array(nums)
            else:
                vals[lhs] = np.array(nums)
    return vals, expect


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ----------------------------------------------------------------------------
# checks (raise AssertionError on failure; reused by the mutation tests)
# ----------------------------------------------------------------------------

def check_gating_golden():
    for name, k, cs, ids, ws in _read_gating_golden():
        z = np.log(np.array([cs], dtype=np.float64))
        idx = O.topk_experts(z, k)
        assert idx[0].tolist() == ids, (name, idx[0].tolist(), ids)
        w = O.gate_weights(z, idx)[0]
        np.testing.assert_allclose(w, [float(x) for x in ws], rtol=1e-14, atol=0, err_msg=name)


def check_topk_brute_force():
    """Unique k-subset S with every member ahead of every non-member in the
    order (logit desc, id asc); slots ordered within S by pairwise dominance."""
    rng = np.random.default_rng(7)
    for trial in range(60):
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, E + 1))
        z = rng.integers(-2, 3, size=(3, E)).astype(np.float64)  # many exact ties
        idx = O.topk_experts(z, k)
        for t in range(z.shape[0]):
            def ahead(a, b):
                return z[t, a] > z[t, b] or (z[t, a] == z[t, b] and a < b)
            good = [S for S in itertools.combinations(range(E), k)
                    if all(ahead(s, o) for s in S for o in range(E) if o not in S)]
            assert len(good) == 1
            S = list(good[0])
            # position of s = number of members ahead of it
            ordered = sorted(S, key=lambda s: sum(ahead(o, s) for o in S))
            assert idx[t].tolist() == ordered, (z[t], k, idx[t], ordered)


def check_zero_input_routing():
    w, inp = _tiny()
    x = np.zeros_like(inp["x"])
    z, idx, g = O.route(x, inp["w_router"], w.k)
    assert (idx == np.arange(w.k)[None, :]).all()
    assert (g == 1.0 / w.k).all()


def check_duplicate_router_columns():
    w, inp = _tiny(k=3)
    wr = inp["w_router"].copy()
    wr[:, 5] = wr[:, 2]
    wr[:, 7] = wr[:, 2]
    z, idx, g = O.route(inp["x"], wr, w.k)
    for t in range(w.T):
        s = idx[t].tolist()
        for dup in (5, 7):
            if dup in s:
                assert 2 in s and s.index(2) < s.index(dup)


def check_k1_and_kE():
    w, inp = _tiny()
    z = O.router_logits(inp["x"], inp["w_router"])
    _, idx1, g1 = O.route(inp["x"], inp["w_router"], 1)
    assert (g1 == 1.0).all()
    assert (idx1[:, 0] == np.argmax(z, axis=1)).all()
    _, idxE, gE = O.route(inp["x"], inp["w_router"], w.E)
    ref = scipy.special.softmax(z, axis=1)
    np.testing.assert_allclose(gE, np.take_along_axis(ref, idxE.astype(np.int64), 1), rtol=1e-13)


def check_weights_sum_to_one():
    w, inp = _tiny(k=3)
    _, _, g = O.route(inp["x"], inp["w_router"], w.k)
    assert np.abs(g.sum(1) - 1).max() < 1e-14
    assert (g > 0).all()


def check_counts_offsets():
    for (k, e_lo, e_hi) in ((2, 0, 8), (3, 2, 6), (1, 7, 8)):
        w, inp = _tiny(k=k, e_lo=e_lo, e_hi=e_hi, E=8)
        _, idx, _ = O.route(inp["x"], inp["w_router"], k)
        c = O.expert_counts(idx, e_lo, e_hi)
        bc = np.bincount(idx.ravel(), minlength=8)[e_lo:e_hi]
        assert (c == bc).all()
        off = O.expert_offsets(c)
        assert off[0] == 0 and (np.diff(off) >= 0).all()
        nloc = int(((idx >= e_lo) & (idx < e_hi)).sum())
        assert off[-1] == nloc
        if (e_lo, e_hi) == (0, 8):
            assert off[-1] == w.T * k


def check_permutation_maps():
    for (k, e_lo, e_hi) in ((2, 0, 8), (3, 2, 6), (1, 0, 8)):
        w, inp = _tiny(k=k, e_lo=e_lo, e_hi=e_hi)
        _, idx, _ = O.route(inp["x"], inp["w_router"], k)
        dest, src = O.permutation_maps(idx, e_lo, e_hi)
        off = O.expert_offsets(O.expert_counts(idx, e_lo, e_hi))
        R = int(off[-1])
        flat = idx.ravel()
        local = (flat >= e_lo) & (flat < e_hi)
        assert (dest[~local] == -1).all()
        assert sorted(dest[local].tolist()) == list(range(R))          # bijection onto [0, R)
        assert (src[dest[local]] == np.nonzero(local)[0] // k).all()    # inverse map
        for e in range(e_hi - e_lo):                                   # tokens ascending per group
            seg = src[off[e]:off[e + 1]]
            assert (np.diff(seg) > 0).all()
        # independent construction: stable argsort of slots by expert id
        slots = np.nonzero(local)[0]
        order = slots[np.argsort(flat[slots], kind="stable")]
        assert (dest[order] == np.arange(R)).all()


def check_permute_unpermute_identity():
    w, inp = _tiny()
    _, idx, _ = O.route(inp["x"], inp["w_router"], w.k)
    dest, src = O.permutation_maps(idx, 0, w.E)
    xp = O.permute_rows(inp["x"], dest, len(src))
    back = O.unpermute_rows(xp, dest, w.T)
    assert (back == w.k * inp["x"].astype(np.float64)).all()
    w1, inp1 = _tiny(k=1)
    _, idx1, _ = O.route(inp1["x"], inp1["w_router"], 1)
    d1, s1 = O.permutation_maps(idx1, 0, w1.E)
    assert (O.unpermute_rows(O.permute_rows(inp1["x"], d1, len(s1)), d1, w1.T) == inp1["x"]).all()


def _dense_masked(x, idx, gw, wg, wu, wd, e_lo, e_hi):
    """Every local expert on every token, then a dense [T, E_l] gate mask."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    M = np.zeros((T, e_hi - e_lo))
    for t in range(T):
        for j in range(idx.shape[1]):
            if e_lo <= idx[t, j] < e_hi:
                M[t, idx[t, j] - e_lo] = gw[t, j]
    y = np.zeros_like(x)
    for e in range(e_hi - e_lo):
        g = x @ np.asarray(wg[e], np.float64).T
        u = x @ np.asarray(wu[e], np.float64).T
        h = g / (1.0 + np.exp(-g)) * u
        y += M[:, e:e + 1] * (h @ np.asarray(wd[e], np.float64).T)
    return y


def check_dense_equals_routed():
    for (k, e_lo, e_hi) in ((2, 0, 8), (3, 2, 5)):
        w, inp = _tiny(k=k, e_lo=e_lo, e_hi=e_hi)
        _, idx, gw = O.route(inp["x"], inp["w_router"], k)
        y = O.moe_forward(inp["x"], idx, gw, inp["w_gate"], inp["w_up"], inp["w_down"], e_lo, e_hi)
        yd = _dense_masked(inp["x"], idx, gw, inp["w_gate"], inp["w_up"], inp["w_down"], e_lo, e_hi)
        assert _rel(y, yd) < 1e-12
        yp = O.moe_forward_pairs(inp["x"][:32], idx[:32], gw[:32], inp["w_gate"], inp["w_up"],
                                 inp["w_down"], e_lo, e_hi)
        assert _rel(yp, y[:32]) < 1e-12


def check_single_expert_is_swiglu_mlp():
    w, inp = _tiny(E=1, k=1, e_lo=0, e_hi=1)
    _, idx, gw = O.route(inp["x"], inp["w_router"], 1)
    y = O.moe_forward(inp["x"], idx, gw, inp["w_gate"], inp["w_up"], inp["w_down"], 0, 1)
    xt = torch.tensor(inp["x"], dtype=torch.float64)
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(xt, torch.tensor(inp["w_gate"][0], dtype=torch.float64)))
        * torch.nn.functional.linear(xt, torch.tensor(inp["w_up"][0], dtype=torch.float64)),
        torch.tensor(inp["w_down"][0], dtype=torch.float64))
    assert _rel(y, ref.numpy()) < 1e-13


def check_zero_projection_gives_zero():
    w, inp = _tiny()
    _, idx, gw = O.route(inp["x"], inp["w_router"], w.k)
    for key in ("w_up", "w_gate"):
        ww = dict(inp)
        ww[key] = np.zeros_like(inp[key])
        y = O.moe_forward(inp["x"], idx, gw, ww["w_gate"], ww["w_up"], ww["w_down"], 0, w.E)
        assert (y == 0).all()


def check_scalar_golden():
    v, ex = _read_scalar_golden()
    x = v["x"].reshape(1, 1)
    wr = v["w_router"].reshape(1, 2)
    wg = v["w_gate"].reshape(2, 1, 1)
    wu = v["w_up"].reshape(2, 1, 1)
    wd = v["w_down"].reshape(2, 1, 1)
    dy = v["dy"].reshape(1, 1)
    k = int(v["k"][0])
    z, idx, gw = O.route(x, wr, k)
    assert idx[0].tolist() == [int(i) for i in ex["idx"]]
    np.testing.assert_allclose(gw[0], ex["w"], rtol=1e-14)
    y = O.moe_forward(x, idx, gw, wg, wu, wd, 0, 2)
    np.testing.assert_allclose(y.ravel(), ex["y"], rtol=1e-13)
    gr = O.moe_backward(x, wr, idx, gw, wg, wu, wd, dy, 0, 2)
    np.testing.assert_allclose(gr["dw"][0], ex["dw"], rtol=1e-13)
    np.testing.assert_allclose(gr["d_logits"][0], ex["d_logits"], rtol=1e-13)
    np.testing.assert_allclose(gr["dw_router"][0], ex["dw_router"], rtol=1e-13)
    np.testing.assert_allclose(gr["dw_down"].ravel(), ex["dw_down"], rtol=1e-13)
    np.testing.assert_allclose(gr["dw_gate"].ravel(), ex["dw_gate"], rtol=1e-13)
    np.testing.assert_allclose(gr["dw_up"].ravel(), ex["dw_up"], rtol=1e-13)
    np.testing.assert_allclose(gr["dx"].ravel(), ex["dx"], rtol=1e-13)


def _torch_forward(x, wr, wg, wu, wd, idx, e_lo, e_hi):
    """Independent float64 torch forward (dense-masked form) for autograd."""
    z = x @ wr
    p = torch.softmax(z, dim=-1)
    psel = p.gather(1, idx)
    gw = psel / psel.sum(1, keepdim=True)
    T = x.shape[0]
    y = torch.zeros_like(x)
    for e in range(e_lo, e_hi):
        m = (idx == e).to(x.dtype)                      # [T, k]
        coef = (gw * m).sum(1, keepdim=True)            # weight of expert e per token
        out = torch.nn.functional.linear(
            torch.nn.functional.silu(torch.nn.functional.linear(x, wg[e - e_lo]))
            * torch.nn.functional.linear(x, wu[e - e_lo]), wd[e - e_lo])
        y = y + coef * out
    return z, gw, y


def check_backward_vs_autograd():
    for (k, e_lo, e_hi) in ((2, 0, 8), (3, 1, 6)):
        w, inp = _tiny(k=k, e_lo=e_lo, e_hi=e_hi, T=96)
        rng = np.random.default_rng(3)
        dy = rng.standard_normal((w.T, w.H))
        _, idx, gw = O.route(inp["x"], inp["w_router"], k)
        gr = O.moe_backward(inp["x"], inp["w_router"], idx, gw, inp["w_gate"], inp["w_up"],
                            inp["w_down"], dy, e_lo, e_hi)
        t = {n: torch.tensor(inp[n], dtype=torch.float64, requires_grad=True)
             for n in ("x", "w_router", "w_gate", "w_up", "w_down")}
        z, g, y = _torch_forward(t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"],
                                 torch.tensor(idx, dtype=torch.int64), e_lo, e_hi)
        z.retain_grad()
        g.retain_grad()
        (y * torch.tensor(dy)).sum().backward()
        assert _rel(gr["dx"], t["x"].grad.numpy()) < 1e-11
        assert _rel(gr["dw_router"], t["w_router"].grad.numpy()) < 1e-11
        assert _rel(gr["dw_gate"], t["w_gate"].grad.numpy()) < 1e-11
        assert _rel(gr["dw_up"], t["w_up"].grad.numpy()) < 1e-11
        assert _rel(gr["dw_down"], t["w_down"].grad.numpy()) < 1e-11
        assert _rel(gr["d_logits"], z.grad.numpy()) < 1e-11
        assert _rel(gr["dw"], g.grad.numpy()) < 1e-11
        assert np.abs(gr["d_logits"].sum(1)).max() < 1e-12       # softmax Jacobian rows sum to 0
        off = np.ones_like(gr["d_logits"], dtype=bool)
        np.put_along_axis(off, idx.astype(np.int64), False, axis=1)
        assert (gr["d_logits"][off] == 0).all()
        nonlocal_ = (idx < e_lo) | (idx >= e_hi)
        assert (gr["dw"][nonlocal_] == 0).all()


def check_finite_differences():
    w, inp = _tiny(T=12, k=2)
    rng = np.random.default_rng(11)
    dy = rng.standard_normal((w.T, w.H))
    z, idx, gw = O.route(inp["x"], inp["w_router"], w.k)
    srt = np.sort(z, axis=1)[:, ::-1]
    assert (srt[:, w.k - 1] - srt[:, w.k] > 1e-3).all()  # routing is stable under the step
    gr = O.moe_backward(inp["x"], inp["w_router"], idx, gw, inp["w_gate"], inp["w_up"],
                        inp["w_down"], dy, 0, w.E)

    def loss(**over):
        p = {n: np.asarray(inp[n], np.float64) for n in ("x", "w_router", "w_gate", "w_up", "w_down")}
        p.update(over)
        zz, ii, gg = O.route(p["x"], p["w_router"], w.k)
        assert (ii == idx).all()
        return float((O.moe_forward(p["x"], ii, gg, p["w_gate"], p["w_up"], p["w_down"], 0, w.E) * dy).sum())

    h = 1e-6
    for name, gname, pos in (("x", "dx", (3, 5)), ("x", "dx", (7, 60)), ("w_router", "dw_router", (10, 4)),
                             ("w_gate", "dw_gate", (int(idx[0, 0]), 2, 9)),
                             ("w_up", "dw_up", (int(idx[1, 0]), 30, 1)),
                             ("w_down", "dw_down", (int(idx[2, 1]), 40, 7))):
        base = np.asarray(inp[name], np.float64)
        p1, m1 = base.copy(), base.copy()
        p1[pos] += h
        m1[pos] -= h
        fd = (loss(**{name: p1}) - loss(**{name: m1})) / (2 * h)
        an = gr[gname][pos]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, pos, fd, an)


def check_router_grads_vs_autograd():
    """router_logit_grad against autograd of sum(dw * softmax(z[idx])) (rows with a
    repeated expert included: that logit is read twice), and router_input_grad
    against autograd of sum(dz * (x . W_r)) with respect to x."""
    rng = np.random.default_rng(21)
    T, E, k, H = 6, 9, 3, 5
    idx = np.array([[4, 1, 7], [2, 2, 5], [0, 8, 0], [3, 6, 1], [5, 5, 5], [8, 7, 6]])
    z = torch.tensor(rng.standard_normal((T, E)), requires_grad=True)
    dw = rng.standard_normal((T, k))
    w = torch.softmax(z.gather(1, torch.tensor(idx)), dim=1)
    (w * torch.tensor(dw)).sum().backward()
    got = O.router_logit_grad(w.detach().numpy(), dw, idx, E)
    assert _rel(got, z.grad.numpy()) < 1e-13
    x = torch.tensor(rng.standard_normal((T, H)), requires_grad=True)
    wr = rng.standard_normal((H, E))
    (torch.tensor(got) * (x @ torch.tensor(wr))).sum().backward()
    assert _rel(O.router_input_grad(got, wr), x.grad.numpy()) < 1e-13


def check_fp8_codes_vs_torch():
    """E4M3 decode of all 256 codes and encode of random values, every code's value
    and every midpoint between neighbours, against torch's float8_e4m3fn."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    dec = O.fp8_e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(dec))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], dec[ok])
    assert dec[0x7E] == 448.0 and dec[0x01] == 2.0 ** -9 and dec[0x08] == 2.0 ** -6
    vals = np.sort(dec[ok & (dec >= 0)])
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-0.03, 0.03, 4000), vals, -vals,
                        (vals[:-1] + vals[1:]) / 2, -(vals[:-1] + vals[1:]) / 2])
    v = v.astype(np.float32).astype(np.float64)
    got = O.fp8_e4m3_encode(v)
    exp = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, exp)


def check_fp8_row_scale_is_minimal():
    """Per-row exponent: amax <= 448 * 2^e and amax > 448 * 2^(e - 1) (brute force over
    values at, just below and just above the boundaries); zero rows get e = 0."""
    rng = np.random.default_rng(6)
    b = 448.0 * np.exp2(np.arange(-30, 30, dtype=np.float64))
    amax = np.concatenate([b, np.nextafter(b, 0), np.nextafter(b, np.inf), rng.uniform(1e-6, 1e6, 500)])
    e = O.fp8_row_exponent(amax)
    assert np.all(amax <= 448.0 * np.exp2(e.astype(np.float64)))
    assert np.all(amax > 448.0 * np.exp2(e.astype(np.float64) - 1))
    assert O.fp8_row_exponent(np.array([0.0]))[0] == 0
    a = rng.standard_normal((7, 33)) * np.exp2(rng.integers(-20, 20, size=(7, 1)))
    a[3] = 0.0
    q, sc = O.quantize_rows_fp8(a)
    back = O.fp8_e4m3_decode(q) * sc[:, None]
    # each value within half a step of its binade (relative 2^-4 for normals)
    assert np.all(np.abs(back - a) <= np.maximum(2.0 ** -4 * np.abs(a), sc[:, None] * 2.0 ** -10))
    assert np.all(np.abs(O.fp8_e4m3_decode(q)).max(axis=1)[[0, 1, 2, 4, 5, 6]] >= 224.0)
    assert (q[3] == 0).all() and sc[3] == 1.0


def check_fp8_matmul_brute_force():
    """fp8_matmul_rows against a per-element loop over decoded codes, with distinct
    row and column scales (catches a scale on the wrong axis)."""
    rng = np.random.default_rng(7)
    aq = rng.integers(0, 256, size=(5, 9)).astype(np.uint8)
    bq = rng.integers(0, 256, size=(4, 9)).astype(np.uint8)
    aq[(aq & 0x7F) == 0x7F] = 0x3C
    bq[(bq & 0x7F) == 0x7F] = 0x41
    sa = np.exp2(rng.integers(-5, 5, size=5).astype(np.float64))
    sb = np.exp2(rng.integers(-5, 5, size=4).astype(np.float64))
    got = O.fp8_matmul_rows(aq, sa, bq, sb)
    da, db = O.fp8_e4m3_decode(aq), O.fp8_e4m3_decode(bq)
    for r in range(5):
        for n in range(4):
            ref = sum(da[r, k] * db[n, k] for k in range(9)) * sa[r] * sb[n]
            assert abs(got[r, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def check_fp8_forward_close_to_exact():
    """The FP8 forward stays near the exact forward: four quantized operands (x, the
    gate / up weights, h, the down weights), each rounded within 2^-4 relative, give
    a rel-L2 well under 12% (an unapplied scale or a dropped factor lands far
    outside).  And on operands that lie on the E4M3 grid with row maximum 448 (scale
    1), the quantized gate / up products equal the plain fp64 ones exactly."""
    w, inp = _tiny(T=64, k=2)
    z, idx, gw = O.route(inp["x"], inp["w_router"], w.k)
    ref = O.moe_forward(inp["x"], idx, gw, inp["w_gate"], inp["w_up"], inp["w_down"], 0, w.E)
    got = O.moe_forward_fp8(inp["x"], idx, gw, inp["w_gate"], inp["w_up"], inp["w_down"], 0, w.E)
    assert _rel(got, ref) < 0.12
    rng = np.random.default_rng(8)
    grid = O.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    pick = lambda *sh: rng.choice(np.concatenate([grid, -grid]), size=sh)
    x, wg, wu, wd = pick(6, 16), pick(1, 8, 16), pick(1, 8, 16), pick(1, 16, 8)
    for a in (x, wg[0], wu[0], wd[0]):
        a[:, 0] = 448.0
    xq, sx = O.quantize_rows_fp8(x)
    assert (sx == 1.0).all()
    qg, sg = O.quantize_expert_weights_fp8(wg)
    qu, su = O.quantize_expert_weights_fp8(wu)
    qd, sd = O.quantize_expert_weights_fp8(wd)
    parts = O.expert_ffn_fp8_parts(xq, sx, qg[0], sg[0], qu[0], su[0], qd[0], sd[0])
    exact = O.expert_ffn_parts(x, wg[0], wu[0], wd[0])
    assert np.array_equal(parts["g"], exact["g"]) and np.array_equal(parts["u"], exact["u"])


def check_fp8_weight_t_scales_per_input_channel():
    """The transposed weight quantization scales each input channel (a column of
    the stored [N, K] weight, over N; for gate / up over both matrices) by the
    smallest power of two that brings its maximum to <= 448, and its codes
    decode to that column within the E4M3 step."""
    rng = np.random.default_rng(9)
    w0 = rng.standard_normal((2, 12, 10)) * np.exp2(rng.integers(-12, 12, size=(2, 1, 10)))
    w1 = rng.standard_normal((2, 12, 10)) * np.exp2(rng.integers(-12, 12, size=(2, 1, 10)))
    for q, sc, cols in ((*O.quantize_expert_weights_t_fp8(w0), np.abs(w0).max(axis=1)),
                        (*O.quantize_expert_weights_t_fp8(w0, w1),
                         np.maximum(np.abs(w0).max(axis=1), np.abs(w1).max(axis=1)))):
        assert q.shape[:2] == (2, 10) and sc.shape == (2, 10)
        assert np.all(cols <= 448.0 * sc) and np.all(cols > 224.0 * sc)
    q, sc = O.quantize_expert_weights_t_fp8(w0, w1)
    back = O.fp8_e4m3_decode(q) * sc[:, :, None]
    ref = np.concatenate([w0.transpose(0, 2, 1), w1.transpose(0, 2, 1)], axis=2)
    assert np.all(np.abs(back - ref) <= np.maximum(2.0 ** -4 * np.abs(ref), sc[:, :, None] * 2.0 ** -10))


def check_fp8_dgrad_close_to_exact():
    """The FP8 data gradients of one expert stay near the exact ones (five
    quantized operands, each within 2^-4 relative: rel-L2 under 12%; a swapped
    gate / up order or a dropped scale lands far outside).  On dy and W_down on
    the E4M3 grid with every quantized row's maximum 448 (scale 1), dh is the
    bf16 of the exact product."""
    rng = np.random.default_rng(10)
    n, H, I = 24, 64, 32
    x = rng.standard_normal((n, H))
    wg, wu = rng.standard_normal((1, I, H)) / 8, rng.standard_normal((1, I, H)) / 8
    wd = rng.standard_normal((1, H, I)) / 6
    dy = rng.standard_normal((n, H))
    g, u = x @ wg[0].T, x @ wu[0].T
    dg, du = O.swiglu_grad(dy @ wd[0], g, u)
    exact = dg @ wg[0] + du @ wu[0]
    dyq, sdy = O.quantize_rows_fp8(dy)
    qd, sd = O.quantize_expert_weights_t_fp8(wd)
    qgu, sgu = O.quantize_expert_weights_t_fp8(wg, wu)
    p = O.expert_dgrad_fp8_parts(dyq, sdy, g, u, qd[0], sd[0], qgu[0], sgu[0])
    assert _rel(p["dx"], exact) < 0.12
    assert np.array_equal(p["dgu"], O.round_bf16(p["dgu"]))
    grid = O.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    pick = lambda *sh: rng.choice(np.concatenate([grid, -grid]), size=sh)
    dy2, wd2 = pick(5, 16), pick(1, 16, 8)
    dy2[:, 0] = 448.0
    wd2[0, 0, :] = 448.0          # every input channel (column) reaches 448
    dyq2, sdy2 = O.quantize_rows_fp8(dy2)
    qd2, sd2 = O.quantize_expert_weights_t_fp8(wd2)
    assert (sdy2 == 1.0).all() and (sd2 == 1.0).all()
    p2 = O.expert_dgrad_fp8_parts(dyq2, sdy2, np.zeros((5, 8)), np.zeros((5, 8)), qd2[0], sd2[0],
                                  np.zeros((16, 16), np.uint8), np.ones(16))
    assert np.array_equal(p2["dh"], O.round_bf16(dy2 @ wd2[0]))


def check_round_bf16_vs_torch():
    """round_bf16 against torch's float32 -> bfloat16 conversion (round to nearest
    even): random values over the whole exponent range, exact half-way cases with an
    even and with an odd kept mantissa, values at and past the largest finite
    bfloat16, float32 subnormals, and -0.  On float64 inputs the rounding is direct:
    a value just past a half-way point goes up even where float32 would first have
    rounded it onto that point."""
    rng = np.random.default_rng(12)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-140, 128, 20000))).astype(np.float32)
    base = torch.tensor(rng.integers(0, 1 << 16, 4000, dtype=np.int64).astype(np.int16)).view(torch.bfloat16)
    base = base[torch.isfinite(base)].float().numpy().astype(np.float32)
    # half-way points above each base value: the low 16 bits 0x8000 exactly
    half = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    half = half[np.isfinite(half)]
    edge = np.array([3.3895314e38, 3.3961776e38, 3.3961778e38, 3.4e38, -3.4e38, np.finfo(np.float32).max,
                     1e-40, -1e-40, 9.2e-41, 1e-45, 2.0 ** -133, 3 * 2.0 ** -134, 2.0 ** -134,
                     -0.0, 0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 3 * 2 ** -8)], dtype=np.float32)
    for arr in (v, half, edge):
        ref = torch.from_numpy(arr).to(torch.bfloat16).double().numpy()
        got = O.round_bf16(arr.astype(np.float64))
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        assert same.all(), (arr[~same][:4], got[~same][:4], ref[~same][:4])
        assert np.array_equal(np.signbit(got), np.signbit(ref))
    odd_mid = 1.0 + 3 * 2.0 ** -8                 # between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6
    assert O.round_bf16(odd_mid) == 1.0 + 2.0 ** -6
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0   # between 1 and 1 + 2^-7: ties to 1
    just_past = 1.0 + 2.0 ** -8 + 2.0 ** -40      # float32 would round this onto the half-way point
    assert np.float32(just_past) == np.float32(1.0 + 2.0 ** -8)
    assert O.round_bf16(just_past) == 1.0 + 2.0 ** -7


def check_pair_values_rows():
    """pair_values on an EP rank (e_lo != 0): each local slot's g, u, h, y equal a
    per-element loop of the SwiGLU expert written out here (sums over H and I
    in Python), non-local slots are NaN, and the gate-weighted sum of a token's
    local slots is moe_forward's output."""
    w, inp = _tiny(T=12, H=8, I=4, E=6, k=3, e_lo=2, e_hi=5)
    z, idx, gw = O.route(inp["x"], inp["w_router"], w.k)
    pv = O.pair_values(inp["x"], idx, inp["w_gate"], inp["w_up"], inp["w_down"], w.e_lo, w.e_hi)
    x = np.asarray(inp["x"], np.float64)
    nloc = 0
    for t in range(w.T):
        for j in range(w.k):
            e = int(idx[t, j])
            if not w.e_lo <= e < w.e_hi:
                assert all(np.isnan(pv[n][t, j]).all() for n in pv)
                continue
            nloc += 1
            Wg, Wu, Wd = (np.asarray(inp[n][e - w.e_lo], np.float64) for n in ("w_gate", "w_up", "w_down"))
            g = [sum(x[t, h] * Wg[i, h] for h in range(w.H)) for i in range(w.I)]
            u = [sum(x[t, h] * Wu[i, h] for h in range(w.H)) for i in range(w.I)]
            hh = [g[i] / (1.0 + math.exp(-g[i])) * u[i] for i in range(w.I)]
            y = [sum(hh[i] * Wd[m, i] for i in range(w.I)) for m in range(w.H)]
            for n, ref in (("g", g), ("u", u), ("h", hh), ("y", y)):
                assert np.allclose(pv[n][t, j], ref, rtol=1e-12, atol=1e-14), (n, t, j)
    assert 0 < nloc < w.T * w.k
    ysum = np.nansum(pv["y"] * np.asarray(gw)[:, :, None], axis=1)
    ref = O.moe_forward(inp["x"], idx, gw, inp["w_gate"], inp["w_up"], inp["w_down"], w.e_lo, w.e_hi)
    assert np.allclose(ysum, ref, rtol=1e-12, atol=1e-14)
    sub = O.pair_values(inp["x"], idx, inp["w_gate"], inp["w_up"], inp["w_down"], w.e_lo, w.e_hi,
                        tokens=[7, 2])
    for n in pv:
        assert np.allclose(sub[n], pv[n][[7, 2]], rtol=1e-12, atol=1e-14, equal_nan=True)


def check_fp8_group_col_scales_literal():
    """Per-(group, column) scales of a hand-built grouped matrix, worked out by hand
    from the rule "smallest power of two 2^e with max|column of the group| <= 448 * 2^e"
    (e = 0 for an all-zero column or an empty group): group 0 (rows 0-1) has column
    maxima 448, 449, 0 -> scales 1, 2, 1; group 1 is empty -> 1, 1, 1; group 2 (rows
    2-4) has maxima 0.875 = 448 * 2^-9, 3584 = 448 * 2^3 and 0.001 -> 2^-9, 8, 2^-18.
    Each code decodes, times its scale, to within one E4M3 step of its value."""
    a = np.array([[448.0, -449.0, 0.0],
                  [-3.0, 100.0, 0.0],
                  [0.5, 3584.0, -0.001],
                  [-0.875, 1.0, 0.0005],
                  [0.25, -7.0, 0.0]])
    codes, sc = O.quantize_group_cols_fp8(a, [0, 2, 2, 5])
    want = np.array([[1.0, 2.0, 1.0], [1.0, 1.0, 1.0], [2.0 ** -9, 8.0, 2.0 ** -18]])
    assert sc.shape == (3, 3) and np.array_equal(sc, want)
    assert [c.shape for c in codes] == [(3, 2), (3, 0), (3, 3)]
    for e, (o0, o1) in enumerate(((0, 2), (2, 2), (2, 5))):
        back = O.fp8_e4m3_decode(codes[e]) * sc[e][:, None]
        ref = a[o0:o1].T
        assert np.all(np.abs(back - ref) <= np.maximum(2.0 ** -4 * np.abs(ref), sc[e][:, None] * 2.0 ** -10))


def _grid_cols(rng, grid, rows, cols, offsets):
    """rows x cols values on the E4M3 grid times a power of two per (group, column),
    each (group, column) reaching 448 times its power exactly (codes then exact)"""
    a = rng.choice(np.concatenate([grid, -grid]), size=(rows, cols))
    for e in range(len(offsets) - 1):
        o0, o1 = offsets[e], offsets[e + 1]
        if o1 == o0:
            continue
        p = np.exp2(rng.integers(-4, 4, size=cols).astype(np.float64))
        a[o0:o1] *= p
        a[o0 + rng.integers(0, o1 - o0, size=cols), np.arange(cols)] = 448.0 * p
    return a


def check_fp8_wgrad_exact_on_grid():
    """On operands whose (group, column) slices lie on the E4M3 grid scaled by a power
    of two with maximum 448 times it, every code is exact, so the FP8 weight gradients
    equal the plain per-expert weight gradients (dW_down[e] = dy_e^T h_e, dW_gate[e] =
    dg_e^T x_e, dW_up[e] = du_e^T x_e over the expert's rows) exactly; an expert with
    no rows gets zeros."""
    rng = np.random.default_rng(21)
    grid = O.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    grid = grid[grid >= 2.0 ** -3]           # keep every product and sum exact in float64
    offsets = [0, 5, 5, 13, 16]
    R, H, I = 16, 12, 8
    x = _grid_cols(rng, grid, R, H, offsets)
    dgu = _grid_cols(rng, grid, R, 2 * I, offsets)
    h = _grid_cols(rng, grid, R, I, offsets)
    dy = _grid_cols(rng, grid, R, H, offsets)
    got = O.moe_wgrad_fp8(x, dgu, h, dy, offsets)
    for e in range(4):
        o0, o1 = offsets[e], offsets[e + 1]
        assert np.array_equal(got["dw_down"][e], dy[o0:o1].T @ h[o0:o1])
        assert np.array_equal(got["dw_gate"][e], dgu[o0:o1, :I].T @ x[o0:o1])
        assert np.array_equal(got["dw_up"][e], dgu[o0:o1, I:].T @ x[o0:o1])
    assert not got["dw_down"][1].any() and not got["dw_gate"][1].any()


def check_fp8_wgrad_close_to_exact():
    """Random operands whose experts differ in magnitude by 2^20: each expert's FP8
    weight gradients stay within the two operands' E4M3 rounding (each within 2^-4
    relative: rel-L2 under 10%) of its exact weight gradients.  Scales shared across
    experts would push the small expert's codes into underflow."""
    rng = np.random.default_rng(22)
    offsets = [0, 40, 90]
    R, H, I = 90, 48, 32
    mag = np.ones((R, 1))
    mag[40:] = 2.0 ** 20
    x, dgu = rng.standard_normal((R, H)) * mag, rng.standard_normal((R, 2 * I)) * mag
    h, dy = rng.standard_normal((R, I)) * mag, rng.standard_normal((R, H)) * mag
    got = O.moe_wgrad_fp8(x, dgu, h, dy, offsets)
    for e in range(2):
        o0, o1 = offsets[e], offsets[e + 1]
        assert _rel(got["dw_down"][e], dy[o0:o1].T @ h[o0:o1]) < 0.10
        assert _rel(got["dw_gate"][e], dgu[o0:o1, :I].T @ x[o0:o1]) < 0.10
        assert _rel(got["dw_up"][e], dgu[o0:o1, I:].T @ x[o0:o1]) < 0.10


ALL_CHECKS = [check_gating_golden, check_topk_brute_force, check_zero_input_routing,
              check_duplicate_router_columns, check_k1_and_kE, check_weights_sum_to_one,
              check_counts_offsets, check_permutation_maps, check_permute_unpermute_identity,
              check_dense_equals_routed, check_single_expert_is_swiglu_mlp,
              check_zero_projection_gives_zero, check_scalar_golden, check_backward_vs_autograd,
              check_finite_differences, check_router_grads_vs_autograd, check_fp8_codes_vs_torch,
              check_fp8_row_scale_is_minimal, check_fp8_matmul_brute_force,
              check_fp8_forward_close_to_exact, check_fp8_weight_t_scales_per_input_channel,
              check_fp8_dgrad_close_to_exact, check_round_bf16_vs_torch, check_pair_values_rows,
              check_fp8_group_col_scales_literal, check_fp8_wgrad_exact_on_grid,
              check_fp8_wgrad_close_to_exact]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check()


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------

def _mut_silu_is_sigmoid(a):
    return OM.sigmoid(a)


def _mut_topk_ties_high(z, k):
    z = np.asarray(z, np.float64)
    T, E = z.shape
    ids = np.broadcast_to(-np.arange(E), (T, E))
    return np.lexsort((ids, -z), axis=-1)[:, :k].astype(np.int32)


def _mut_no_renorm(z, idx):
    return np.take_along_axis(OM.softmax(z), np.asarray(idx, np.int64), axis=1)


def _mut_group_tokens_descending(idx, e_lo, e_hi):
    dest, src = _ORIG["permutation_maps"](idx, e_lo, e_hi)
    idx = np.asarray(idx)
    off = OM.expert_offsets(OM.expert_counts(idx, e_lo, e_hi))
    for e in range(e_hi - e_lo):
        src[off[e]:off[e + 1]] = src[off[e]:off[e + 1]][::-1].copy()
    k = idx.shape[1]
    for r, t in enumerate(src):
        for j in range(k):
            if idx[t, j] - e_lo == np.searchsorted(off, r, side="right") - 1:
                dest[t * k + j] = r
    return dest, src


def _mut_backward_sign(*a, **kw):
    g = _ORIG["moe_backward"](*a, **kw)
    g["d_logits"] = -g["d_logits"]
    return g


def _mut_backward_drop_router_dx(x, w_router, idx, w, *rest):
    g = _ORIG["moe_backward"](x, np.zeros_like(np.asarray(w_router)), idx, w, *rest)
    g["dw_router"] = _ORIG["moe_backward"](x, w_router, idx, w, *rest)["dw_router"]
    return g


def _mut_ffn_drops_up(v, wg, wu, wd):
    p = _ORIG["expert_ffn_parts"](v, wg, wu, wd)
    p["h"] = OM.silu(p["g"])          # dropped factor: the up projection
    p["y"] = p["h"] @ np.asarray(wd, np.float64).T
    return p


def _mut_repeated_expert_overwrites(w, dw, idx, E):
    w, dw = np.asarray(w, np.float64), np.asarray(dw, np.float64)
    dz = np.zeros((w.shape[0], E))
    np.put_along_axis(dz, np.asarray(idx, np.int64), w * (dw - np.sum(w * dw, 1, keepdims=True)), 1)
    return dz


def _mut_router_dx_transposed_sign(dz, w_router):
    return -np.asarray(dz, np.float64) @ np.asarray(w_router, np.float64).T


def _mut_fp8_round_half_away(v):
    v = np.asarray(v, np.float64)
    out = _ORIG["fp8_e4m3_encode"](v)
    dec = OM.fp8_e4m3_decode(out)
    nxt = OM.fp8_e4m3_decode(np.where(out & 0x7F == 0x7E, out, out + 1).astype(np.uint8))
    tie = np.abs(np.abs(v) - (np.abs(dec) + np.abs(nxt)) / 2) == 0
    return np.where(tie & (np.abs(v) > np.abs(dec)), out + 1, out).astype(np.uint8)


def _mut_fp8_exponent_one_high(amax):
    e = _ORIG["fp8_row_exponent"](amax)
    return np.where(np.asarray(amax) == 0, 0, e + 1)


def _mut_fp8_scale_wrong_axis(aq, sa, bq, sb):
    acc = OM.fp8_e4m3_decode(aq) @ OM.fp8_e4m3_decode(bq).T
    n = min(len(sa), len(sb))
    return acc * np.asarray(sa, np.float64)[:, None] * np.asarray(sb, np.float64)[:n].mean()


def _mut_fp8_t_gate_up_swapped(w0, w1=None):
    return _ORIG["quantize_expert_weights_t_fp8"](w1, w0) if w1 is not None else \
        _ORIG["quantize_expert_weights_t_fp8"](w0)


def _mut_fp8_t_scales_per_output_channel(w0, w1=None):
    """codes of the transposed layout, but each scale taken over the output channel"""
    a = [np.asarray(w0, np.float64)] + ([] if w1 is None else [np.asarray(w1, np.float64)])
    a = np.concatenate([m.transpose(0, 2, 1) for m in a], axis=2)
    El, K, N = a.shape
    amax = np.abs(a).max(axis=1, keepdims=True)              # over K, per output channel
    sc = np.exp2(OM.fp8_row_exponent(amax.reshape(-1)).astype(np.float64)).reshape(El, 1, N)
    q = OM.fp8_e4m3_encode(a / sc)
    return q, np.broadcast_to(sc.max(axis=2), (El, K)).copy()


def _mut_bf16_truncates(a):
    a32 = np.asarray(a, np.float32)
    return (a32.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def _mut_bf16_ties_away(a):
    a32 = np.asarray(a, np.float32)
    b = a32.view(np.uint32).astype(np.uint64)
    return ((b + 0x8000) >> 16 << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def _mut_bf16_via_float32(a):
    """rounds to float32 first, then to bfloat16 (double rounding)"""
    return _ORIG["round_bf16"](np.asarray(a, np.float32).astype(np.float64))


def _mut_pair_values_global_index(x, idx, w_gate, w_up, w_down, e_lo, e_hi, tokens=None):
    """indexes the local weight stacks by the global expert id"""
    E_l = e_hi - e_lo
    roll = lambda wt: np.roll(np.asarray(wt), -e_lo % E_l, axis=0)
    return _ORIG["pair_values"](x, idx, roll(w_gate), roll(w_up), roll(w_down), e_lo, e_hi, tokens)


def _mut_pair_values_slot_order(x, idx, w_gate, w_up, w_down, e_lo, e_hi, tokens=None):
    out = _ORIG["pair_values"](x, idx, w_gate, w_up, w_down, e_lo, e_hi, tokens)
    return {n: v[:, ::-1].copy() for n, v in out.items()}


def _mut_group_cols_shared_scale(a, offsets):
    """scales from the column maxima over all rows instead of each group's rows"""
    a = np.asarray(a, np.float64)
    s = np.exp2(OM.fp8_row_exponent(np.abs(a).max(axis=0) if len(a) else np.zeros(a.shape[1]))
                .astype(np.float64))
    off = np.asarray(offsets, np.int64)
    codes = [OM.fp8_e4m3_encode(a[off[e]:off[e + 1]].T / s[:, None]) for e in range(len(off) - 1)]
    return codes, np.broadcast_to(s, (len(off) - 1, a.shape[1])).copy()


def _mut_group_cols_one_scale_per_group(a, offsets):
    """one scale per group (its largest column) instead of one per (group, column)"""
    a = np.asarray(a, np.float64)
    off = np.asarray(offsets, np.int64)
    codes, scales = [], []
    for e in range(len(off) - 1):
        blk = a[off[e]:off[e + 1]]
        s = 2.0 ** float(OM.fp8_row_exponent(np.array([np.abs(blk).max() if blk.size else 0.0]))[0])
        codes.append(OM.fp8_e4m3_encode(blk.T / s))
        scales.append(np.full(a.shape[1], s))
    return codes, np.stack(scales)


def _mut_wgrad_gate_up_swapped(x_perm, dgu, h_perm, dy_perm, offsets):
    out = _ORIG["moe_wgrad_fp8"](x_perm, dgu, h_perm, dy_perm, offsets)
    return {"dw_gate": out["dw_up"], "dw_up": out["dw_gate"], "dw_down": out["dw_down"]}


def _mut_wgrad_down_from_x(x_perm, dgu, h_perm, dy_perm, offsets):
    """dW_down from the columns of x in place of dy"""
    return _ORIG["moe_wgrad_fp8"](x_perm, dgu, h_perm, x_perm, offsets)


_ORIG = {n: getattr(OM, n) for n in ("silu", "topk_experts", "gate_weights", "permutation_maps",
                                     "moe_backward", "expert_ffn_parts", "fp8_e4m3_encode",
                                     "fp8_row_exponent", "quantize_expert_weights_t_fp8",
                                     "round_bf16", "pair_values", "quantize_group_cols_fp8",
                                     "moe_wgrad_fp8")}

MUTATIONS = [("silu", _mut_silu_is_sigmoid), ("topk_experts", _mut_topk_ties_high),
             ("gate_weights", _mut_no_renorm), ("permutation_maps", _mut_group_tokens_descending),
             ("moe_backward", _mut_backward_sign), ("moe_backward", _mut_backward_drop_router_dx),
             ("expert_ffn_parts", _mut_ffn_drops_up),
             ("router_logit_grad", _mut_repeated_expert_overwrites),
             ("router_input_grad", _mut_router_dx_transposed_sign),
             ("fp8_e4m3_encode", _mut_fp8_round_half_away),
             ("fp8_row_exponent", _mut_fp8_exponent_one_high),
             ("fp8_matmul_rows", _mut_fp8_scale_wrong_axis),
             ("quantize_expert_weights_t_fp8", _mut_fp8_t_gate_up_swapped),
             ("quantize_expert_weights_t_fp8", _mut_fp8_t_scales_per_output_channel),
             ("round_bf16", _mut_bf16_truncates), ("round_bf16", _mut_bf16_ties_away),
             ("round_bf16", _mut_bf16_via_float32),
             ("pair_values", _mut_pair_values_global_index),
             ("pair_values", _mut_pair_values_slot_order),
             ("quantize_group_cols_fp8", _mut_group_cols_shared_scale),
             ("quantize_group_cols_fp8", _mut_group_cols_one_scale_per_group),
             ("moe_wgrad_fp8", _mut_wgrad_gate_up_swapped),
             ("moe_wgrad_fp8", _mut_wgrad_down_from_x)]


@pytest.mark.parametrize("name,mut", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, mut):
    monkeypatch.setattr(OM, name, mut)
    monkeypatch.setattr(O, name, mut, raising=False)
    failed = []
    for chk in ALL_CHECKS:
        try:
            chk()
        except Exception:          # a pin that fails or breaks on the mistake catches it
            failed.append(chk.__name__)
    assert failed, f"no pin caught the planted mistake in {name}"
