#!/usr/bin/env python3
"""Benchmark of the per-GPU MoE expert layer on one MI355X.

One step = the whole layer on one batch of seeded synthetic inputs already
resident in HBM: router GEMM + top-k, permute, grouped SwiGLU FFN, combine,
and (for training workloads) the backward of every one of them.  The default
workload is the training step of one EP rank's share of the 128-expert
Qwen3-MoE-30B-A3B-shaped layer (T=8192 tokens, H=2048, I=768, 16 local experts
of 128, top-8, bf16, fp32 accumulation and fp32 weight gradients).

Prints ONE JSON line.  value = algorithmic TFLOP/s of the whole step
(router 2THE, expert FFN 6RHI forward and 12RHI backward, router backward
2THE + 2TkH; R = routed rows kept on this GPU).
"""
import argparse
import ctypes
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (vector/matrix)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

METRIC = "MoE layer fwd+bwd TFLOP/s and tokens/s, 128e/H2048/I768 top-8 bf16"
# the 128-expert full layer whose forward the secondary measurement times
SECONDARY_WORKLOAD = "full_t16384_h2048_i768_e128_k8"

KERNELS = ["ROUTE", "PERMUTE_HIST", "PERMUTE_SCAN", "PERMUTE_SCATTER", "FFN_GATEUP", "FFN_DOWN",
           "COMBINE", "COMBINE_BWD", "ROUTE_BWD_DZ", "ROUTE_BWD_DW", "FFN_DOWN_DGRAD",
           "FFN_DOWN_WGRAD", "FFN_GATEUP_DGRAD", "FFN_GATEUP_WGRAD", "COMBINE_DX", "ROUTE_BWD_DX",
           "COMBINE_ADD", "FFN_WGRAD_REDUCE"]


def step_flops(w, R):
    f = 2.0 * w.T * w.H * w.E + 6.0 * R * w.H * w.I
    if w.train:
        f += 12.0 * R * w.H * w.I + 2.0 * w.T * w.H * w.E + 2.0 * w.T * w.k * w.H
    return f


def kernel_work(name, w, R, launches, A=None, gather=False):
    """Algorithmic (flops, HBM bytes) of ONE launch of a kernel.  R = routed rows
    kept on this GPU, A = tokens with at least one of them (rows of x, dy that
    the scatter and the combine backward must read; all T when not given).
    gather: the layer's permute writes the maps alone and the gate/up product
    reads the token rows through src_row (each row once from HBM)."""
    T, H, I, E, k, El = w.T, w.H, w.I, w.E, w.k, w.E_l
    A = T if A is None else A
    b = 2 if w.dtype == "bf16" else 4
    gu = 2 * I * b * R if w.train else 0
    tab = {
        "ROUTE": (2.0 * T * H * E, T * H * b + H * E * b + T * E * 4 + T * k * 8),
        "PERMUTE_HIST": (0, T * k * 8 + (T // 256 + 1) * El * 4),
        "PERMUTE_SCAN": (0, 2 * (T // 256 + 1) * El * 4),
        "PERMUTE_SCATTER": (0, A * H * b + R * H * b + T * k * 12 + R * 4),
        "FFN_GATEUP": (4.0 * R * H * I, R * H * b + 2 * El * I * H * b + R * I * b + gu),
        "FFN_DOWN": (2.0 * R * H * I, R * I * b + El * H * I * b + R * H * b),
        "COMBINE_BWD": (0, A * H * b + 2 * R * H * b + T * k * 12),
        "ROUTE_BWD_DZ": (0, T * k * 12 + T * E * 4 + T * 2 * E * 2),
        "COMBINE_DX": (2.0 * T * k * H, R * H * b + E * H * b + T * k * 16 + T * H * b),
        # dense product over all E columns (the method's work is the k kept ones)
        "ROUTE_BWD_DX": (2.0 * T * k * H, T * 2 * E * 2 + H * E * b + T * H * 4),
        # unweighted unpermute-reduce plus an fp32 addend row per token
        "COMBINE_ADD": (0, R * H * b + T * k * 4 + T * H * 4 + T * H * b),
        # split experts' partial slots (none on balanced loads): priced at zero
        "FFN_WGRAD_REDUCE": (0, 0),
        "ROUTE_BWD_DW": (2.0 * T * H * E, T * H * b + T * 2 * E * 2 + H * E * 4),
        "FFN_DOWN_DGRAD": (2.0 * R * H * I, R * H * b + El * H * I * b + 2 * R * 2 * I * b),
        "FFN_DOWN_WGRAD": (2.0 * R * H * I, R * H * b + R * I * b + El * H * I * 4),
        "FFN_GATEUP_DGRAD": (4.0 * R * H * I, R * 2 * I * b + 2 * El * I * H * b + R * H * b),
        "FFN_GATEUP_WGRAD": (4.0 * R * H * I, R * 2 * I * b + R * H * b + 2 * El * I * H * 4),
    }
    if gather:
        tab["PERMUTE_SCATTER"] = (0, T * k * 12 + R * 4)
        tab["FFN_GATEUP"] = (4.0 * R * H * I, A * H * b + 2 * El * I * H * b + R * I * b + gu)
    if name == "COMBINE":
        return 0.0, R * H * b + T * k * 8 + T * H * b
    return tab[name]


# Measured HBM traffic per launch (rocprofv3 FETCH_SIZE and WRITE_SIZE passes,
# scaled by what the same counters read for a plain copy of known size): a
# committed summary under profiles/, valid only for the kernel sources it was
# taken with.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_ep16_train_t8192.md")


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_expert_layer_router_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed summary, or None."""
    try:
        text = open(TRAFFIC_FILE, encoding="utf-8").read()
    except OSError:
        return None
    m = re.search(r"kernel source hash: `([0-9a-f]+)`", text)
    if not m or m.group(1) != kernel_source_hash() or f"workload: `{workload}`" not in text:
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 5 and cells[0] == kernel:
            try:
                return int(float(cells[4]))
            except ValueError:
                return None
    return None


def roofline_of(name, w, R, avg_us, launches, A=None, gather=False):
    flops, nbytes = kernel_work(name, w, R, launches, A, gather)
    peak_f = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    t_f = flops / (peak_f * 1e12)
    t_b = nbytes / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(name, w.name)
    if flops > 0 and t_f >= t_b:
        ach = flops / (avg_us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_f, "unit": "TFLOP/s",
                "frac": round(ach / peak_f, 4), "traffic": traffic,
                "kernel": name, "algorithmic_per_launch": flops, "avg_us": round(avg_us, 2),
                "hbm_floor_us": round(t_b * 1e6, 2), "mfma_floor_us": round(t_f * 1e6, 2)}
    ach = nbytes / (avg_us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": name, "algorithmic_per_launch": nbytes, "avg_us": round(avg_us, 2),
            "hbm_floor_us": round(t_b * 1e6, 2), "mfma_floor_us": round(t_f * 1e6, 2)}


def cpu_baseline(w, inp, target_s=12.0):
    """The CPU oracle as it stands, on the first Ts tokens of the same workload."""
    import numpy as np

    import oracle as O
    avail = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = avail
    cores = min(avail, blas)
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass

    def run(Ts):
        x = inp["x"][:Ts]
        t0 = time.perf_counter()
        z, idx, gw = O.route(x, inp["w_router"], w.k, inp.get("bias"))
        O.moe_forward(x, idx, gw, inp["w_gate"], inp["w_up"], inp["w_down"], w.e_lo, w.e_hi)
        if w.train:
            O.moe_backward(x, inp["w_router"], idx, gw, inp["w_gate"], inp["w_up"], inp["w_down"],
                           inp["dy"][:Ts], w.e_lo, w.e_hi)
        dt = time.perf_counter() - t0
        R = int(((idx >= w.e_lo) & (idx < w.e_hi)).sum())
        return dt, R

    Ts = min(w.T, 128)
    dt, R = run(Ts)
    # the oracle has a fixed cost per call (per-expert set-up), so a small
    # sample's rate understates larger ones: rescale until the sample is long
    # enough or the whole workload, then repeat the run to fill the budget
    while dt < target_s / 4 and Ts < w.T:
        Ts = int(min(w.T, max(2 * Ts, Ts * target_s / max(dt, 1e-3))))
        dt, R = run(Ts)
    reps = max(1, min(20, int(target_s / max(dt, 1e-3))))
    for _ in range(reps - 1):
        dt += run(Ts)[0]
    dt /= reps
    sub = w.scaled(T=Ts)
    fl = step_flops(sub, R)
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "cores_available": avail, "blas_threads": int(blas), "cpu_model": model,
            "kind": "oracle", "tokens_per_s": round(Ts / dt, 1), "seconds": round(dt * reps, 2),
            "sample": f"first {Ts} of {w.T} tokens of {w.name}, float64 NumPy "
                      f"{'forward+backward' if w.train else 'forward'}, mean of {reps} run(s)"}


def _kernel_avg_us(moe, torch, kid, fn, n):
    """Average duration of kernel `kid` over n calls of fn (library events on its stream)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in starts + stops:
        e.record()
    torch.cuda.synchronize()
    arr_s = (ctypes.c_void_p * n)(*[ctypes.c_void_p(e.cuda_event) for e in starts])
    arr_e = (ctypes.c_void_p * n)(*[ctypes.c_void_p(e.cuda_event) for e in stops])
    moe.lib.moe_profile_kernel(kid, arr_s, arr_e, n)
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    cnt = moe.lib.moe_profile_recorded()
    moe.lib.moe_profile_kernel(-1, None, None, 0)
    return sum(starts[i].elapsed_time(stops[i]) * 1e3 for i in range(cnt)) / max(cnt, 1)


def fp8_ffn_bench(w, args):
    """Grouped SwiGLU FFN forward, bf16 versus the FP8 recipe (E4M3 codes, one
    power-of-two scale per row), on the routing of the bf16 router.  FLOPs are
    the algorithmic 6 R H I of the FFN; the FP8 time includes its schedule, row-
    scale gather and the quantization of h (the activation quantization before
    the permute is timed on its own)."""
    import torch

    import moe_expert_layer_router_amd as moe
    from workloads import make_inputs

    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    t = {n: torch.from_numpy(v).to(dev).to(torch.bfloat16).contiguous() for n, v in inp.items()
         if n not in ("bias", "dy")}
    bias = torch.from_numpy(inp["bias"]).to(dev) if "bias" in inp else None
    idx, _, _ = moe.moe_route(t["x"], t["w_router"], w.k, bias=bias)
    pb = moe.moe_permute(t["x"], idx, w.E, w.e_lo, w.e_hi)
    xq, sx = moe.moe_quantize_fp8(t["x"])
    pq = moe.moe_permute(xq, idx, w.E, w.e_lo, w.e_hi)
    wq = {}
    for n in ("w_gate", "w_up", "w_down"):
        El, N, K = t[n].shape
        q, s8 = moe.moe_quantize_fp8(t[n].view(El * N, K))
        wq[n] = (q.view(El, N, K), s8.view(El, N))
    torch.cuda.synchronize()
    R = int(pb["offsets"][-1].item())
    ob = moe.moe_grouped_ffn_fwd(pb["x_perm"], pb["offsets"], t["w_gate"], t["w_up"], t["w_down"],
                                 save_gu=False)
    o8 = moe.moe_grouped_ffn_fwd_fp8(pq["x_perm"], sx, pq["src_row"], pq["offsets"], wq["w_gate"],
                                     wq["w_up"], wq["w_down"])
    f_b = lambda: moe.moe_grouped_ffn_fwd(pb["x_perm"], pb["offsets"], t["w_gate"], t["w_up"],
                                          t["w_down"], save_gu=False, out=ob)
    f_8 = lambda: moe.moe_grouped_ffn_fwd_fp8(pq["x_perm"], sx, pq["src_row"], pq["offsets"],
                                              wq["w_gate"], wq["w_up"], wq["w_down"], out=o8)
    f_q = lambda: moe.moe_quantize_fp8(t["x"], out={"q": xq, "scale": sx})

    def timed(fn, n):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    n = args.steps
    us_b, us_8, us_q = timed(f_b, n), timed(f_8, n), timed(f_q, n)
    flops = 6.0 * R * w.H * w.I
    kern = {}
    for name, kid, fl in (("FFN_GATEUP", 4, 4.0 * R * w.H * w.I), ("FFN_DOWN", 5, 2.0 * R * w.H * w.I)):
        for tag, fn, peak in (("bf16", f_b, PEAK_BF16_TFLOPS), ("fp8", f_8, PEAK_FP8_TFLOPS)):
            avg = _kernel_avg_us(moe, torch, kid, fn, n)
            ach = fl / (avg * 1e-6) / 1e12
            kern[f"{name}_{tag}"] = {"avg_us": round(avg, 2), "achieved_tflops": round(ach, 1),
                                     "peak_tflops": peak, "frac": round(ach / peak, 4)}
    tf8 = flops / (us_8 * 1e-6) / 1e12
    dgrad = fp8_dgrad_bench(w, args, moe, torch, t, pb, timed, n)
    dom = max(("FFN_GATEUP_fp8", "FFN_DOWN_fp8"), key=lambda k: kern[k]["avg_us"])
    return {
        "metric": "grouped expert FFN forward TFLOP/s, FP8 recipe vs bf16",
        "value": round(tf8, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "higher_is_better": True, "vs_baseline": None,
        "dtype": "fp8 e4m3 operands (row scales), fp32 accumulate, bf16 out",
        "data": "synthetic (seeded normal draws, random-init weights)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "k": w.k,
                   "local_experts": [w.e_lo, w.e_hi], "routed_rows": R},
        "us_per_ffn_forward": {"fp8": round(us_8, 2), "bf16": round(us_b, 2)},
        "bf16_tflops": round(flops / (us_b * 1e-6) / 1e12, 2),
        "speedup_vs_bf16": round(us_b / us_8, 3),
        "activation_quantize_us": round(us_q, 2),
        "kernels": kern,
        "data_gradients": dgrad,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": kern[dom]["achieved_tflops"],
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": kern[dom]["frac"],
                     "traffic": None},
    }


def fp8_dgrad_bench(w, args, moe, torch, t, pb, timed, n):
    """The two data-gradient products of the expert FFN, bf16 (those of
    moe_grouped_ffn_bwd_split, with the weight-gradient stream held back by a
    sleep kernel so that they run alone) versus moe_grouped_ffn_dgrad_fp8 (both
    FP8 products, the SiLU derivative and the row quantization of [dg | du]).
    FLOPs: 6 R H I.  The quantization of dy_perm and of the transposed weights
    is timed on its own."""
    dev = torch.device("cuda:0")
    R_cap, H, I = w.T * w.k, w.H, w.I
    E_l = w.e_hi - w.e_lo
    offsets = pb["offsets"]
    R = int(offsets[-1].item())
    g = torch.Generator().manual_seed(11)
    dy = (torch.randn(R_cap, H, generator=g) * 0.05).to(dev).to(torch.bfloat16)
    fw = moe.moe_grouped_ffn_fwd(pb["x_perm"], offsets, t["w_gate"], t["w_up"], t["w_down"],
                                 save_gu=True)
    gu, h_perm = fw["gu"], fw["h_perm"]
    dyq, sdy = moe.moe_quantize_fp8(dy, nrows=offsets[E_l:])
    wdt = moe.moe_quantize_fp8_t(t["w_down"])
    wgut = moe.moe_quantize_fp8_t(t["w_gate"], t["w_up"])
    o8 = moe.moe_grouped_ffn_dgrad_fp8(dyq, sdy, gu, offsets, wdt, wgut)
    bufs = {"dx": torch.empty_like(pb["x_perm"]),
            "dwg": torch.empty((E_l, I, H), dtype=torch.float32, device=dev),
            "dwu": torch.empty((E_l, I, H), dtype=torch.float32, device=dev),
            "dwd": torch.empty((E_l, H, I), dtype=torch.float32, device=dev)}
    nb = moe.lib.moe_workspace_bytes(moe.MOE_OP_FFN_BWD, R_cap, H, I, max(E_l, 1), 1, 0, E_l, moe.MOE_BF16)
    ws = torch.empty(int(nb), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream(device=dev)
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    main = torch.cuda.current_stream()

    def f_bd():
        with torch.cuda.stream(side):
            torch.cuda._sleep(20_000_000)  # the weight gradients start after the data gradients
        rc = moe.lib.moe_grouped_ffn_bwd_split(
            P(dy), P(pb["x_perm"]), P(gu), P(h_perm), P(offsets), E_l, R_cap, H, I, P(t["w_gate"]),
            P(t["w_up"]), P(t["w_down"]), moe.MOE_BF16, P(bufs["dx"]), P(bufs["dwg"]), P(bufs["dwu"]),
            P(bufs["dwd"]), 0, P(ws), ctypes.c_size_t(ws.numel()), ctypes.c_void_p(main.cuda_stream),
            ctypes.c_void_p(side.cuda_stream))
        assert rc == 0, moe.lib.moe_last_error()
        main.wait_stream(side)

    f_8 = lambda: moe.moe_grouped_ffn_dgrad_fp8(dyq, sdy, gu, offsets, wdt, wgut, out=o8)
    f_qdy = lambda: moe.moe_quantize_fp8(dy, nrows=offsets[E_l:], out={"q": dyq, "scale": sdy})
    f_qw = lambda: (moe.moe_quantize_fp8_t(t["w_down"], out={"q": wdt[0], "scale": wdt[1]}),
                    moe.moe_quantize_fp8_t(t["w_gate"], t["w_up"], out={"q": wgut[0], "scale": wgut[1]}))
    us_8 = timed(f_8, n)
    kid = {k: KERNELS.index(k) for k in ("FFN_DOWN_DGRAD", "FFN_GATEUP_DGRAD")}
    fl = {"FFN_DOWN_DGRAD": 2.0 * R * H * I, "FFN_GATEUP_DGRAD": 4.0 * R * H * I}
    kern = {}
    for name in kid:
        for tag, fn, peak in (("bf16", f_bd, PEAK_BF16_TFLOPS), ("fp8", f_8, PEAK_FP8_TFLOPS)):
            avg = _kernel_avg_us(moe, torch, kid[name], fn, n)
            ach = fl[name] / (avg * 1e-6) / 1e12
            kern[f"{name}_{tag}"] = {"avg_us": round(avg, 2), "achieved_tflops": round(ach, 1),
                                     "peak_tflops": peak, "frac": round(ach / peak, 4)}
    us_b = kern["FFN_DOWN_DGRAD_bf16"]["avg_us"] + kern["FFN_GATEUP_DGRAD_bf16"]["avg_us"]
    flops = 6.0 * R * H * I
    # the whole expert backward: bf16 (moe_grouped_ffn_bwd, data and weight
    # gradients on two streams) against the FP8 data gradients followed by the
    # FP8 weight gradients (their operand quantization included)
    f_bb = lambda: moe.moe_grouped_ffn_bwd(dy, pb["x_perm"], gu, h_perm, offsets, t["w_gate"], t["w_up"],
                                           t["w_down"], ws=ws, out={"dx_perm": bufs["dx"],
                                                                    "dw_gate": bufs["dwg"],
                                                                    "dw_up": bufs["dwu"],
                                                                    "dw_down": bufs["dwd"]})
    ow = moe.moe_grouped_ffn_wgrad_fp8(pb["x_perm"], None, o8["dgu"], h_perm, dy, offsets, E_l)
    nbw = moe.lib.moe_workspace_bytes(moe.MOE_OP_FFN_WGRAD_FP8, R_cap, H, I, max(E_l, 1), 1, 0, E_l,
                                      moe.MOE_BF16)
    wsw = torch.empty(int(nbw), dtype=torch.uint8, device=dev)
    f_w8 = lambda: moe.moe_grouped_ffn_wgrad_fp8(pb["x_perm"], None, o8["dgu"], h_perm, dy, offsets, E_l,
                                                 ws=wsw, out=ow)

    def f_b8():
        f_8()
        f_w8()
    us_bb, us_w8, us_b8 = timed(f_bb, n), timed(f_w8, n), timed(f_b8, n)
    backward = {"us": {"bf16": round(us_bb, 2), "fp8": round(us_b8, 2), "fp8_weight_gradients": round(us_w8, 2)},
                "bf16_tflops": round(2 * flops / (us_bb * 1e-6) / 1e12, 1),
                "fp8_tflops": round(2 * flops / (us_b8 * 1e-6) / 1e12, 1),
                "speedup_vs_bf16": round(us_bb / us_b8, 3),
                "note": "fp8 = data gradients (with the SiLU' pass and [dg|du] codes) + weight gradients "
                        "(with the per-(expert, column) quantization of their four operands); the dy_perm "
                        "rows and the transposed weights are quantized outside (timed below)"}
    return {"us": {"fp8": round(us_8, 2), "bf16_products": round(us_b, 2)},
            "fp8_tflops": round(flops / (us_8 * 1e-6) / 1e12, 1),
            "bf16_tflops": round(flops / (us_b * 1e-6) / 1e12, 1),
            "speedup_vs_bf16": round(us_b / us_8, 3),
            "dy_quantize_us": round(timed(f_qdy, n), 2),
            "weight_quantize_t_us": round(timed(f_qw, n), 2),
            "kernels": kern,
            "backward": backward}


def step_stats(run, n, dev):
    """Per-step times after the timed region: each step bracketed by its own
    event pair, median / p10 / p90 over n steps.  "warm": back to back, so the
    weights stay in the 256 MiB Infinity Cache and L2 between steps.  "cold":
    a 512 MiB buffer is written before each step's start event (outside the
    bracket), which evicts the previous step's data from both caches."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = {}
    for mode in ("warm", "cold"):
        ts = []
        for i in range(n):
            if mode == "cold":
                flush.fill_(i & 0xff)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        q = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]
        out[mode] = {"median": round(q(0.5), 4), "p10": round(q(0.1), 4), "p90": round(q(0.9), 4)}
    del flush
    return out


def live_kernel_times(moe, torch, step, n):
    """Live per-kernel durations: events the library records around each launch
    of one kernel, on the stream it is launched on, over n eager steps."""
    kt = {}
    for kid, name in enumerate(KERNELS):
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(4 * n)]
        stops = [torch.cuda.Event(enable_timing=True) for _ in range(4 * n)]
        # torch creates the HIP event on first record; the library records it again
        for e in starts + stops:
            e.record()
        torch.cuda.synchronize()
        arr_s = (ctypes.c_void_p * (4 * n))(*[ctypes.c_void_p(e.cuda_event) for e in starts])
        arr_e = (ctypes.c_void_p * (4 * n))(*[ctypes.c_void_p(e.cuda_event) for e in stops])
        moe.lib.moe_profile_kernel(kid, arr_s, arr_e, 4 * n)
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        cnt = moe.lib.moe_profile_recorded()
        moe.lib.moe_profile_kernel(-1, None, None, 0)
        if cnt == 0:
            continue
        times = [starts[i].elapsed_time(stops[i]) * 1e3 for i in range(cnt)]
        kt[name] = {"avg_us": sum(times) / cnt, "launches_per_step": cnt // n,
                    "us_per_step": sum(times) / n}
    return kt


def secondary_forward(w, args, moe, torch):
    """The forward of the full 128-expert layer (every expert local, T = 16384):
    graph-replayed layer time and each forward kernel's live time against its
    roofline (router, permute and combine against HBM, the grouped products
    against bf16 MFMA).  The layer's permute writes the maps alone and its
    gate/up product reads the token rows through src_row.  The same forward on
    the materialized grouped copy is timed beside it ("ms_per_step_grouped_copy"),
    and its permute launches in it ("permute_copy": the scatter, and the three
    launches together, "PERMUTE", priced at the copy's algorithmic bytes)."""
    from workloads import make_inputs
    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    t = {n: torch.from_numpy(v).to(dev).to(torch.bfloat16).contiguous() for n, v in inp.items()
         if n != "bias"}

    def graph_ms(layer):
        step = lambda: layer.forward(t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"])
        for _ in range(max(args.warmup, 1)):
            step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps, step

    layer = moe.MoELayer(w.T, w.H, w.I, w.E, w.k, w.e_lo, w.e_hi, torch.bfloat16, dev, train=False)
    gather = layer.gather
    ms, step = graph_ms(layer)
    R = int(layer.buf["offsets"][-1].item())
    kt = live_kernel_times(moe, torch, step, args.steps)
    roof = {}
    for k, v in kt.items():
        r = roofline_of(k, w, R, v["avg_us"], v["launches_per_step"], gather=gather)
        roof[k] = {kk: r[kk] for kk in ("bound", "achieved", "unit", "frac", "avg_us")}
    del layer
    # the permute that writes the grouped copy, alone, and the forward on it
    ref = moe.MoELayer(w.T, w.H, w.I, w.E, w.k, w.e_lo, w.e_hi, torch.bfloat16, dev, train=False,
                       gather=False)
    ms_copy, step_copy = graph_ms(ref)
    kp = live_kernel_times(moe, torch, step_copy, args.steps)
    pc = {}
    for k in ("PERMUTE_HIST", "PERMUTE_SCAN", "PERMUTE_SCATTER"):
        if k in kp:
            r = roofline_of(k, w, R, kp[k]["avg_us"], kp[k]["launches_per_step"])
            pc[k] = {kk: r[kk] for kk in ("bound", "achieved", "unit", "frac", "avg_us")}
    if pc:
        us = sum(v["avg_us"] for v in pc.values())
        nb = kernel_work("PERMUTE_SCATTER", w, R, 1)[1]
        pc["PERMUTE"] = {"bound": "hbm", "achieved": round(nb / (us * 1e-6) / 1e9, 1), "unit": "GB/s",
                         "frac": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "avg_us": round(us, 2)}
    del ref
    flops = step_flops(w, R)
    return {"workload": w.name, "pass": "forward", "timing": "hip-graph replay", "steps": args.steps,
            "ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "tokens_per_s": round(w.T / (ms * 1e-3), 1), "routed_rows": R,
            "permute": "maps only, gate/up gathers x through src_row" if gather else "grouped copy",
            "roofline": roof, "ms_per_step_grouped_copy": round(ms_copy, 4), "permute_copy": pc}


def fp8_step(w, t, bias, args, moe, torch):
    """The same training step with the expert FFN in the FP8 recipe (MoELayer with
    fp8=True: token, weight, dy and [dg | du] quantization included in the step),
    graph-replayed on the same inputs; checked bit for bit against its eager run."""
    dev = torch.device("cuda:0")
    layer = moe.MoELayer(w.T, w.H, w.I, w.E, w.k, w.e_lo, w.e_hi, torch.bfloat16, dev, train=True,
                         fp8=True)

    def step():
        layer.forward(t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], bias=bias)
        layer.backward(t["dy"], t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"])

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    ref = layer.buf["dx"].clone()
    R = int(layer.buf["offsets"][-1].item())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    same = torch.equal(layer.buf["dx"].view(torch.int16), ref.view(torch.int16))
    run = g.replay if same else step
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = step_flops(w, R)
    out = {"workload": w.name, "pass": "forward+backward", "ffn": "fp8 e4m3 (per-row / per-channel "
           "power-of-two scales), router and combine bf16", "timing": "hip-graph replay" if same else
           "eager launches", "steps": args.steps, "ms_per_step": round(ms, 4),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
           "routed_rows": R}
    del layer, g
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ep16_train_t8192_h2048_i768_e128_k8")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-times", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the forward of the full 128-expert layer timed after the main step")
    ap.add_argument("--no-step-stats", action="store_true",
                    help="skip the per-step warm / cold (cache-flushed) timing pass")
    ap.add_argument("--fp8", action="store_true",
                    help="run the layer with the FP8 expert FFN (MoELayer(fp8=True)) as the main step")
    ap.add_argument("--no-fp8-step", action="store_true",
                    help="skip the training step with the FP8 expert FFN timed after the main step")
    ap.add_argument("--fp8-ffn", action="store_true",
                    help="instead of the layer step: time the grouped FFN forward in bf16 and in the "
                         "FP8 recipe on the same routing (default workload: the full 128-expert layer)")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="after the warm-up, copy 256 MiB device to device once (outside the timed "
                         "region): the copy kernel's FETCH_SIZE / WRITE_SIZE calibrate counter runs")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this layer build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_expert_layer_router_amd as moe
    from workloads import WORKLOADS, make_inputs

    if args.fp8_ffn:
        wl = args.workload if args.workload != ap.get_default("workload") else "full_t16384_h2048_i768_e128_k8"
        print(json.dumps(fp8_ffn_bench(WORKLOADS[wl], args)), flush=True)
        return

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    inp = make_inputs(w)
    t = {n: torch.from_numpy(v).to(dev).to(dt).contiguous() for n, v in inp.items() if n != "bias"}
    bias = torch.from_numpy(inp["bias"]).to(dev) if "bias" in inp else None
    if args.fp8 and w.dtype != "bf16":
        print("--fp8 needs a bf16 workload", file=sys.stderr)
        sys.exit(2)
    layer = moe.MoELayer(w.T, w.H, w.I, w.E, w.k, w.e_lo, w.e_hi, dt, dev, train=w.train, fp8=args.fp8)

    def step():
        layer.forward(t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], bias=bias)
        if w.train:
            layer.backward(t["dy"], t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"])

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    R = int(layer.buf["offsets"][-1].item())
    A = int((layer.buf["dest_row"].view(w.T, w.k) >= 0).any(dim=1).sum().item())
    ref_out = (layer.buf["dx"] if w.train else layer.buf["y"]).clone()
    if args.pmc_calibration:
        src = torch.ones(128 << 20, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        out = layer.buf["dx"] if w.train else layer.buf["y"]
        if not torch.equal(out.view(torch.int16) if dt == torch.bfloat16 else out, ref_out.view(torch.int16)
                           if dt == torch.bfloat16 else ref_out):
            print("graph replay differs from eager result; timing eager launches", file=sys.stderr)
            graph = None

    run = graph.replay if graph is not None else step
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / args.steps

    flops = step_flops(w, R)
    result = {
        "metric": (METRIC if w.train else METRIC.replace("fwd+bwd", "fwd")).replace(
            "bf16", "FP8 expert FFN" if args.fp8 else "bf16"),
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp8-e4m3 expert FFN, bf16 router/combine" if args.fp8 else "bf16")
                 if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded normal draws, random-init weights)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "k": w.k,
                   "local_experts": [w.e_lo, w.e_hi], "routed_rows": R,
                   "tokens_with_local_slots": A,
                   "pass": "forward+backward" if w.train else "forward",
                   "timing": "hip-graph replay" if graph is not None else "eager launches"},
        "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "flops_per_step": flops,
        "wall_s_timed_region": round(wall, 3),
    }

    if not args.no_step_stats:
        result["step_ms"] = step_stats(run, args.steps, dev)

    if not args.no_kernel_times:
        kt = live_kernel_times(moe, torch, step, args.steps)
        result["kernels_us_per_step"] = {k: round(v["us_per_step"], 2) for k, v in kt.items()}
        dom = max(kt, key=lambda k: kt[k]["us_per_step"])
        result["roofline"] = roofline_of(dom, w, R, kt[dom]["avg_us"], kt[dom]["launches_per_step"], A)
        result["roofline_all"] = {k: {kk: vv for kk, vv in
                                      roofline_of(k, w, R, v["avg_us"], v["launches_per_step"], A).items()
                                      if kk in ("bound", "achieved", "unit", "frac", "avg_us")}
                                  for k, v in kt.items()}

    if not args.no_secondary and w.name != SECONDARY_WORKLOAD:
        del layer, graph
        torch.cuda.empty_cache()
        layer = graph = None
        result["secondary"] = secondary_forward(WORKLOADS[SECONDARY_WORKLOAD], args, moe, torch)

    if not args.no_fp8_step and not args.fp8 and w.train and w.dtype == "bf16":
        del layer, graph
        torch.cuda.empty_cache()
        layer = graph = None
        fp = fp8_step(w, t, bias, args, moe, torch)
        fp["vs_bf16_step"] = round(ms / fp["ms_per_step"], 3)
        result["fp8_step"] = fp

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
