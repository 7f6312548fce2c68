"""Seeded synthetic inputs for the per-GPU MoE expert layer.

This module only draws random numbers and casts them; it holds none of the
layer's arithmetic, so both the CPU oracle's tests and the HIP path's tests
and bench draw the very same tensors from here.

Shapes follow the Qwen3-MoE-30B-A3B expert layer described on the page
"Qwen3-MoE-30B-A3B模型EP+FSDP2并行方案" (section "Qwen3-MoE-30B-A3B模型":
128 experts, hidden 2048, intermediate 768; expert tensors laid out
[E, I, H] for gate/up and [E, H, I] for down) and one EP rank's slice of it
(section "完整并行流程": 128/8 = 16 experts per rank, [16, 2048, 768]).

Draw recipe (fixed order, one generator per workload):
  rng = numpy.random.default_rng(seed)        # PCG64
  X       [T,H]      ~ N(0, 1)
  W_r     [H,E]      ~ N(0, 1/H)   (variance 1/H, i.e. std H**-0.5)
  W_gate  [E_l,I,H]  ~ N(0, 0.02²) (std 0.02)
  W_up    [E_l,I,H]  ~ N(0, 0.02²)
  W_down  [E_l,H,I]  ~ N(0, 0.02²)
  rank    [E]        = rng.permutation(E)        (skewed workload only)
  dY      [T,H]      ~ N(0, 1)                   (training workload only)
All draws are float32 (``standard_normal(dtype=float32)`` times the std);
bf16 workloads then round every tensor to bf16 with round-to-nearest-even
and keep it as float32 holding exactly representable bf16 values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    e_lo: int
    e_hi: int
    dtype: str            # "f32" or "bf16"
    skew: bool = False    # add a Zipf-like per-expert router bias
    train: bool = False   # also draw an upstream gradient dY
    seed: int = 0

    @property
    def E_l(self) -> int:
        return self.e_hi - self.e_lo

    def scaled(self, **kw) -> "Workload":
        """A copy with some fields replaced (used for small parity cases)."""
        return dataclasses.replace(self, **kw)


# The workloads: a tiny fp32 correctness case, one EP rank's share of the
# 128-expert layer (forward), the full single-GPU layer, a skewed-load
# variant, the EP rank's training step (forward + backward) and that step
# under the skewed load.
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_fp32_t256_h64_i32_e8_k2", 256, 64, 32, 8, 2, 0, 8, "f32"),
        Workload("ep16_share_t4096_h2048_i768_e128_k8", 4096, 2048, 768, 128, 8, 0, 16, "bf16"),
        Workload("full_t16384_h2048_i768_e128_k8", 16384, 2048, 768, 128, 8, 0, 128, "bf16"),
        Workload("skewed_t32768_h2048_i768_e128_k8", 32768, 2048, 768, 128, 8, 0, 128, "bf16",
                 skew=True),
        Workload("ep16_train_t8192_h2048_i768_e128_k8", 8192, 2048, 768, 128, 8, 0, 16, "bf16",
                 train=True),
        # the training step under the skewed router bias, on the EP rank whose
        # 16 local experts [80, 96) hold the hottest expert of this seed's
        # ranking (8191 of its 8747 routed rows; 10 local experts get none)
        Workload("ep16_train_skewed_t8192_h2048_i768_e128_k8", 8192, 2048, 768, 128, 8, 80, 96,
                 "bf16", skew=True, train=True),
    ]
}

TINY = WORKLOADS["tiny_fp32_t256_h64_i32_e8_k2"]
EP_SHARE = WORKLOADS["ep16_share_t4096_h2048_i768_e128_k8"]
FULL = WORKLOADS["full_t16384_h2048_i768_e128_k8"]
SKEWED = WORKLOADS["skewed_t32768_h2048_i768_e128_k8"]
TRAIN = WORKLOADS["ep16_train_t8192_h2048_i768_e128_k8"]
TRAIN_SKEWED = WORKLOADS["ep16_train_skewed_t8192_h2048_i768_e128_k8"]

SKEW_BIAS_SCALE = 2.0


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    Works on the bit pattern: add 0x7FFF plus the lowest kept bit, then clear
    the 16 dropped bits.  Inputs here are finite normal draws.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw the workload's tensors (float32 arrays; bf16-exact for bf16 workloads).

    Keys: x, w_router, w_gate, w_up, w_down, and optionally bias (skewed
    workload: -SKEW_BIAS_SCALE*ln(rank_e+1), float32) and dy (training).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    f32 = np.float32
    out: Dict[str, np.ndarray] = {}
    out["x"] = rng.standard_normal((w.T, w.H), dtype=f32)
    out["w_router"] = rng.standard_normal((w.H, w.E), dtype=f32) * f32(1.0 / math.sqrt(w.H))
    out["w_gate"] = rng.standard_normal((w.E_l, w.I, w.H), dtype=f32) * f32(0.02)
    out["w_up"] = rng.standard_normal((w.E_l, w.I, w.H), dtype=f32) * f32(0.02)
    out["w_down"] = rng.standard_normal((w.E_l, w.H, w.I), dtype=f32) * f32(0.02)
    if w.skew:
        rank = rng.permutation(w.E)
        out["bias"] = (-SKEW_BIAS_SCALE * np.log(rank.astype(np.float64) + 1.0)).astype(f32)
    if w.train:
        out["dy"] = rng.standard_normal((w.T, w.H), dtype=f32)
    if w.dtype == "bf16":
        for key in ("x", "w_router", "w_gate", "w_up", "w_down", "dy"):
            if key in out:
                out[key] = round_bf16(out[key])
    return out
