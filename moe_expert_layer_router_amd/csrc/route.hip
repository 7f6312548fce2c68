// Router GEMM + top-k softmax gating for gfx950.
//
// The pages leave the router open; the layer uses the plain top-k router:
// logits z = x . W_r (+ bias), the k largest logits per token (equal logits go
// to the lower expert id, slot order = logit descending then id ascending),
// gate weights = softmax over the kept logits (identical to a softmax over all
// experts renormalised over the kept ones).
//
// bf16 path, two launches.  (1) A workgroup of four waves takes 128 tokens and
// one slice of HS rows of W_r (all E experts): the slice is copied once into
// LDS, so the L2 traffic for W_r is one slice per 128 tokens, and each wave
// multiplies its 32 tokens' x fragments (all of the slice's loads in flight
// at once, straight from global memory) by the slice with bf16 32x32x16
// MFMAs, reading the W_r fragments with transposing LDS reads.  Each wave
// stores its fp32 partial logits.  (2) One half wave per token adds the
// slices' partials in slice order (+ bias), stores the logits, and takes the
// top k: every lane holds up to eight logits (expert e = lane % 32 + 32 i)
// and k rounds of a branch-free arg-max over unique (logit, id) keys pick the
// experts.  Every sum runs in a fixed order, so logits are deterministic.
#include "common.h"

#include <math.h>

namespace moe {

// Selection key of (logit, expert): the unsigned order of keys is logit
// descending, then expert id ascending, so every key is unique and the k
// largest keys are the k kept experts in slot order.  -0 is folded into +0 so
// equal logits tie on the id.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xffff - e);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return 0xffff - (int)(uint32_t)key; }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  return ((uint64_t)dpp32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Lane permutations of one 32-lane half: xor 1 and xor 2 inside a quad (DPP
// quad_perm), i <-> 7 - i inside 8 lanes (row_half_mirror), i <-> 15 - i
// inside 16 lanes (row_mirror), then the two 16-lane rows of the half swap
// (v_permlane16_swap with both operands the same value returns the values of
// the row pair).  Each step pairs disjoint lane groups, so after the five
// steps every lane holds the reduction over its half.
constexpr int kDppXor1 = 0xb1, kDppXor2 = 0x4e, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ uint64_t half_max_u64(uint64_t k) {
  k = max_u64(k, dpp64<kDppXor1>(k));
  k = max_u64(k, dpp64<kDppXor2>(k));
  k = max_u64(k, dpp64<kDppHalfMirror>(k));
  k = max_u64(k, dpp64<kDppMirror>(k));
  const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)k, (uint32_t)k, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(k >> 32), (uint32_t)(k >> 32), false, false);
  return max_u64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);
}

__device__ __forceinline__ float half_sum_f32(float v) {
  v += __uint_as_float(dpp32<kDppXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<kDppXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<kDppHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<kDppMirror>(__float_as_uint(v)));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// k-round selection + softmax of one token held by 32 lanes (half a wave;
// both halves of a wave run the same instructions on their own tokens).
// v[i] is the logit of expert e = h + 32*i, h = lane % 32 (e >= E ignored).
// Each round takes the largest remaining key of the half (branch-free), and
// half-lane j keeps the key of round j; half-lane j (< k) writes slot j.
template <int NV>
__device__ __forceinline__ void topk_softmax_half(const float (&v)[NV], int E, int k, bool active,
                                                  int32_t* idx_out, float* w_out) {
  const int h = lane_id() & 31;
  uint64_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) key[i] = (h + 32 * i) < E ? topk_key(v[i], h + 32 * i) : 0ull;
  uint64_t mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) best = max_u64(best, key[i]);
    best = half_max_u64(best);
    mine = (h == j) ? best : mine;
#pragma unroll
    for (int i = 0; i < NV; ++i) key[i] = (key[i] == best) ? 0ull : key[i];
  }
  const float z = key_value(mine);
  const float zmax = __shfl(z, lane_id() & 32, kWave);  // slot 0 of this half
  const float ex = (h < k) ? expf(z - zmax) : 0.f;
  const float sum = half_sum_f32(ex);
  if (active && h < k) {
    idx_out[h] = key_expert(mine);
    w_out[h] = ex / sum;
  }
}

int route_nb(int E) { return E <= 32 ? 1 : E <= 64 ? 2 : E <= 128 ? 4 : 8; }

// ---------------------------------------------------------------------------
// bf16: sliced router GEMM (partial logits), then sum + top-k
// ---------------------------------------------------------------------------
constexpr int kRtTokens = 128;  // tokens per workgroup: 4 waves x 32
constexpr int kRtMaxRows = 512;  // rows of W_r per slice at most (x fragments held in registers)

// Slice count S (slice HS = H / S rows, a multiple of 64): the fewest slices
// whose W_r copy fits 128 KB of LDS and whose x fragments fit the registers,
// then more while the grid has fewer workgroups than CUs.
int route_slices(int T, int H, int E) {
  const int EP = 32 * route_nb(E);
  const int units = H / 64;
  const int tiles = (T + kRtTokens - 1) / kRtTokens;
  int S = units;
  for (int d = 1; d <= units; ++d) {
    const int HS = H / d;
    if (units % d == 0 && HS <= kRtMaxRows && (size_t)HS * EP * 2 <= 128 * 1024) {
      S = d;
      break;
    }
  }
  for (int d = S + 1; d <= units && tiles * S < kCUs; ++d)
    if (units % d == 0) S = d;
  return S;
}
size_t route_ws_bytes(int T, int H, int E) {
  return (size_t)route_slices(T, H, E) * T * E * sizeof(float);
}

// LDS copy of a W_r slice: row h (= k of the product) holds EP bf16 (experts,
// zero past E) as 16-byte chunks; logical chunk c sits at c ^ swz(h), which
// spreads the four rows a transposing read touches over the bank line.
template <int NB>
__device__ __forceinline__ int rt_swz(int h) { return ((h & 3) << 2) & (4 * NB - 1); }

// B fragment of k16-step j, expert block nb: lane l gets expert 32 nb + l % 32,
// k = 16 j + 8 (l / 32) + 0..7, from two transposing reads (rows k and k + 4
// of each 16-lane group): within a group, lane i points at row
// 16 j + 8 (g / 2) + i / 4 and column 32 nb + 16 (g % 2) + 4 (i % 4).
template <int NB>
__device__ __forceinline__ bf16x8_t rt_frag(const bf16_t* s_w, int j, int nb, int lane) {
  constexpr int EP = 32 * NB;
  const int g = lane >> 4, i = lane & 15;
  const int h = 16 * j + 8 * (g >> 1) + (i >> 2);  // h % 4 == (i >> 2) % 4, also for h + 4
  const int c = (4 * nb + 2 * (g & 1) + ((i & 3) >> 1)) ^ rt_swz<NB>(h);
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const auto* q = (const __attribute__((address_space(3))) char*)(
      (const __attribute__((address_space(3))) void*)s_w) + (h * EP + c * 8 + 4 * (i & 1)) * 2;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)q);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 4 * EP * 2));
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// part[(s T + t) E + e] = sum over h in slice s (ascending, in MFMA k-steps) of x[t][h] W_r[h][e].
template <int NB, int NSMAX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void route_part_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int T, int H,
                       int E, int HS, float* __restrict__ part) {
  constexpr int EP = 32 * NB;
  constexpr int CPR = EP / 8;  // 16-byte chunks per LDS row
  extern __shared__ __align__(16) bf16_t s_w[];  // [HS][EP]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int sl = blockIdx.y, h0 = sl * HS;
  const int nstep = HS / 16;
  const int t0 = blockIdx.x * kRtTokens + wave * 32;

  // Load order: this thread's chunks of the W_r slice (at most 32: the slice
  // is at most 128 KB), then the x fragments of the whole slice, all in
  // flight together; the LDS stores of the slice wait only for the W_r loads
  // (older in the in-order memory counter), and each MFMA step only for its
  // own x fragment, so the MFMAs overlap the x stream.
  //   x: lane row t0 + l % 32 (clamped into range; rows past T are computed but
  //   never stored), k = 16 j + 8 (l / 32) + 0..7.
  const int nchunk = HS * CPR;
  constexpr int kMaxChunks = 128 * 1024 / 16 / 256;
  const bool vec = E % 8 == 0;
  u32x4_t wv[kMaxChunks];
  if (vec) {
#pragma unroll
    for (int u = 0; u < kMaxChunks; ++u) {
      const int c = threadIdx.x + u * 256;
      const int h = c / CPR, ch = c % CPR;
      wv[u] = (c < nchunk && ch * 8 < E)
                  ? *reinterpret_cast<const u32x4_t*>(w + (size_t)(h0 + h) * E + ch * 8)
                  : u32x4_t{};
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  int trow = min(t0 + (lane & 31), T - 1);
  const bf16_t* xa = x + (size_t)trow * H + h0 + (lane >> 5) * 8;
  bf16x8_t a[NSMAX];
#pragma unroll
  for (int j = 0; j < NSMAX; ++j) a[j] = *reinterpret_cast<const bf16x8_t*>(xa + 16 * min(j, nstep - 1));
  __builtin_amdgcn_sched_barrier(0);

  // W_r[h0 .. h0 + HS) -> s_w
  if (vec) {
#pragma unroll
    for (int u = 0; u < kMaxChunks; ++u) {
      const int c = threadIdx.x + u * 256;
      if (c >= nchunk) break;
      const int h = c / CPR, ch = c % CPR;
      *reinterpret_cast<u32x4_t*>(s_w + h * EP + ((ch ^ rt_swz<NB>(h)) * 8)) = wv[u];
    }
  } else {
    for (int i = threadIdx.x; i < HS * EP; i += 256) {
      const int h = i / EP, e = i % EP;
      s_w[h * EP + (((e >> 3) ^ rt_swz<NB>(h)) << 3) + (e & 7)] =
          e < E ? w[(size_t)(h0 + h) * E + e] : bf16_t(0);
    }
  }
  __syncthreads();

  f32x16_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16_t{};
#pragma unroll
  for (int j = 0; j < NSMAX; ++j) {
    // steps past the slice multiply zeros (by a fragment of step 0)
    const bool on = j < nstep;
    const bf16x8_t av = on ? a[j] : bf16x8_t{};
    const int js = on ? j : 0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, rt_frag<NB>(s_w, js, nb, lane), acc[nb], 0,
                                                        0, 0);
  }
  float* ps = part + (size_t)sl * T * E;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int t = t0 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      const int e = nb * 32 + (lane & 31);
      if (t < T && e < E) ps[(size_t)t * E + e] = acc[nb][q];
    }
}

// Logits z[t][e] = sum over slices s (ascending) of part[s][t][e] (+ bias[e]),
// then the top-k.  Two tokens per wave, one per half.
template <int NB>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ part, int S,
                                                         int T, int E, int k,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (2 * pair >= T) return;
  const int t = 2 * pair + ((threadIdx.x >> 5) & 1);
  const bool active = t < T;
  const int tr = active ? t : T - 1;
  const int h32 = lane_id() & 31;
  float v[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) v[i] = 0.f;
  // four slices' loads in flight at a time, added in slice order
  for (int s0 = 0; s0 < S; s0 += 4) {
    float pv[4][NB];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* ps = part + ((size_t)min(s0 + u, S - 1) * T + tr) * E;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int e = h32 + 32 * i;
        pv[u][i] = (e < E) ? ps[e] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + u < S) {
#pragma unroll
        for (int i = 0; i < NB; ++i) v[i] += pv[u][i];
      }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int e = h32 + 32 * i;
    if (e < E) {
      if (bias != nullptr) v[i] += bias[e];
      if (logits != nullptr && active) logits[(size_t)t * E + e] = v[i];
    }
  }
  topk_softmax_half<NB>(v, E, k, active, topk_idx + (size_t)tr * k, topk_w + (size_t)tr * k);
}

// ---------------------------------------------------------------------------
// fp32: one wave per token, plain FMA dot products in h order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_f32_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ w_router,
                                                        const float* __restrict__ bias, int T,
                                                        int H, int E, int k,
                                                        float* __restrict__ logits,
                                                        int32_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_w) {
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);  // two tokens per wave
  if (2 * pair >= T) return;
  const int t = 2 * pair + ((threadIdx.x >> 5) & 1);
  const bool active = t < T;
  const int tr = active ? t : T - 1;
  const int h32 = lane_id() & 31;
  const float* xr = x + (size_t)tr * H;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = h32 + 32 * i;
    float z = 0.f;
    if (e < E) {
      for (int h = 0; h < H; ++h) z = fmaf(xr[h], w_router[(size_t)h * E + e], z);
      if (bias != nullptr) z += bias[e];
      if (logits != nullptr && active) logits[(size_t)t * E + e] = z;
    }
    v[i] = z;
  }
  topk_softmax_half<8>(v, E, k, active, topk_idx + (size_t)tr * k, topk_w + (size_t)tr * k);
}

__global__ __launch_bounds__(256) void route_from_logits_kernel(const float* __restrict__ logits,
                                                                int T, int E, int k,
                                                                int32_t* __restrict__ topk_idx,
                                                                float* __restrict__ topk_w) {
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (2 * pair >= T) return;
  const int t = 2 * pair + ((threadIdx.x >> 5) & 1);
  const bool active = t < T;
  const int tr = active ? t : T - 1;
  const int h32 = lane_id() & 31;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = h32 + 32 * i;
    v[i] = (e < E) ? logits[(size_t)tr * E + e] : 0.f;
  }
  topk_softmax_half<8>(v, E, k, active, topk_idx + (size_t)tr * k, topk_w + (size_t)tr * k);
}

// ---------------------------------------------------------------------------
// Transpose [rows, cols] -> [cols, rows] through a 32x33 LDS tile.
// ---------------------------------------------------------------------------
template <typename U>
__global__ __launch_bounds__(256) void transpose_kernel(const U* __restrict__ src,
                                                        U* __restrict__ dst, int rows, int cols) {
  __shared__ U tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[(size_t)r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) dst[(size_t)c * rows + r] = tile[tx][i];
  }
}

hipError_t launch_transpose(const void* src, void* dst, int rows, int cols, int elem_bytes,
                            hipStream_t s) {
  const dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  if (elem_bytes == 2)
    transpose_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, rows,
                                                     cols);
  else
    transpose_kernel<uint32_t><<<grid, 256, 0, s>>>((const uint32_t*)src, (uint32_t*)dst, rows,
                                                     cols);
  return hipGetLastError();
}

hipError_t launch_route_bf16(const bf16_t* x, const bf16_t* w_router, const float* bias, int T,
                             int H, int E, int k, float* logits, int32_t* topk_idx, float* topk_w,
                             float* part_ws, hipStream_t s) {
  const int nb = route_nb(E);
  const int S = route_slices(T, H, E);
  const int HS = H / S;
  const dim3 grid((T + kRtTokens - 1) / kRtTokens, S);
  const size_t lds = (size_t)HS * 32 * nb * sizeof(bf16_t);
  ProfScope ps(MOE_KERNEL_ROUTE, s);
#define MOE_RT_CASE(NB)                                                                        \
  do {                                                                                         \
    if (HS <= 256)                                                                             \
      route_part_kernel<NB, 16><<<grid, 256, lds, s>>>(x, w_router, T, H, E, HS, part_ws);     \
    else                                                                                       \
      route_part_kernel<NB, 32><<<grid, 256, lds, s>>>(x, w_router, T, H, E, HS, part_ws);     \
    route_topk_kernel<NB><<<(T + 7) / 8, 256, 0, s>>>(part_ws, S, T, E, k, bias, logits,       \
                                                      topk_idx, topk_w);                      \
  } while (0)
  if (nb == 1) MOE_RT_CASE(1);
  else if (nb == 2) MOE_RT_CASE(2);
  else if (nb == 4) MOE_RT_CASE(4);
  else MOE_RT_CASE(8);
#undef MOE_RT_CASE
  return hipGetLastError();
}

hipError_t launch_route_f32(const float* x, const float* w_router, const float* bias, int T, int H,
                            int E, int k, float* logits, int32_t* topk_idx, float* topk_w,
                            hipStream_t s) {
  ProfScope ps(MOE_KERNEL_ROUTE, s);
  route_f32_kernel<<<(T + 7) / 8, 256, 0, s>>>(x, w_router, bias, T, H, E, k, logits, topk_idx,
                                                topk_w);
  return hipGetLastError();
}

hipError_t launch_route_from_logits(const float* logits, int T, int E, int k, int32_t* topk_idx,
                                    float* topk_w, hipStream_t s) {
  route_from_logits_kernel<<<(T + 7) / 8, 256, 0, s>>>(logits, T, E, k, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
