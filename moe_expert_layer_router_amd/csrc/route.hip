// Router GEMM + top-k softmax gating for gfx950.
//
// The pages leave the router open; the layer uses the plain top-k router:
// logits z = x . W_r (+ bias), the k largest logits per token (equal logits go
// to the lower expert id, slot order = logit descending then id ascending),
// gate weights = softmax over the kept logits (identical to a softmax over all
// experts renormalised over the kept ones).
//
// bf16 path: one workgroup (8 waves) owns 32 tokens and all E <= 256 experts.
// The eight waves split the hidden dimension H into interleaved 64-wide
// chunks and run bf16 32x32x16 MFMAs straight from global memory (x rows, and
// W_r repacked in MFMA fragment order, which is small and stays in L2), with
// the next chunk's loads in flight during the current chunk's MFMAs; the
// partial logit tiles are summed through LDS in a fixed order, so logits are
// deterministic.  Then each half wave takes one token: every lane holds up to
// eight logits (expert e = lane % 32 + 32 i) and k rounds of a branch-free
// arg-max over unique (logit, id) keys pick the experts.
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

// W_r [H, E] -> MFMA B fragments: for every k16-step sg and 32-expert block nb
// one 1 KB record whose lane l holds W_r[16 sg + 8 (l / 32) + q][32 nb + l % 32],
// q = 0..7 (zero for experts >= E), so each fragment load of the router is
// one contiguous 1 KB read.
__global__ __launch_bounds__(256) void pack_router_kernel(const bf16_t* __restrict__ w,
                                                          bf16_t* __restrict__ wp, int H, int E,
                                                          int NB) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= (H / 16) * NB * 64) return;
  const int l = i & 63, nb = (i >> 6) % NB, sg = (i >> 6) / NB;
  const int e = nb * 32 + (l & 31);
  const int h0 = sg * 16 + (l >> 5) * 8;
  u32x4_t out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = e < E ? w[(size_t)(h0 + 2 * q) * E + e] : 0u;
    const uint32_t hi = e < E ? w[(size_t)(h0 + 2 * q + 1) * E + e] : 0u;
    out[q] = lo | (hi << 16);
  }
  *reinterpret_cast<u32x4_t*>(wp + (size_t)i * 8) = out;
}

int route_nb(int E) { return E <= 32 ? 1 : E <= 64 ? 2 : E <= 128 ? 4 : 8; }
size_t route_ws_bytes(int H, int E) { return (size_t)H * 32 * route_nb(E) * sizeof(bf16_t); }

// ---------------------------------------------------------------------------
// bf16: MFMA router GEMM fused with top-k
// ---------------------------------------------------------------------------
constexpr int kRouteTB = 32;  // tokens per workgroup
constexpr int kRouteWaves = 8;

// Operands of one k chunk (CH k16-steps) for the 32 tokens x (32 NB) experts
// tile: A fragments (x rows) and B fragments (rows of W_r^T).
template <int CH, int NB>
struct RouteChunk {
  bf16x8_t a[CH];
  bf16x8_t b[CH][NB];
};

// x fragments: xa points at this lane's row and k offset 8 (lane / 32);
// W fragments: wpl points at this lane's 16 bytes of the packed record of
// (k16-step 0, block 0); records are 512 elements apart.
template <int CH, int NB>
__device__ __forceinline__ void route_load(RouteChunk<CH, NB>& c, const bf16_t* xa,
                                           const bf16_t* wpl, int k0) {
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    c.a[s] = *reinterpret_cast<const bf16x8_t*>(xa + k0 + 16 * s);
    const bf16_t* rec = wpl + (size_t)((k0 >> 4) + s) * NB * 512;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) c.b[s][nb] = *reinterpret_cast<const bf16x8_t*>(rec + nb * 512);
  }
}

// MFMAs of one chunk; a chunk past the end of H (valid == false, uniform)
// contributes zero operands.
template <int CH, int NB>
__device__ __forceinline__ void route_mma(const RouteChunk<CH, NB>& c, bool valid,
                                          f32x16_t (&acc)[NB]) {
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    const bf16x8_t a = valid ? c.a[s] : bf16x8_t{};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, c.b[s][nb], acc[nb], 0, 0, 0);
  }
}

template <int NB>  // NB = number of 32-expert column blocks (E <= 32*NB)
__global__ __launch_bounds__(kRouteWaves * kWave)
__attribute__((amdgpu_waves_per_eu(2, 2))) void route_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wp, const float* __restrict__ bias,
    int T, int H, int E, int k, float* __restrict__ logits, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  constexpr int EP = NB * 32;
  constexpr int CH = NB <= 4 ? 4 : 1;  // k16-steps per chunk (register budget)
  constexpr int KC = 16 * CH;
  constexpr int NTH = kRouteWaves * kWave;
  extern __shared__ float s_part[];  // [4][kRouteTB][EP]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouteTB;
  const int nC = H / KC;  // H % 64 == 0

  int trow = t0 + (lane & 31);
  if (trow >= T) trow = T - 1;  // ragged last block: duplicate a valid row, never stored
  const bf16_t* xa = x + (size_t)trow * H + (lane >> 5) * 8;
  const bf16_t* wpl = wp + lane * 8;  // packed W_r fragments (zero for experts >= E)
  f32x16_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16_t{};

  // Wave w takes chunks w, w + 8, w + 16, ...  Two register buffers alternate
  // (no copies between them) and every wave runs the same trip count with
  // every load issued unconditionally from a clamped, always valid chunk, so
  // each load has a use on every path and stays where it is issued: one chunk
  // is in flight while the previous one feeds the MFMAs.  Chunks past the end
  // of H are multiplied as zeros.
  RouteChunk<CH, NB> A, B;
  const int n_it = (nC + 2 * kRouteWaves - 1) / (2 * kRouteWaves);
  route_load<CH, NB>(A, xa, wpl, min(wave, nC - 1) * KC);
  for (int it = 0; it < n_it; ++it) {
    const int ch = wave + it * 2 * kRouteWaves;
    // The scheduling barriers keep each chunk's loads ahead of the previous
    // chunk's MFMAs (the scheduler would otherwise sink them to their uses).
    route_load<CH, NB>(B, xa, wpl, min(ch + kRouteWaves, nC - 1) * KC);
    __builtin_amdgcn_sched_barrier(0);
    route_mma<CH, NB>(A, ch < nC, acc);
    __builtin_amdgcn_sched_barrier(0);
    route_load<CH, NB>(A, xa, wpl, min(ch + 2 * kRouteWaves, nC - 1) * KC);
    __builtin_amdgcn_sched_barrier(0);
    route_mma<CH, NB>(B, ch + kRouteWaves < nC, acc);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Fixed-order reduction of the eight partial tiles: waves 4..7 store, waves
  // 0..3 add their partner's tile to their own and store, then
  // z = ((s0 + s1) + s2) + s3.
  float* slot = s_part + (wave & 3) * kRouteTB * EP;
  if (wave >= 4) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        slot[row * EP + nb * 32 + (lane & 31)] = acc[nb][q];
      }
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        float* p = slot + row * EP + nb * 32 + (lane & 31);
        *p = acc[nb][q] + *p;
      }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kRouteTB * EP; i += NTH) {
    const int row = i / EP, e = i % EP;
    float z = s_part[i] + s_part[kRouteTB * EP + i];
    z += s_part[2 * kRouteTB * EP + i];
    z += s_part[3 * kRouteTB * EP + i];
    if (bias != nullptr && e < E) z += bias[e];
    s_part[i] = z;
    if (logits != nullptr && e < E && t0 + row < T) logits[(size_t)(t0 + row) * E + e] = z;
  }
  __syncthreads();
  // two tokens per wave: half 0 takes token tt, half 1 token tt + 1
  for (int tt = 2 * wave; tt < kRouteTB; tt += 2 * kRouteWaves) {
    const int ts = tt + (lane >> 5);
    const int t = t0 + ts;
    if (t0 + tt >= T) break;  // wave-uniform
    float v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int e = (lane & 31) + 32 * i;
      v[i] = (e < E) ? s_part[ts * EP + e] : 0.f;
    }
    const bool active = t < T;
    topk_softmax_half<NB>(v, E, k, active, topk_idx + (size_t)(active ? t : 0) * k,
                          topk_w + (size_t)(active ? t : 0) * k);
  }
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
                             bf16_t* wp_ws, hipStream_t s) {
  const int nb = route_nb(E);
  const int nrec = (H / 16) * nb * 64;
  pack_router_kernel<<<(nrec + 255) / 256, 256, 0, s>>>(w_router, wp_ws, H, E, nb);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int blocks = (T + kRouteTB - 1) / kRouteTB;
  ProfScope ps(MOE_KERNEL_ROUTE, s);
#define MOE_ROUTE_CASE(NB)                                                                  \
  route_bf16_kernel<NB><<<blocks, kRouteWaves * kWave, 4 * kRouteTB * NB * 32 * sizeof(float), \
                          s>>>(x, wp_ws, bias, T, H, E, k, logits, topk_idx, topk_w)
  if (nb == 1) MOE_ROUTE_CASE(1);
  else if (nb == 2) MOE_ROUTE_CASE(2);
  else if (nb == 4) MOE_ROUTE_CASE(4);
  else MOE_ROUTE_CASE(8);
#undef MOE_ROUTE_CASE
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
