// Router GEMM + top-k softmax gating for gfx950.
//
// The pages leave the router open; the layer uses the plain top-k router:
// logits z = x . W_r (+ bias), the k largest logits per token (equal logits go
// to the lower expert id, slot order = logit descending then id ascending),
// gate weights = softmax over the kept logits (identical to a softmax over all
// experts renormalised over the kept ones).
//
// bf16 path: one workgroup (4 waves) owns 32 tokens and all E <= 256 experts.
// The four waves split the hidden dimension H into quarters and run bf16
// 32x32x16 MFMAs straight from global memory (x rows and the transposed router
// weight W_r^T, which is small and stays in L2); the four partial logit tiles
// are summed through LDS in a fixed order, so logits are deterministic.  Then
// each wave takes one token at a time: every lane holds up to four logits
// (expert e = lane + 64 i) and k rounds of a wave-wide arg-max butterfly pick
// the experts.
#include "common.h"

#include <math.h>

namespace moe {

// k-round selection + softmax of one token held by one wave.  v[i] is the
// logit of expert e = lane + 64*i (entries with e >= E are ignored).  Lane j
// (< k) writes slot j of idx_out / w_out.
__device__ __forceinline__ void topk_softmax_wave(const float (&v)[4], int E, int k,
                                                  int32_t* idx_out, float* w_out) {
  const int lane = lane_id();
  bool alive[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) alive[i] = (lane + 64 * i) < E;
  float my_val = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (alive[i] && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
    // (value desc, id asc) is a total order, so the butterfly leaves every
    // lane holding the same winner.
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == j) {
      my_val = bv;
      my_id = bi;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (bi == lane + 64 * i) alive[i] = false;
  }
  const float zmax = __shfl(my_val, 0, kWave);
  const float ex = (lane < k) ? expf(my_val - zmax) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    idx_out[lane] = my_id;
    w_out[lane] = ex / sum;
  }
}

// ---------------------------------------------------------------------------
// bf16: MFMA router GEMM fused with top-k
// ---------------------------------------------------------------------------
constexpr int kRouteTB = 32;  // tokens per workgroup

template <int NB>  // NB = number of 32-expert column blocks (E <= 32*NB)
__global__ __launch_bounds__(256) void route_bf16_kernel(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ wt,
                                                         const float* __restrict__ bias, int T,
                                                         int H, int E, int k,
                                                         float* __restrict__ logits,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  constexpr int EP = NB * 32;
  extern __shared__ float s_part[];  // [4 waves][kRouteTB][EP]
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouteTB;
  const int kq = H >> 2;
  const int kbeg = wave * kq;

  int trow = t0 + (lane & 31);
  if (trow >= T) trow = T - 1;  // ragged last block: duplicate a valid row, never stored
  const bf16_t* xa = x + (size_t)trow * H + kbeg + (lane >> 5) * 8;
  const bf16_t* wb[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int e = nb * 32 + (lane & 31);
    if (e >= E) e = E - 1;  // padded experts: valid row, masked below
    wb[nb] = wt + (size_t)e * H + kbeg + (lane >> 5) * 8;
  }
  f32x16_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16_t{};

#pragma unroll 4
  for (int kk = 0; kk < kq; kk += 16) {
    const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xa + kk);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(wb[nb] + kk);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[nb], 0, 0, 0);
    }
  }

  float* mine = s_part + wave * kRouteTB * EP;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      mine[row * EP + nb * 32 + (lane & 31)] = acc[nb][q];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kRouteTB * EP; i += 256) {
    const int row = i / EP, e = i % EP;
    float z = s_part[i] + s_part[kRouteTB * EP + i];
    z += s_part[2 * kRouteTB * EP + i];
    z += s_part[3 * kRouteTB * EP + i];
    if (bias != nullptr && e < E) z += bias[e];
    s_part[i] = z;
    if (logits != nullptr && e < E && t0 + row < T) logits[(size_t)(t0 + row) * E + e] = z;
  }
  __syncthreads();
  for (int tt = wave; tt < kRouteTB; tt += 4) {
    const int t = t0 + tt;
    if (t >= T) break;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      v[i] = (e < E) ? s_part[tt * EP + e] : 0.f;
    }
    topk_softmax_wave(v, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
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
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const float* xr = x + (size_t)t * H;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    float z = 0.f;
    if (e < E) {
      for (int h = 0; h < H; ++h) z = fmaf(xr[h], w_router[(size_t)h * E + e], z);
      if (bias != nullptr) z += bias[e];
      if (logits != nullptr) logits[(size_t)t * E + e] = z;
    }
    v[i] = z;
  }
  topk_softmax_wave(v, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
}

__global__ __launch_bounds__(256) void route_from_logits_kernel(const float* __restrict__ logits,
                                                                int T, int E, int k,
                                                                int32_t* __restrict__ topk_idx,
                                                                float* __restrict__ topk_w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? logits[(size_t)t * E + e] : 0.f;
  }
  topk_softmax_wave(v, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
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
                             bf16_t* wt_ws, hipStream_t s) {
  hipError_t err = launch_transpose(w_router, wt_ws, H, E, 2, s);
  if (err != hipSuccess) return err;
  const int blocks = (T + kRouteTB - 1) / kRouteTB;
  const int nb = (E + 31) / 32;
  ProfScope ps(MOE_KERNEL_ROUTE, s);
#define MOE_ROUTE_CASE(NB)                                                                  \
  route_bf16_kernel<NB><<<blocks, 256, 4 * kRouteTB * NB * 32 * sizeof(float), s>>>(        \
      x, wt_ws, bias, T, H, E, k, logits, topk_idx, topk_w)
  if (nb <= 1) MOE_ROUTE_CASE(1);
  else if (nb <= 2) MOE_ROUTE_CASE(2);
  else if (nb <= 4) MOE_ROUTE_CASE(4);
  else MOE_ROUTE_CASE(8);
#undef MOE_ROUTE_CASE
  return hipGetLastError();
}

hipError_t launch_route_f32(const float* x, const float* w_router, const float* bias, int T, int H,
                            int E, int k, float* logits, int32_t* topk_idx, float* topk_w,
                            hipStream_t s) {
  ProfScope ps(MOE_KERNEL_ROUTE, s);
  route_f32_kernel<<<(T + 3) / 4, 256, 0, s>>>(x, w_router, bias, T, H, E, k, logits, topk_idx,
                                                topk_w);
  return hipGetLastError();
}

hipError_t launch_route_from_logits(const float* logits, int T, int E, int k, int32_t* topk_idx,
                                    float* topk_w, hipStream_t s) {
  route_from_logits_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
