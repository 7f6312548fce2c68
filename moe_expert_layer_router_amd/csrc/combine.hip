// Combine (weighted unpermute) and the gating backward for gfx950.
//
// The "unpermute" of the dispatcher table (page "FSDPTurbo EP/EFSDP and
// LlamaFactory FSDP2/CP Design", section 3) becomes a per-token gather-reduce:
// one wave owns one token, reads its k grouped rows with 16-byte vectors and
// sums them in fp32 in slot order j = 0..k-1.  No atomics, so the result is
// deterministic and independent of the launch shape.
#include "common.h"

namespace moe {

// 16 bytes of a row as fp32: 8 bf16 or 4 fp32 elements.
template <bool BF16>
struct Vec {
  static constexpr int N = BF16 ? 8 : 4;
  __device__ static void load(const void* base, size_t elem, float* f) {
    const uint4 v = *reinterpret_cast<const uint4*>((const char*)base + elem * (BF16 ? 2 : 4));
    if constexpr (BF16) {
      unpack8(v, f);
    } else {
      f[0] = __uint_as_float(v.x);
      f[1] = __uint_as_float(v.y);
      f[2] = __uint_as_float(v.z);
      f[3] = __uint_as_float(v.w);
    }
  }
  __device__ static void store(void* base, size_t elem, const float* f) {
    uint4 v;
    if constexpr (BF16) {
      v = pack8(f);
    } else {
      v = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                     __float_as_uint(f[3]));
    }
    *reinterpret_cast<uint4*>((char*)base + elem * (BF16 ? 2 : 4)) = v;
  }
};

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_perm,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ dest_row,
                                                      const float* __restrict__ addend, int T,
                                                      int H, int k, void* __restrict__ y) {
  using V = Vec<BF16>;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  int d = -1;
  float w = 1.f;
  if (lane < k) {
    d = dest_row[(size_t)t * k + lane];
    if (topk_w != nullptr) w = topk_w[(size_t)t * k + lane];
  }
  const int nch = H / V::N;
  // Wave-uniform trip count: every lane joins every shuffle.
  for (int c0 = 0; c0 < nch; c0 += kWave) {
    const int c = c0 + lane;
    const bool on = c < nch;
    float acc[V::N];
#pragma unroll
    for (int i = 0; i < V::N; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int dj = __shfl(d, j, kWave);
      const float wj = __shfl(w, j, kWave);
      if (dj < 0 || !on) continue;
      float v[V::N];
      V::load(y_perm, (size_t)dj * H + (size_t)c * V::N, v);
#pragma unroll
      for (int i = 0; i < V::N; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
    }
    if (!on) continue;
    if (addend != nullptr) {
      const float4* ad = reinterpret_cast<const float4*>(addend + (size_t)t * H + (size_t)c * V::N);
#pragma unroll
      for (int q = 0; q < V::N / 4; ++q) {
        const float4 a = ad[q];
        acc[4 * q] += a.x;
        acc[4 * q + 1] += a.y;
        acc[4 * q + 2] += a.z;
        acc[4 * q + 3] += a.w;
      }
    }
    V::store(y, (size_t)t * H + (size_t)c * V::N, acc);
  }
}

// dy_perm[dest] = w * dy[t];  d_topk_w[t, j] = <dy[t], y_perm[dest]>.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const void* __restrict__ dy,
                                                          const void* __restrict__ y_perm,
                                                          const float* __restrict__ topk_w,
                                                          const int32_t* __restrict__ dest_row,
                                                          int T, int H, int k,
                                                          void* __restrict__ dy_perm,
                                                          float* __restrict__ d_topk_w) {
  using V = Vec<BF16>;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const int nch = H / V::N;
  for (int j = 0; j < k; ++j) {
    const int d = dest_row[(size_t)t * k + j];
    if (d < 0) {
      if (lane == 0) d_topk_w[(size_t)t * k + j] = 0.f;
      continue;
    }
    const float w = topk_w[(size_t)t * k + j];
    float dot = 0.f;
    for (int c = lane; c < nch; c += kWave) {
      float g[V::N], v[V::N];
      V::load(dy, (size_t)t * H + (size_t)c * V::N, g);
      V::load(y_perm, (size_t)d * H + (size_t)c * V::N, v);
#pragma unroll
      for (int i = 0; i < V::N; ++i) {
        dot = fmaf(g[i], v[i], dot);
        g[i] *= w;
      }
      V::store(dy_perm, (size_t)d * H + (size_t)c * V::N, g);
    }
    dot = wave_sum(dot);
    if (lane == 0) d_topk_w[(size_t)t * k + j] = dot;
  }
}

// Router backward, one wave per token:
//   dz_j = w_j (dw_j - sum_l w_l dw_l) on the kept experts, 0 elsewhere;
//   dx_router[t] = sum_j dz_j * W_r[:, idx_j]   (rows of the transposed W_r);
//   bf16 path also writes dz split as bf16 hi + lo ([T, 2E]) for the MFMA
//   product x^T . dz.
template <bool BF16>
__global__ __launch_bounds__(256) void route_bwd_dz_kernel(
    const float* __restrict__ d_topk_w, const float* __restrict__ topk_w,
    const int32_t* __restrict__ topk_idx, const void* __restrict__ w_router_t, int T, int H,
    int E, int k, float* __restrict__ d_logits, float* __restrict__ dx_router,
    bf16_t* __restrict__ dz_hilo) {
  using V = Vec<BF16>;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  float w = 0.f, dw = 0.f;
  int id = -1;
  if (lane < k) {
    w = topk_w[(size_t)t * k + lane];
    dw = d_topk_w[(size_t)t * k + lane];
    id = topk_idx[(size_t)t * k + lane];
  }
  const float inner = wave_sum(w * dw);
  const float dz = w * (dw - inner);
  for (int e0 = 0; e0 < E; e0 += kWave) {
    const int e = e0 + lane;
    float v = 0.f;
    for (int j = 0; j < k; ++j) {
      const int ij = __shfl(id, j, kWave);
      const float dj = __shfl(dz, j, kWave);
      if (ij == e) v = dj;
    }
    if (e >= E) continue;
    d_logits[(size_t)t * E + e] = v;
    if (dz_hilo != nullptr) {
      const bf16_t hi = f2bf(v);
      const bf16_t lo = f2bf(v - bf2f(hi));
      dz_hilo[(size_t)t * 2 * E + e] = hi;
      dz_hilo[(size_t)t * 2 * E + E + e] = lo;
    }
  }
  if (dx_router == nullptr) return;
  const int nch = H / V::N;
  for (int c0 = 0; c0 < nch; c0 += kWave) {
    const int c = c0 + lane;
    const bool on = c < nch;
    float acc[V::N];
#pragma unroll
    for (int i = 0; i < V::N; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int ij = __shfl(id, j, kWave);
      const float dj = __shfl(dz, j, kWave);
      if (!on) continue;
      float v[V::N];
      V::load(w_router_t, (size_t)ij * H + (size_t)c * V::N, v);
#pragma unroll
      for (int i = 0; i < V::N; ++i) acc[i] = fmaf(dj, v[i], acc[i]);
    }
    if (!on) continue;
    float4* out = reinterpret_cast<float4*>(dx_router + (size_t)t * H + (size_t)c * V::N);
#pragma unroll
    for (int q = 0; q < V::N / 4; ++q)
      out[q] = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  }
}

// fp32 path: dw_router[h, e] = sum_t x[t, h] * d_logits[t, e], t ascending.
__global__ __launch_bounds__(256) void dw_router_f32_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ dz, int T,
                                                            int H, int E,
                                                            float* __restrict__ dw) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= H * E) return;
  const int h = i / E, e = i % E;
  float acc = 0.f;
  for (int t = 0; t < T; ++t) acc = fmaf(x[(size_t)t * H + h], dz[(size_t)t * E + e], acc);
  dw[i] = acc;
}

// dw_router[h, e] = sum over splits s (ascending) of P[s][h][e] + P[s][h][E + e].
__global__ __launch_bounds__(256) void dw_router_reduce_kernel(const float* __restrict__ part,
                                                               int nsplit, int H, int E,
                                                               float* __restrict__ dw) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= H * E) return;
  const int h = i / E, e = i % E;
  float acc = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float* p = part + ((size_t)sp * H + h) * 2 * E;
    acc += p[e];
    acc += p[E + e];
  }
  dw[i] = acc;
}

hipError_t launch_combine(const void* y_perm, const float* topk_w, const int32_t* dest_row,
                          const float* addend, int T, int H, int k, bool bf16, void* y,
                          hipStream_t s) {
  const int blocks = (T + 3) / 4;
  ProfScope ps(MOE_KERNEL_COMBINE, s);
  if (bf16)
    combine_kernel<true><<<blocks, 256, 0, s>>>(y_perm, topk_w, dest_row, addend, T, H, k, y);
  else
    combine_kernel<false><<<blocks, 256, 0, s>>>(y_perm, topk_w, dest_row, addend, T, H, k, y);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dy, const void* y_perm, const float* topk_w,
                              const int32_t* dest_row, int T, int H, int k, bool bf16,
                              void* dy_perm, float* d_topk_w, hipStream_t s) {
  const int blocks = (T + 3) / 4;
  ProfScope ps(MOE_KERNEL_COMBINE_BWD, s);
  if (bf16)
    combine_bwd_kernel<true><<<blocks, 256, 0, s>>>(dy, y_perm, topk_w, dest_row, T, H, k,
                                                     dy_perm, d_topk_w);
  else
    combine_bwd_kernel<false><<<blocks, 256, 0, s>>>(dy, y_perm, topk_w, dest_row, T, H, k,
                                                      dy_perm, d_topk_w);
  return hipGetLastError();
}

hipError_t launch_route_bwd_dz(const float* d_topk_w, const float* topk_w,
                               const int32_t* topk_idx, const void* w_router_t, int T, int H, int E,
                               int k, bool bf16, float* d_logits, float* dx_router,
                               bf16_t* dz_hilo, hipStream_t s) {
  const int blocks = (T + 3) / 4;
  ProfScope ps(MOE_KERNEL_ROUTE_BWD_DZ, s);
  if (bf16)
    route_bwd_dz_kernel<true><<<blocks, 256, 0, s>>>(d_topk_w, topk_w, topk_idx, w_router_t, T,
                                                      H, E, k, d_logits, dx_router, dz_hilo);
  else
    route_bwd_dz_kernel<false><<<blocks, 256, 0, s>>>(d_topk_w, topk_w, topk_idx, w_router_t, T,
                                                       H, E, k, d_logits, dx_router, dz_hilo);
  return hipGetLastError();
}

hipError_t launch_dw_router_f32(const float* x, const float* d_logits, int T, int H, int E,
                                float* dw_router, hipStream_t s) {
  dw_router_f32_kernel<<<(H * E + 255) / 256, 256, 0, s>>>(x, d_logits, T, H, E, dw_router);
  return hipGetLastError();
}

hipError_t launch_dw_router_reduce(const float* partials, int nsplit, int H, int E,
                                   float* dw_router, hipStream_t s) {
  dw_router_reduce_kernel<<<(H * E + 255) / 256, 256, 0, s>>>(partials, nsplit, H, E,
                                                               dw_router);
  return hipGetLastError();
}

}  // namespace moe
