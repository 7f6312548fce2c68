// Combine (weighted unpermute) and the gating backward for gfx950.
//
// The "unpermute" of the dispatcher table (page "FSDPTurbo EP/EFSDP and
// LlamaFactory FSDP2/CP Design", section 3) becomes a per-token gather-reduce:
// one wave owns one token, packs its local slots into the low lanes, issues
// the 16-byte loads of up to four grouped rows x four chunks per lane at once
// and sums them in fp32 in slot order j = 0..k-1.  No atomics, so the result is
// deterministic and independent of the launch shape.
#include "common.h"

namespace moe {

// 16 bytes of a row: 8 bf16 or 4 fp32 elements, held as a native vector.
template <bool BF16>
struct Row {
  static constexpr int N = BF16 ? 8 : 4;
  static constexpr int EB = BF16 ? 2 : 4;
  __device__ static u32x4_t ld(const void* base, size_t elem) {
    return *reinterpret_cast<const u32x4_t*>((const char*)base + elem * EB);
  }
  __device__ static void st(void* base, size_t elem, u32x4_t v) {
    *reinterpret_cast<u32x4_t*>((char*)base + elem * EB) = v;
  }
  // Streaming (non-temporal) forms for rows touched once per call: grouped
  // rows, token rows and the outputs.  They keep the caches for what is
  // re-read (the router weight rows); on the full 128-expert layer they raise
  // the combine from 0.64 to 0.76 of HBM.
  __device__ static u32x4_t ld_s(const void* base, size_t elem) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>((const char*)base + elem * EB));
  }
  __device__ static void st_s(void* base, size_t elem, u32x4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>((char*)base + elem * EB));
  }
  __device__ static void to_f32(u32x4_t v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (BF16) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
      } else {
        f[i] = __uint_as_float(v[i]);
      }
    }
  }
  __device__ static u32x4_t from_f32(const float* f) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = BF16 ? pack_bf2(f[2 * i], f[2 * i + 1]) : __float_as_uint(f[i]);
    return v;
  }
};

// Chunks of 16 bytes per lane per pass and slots whose rows are loaded
// together: all CU x SG row loads of a pass are in flight at once.  Eight
// slots (a top-8 token in one round trip) double the load registers and halve
// the waves per SIMD, which costs more on an EP share (about one local slot
// per token) than it gains on the full layer.
constexpr int kCU = 4;
constexpr int kSG = 4;

// Moves the lanes holding a local slot (d >= 0; lanes >= k hold d = -1) to
// lanes 0..n-1, keeping slot order; returns n.  Lane i then holds that slot's
// row d, weight w and slot index j.  Lanes without a slot all send to lane
// 63, which is never read (n <= k <= 32).
__device__ __forceinline__ int pack_slots(int d, float w, int& dc, float& wc, int& jc) {
  const int lane = lane_id();
  const uint64_t m = __ballot(d >= 0);
  const int rank = __popcll(m & ((1ull << lane) - 1ull));
  const int to = (d >= 0 ? rank : 63) << 2;
  dc = __builtin_amdgcn_ds_permute(to, d);
  wc = __int_as_float(__builtin_amdgcn_ds_permute(to, __float_as_int(w)));
  jc = __builtin_amdgcn_ds_permute(to, lane);
  return __popcll(m);
}

// out[c] = sum over packed slots j < n (ascending) of wc_j * rows[dc_j][c] for
// this lane's chunks c0 + u * 64 + lane; fp32 accumulation.  STREAM: the rows
// are read once (streaming loads).
template <bool BF16, bool STREAM>
__device__ __forceinline__ void gather_rows(const void* __restrict__ rows, int H, int nch, int c0,
                                            int n, int dc, float wc,
                                            float (&acc)[kCU][Row<BF16>::N]) {
  using R = Row<BF16>;
  const int lane = lane_id();
  for (int j0 = 0; j0 < n; j0 += kSG) {
    u32x4_t raw[kSG][kCU];
    float wj[kSG];
#pragma unroll
    for (int s = 0; s < kSG; ++s) {
      const int j = j0 + s;  // < 36: a valid lane index
      const int dj = __shfl(dc, j, kWave);
      wj[s] = (j < n) ? __shfl(wc, j, kWave) : 0.f;
#pragma unroll
      for (int u = 0; u < kCU; ++u) {
        const int c = c0 + u * kWave + lane;
        const size_t e = (size_t)dj * H + (size_t)c * R::N;
        raw[s][u] = (j < n && c < nch) ? (STREAM ? R::ld_s(rows, e) : R::ld(rows, e)) : u32x4_t{};
      }
    }
#pragma unroll
    for (int s = 0; s < kSG; ++s)
#pragma unroll
      for (int u = 0; u < kCU; ++u) {
        float v[R::N];
        R::to_f32(raw[s][u], v);
#pragma unroll
        for (int i = 0; i < R::N; ++i) acc[u][i] = fmaf(wj[s], v[i], acc[u][i]);
      }
  }
}

// y[t] = sum over local slots j (ascending) of w_j * y_perm[dest_j] (+ addend[t]).
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_perm,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ dest_row,
                                                      const float* __restrict__ addend, int T,
                                                      int H, int k, void* __restrict__ y) {
  using R = Row<BF16>;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  int d = -1;
  float w = 1.f;
  if (lane < k) {
    d = dest_row[(size_t)t * k + lane];
    if (topk_w != nullptr) w = topk_w[(size_t)t * k + lane];
  }
  int dc, jc;
  float wc;
  const int n = pack_slots(d, w, dc, wc, jc);
  const int nch = H / R::N;
  for (int c0 = 0; c0 < nch; c0 += kWave * kCU) {
    float acc[kCU][R::N];
#pragma unroll
    for (int u = 0; u < kCU; ++u)
#pragma unroll
      for (int i = 0; i < R::N; ++i) acc[u][i] = 0.f;
    f32x4_t add[kCU][R::N / 4];
    if (addend != nullptr) {
#pragma unroll
      for (int u = 0; u < kCU; ++u) {
        const int c = c0 + u * kWave + lane;
#pragma unroll
        for (int q = 0; q < R::N / 4; ++q)
          add[u][q] = c < nch ? *reinterpret_cast<const f32x4_t*>(addend + (size_t)t * H +
                                                                   (size_t)c * R::N + 4 * q)
                              : f32x4_t{};
      }
    }
    gather_rows<BF16, true>(y_perm, H, nch, c0, n, dc, wc, acc);
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c >= nch) continue;
      if (addend != nullptr) {
#pragma unroll
        for (int i = 0; i < R::N; ++i) acc[u][i] += add[u][i / 4][i % 4];
      }
      R::st_s(y, (size_t)t * H + (size_t)c * R::N, R::from_f32(acc[u]));
    }
  }
}

// dy_perm[dest_j] = w_j * dy[t];  d_topk_w[t, j] = <dy[t], y_perm[dest_j]>
// (0 for slots of other experts).
template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const void* __restrict__ dy,
                                                          const void* __restrict__ y_perm,
                                                          const float* __restrict__ topk_w,
                                                          const int32_t* __restrict__ dest_row,
                                                          int T, int H, int k,
                                                          void* __restrict__ dy_perm,
                                                          float* __restrict__ d_topk_w) {
  using R = Row<BF16>;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  int d = -1;
  float w = 0.f;
  if (lane < k) {
    d = dest_row[(size_t)t * k + lane];
    w = topk_w[(size_t)t * k + lane];
    if (d < 0) d_topk_w[(size_t)t * k + lane] = 0.f;
  }
  int dc, jc;
  float wc;
  const int n = pack_slots(d, w, dc, wc, jc);
  const int nch = H / R::N;
  for (int j0 = 0; j0 < n; j0 += kSG) {
    int dj[kSG];
    float wj[kSG], dot[kSG];
#pragma unroll
    for (int s = 0; s < kSG; ++s) {
      dj[s] = __shfl(dc, j0 + s, kWave);
      wj[s] = __shfl(wc, j0 + s, kWave);
      dot[s] = 0.f;
    }
    for (int c0 = 0; c0 < nch; c0 += kWave * kCU) {
      u32x4_t g[kCU], raw[kSG][kCU];
#pragma unroll
      for (int u = 0; u < kCU; ++u) {
        const int c = c0 + u * kWave + lane;
        g[u] = c < nch ? R::ld_s(dy, (size_t)t * H + (size_t)c * R::N) : u32x4_t{};
#pragma unroll
        for (int s = 0; s < kSG; ++s)
          raw[s][u] = (j0 + s < n && c < nch) ? R::ld_s(y_perm, (size_t)dj[s] * H + (size_t)c * R::N)
                                              : u32x4_t{};
      }
#pragma unroll
      for (int u = 0; u < kCU; ++u) {
        const int c = c0 + u * kWave + lane;
        float gf[R::N];
        R::to_f32(g[u], gf);
#pragma unroll
        for (int s = 0; s < kSG; ++s) {
          float v[R::N], o[R::N];
          R::to_f32(raw[s][u], v);
#pragma unroll
          for (int i = 0; i < R::N; ++i) {
            dot[s] = fmaf(gf[i], v[i], dot[s]);
            o[i] = wj[s] * gf[i];
          }
          if (j0 + s < n && c < nch) R::st_s(dy_perm, (size_t)dj[s] * H + (size_t)c * R::N, R::from_f32(o));
        }
      }
    }
#pragma unroll
    for (int s = 0; s < kSG; ++s) {
      const float sum = wave_sum(dot[s]);
      const int js = __shfl(jc, j0 + s, kWave);
      if (lane == 0 && j0 + s < n) d_topk_w[(size_t)t * k + js] = sum;
    }
  }
}

// Input gradient, one wave per token:
//   dx[t] = sum over local slots of dx_perm[dest_j]  +  sum_j dz_j * W_r^T[idx_j]
// with dz_j = w_j (dw_j - sum_l w_l dw_l) computed in the wave (lanes >= k
// hold w = 0, so their dz is 0).
template <bool BF16>
__global__ __launch_bounds__(256) void combine_dx_kernel(
    const void* __restrict__ dx_perm, const int32_t* __restrict__ dest_row,
    const float* __restrict__ d_topk_w, const float* __restrict__ topk_w,
    const int32_t* __restrict__ topk_idx, const void* __restrict__ w_router_t, int T, int H,
    int k, void* __restrict__ dx) {
  using R = Row<BF16>;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  int d = -1, id = -1;
  float w = 0.f, dw = 0.f;
  if (lane < k) {
    d = dest_row[(size_t)t * k + lane];
    w = topk_w[(size_t)t * k + lane];
    dw = d_topk_w[(size_t)t * k + lane];
    id = topk_idx[(size_t)t * k + lane];
  }
  const float inner = wave_sum(w * dw);
  const float dz = w * (dw - inner);
  int dc, jc;
  float wc;
  const int n = pack_slots(d, 1.f, dc, wc, jc);
  const int nch = H / R::N;
  for (int c0 = 0; c0 < nch; c0 += kWave * kCU) {
    float acc[kCU][R::N];
#pragma unroll
    for (int u = 0; u < kCU; ++u)
#pragma unroll
      for (int i = 0; i < R::N; ++i) acc[u][i] = 0.f;
    gather_rows<BF16, true>(dx_perm, H, nch, c0, n, dc, wc, acc);
    gather_rows<BF16, false>(w_router_t, H, nch, c0, k, id, dz, acc);
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < nch) R::st_s(dx, (size_t)t * H + (size_t)c * R::N, R::from_f32(acc[u]));
    }
  }
}

// Router backward, one wave per token:
//   dz_j = w_j (dw_j - sum_l w_l dw_l) on the kept experts, 0 elsewhere;
//   dx_router[t] = sum_j dz_j * W_r[:, idx_j]   (rows of the transposed W_r);
//   bf16 path also writes dz split as bf16 hi + lo ([T, 2E]) for the MFMA
//   product x^T . dz.
// DX: the router input gradient is wanted (its row gather needs registers the
// logit-gradient-only form does without).
template <bool BF16, bool DX>
__global__ __launch_bounds__(256) void route_bwd_dz_kernel(
    const float* __restrict__ d_topk_w, const float* __restrict__ topk_w,
    const int32_t* __restrict__ topk_idx, const void* __restrict__ w_router_t, int T, int H,
    int E, int k, float* __restrict__ d_logits, float* __restrict__ dx_router,
    bf16_t* __restrict__ dz_hilo) {
  using R = Row<BF16>;
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
    // slot j's (expert, dz) broadcast from lane j (uniform j: a scalar read);
    // an expert named by several slots gets their sum, in slot order
    for (int j = 0; j < k; ++j) {
      const int ij = __builtin_amdgcn_readlane(id, j);
      const float dj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dz), j));
      v += (ij == e) ? dj : 0.f;
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
  if constexpr (!DX) return;
  const int nch = H / R::N;
  for (int c0 = 0; c0 < nch; c0 += kWave * kCU) {
    float acc[kCU][R::N];
#pragma unroll
    for (int u = 0; u < kCU; ++u)
#pragma unroll
      for (int i = 0; i < R::N; ++i) acc[u][i] = 0.f;
    gather_rows<BF16, false>(w_router_t, H, nch, c0, k, id, dz, acc);
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c >= nch) continue;
#pragma unroll
      for (int q = 0; q < R::N / 4; ++q)
        *reinterpret_cast<f32x4_t*>(dx_router + (size_t)t * H + (size_t)c * R::N + 4 * q) =
            f32x4_t{acc[u][4 * q], acc[u][4 * q + 1], acc[u][4 * q + 2], acc[u][4 * q + 3]};
    }
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

// dw_router[h, e] = sum over splits s (ascending) of P[s][h][e] (folded
// partials [nsplit, H, E], hi + lo added by the product) or of
// P[s][h][e] + P[s][h][E + e] ([nsplit, H, 2E]).
__global__ __launch_bounds__(256) void dw_router_reduce_kernel(const float* __restrict__ part,
                                                               int nsplit, int H, int E,
                                                               int folded,
                                                               float* __restrict__ dw) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= H * E) return;
  float acc = 0.f;
  if (folded) {
    for (int sp = 0; sp < nsplit; ++sp) acc += part[(size_t)sp * H * E + i];
  } else {
    const int h = i / E, e = i % E;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float* p = part + ((size_t)sp * H + h) * 2 * E;
      acc += p[e];
      acc += p[E + e];
    }
  }
  dw[i] = acc;
}

// Folded partials, 4 outputs per lane: 64 float4 outputs per workgroup, wave
// w summing splits w, w + 4, ... (ascending), then the four wave sums in wave
// order.  Every wave keeps its split loads in flight together.
__global__ __launch_bounds__(256) void dw_router_reduce4_kernel(const f32x4_t* __restrict__ part,
                                                                int nsplit, int n4,
                                                                f32x4_t* __restrict__ dw) {
  __shared__ f32x4_t s[3][64];
  const int c = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + c;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (i < n4) {
    int sp = w;
    for (; sp + 12 < nsplit; sp += 16) {  // four splits of this wave at a time
      const f32x4_t a = part[(size_t)sp * n4 + i], b = part[(size_t)(sp + 4) * n4 + i];
      const f32x4_t d = part[(size_t)(sp + 8) * n4 + i], e = part[(size_t)(sp + 12) * n4 + i];
      acc += a;
      acc += b;
      acc += d;
      acc += e;
    }
    for (; sp < nsplit; sp += 4) acc += part[(size_t)sp * n4 + i];
  }
  if (w > 0) s[w - 1][c] = acc;
  __syncthreads();
  if (w == 0 && i < n4) dw[i] = ((acc + s[0][c]) + s[1][c]) + s[2][c];
}

hipError_t launch_combine(const void* y_perm, const float* topk_w, const int32_t* dest_row,
                          const float* addend, int T, int H, int k, bool bf16, void* y,
                          hipStream_t s) {
  const int blocks = (T + 3) / 4;
  ProfScope ps(addend != nullptr ? MOE_KERNEL_COMBINE_ADD : MOE_KERNEL_COMBINE, s);
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

hipError_t launch_combine_dx(const void* dx_perm, const int32_t* dest_row, const float* d_topk_w,
                             const float* topk_w, const int32_t* topk_idx, const void* w_router_t,
                             int T, int H, int k, bool bf16, void* dx, hipStream_t s) {
  const int blocks = (T + 3) / 4;
  ProfScope ps(MOE_KERNEL_COMBINE_DX, s);
  if (bf16)
    combine_dx_kernel<true><<<blocks, 256, 0, s>>>(dx_perm, dest_row, d_topk_w, topk_w, topk_idx,
                                                    w_router_t, T, H, k, dx);
  else
    combine_dx_kernel<false><<<blocks, 256, 0, s>>>(dx_perm, dest_row, d_topk_w, topk_w, topk_idx,
                                                     w_router_t, T, H, k, dx);
  return hipGetLastError();
}

hipError_t launch_route_bwd_dz(const float* d_topk_w, const float* topk_w,
                               const int32_t* topk_idx, const void* w_router_t, int T, int H, int E,
                               int k, bool bf16, float* d_logits, float* dx_router,
                               bf16_t* dz_hilo, hipStream_t s) {
  const int blocks = (T + 3) / 4;
  ProfScope ps(MOE_KERNEL_ROUTE_BWD_DZ, s);
#define MOE_DZ(B, D)                                                                             \
  route_bwd_dz_kernel<B, D><<<blocks, 256, 0, s>>>(d_topk_w, topk_w, topk_idx, w_router_t, T, H, E, \
                                                   k, d_logits, dx_router, dz_hilo)
  if (bf16) {
    if (dx_router != nullptr) MOE_DZ(true, true); else MOE_DZ(true, false);
  } else {
    if (dx_router != nullptr) MOE_DZ(false, true); else MOE_DZ(false, false);
  }
#undef MOE_DZ
  return hipGetLastError();
}

hipError_t launch_dw_router_f32(const float* x, const float* d_logits, int T, int H, int E,
                                float* dw_router, hipStream_t s) {
  dw_router_f32_kernel<<<(H * E + 255) / 256, 256, 0, s>>>(x, d_logits, T, H, E, dw_router);
  return hipGetLastError();
}

hipError_t launch_dw_router_reduce(const float* partials, int nsplit, int H, int E, bool folded,
                                   float* dw_router, hipStream_t s) {
  if (folded && (H * E) % 4 == 0 && ((uintptr_t)dw_router & 15) == 0 &&
      ((uintptr_t)partials & 15) == 0) {
    const int n4 = H * E / 4;
    dw_router_reduce4_kernel<<<(n4 + 63) / 64, 256, 0, s>>>(
        reinterpret_cast<const f32x4_t*>(partials), nsplit, n4, reinterpret_cast<f32x4_t*>(dw_router));
  } else {
    dw_router_reduce_kernel<<<(H * E + 255) / 256, 256, 0, s>>>(partials, nsplit, H, E,
                                                                 folded ? 1 : 0, dw_router);
  }
  return hipGetLastError();
}

}  // namespace moe
