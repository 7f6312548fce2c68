// fp32 expert FFN, forward and backward: plain kernels, one thread per output
// element, reductions in index order.  This path serves fp32 layers (small
// correctness-sized workloads); the bf16 path runs the MFMA kernels of gemm.hip.
#include "common.h"

namespace moe {

// Expert owning grouped row r: largest e with offsets[e] <= r.
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E_l, int r) {
  int lo = 0, hi = E_l - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void gateup_f32_kernel(const float* __restrict__ x, const int32_t* __restrict__ offsets,
                                  int E_l, int R_cap, int H, int I, const float* __restrict__ wg,
                                  const float* __restrict__ wu, float* __restrict__ gu,
                                  float* __restrict__ hout) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int r = (int)(i / I), c = (int)(i % I);
  if (r >= R_cap || r >= offsets[E_l]) return;
  const int e = expert_of_row(offsets, E_l, r);
  const float* xr = x + (long)r * H;
  const float* g_row = wg + ((long)e * I + c) * H;
  const float* u_row = wu + ((long)e * I + c) * H;
  float g = 0.f, u = 0.f;
  for (int h = 0; h < H; ++h) {
    g = fmaf(xr[h], g_row[h], g);
    u = fmaf(xr[h], u_row[h], u);
  }
  hout[(long)r * I + c] = g / (1.f + expf(-g)) * u;
  if (gu != nullptr) {
    gu[(long)r * 2 * I + c] = g;
    gu[(long)r * 2 * I + I + c] = u;
  }
}

__global__ void down_f32_kernel(const float* __restrict__ hin, const int32_t* __restrict__ offsets,
                                int E_l, int R_cap, int H, int I, const float* __restrict__ wd,
                                float* __restrict__ y) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int r = (int)(i / H), n = (int)(i % H);
  if (r >= R_cap || r >= offsets[E_l]) return;
  const int e = expert_of_row(offsets, E_l, r);
  const float* hr = hin + (long)r * I;
  const float* w = wd + ((long)e * H + n) * I;
  float acc = 0.f;
  for (int c = 0; c < I; ++c) acc = fmaf(hr[c], w[c], acc);
  y[(long)r * H + n] = acc;
}

// [dG dU] from dh = dY_e W_down[e].
__global__ void down_dgrad_f32_kernel(const float* __restrict__ dy,
                                      const int32_t* __restrict__ offsets, int E_l, int R_cap,
                                      int H, int I, const float* __restrict__ wd,
                                      const float* __restrict__ gu, float* __restrict__ dgu) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int r = (int)(i / I), c = (int)(i % I);
  if (r >= R_cap || r >= offsets[E_l]) return;
  const int e = expert_of_row(offsets, E_l, r);
  float dh = 0.f;
  for (int h = 0; h < H; ++h) dh = fmaf(dy[(long)r * H + h], wd[((long)e * H + h) * I + c], dh);
  const float g = gu[(long)r * 2 * I + c], u = gu[(long)r * 2 * I + I + c];
  const float s = 1.f / (1.f + expf(-g));
  dgu[(long)r * 2 * I + c] = dh * u * s * (1.f + g * (1.f - s));
  dgu[(long)r * 2 * I + I + c] = dh * g * s;
}

__global__ void gateup_dgrad_f32_kernel(const float* __restrict__ dgu,
                                        const int32_t* __restrict__ offsets, int E_l, int R_cap,
                                        int H, int I, const float* __restrict__ wg,
                                        const float* __restrict__ wu, float* __restrict__ dx) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int r = (int)(i / H), n = (int)(i % H);
  if (r >= R_cap || r >= offsets[E_l]) return;
  const int e = expert_of_row(offsets, E_l, r);
  float acc = 0.f;
  for (int c = 0; c < I; ++c)
    acc = fmaf(dgu[(long)r * 2 * I + c], wg[((long)e * I + c) * H + n], acc);
  for (int c = 0; c < I; ++c)
    acc = fmaf(dgu[(long)r * 2 * I + I + c], wu[((long)e * I + c) * H + n], acc);
  dx[(long)r * H + n] = acc;
}

// out[e][m][n] (+)= sum over the expert's rows r of A[r][m] * B[r][n].
__global__ void wgrad_f32_kernel(const float* __restrict__ A, long lda, const float* __restrict__ B,
                                 long ldb, const int32_t* __restrict__ offsets, int E_l, int M,
                                 int N, float* __restrict__ out0, float* __restrict__ out1,
                                 int m_split, int accumulate) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long per = (long)M * N;
  if (i >= per * E_l) return;
  const int e = (int)(i / per);
  const int m = (int)((i % per) / N), n = (int)(i % N);
  float acc = 0.f;
  for (int r = offsets[e]; r < offsets[e + 1]; ++r) acc = fmaf(A[r * lda + m], B[r * ldb + n], acc);
  const long mm = (m < m_split) ? m : m - m_split;
  const long rows = (m < m_split) ? m_split : M - m_split;
  float* dst = ((m < m_split) ? out0 : out1) + ((long)e * rows + mm) * N + n;
  if (accumulate) *dst += acc; else *dst = acc;
}

static inline unsigned nblocks(long n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_ffn_fwd_f32(const float* x_perm, const int32_t* offsets, int E_l, int R_cap,
                              int H, int I, const float* w_gate, const float* w_up,
                              const float* w_down, float* gu, float* h_perm, float* y_perm,
                              hipStream_t s) {
  {
    ProfScope ps(MOE_KERNEL_FFN_GATEUP, s);
    gateup_f32_kernel<<<nblocks((long)R_cap * I), 256, 0, s>>>(x_perm, offsets, E_l, R_cap, H, I,
                                                             w_gate, w_up, gu, h_perm);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    ProfScope ps(MOE_KERNEL_FFN_DOWN, s);
    down_f32_kernel<<<nblocks((long)R_cap * H), 256, 0, s>>>(h_perm, offsets, E_l, R_cap, H, I,
                                                           w_down, y_perm);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_bwd_f32(const float* dy_perm, const float* x_perm, const float* gu,
                              const float* h_perm, const int32_t* offsets, int E_l, int R_cap,
                              int H, int I, const float* w_gate, const float* w_up,
                              const float* w_down, float* dx_perm, float* dw_gate, float* dw_up,
                              float* dw_down, bool accumulate, float* dgu_ws, hipStream_t s) {
  {
    ProfScope ps(MOE_KERNEL_FFN_DOWN_DGRAD, s);
    down_dgrad_f32_kernel<<<nblocks((long)R_cap * I), 256, 0, s>>>(dy_perm, offsets, E_l, R_cap, H,
                                                                 I, w_down, gu, dgu_ws);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  wgrad_f32_kernel<<<nblocks((long)E_l * H * I), 256, 0, s>>>(
      dy_perm, H, h_perm, I, offsets, E_l, H, I, dw_down, nullptr, H, accumulate ? 1 : 0);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    ProfScope ps(MOE_KERNEL_FFN_GATEUP_DGRAD, s);
    gateup_dgrad_f32_kernel<<<nblocks((long)R_cap * H), 256, 0, s>>>(dgu_ws, offsets, E_l, R_cap, H,
                                                                   I, w_gate, w_up, dx_perm);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  wgrad_f32_kernel<<<nblocks((long)E_l * 2 * I * H), 256, 0, s>>>(
      dgu_ws, 2 * I, x_perm, H, offsets, E_l, 2 * I, H, dw_gate, dw_up, I, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
