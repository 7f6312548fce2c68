// E4M3 quantization of rows with one power-of-two scale per row, the FP8
// recipe of the expert FFN (the pages name FP8 as their kernel-level speed
// lever, page "Qwen3-MoE-30B-A3B模型EP+FSDP2并行方案", closing throughput
// table; the format and the scaling are this library's reading).
//
// Row scale s = 2^e, e the smallest integer with max|row| <= 448 * 2^e
// (e = 0 for a zero row): with max|row| = f * 2^E, f in [0.5, 1), and
// 448 = 0.875 * 2^9, e = E - 9 + (f > 0.875).  Codes are the E4M3 values
// nearest to v / s (ties to even) from the gfx950 conversion instruction;
// v / s is exact (a power-of-two scaling), so the codes are those of an exact
// rounding.  One wave per row: a pass for the maximum, a pass (from cache)
// for the codes.
#include "common.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_rows_fp8_kernel(const void* __restrict__ src,
                                                                int rows, int cols,
                                                                const int32_t* __restrict__ nrows,
                                                                uint8_t* __restrict__ q,
                                                                float* __restrict__ scale) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (row >= rows) return;
  if (nrows != nullptr && row >= *nrows) return;
  // 8 values per lane step: one 16-byte load (bf16) or two (fp32)
  const int nch = cols / 8;
  float amax = 0.f;
  for (int c = lane; c < nch; c += kWave) {
    float v[8];
    if constexpr (BF16) {
      unpack8(*reinterpret_cast<const uint4*>((const bf16_t*)src + (size_t)row * cols + c * 8), v);
    } else {
      const float4* f = reinterpret_cast<const float4*>((const float*)src + (size_t)row * cols + c * 8);
      const float4 a = f[0], b = f[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  int E;
  const float f = frexpf(amax, &E);
  const int e = amax == 0.f ? 0 : E - 9 + (f > 0.875f ? 1 : 0);
  if (lane == 0) scale[row] = ldexpf(1.f, e);
  for (int c = lane; c < nch; c += kWave) {
    float v[8];
    if constexpr (BF16) {
      unpack8(*reinterpret_cast<const uint4*>((const bf16_t*)src + (size_t)row * cols + c * 8), v);
    } else {
      const float4* fp = reinterpret_cast<const float4*>((const float*)src + (size_t)row * cols + c * 8);
      const float4 a = fp[0], b = fp[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    int w0 = 0, w1 = 0;
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -e), ldexpf(v[1], -e), w0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -e), ldexpf(v[3], -e), w0, true);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4], -e), ldexpf(v[5], -e), w1, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[6], -e), ldexpf(v[7], -e), w1, true);
    *reinterpret_cast<uint2*>(q + (size_t)row * cols + c * 8) = make_uint2((uint32_t)w0, (uint32_t)w1);
  }
}

hipError_t launch_quantize_fp8(const void* src, int rows, int cols, bool bf16,
                               const int32_t* nrows, uint8_t* q, float* scale, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int blocks = (rows + 3) / 4;
  if (bf16)
    quantize_rows_fp8_kernel<true><<<blocks, 256, 0, s>>>(src, rows, cols, nrows, q, scale);
  else
    quantize_rows_fp8_kernel<false><<<blocks, 256, 0, s>>>(src, rows, cols, nrows, q, scale);
  return hipGetLastError();
}

}  // namespace moe
