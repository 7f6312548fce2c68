// E4M3 quantization of rows with one power-of-two scale per row, the FP8
// recipe of the expert FFN (the pages name FP8 as their kernel-level speed
// lever, page "TorchTitan FSDP2 完全指南", section "性能表现", H100 benchmark
// table, row FSDP + compile + FP8; the format and the scaling are this
// library's reading).
//
// Row scale s = 2^e, e the smallest integer with max|row| <= 448 * 2^e
// (e = 0 for a zero row): with max|row| = f * 2^E, f in [0.5, 1), and
// 448 = 0.875 * 2^9, e = E - 9 + (f > 0.875).  Codes are the E4M3 values
// nearest to v / s (ties to even) from the gfx950 conversion instruction;
// v / s is exact (a power-of-two scaling), so the codes are those of an exact
// rounding.  One wave per row: a pass for the maximum, a pass (from cache)
// for the codes.
#include <algorithm>

#include "common.h"

namespace moe {

// Exponent of the row scale for a row maximum amax (0 for a zero row).
__device__ __forceinline__ int fp8_exponent(float amax) {
  int E;
  const float f = frexpf(amax, &E);
  return amax == 0.f ? 0 : E - 9 + (f > 0.875f ? 1 : 0);
}

// Eight values -> eight E4M3 codes of v * 2^-e (two dwords).
__device__ __forceinline__ uint2 fp8_codes8(const float* v, int e) {
  int w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -e), ldexpf(v[1], -e), w0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -e), ldexpf(v[3], -e), w0, true);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4], -e), ldexpf(v[5], -e), w1, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[6], -e), ldexpf(v[7], -e), w1, true);
  return make_uint2((uint32_t)w0, (uint32_t)w1);
}

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
  const int e = fp8_exponent(amax);
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
    *reinterpret_cast<uint2*>(q + (size_t)row * cols + c * 8) = fp8_codes8(v, e);
  }
}

// Per-input-channel codes of expert weights for the data-gradient products:
// src0 (and src1) [B][N][K] bf16 -> q [B][K][n N], row k = the column k of
// src0 followed by the column k of src1, scaled by one power of two per k.
// A workgroup takes 64 columns of one batch: pass 1 the column maxima (each
// thread 8 columns of every 32nd row, then an LDS reduction), pass 2 the
// codes, through 64 x 64 tiles in LDS so that each thread writes 16
// consecutive codes of one output row.  N % 64 == 0, K % 64 == 0.
__global__ __launch_bounds__(256) void quantize_t_fp8_kernel(const bf16_t* __restrict__ src0,
                                                             const bf16_t* __restrict__ src1,
                                                             int N, int K,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ scale) {
  __shared__ float s_max[32][65];
  __shared__ int s_e[64];
  __shared__ __align__(16) bf16_t s_tile[64][64];
  const int b = blockIdx.y, c0 = blockIdx.x * 64, t = threadIdx.x;
  const int nsrc = src1 != nullptr ? 2 : 1;
  const int cc = t & 7, r0 = t >> 3;  // 8 columns 8 cc .. + 7 of rows r0, r0 + 32, ...
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int si = 0; si < nsrc; ++si) {
    const bf16_t* src = (si == 0 ? src0 : src1) + (size_t)b * N * K + c0 + 8 * cc;
    for (int r = r0; r < N; r += 32) {
      float v[8];
      unpack8(*reinterpret_cast<const uint4*>(src + (size_t)r * K), v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(v[i]));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) s_max[r0][8 * cc + i] = m[i];
  __syncthreads();
  if (t < 64) {
    float a = 0.f;
    for (int r = 0; r < 32; ++r) a = fmaxf(a, s_max[r][t]);
    const int e = fp8_exponent(a);
    s_e[t] = e;
    scale[(size_t)b * K + c0 + t] = ldexpf(1.f, e);
  }
  __syncthreads();
  const int oc = t & 63, og = t >> 6;  // output row c0 + oc, 16 source rows 16 og .. + 15
  const int e = s_e[oc];
  uint8_t* qrow = q + ((size_t)b * K + c0 + oc) * (size_t)(nsrc * N);
  for (int si = 0; si < nsrc; ++si) {
    const bf16_t* src = (si == 0 ? src0 : src1) + (size_t)b * N * K + c0;
    for (int n0 = 0; n0 < N; n0 += 64) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = (t >> 3) + 32 * h;
        *reinterpret_cast<uint4*>(&s_tile[r][8 * cc]) =
            *reinterpret_cast<const uint4*>(src + (size_t)(n0 + r) * K + 8 * cc);
      }
      __syncthreads();
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = bf2f(s_tile[16 * og + i][oc]);
      const uint2 lo = fp8_codes8(v, e), hi = fp8_codes8(v + 8, e);
      *reinterpret_cast<uint4*>(qrow + (size_t)si * N + n0 + 16 * og) = make_uint4(lo.x, lo.y, hi.x, hi.y);
      __syncthreads();
    }
  }
}

hipError_t launch_quantize_t_fp8(const bf16_t* src0, const bf16_t* src1, int batch, int N, int K,
                                 uint8_t* q, float* scale, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  quantize_t_fp8_kernel<<<dim3(K / 64, batch), 256, 0, s>>>(src0, src1, N, K, q, scale);
  return hipGetLastError();
}

// Both code layouts of expert weights from the same two reads: the rows of
// w0 (and w1) [B][N][K] as quantize_rows_fp8 makes them (forward) and the
// per-input-channel rows of [w0^T | w1^T] as quantize_t_fp8 makes them (data
// gradients), bit for bit: the same exponent rule and conversion on the same
// maxima (a maximum is exact in any order).  Three launches over 128 x 128
// tiles: (1) each tile's row maxima (over its 128 columns) and column maxima
// (over its 128 rows) to fp32 partials in the workspace; (2) one thread per
// row and per input channel reduces its partials to the scale exponent (and
// writes the scale); (3) each tile goes out twice, as rows of codes (two
// threads per row, 64 consecutive codes each) and, through LDS, as rows of
// the transposed layout (two threads per input channel), so that every
// 128-byte line of either output is written by one workgroup.
// N % 128 == 0, K % 128 == 0.
constexpr int kQwT = 128;  // tile edge
struct QuantW {
  const bf16_t* w[2];
  uint8_t* q[2];      // row codes [B][N][K] of w0 / w1
  float* s[2];        // row scales [B][N]
  uint8_t* qt;        // transposed codes [B][K][nsrc N], or null
  float* st;          // per-input-channel scales [B][K]
  float* rowp;        // [nsrc][B][N][K / 128] row partial maxima
  float* colp;        // [B][K][nsrc N / 128] column partial maxima
  int* erow;          // [nsrc][B][N] row exponents
  int* ecol;          // [B][K] input-channel exponents
  int nsrc, B, N, K;
};

// Thread t of a tile holds the 16-byte chunk t % 16 (columns 8 (t % 16) ..
// + 7) of rows t / 16 + 16 i, i < 8: each load instruction of a wave reads
// four whole 256-byte rows.  The chunks are also copied into the LDS tile.
__device__ __forceinline__ void load_tile128(const bf16_t* src, int K, int t,
                                             bf16_t (*tile)[kQwT + 8], uint4 (&raw)[8]) {
  const int r0 = t >> 4, c = (t & 15) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) raw[i] = *reinterpret_cast<const uint4*>(src + (size_t)(r0 + 16 * i) * K + c);
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(&tile[r0 + 16 * i][c]) = raw[i];
}

__global__ __launch_bounds__(256) void quantize_w_max_kernel(const QuantW a) {
  __shared__ float s_col[4][kQwT];
  const int kb = blockIdx.x, nb_all = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int nbs = a.N / kQwT, src = nb_all / nbs, nb = nb_all % nbs;
  const bf16_t* w = a.w[src] + ((size_t)b * a.N + nb * kQwT) * a.K + kb * kQwT;
  // thread t: columns 8 (t % 16) .. + 7 of rows t / 16 + 16 i (as load_tile128)
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    raw[i] = *reinterpret_cast<const uint4*>(w + (size_t)((t >> 4) + 16 * i) * a.K + (t & 15) * 8);
  float mc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // rows: maximum over the tile's 128 columns (the 16 lanes of the row)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v[8];
    unpack8(raw[i], v);
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      m = fmaxf(m, fabsf(v[j]));
      mc[j] = fmaxf(mc[j], fabsf(v[j]));
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    if ((t & 15) == 0)
      a.rowp[(((size_t)src * a.B + b) * a.N + nb * kQwT + (t >> 4) + 16 * i) * (a.K / kQwT) + kb] = m;
  }
  if (a.qt == nullptr) return;
  // columns: the four lanes of a wave with the same chunk, then the four waves
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mc[j] = fmaxf(mc[j], __shfl_xor(mc[j], 16, kWave));
    mc[j] = fmaxf(mc[j], __shfl_xor(mc[j], 32, kWave));
  }
  if ((t & 63) < 16)
#pragma unroll
    for (int j = 0; j < 8; ++j) s_col[t >> 6][(t & 15) * 8 + j] = mc[j];
  __syncthreads();
  if (t < kQwT) {
    const float m = fmaxf(fmaxf(s_col[0][t], s_col[1][t]), fmaxf(s_col[2][t], s_col[3][t]));
    a.colp[((size_t)b * a.K + kb * kQwT + t) * (a.nsrc * nbs) + nb_all] = m;
  }
}

// One thread per row (first nsrc B N threads) and per input channel (next B K).
__global__ __launch_bounds__(256) void quantize_w_exp_kernel(const QuantW a) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long nrow = (long)a.nsrc * a.B * a.N;
  if (i < nrow) {
    const float* p = a.rowp + i * (a.K / kQwT);
    float m = 0.f;
    for (int j = 0; j < a.K / kQwT; ++j) m = fmaxf(m, p[j]);
    const int e = fp8_exponent(m);
    a.erow[i] = e;
    const long src = i / ((long)a.B * a.N);
    a.s[src][i - src * a.B * a.N] = ldexpf(1.f, e);
    return;
  }
  const long c = i - nrow;
  if (a.qt == nullptr || c >= (long)a.B * a.K) return;
  const int np = a.nsrc * (a.N / kQwT);
  const float* p = a.colp + c * np;
  float m = 0.f;
  for (int j = 0; j < np; ++j) m = fmaxf(m, p[j]);
  const int e = fp8_exponent(m);
  a.ecol[c] = e;
  a.st[c] = ldexpf(1.f, e);
}

__global__ __launch_bounds__(256) void quantize_w_codes_kernel(const QuantW a) {
  __shared__ __align__(16) bf16_t tile[kQwT][kQwT + 8];
  const int kb = blockIdx.x, nb_all = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int nbs = a.N / kQwT, src = nb_all / nbs, nb = nb_all % nbs;
  const bf16_t* w = a.w[src] + ((size_t)b * a.N + nb * kQwT) * a.K + kb * kQwT;
  uint4 raw[8];
  load_tile128(w, a.K, t, tile, raw);
  // row codes: eight codes of each of the thread's rows (a wave's store
  // instruction writes four whole 128-byte code rows of the tile)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (t >> 4) + 16 * i;
    const int e = a.erow[((size_t)src * a.B + b) * a.N + nb * kQwT + r];
    float v[8];
    unpack8(raw[i], v);
    *reinterpret_cast<uint2*>(a.q[src] + ((size_t)b * a.N + nb * kQwT + r) * a.K + kb * kQwT +
                              (t & 15) * 8) = fp8_codes8(v, e);
  }
  if (a.qt == nullptr) return;
  __syncthreads();
  {  // transposed codes: input channel t % 128, 64 consecutive rows from 64 (t / 128)
    const int c = t & (kQwT - 1), g = t >> 7;
    const int e = a.ecol[(size_t)b * a.K + kb * kQwT + c];
    uint8_t* dst = a.qt + ((size_t)b * a.K + kb * kQwT + c) * (size_t)(a.nsrc * a.N) + (size_t)src * a.N +
                   nb * kQwT + 64 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = bf2f(tile[64 * g + 16 * i + j][c]);
      const uint2 lo = fp8_codes8(v, e), hi = fp8_codes8(v + 8, e);
      *reinterpret_cast<uint4*>(dst + 16 * i) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
}

static size_t qw_align(size_t b) { return (b + 255) & ~(size_t)255; }

size_t quantize_w_fp8_ws_bytes(int batch, int N, int K, int nsrc) {
  const size_t parts = (size_t)nsrc * batch * N * (K / kQwT);
  return 2 * qw_align(parts * 4) + qw_align((size_t)nsrc * batch * N * 4) + qw_align((size_t)batch * K * 4);
}

hipError_t launch_quantize_w_fp8(const bf16_t* w0, const bf16_t* w1, int batch, int N, int K,
                                 uint8_t* q0, float* s0, uint8_t* q1, float* s1, uint8_t* qt,
                                 float* st, void* ws, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  QuantW a{};
  a.nsrc = w1 != nullptr ? 2 : 1;
  a.w[0] = w0;
  a.w[1] = w1;
  a.q[0] = q0;
  a.q[1] = q1;
  a.s[0] = s0;
  a.s[1] = s1;
  a.qt = qt;
  a.st = st;
  a.B = batch;
  a.N = N;
  a.K = K;
  const size_t parts = qw_align((size_t)a.nsrc * batch * N * (K / kQwT) * 4);
  char* p = (char*)ws;
  a.rowp = (float*)p;
  a.colp = (float*)(p + parts);
  a.erow = (int*)(p + 2 * parts);
  a.ecol = (int*)(p + 2 * parts + qw_align((size_t)a.nsrc * batch * N * 4));
  const dim3 grid(K / kQwT, a.nsrc * (N / kQwT), batch);
  quantize_w_max_kernel<<<grid, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long threads = (long)a.nsrc * batch * N + (qt != nullptr ? (long)batch * K : 0);
  quantize_w_exp_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  quantize_w_codes_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// Columns of grouped rows quantized per (group, column) for the FP8 weight
// gradients, which sum over a group's rows: for group g (rows offsets[g] ..
// offsets[g + 1] - 1) and column c, scale = 2^e by the row rule above applied
// to the column restricted to the group, and the codes of that column go to
// row c of the transposed output, columns poff[g] .. poff[g] + n_g - 1, with
// zero codes up to the next multiple of 64 (poff[g] = the sum of the earlier
// groups' row counts rounded up to 64, also written out).
//
// Three launches, each over column strips of 64 (the tensors' strips numbered
// one after the other) and, in the grid's second dimension, a stride over a
// list of row chunks (every group's rows cut into chunks; an empty group is
// one empty chunk), so that a hot group spreads over as many workgroups as its
// rows need:
//   1. zero the scales (and the caller's tile counters);
//   2. per (64 columns, chunk of kGtMaxRows rows): the chunk's column maxima,
//      and the scale 2^e they call for merged into the group's scale by an
//      atomic max on its bits: e never falls as the maximum grows, and 2^e
//      (down to 2^-141 for the smallest bf16, a float subnormal) orders like
//      its bit pattern, so the merge is the scale of the group's maximum, bit
//      for bit, in any order (0 for a zero column);
//   3. per (64 columns, chunk of kGtCodesRows rows): e read back from the
//      scale (0: e = 0, and the group's first chunk stores the scale 1), and
//      the codes.  Thread (cg, rg) holds 8 columns (c0 + 8 cg ..) of 16
//      consecutive chunk rows (16 rg ..) and writes per column one 16-byte
//      piece of that column's output row, so that eight threads of a wave
//      write a whole 128-byte line, with no LDS transposition.  A thread's 16
//      rows lie wholly inside or wholly past the group's padded rows.
// (Holding a group's rows in registers from the maxima to the codes, one read
// instead of two, needs chunks as long as the groups: at 1024 rows half of
// each workgroup idled on this layer's ~512-row groups and the pass was
// slower.)
constexpr int kGtMaxRows = 256;    // rows per chunk of the maxima pass
constexpr int kGtCodesRows = 512;  // rows per chunk of the codes pass

struct GtChunk {
  int g;     // group, -1 past the last chunk
  int rbeg;  // first row of the chunk within the group
  int n;     // rows in the chunk
  int o0;    // offsets[g]
  int poff;  // padded start of the group
  int ng;    // rows in the group
};

// Chunk c of the list of CH-row chunks of the groups (group order; an empty
// group is one empty chunk), found by wave 0 with scans over 64 groups at a
// time; the result reaches the whole workgroup through LDS.
template <int CH>
__device__ GtChunk gt_find_chunk(const int32_t* offsets, int E_l, int c, int t, GtChunk* s_c) {
  if (t < kWave) {
    int base_c = 0, base_p = 0;
    bool found = false;
    for (int j0 = 0; j0 < E_l && !found; j0 += kWave) {
      const int j = j0 + t;
      const int n = j < E_l ? offsets[j + 1] - offsets[j] : 0;
      const int nc = j < E_l ? max(1, (n + CH - 1) / CH) : 0;
      const int pd = (n + 63) & ~63;
      int ic = nc, ip = pd;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int xc = __shfl_up(ic, o, kWave), xp = __shfl_up(ip, o, kWave);
        if (t >= o) {
          ic += xc;
          ip += xp;
        }
      }
      const int ec = base_c + ic - nc;
      if (nc > 0 && c >= ec && c < ec + nc) {
        const int k = c - ec;
        *s_c = GtChunk{j, k * CH, min(n - k * CH, CH), offsets[j], base_p + ip - pd, n};
      }
      const int tc = __shfl(ic, kWave - 1, kWave), tp = __shfl(ip, kWave - 1, kWave);
      found = c < base_c + tc;
      base_c += tc;
      base_p += tp;
    }
    if (!found && t == 0) s_c->g = -1;
  }
  __syncthreads();
  const GtChunk r = *s_c;
  __syncthreads();  // s_c is rewritten by the next lookup
  return r;
}

// the tensor and 64-column strip of blockIdx.x
__device__ __forceinline__ const QuantGroupTensor& gt_tensor(const QuantGroupT& a, int& c0) {
  int ti = 0, strip = blockIdx.x;
  while (ti + 1 < a.nt && strip >= a.t[ti].C / 64) {
    strip -= a.t[ti].C / 64;
    ++ti;
  }
  c0 = strip * 64;
  return a.t[ti];
}

// 16 rows of 8 columns of a chunk (zeros past its n rows)
__device__ __forceinline__ void gt_load16(const QuantGroupTensor& T, const GtChunk& k, int r0, int col,
                                          uint4* v) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + i;
    v[i] = make_uint4(0u, 0u, 0u, 0u);
    if (r < k.n) {
      const long row = T.rows != nullptr ? T.rows[k.o0 + k.rbeg + r] : k.o0 + k.rbeg + r;
      v[i] = *reinterpret_cast<const uint4*>(T.src + row * T.ld + col);
    }
  }
}

// the codes of column j (0..7) of 16 rows, as one 16-byte piece
__device__ __forceinline__ uint4 gt_codes16(const uint4* v, int j, int e) {
  float f[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w = (&v[i].x)[j >> 1];
    f[i] = __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  const uint2 lo = fp8_codes8(f, e), hi = fp8_codes8(f + 8, e);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// e of a scale 2^e from its bits (normal or subnormal); 0 for a zero scale
__device__ __forceinline__ int gt_scale_exponent(uint32_t b) {
  if (b == 0u) return 0;
  if (b >= 0x00800000u) return (int)(b >> 23) - 127;
  return (31 - __clz(b)) - 149;
}

__global__ __launch_bounds__(256) void quantize_group_t_zero_kernel(const QuantGroupT a) {
  const QuantGroupTensor& T = a.t[blockIdx.y];
  const long n = (long)a.E_l * T.C;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    T.scale[i] = 0.f;
  if (a.ctrs != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && (int)threadIdx.x < a.nctrs)
    a.ctrs[threadIdx.x] = 0;
}

__global__ __launch_bounds__(256) void quantize_group_t_max_kernel(const QuantGroupT a) {
  __shared__ float s_max[32][65];
  __shared__ GtChunk s_c;
  const int t = threadIdx.x, cc = t & 7, r0 = t >> 3;
  int c0;
  const QuantGroupTensor& T = gt_tensor(a, c0);
  for (int c = blockIdx.y;; c += gridDim.y) {
    const GtChunk k = gt_find_chunk<kGtMaxRows>(a.offsets, a.E_l, c, t, &s_c);
    if (k.g < 0) break;
    uint4 v[kGtMaxRows / 32];
#pragma unroll
    for (int i = 0; i < kGtMaxRows / 32; ++i) {
      const int r = k.rbeg + r0 + 32 * i;
      v[i] = make_uint4(0u, 0u, 0u, 0u);
      if (r0 + 32 * i < k.n) {
        const long row = T.rows != nullptr ? T.rows[k.o0 + r] : k.o0 + r;
        v[i] = *reinterpret_cast<const uint4*>(T.src + row * T.ld + c0 + 8 * cc);
      }
    }
    // |x| of a bf16 orders like its bits with the sign cleared: the maxima on
    // the packed words (column 2w in the low half of word w, 2w + 1 in the high;
    // a NaN, above inf in these bits, wins)
    uint32_t m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kGtMaxRows / 32; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = (&v[i].x)[w];
        m[2 * w] = max(m[2 * w], x & 0x7fffu);
        m[2 * w + 1] = max(m[2 * w + 1], x & 0x7fff0000u);
      }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s_max[r0][8 * cc + 2 * w] = __uint_as_float(m[2 * w] << 16);
      s_max[r0][8 * cc + 2 * w + 1] = __uint_as_float(m[2 * w + 1]);
    }
    __syncthreads();
    if (t < 64) {
      float mx = 0.f;
      for (int r = 0; r < 32; ++r) mx = fmaxf(mx, s_max[r][t]);
      if (mx > 0.f)
        atomicMax(reinterpret_cast<unsigned int*>(T.scale + (size_t)k.g * T.C + c0 + t),
                  __float_as_uint(ldexpf(1.f, fp8_exponent(mx))));
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void quantize_group_t_codes_kernel(const QuantGroupT a) {
  __shared__ GtChunk s_c;
  const int t = threadIdx.x, cg = t & 7, rg = t >> 3, r0 = 16 * rg;
  int c0;
  const QuantGroupTensor& T = gt_tensor(a, c0);
  for (int c = blockIdx.y;; c += gridDim.y) {
    const GtChunk k = gt_find_chunk<kGtCodesRows>(a.offsets, a.E_l, c, t, &s_c);
    if (k.g < 0) break;
    if (blockIdx.x == 0 && k.rbeg == 0 && t == 0) {
      a.poff[k.g] = k.poff;
      if (k.g == a.E_l - 1) a.poff[a.E_l] = k.poff + ((k.ng + 63) & ~63);
    }
    float* sp = T.scale + (size_t)k.g * T.C + c0 + 8 * cg;
    if (k.n == 0) {  // an empty group: every column is a zero column
      if (rg == 0)
#pragma unroll
        for (int j = 0; j < 8; ++j) sp[j] = 1.f;
      continue;
    }
    if (r0 >= ((k.n + 63) & ~63)) continue;
    uint4 v[16];
    gt_load16(T, k, r0, c0 + 8 * cg, v);
    int e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = __float_as_uint(sp[j]);
      e[j] = gt_scale_exponent(b);
      if (b == 0u && k.rbeg == 0 && rg == 0) sp[j] = 1.f;  // a zero column
    }
    uint8_t* q = T.q + (size_t)(c0 + 8 * cg) * a.Kp + k.poff + k.rbeg + r0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4*>(q + (size_t)j * a.Kp) = gt_codes16(v, j, e[j]);
  }
}

hipError_t launch_quantize_group_t_fp8(const QuantGroupT& q, hipStream_t s) {
  int strips = 0;
  for (int i = 0; i < q.nt; ++i) strips += q.t[i].C / 64;
  if (strips == 0 || q.E_l <= 0) return hipSuccess;
  long zero_max = 0;
  for (int i = 0; i < q.nt; ++i) zero_max = std::max(zero_max, (long)q.E_l * q.t[i].C);
  const unsigned zero_x = (unsigned)std::min<long>((zero_max + 4095) / 4096, 256);
  quantize_group_t_zero_kernel<<<dim3(zero_x, q.nt), 256, 0, s>>>(q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the grids' second dimension: at most the chunk list's length (one chunk
  // per group plus one per ch rows), at most 64 (the workgroups stride over
  // the list)
  const auto grid = [&](int ch) {
    const long chunks = ((long)q.max_rows + ch - 1) / ch + q.E_l;
    return dim3(strips, (unsigned)std::min<long>(chunks, 64));
  };
  quantize_group_t_max_kernel<<<grid(kGtMaxRows), 256, 0, s>>>(q);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  quantize_group_t_codes_kernel<<<grid(kGtCodesRows), 256, 0, s>>>(q);
  return hipGetLastError();
}

// Gradients of h = SiLU(g) * u for the FP8 gate / up data gradient, one wave
// per grouped row r < nrows: dg = dh u s (1 + g (1 - s)), du = dh SiLU(g),
// s = sigmoid(g), in fp32 from the bf16 dh and the saved g, u; [dg | du] is
// stored in bf16 (for the weight gradients) and its row, as rounded,
// quantized like quantize_rows_fp8 (codes + scale).  I % 8 == 0, I <= 2048.
constexpr int kSwiMaxChunks = 4;  // chunks of 8 columns per lane: I <= 64 * 8 * 4
__global__ __launch_bounds__(256) void swiglu_bwd_fp8_kernel(const bf16_t* __restrict__ dh,
                                                             const bf16_t* __restrict__ gu,
                                                             int rows, int I,
                                                             const int32_t* __restrict__ nrows,
                                                             bf16_t* __restrict__ dgu,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ scale) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (row >= rows || row >= *nrows) return;
  const int nch = I / 8;
  float dg[kSwiMaxChunks][8], du[kSwiMaxChunks][8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kSwiMaxChunks; ++j) {
    const int c = lane + kWave * j;
    if (c >= nch) break;
    float d[8], g[8], u[8];
    unpack8(*reinterpret_cast<const uint4*>(dh + (size_t)row * I + 8 * c), d);
    unpack8(*reinterpret_cast<const uint4*>(gu + (size_t)row * 2 * I + 8 * c), g);
    unpack8(*reinterpret_cast<const uint4*>(gu + (size_t)row * 2 * I + I + 8 * c), u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sg = fast_rcp(1.f + __expf(-g[i]));
      dg[j][i] = d[i] * u[i] * sg * (1.f + g[i] * (1.f - sg));
      du[j][i] = d[i] * g[i] * sg;
    }
    const uint4 pg = pack8(dg[j]), pu = pack8(du[j]);
    *reinterpret_cast<uint4*>(dgu + (size_t)row * 2 * I + 8 * c) = pg;
    *reinterpret_cast<uint4*>(dgu + (size_t)row * 2 * I + I + 8 * c) = pu;
    unpack8(pg, dg[j]);  // the rounded values are what gets quantized
    unpack8(pu, du[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fmaxf(fabsf(dg[j][i]), fabsf(du[j][i])));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  const int e = fp8_exponent(amax);
  if (lane == 0) scale[row] = ldexpf(1.f, e);
#pragma unroll
  for (int j = 0; j < kSwiMaxChunks; ++j) {
    const int c = lane + kWave * j;
    if (c >= nch) break;
    *reinterpret_cast<uint2*>(q + (size_t)row * 2 * I + 8 * c) = fp8_codes8(dg[j], e);
    *reinterpret_cast<uint2*>(q + (size_t)row * 2 * I + I + 8 * c) = fp8_codes8(du[j], e);
  }
}

hipError_t launch_swiglu_bwd_fp8(const bf16_t* dh, const bf16_t* gu, int rows, int I,
                                 const int32_t* nrows, bf16_t* dgu, uint8_t* q, float* scale,
                                 hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  swiglu_bwd_fp8_kernel<<<(rows + 3) / 4, 256, 0, s>>>(dh, gu, rows, I, nrows, dgu, q, scale);
  return hipGetLastError();
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
