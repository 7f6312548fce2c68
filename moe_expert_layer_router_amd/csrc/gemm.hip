// Grouped bf16 GEMMs of the expert FFN on gfx950 MFMA (the "grouped matmul"
// of the dispatcher table on the page "FSDPTurbo EP/EFSDP and LlamaFactory
// FSDP2/CP Design", section 3; expert shapes from the page
// "Qwen3-MoE-30B-A3B模型EP+FSDP2并行方案", section "Qwen3-MoE-30B-A3B模型").
//
// One persistent kernel template covers the five product shapes of the
// forward and backward:
//   GATEUP_FWD   h = SiLU(X_e W_gate^T) * (X_e W_up^T)      M-grouped, fused SwiGLU epilogue
//   DOWN_FWD     Y_e = h_e W_down^T                         M-grouped
//   DOWN_DGRAD   [dG dU] = SiLU'(dY_e W_down)               M-grouped, fused SiLU' epilogue
//   GATEUP_DGRAD dX_e = dG W_gate + dU W_up                 M-grouped
//   WGRAD        dW_e = A_e^T B_e over the expert's rows    K-grouped, fp32 out
// "M-grouped": each expert owns a contiguous row range of the grouped buffer
// and the tile table (built on the device from the offsets) maps M tiles to
// experts.  "K-grouped": the reduction runs over an expert's rows.
//
// Tiling: 256 threads = 4 waves in a 2x2 grid, block tile 128x128, K step 64,
// each wave a 64x64 sub-tile of 2x2 MFMA 32x32x16 bf16 blocks with fp32
// accumulators.  Operand tiles are staged through LDS (double buffered, one
// barrier per K step) as rows of 64 bf16 with the 16-byte chunks of each row
// XOR-swizzled so that both the MFMA fragment reads and the staging writes
// spread over the LDS banks.  Operands whose reduction dimension is not
// contiguous in memory (weights in the data-gradient products, both operands
// of the weight-gradient products) are read as 8x8 blocks and transposed in
// registers before the LDS write.
#include "common.h"

#include <algorithm>

namespace moe {

constexpr int BM = 128, BN = 128, BK = 64, NTH = 256;
constexpr int kStage = 128 * BK;  // elements of one operand stage in LDS
constexpr int kPersistentBlocks = 512;  // 256 CUs x 2 resident workgroups

enum GemmKind { K_GATEUP_FWD = 0, K_DOWN_FWD = 1, K_DOWN_DGRAD = 2, K_GATEUP_DGRAD = 3, K_WGRAD = 4 };

struct GemmArgs {
  const bf16_t* a;
  long lda;
  const bf16_t* b0;  // B operand (gate / the only one)
  const bf16_t* b1;  // second B tensor (up), or null
  long ldb;
  long b_group_stride;      // elements between experts in b0 / b1
  const int32_t* offsets;   // group row offsets [groups + 1], or null for even splits
  const int32_t* sched;     // M-grouped tile table: [0] = count, then (expert, row0, row1)
  int groups;               // K-grouped: number of groups
  int split_rows;           // K-grouped with offsets == null: rows per group
  int ktot;                 // K-grouped with offsets == null: total rows
  int M, N, K, I;
  int n_mtiles, n_ntiles;
  bf16_t* c0;
  bf16_t* c1;
  long ldc;
  const bf16_t* gu;         // DOWN_DGRAD: saved g / u
  float* f0;
  float* f1;
  int m_split;
  long f_group_stride;
  int accumulate;
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_idx(int r, int c) { return r * BK + ((c ^ swz(r)) << 3); }

// 8x8 bf16 transpose in registers: in[i] holds 8 elements of row i; out[j]
// holds element j of every row.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4& lo = in[2 * q];
      const uint4& hi = in[2 * q + 1];
      const uint32_t wl = (j >> 1) == 0 ? lo.x : (j >> 1) == 1 ? lo.y : (j >> 1) == 2 ? lo.z : lo.w;
      const uint32_t wh = (j >> 1) == 0 ? hi.x : (j >> 1) == 1 ? hi.y : (j >> 1) == 2 ? hi.z : hi.w;
      d[q] = (j & 1) ? ((wl >> 16) | (wh & 0xffff0000u)) : ((wl & 0xffffu) | (wh << 16));
    }
    out[j] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

template <int KIND>
__global__ __launch_bounds__(NTH) void gemm_kernel(const GemmArgs p) {
  constexpr bool A_KC = KIND != K_WGRAD;                                  // A rows contiguous in K
  constexpr bool B_KC = KIND == K_GATEUP_FWD || KIND == K_DOWN_FWD;       // B rows contiguous in K
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][kStage];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // K-contiguous staging: thread owns chunk kc of rows (tid >> 3) + 32 i.
  const int kc = tid & 7;
  const int rbase = tid >> 3;
  // MN-contiguous staging: thread owns one 8x8 block (k rows kb*8.., mn cols mb*8..).
  const int blk = tid & 127;
  const int kb = blk >> 4, mb = blk & 15;

  int total;
  if constexpr (KIND == K_WGRAD)
    total = p.groups * p.n_mtiles * p.n_ntiles;
  else
    total = p.sched[0] * p.n_ntiles;

  for (int work = xcd_remap(blockIdx.x, gridDim.x); work < total; work += gridDim.x) {
    // ------------------------------------------------------------------ tile
    int e, nt, row0 = 0, row1 = 0, m0 = 0, kbeg = 0, kend = 0;
    if constexpr (KIND == K_WGRAD) {
      e = work / (p.n_mtiles * p.n_ntiles);
      const int rem = work - e * p.n_mtiles * p.n_ntiles;
      m0 = (rem / p.n_ntiles) * BM;
      nt = rem % p.n_ntiles;
      if (p.offsets != nullptr) {
        kbeg = p.offsets[e];
        kend = p.offsets[e + 1];
      } else {
        kbeg = min(e * p.split_rows, p.ktot);
        kend = min(kbeg + p.split_rows, p.ktot);
      }
    } else {
      const int mt = work / p.n_ntiles;
      nt = work - mt * p.n_ntiles;
      e = p.sched[1 + 3 * mt];
      row0 = p.sched[2 + 3 * mt];
      row1 = p.sched[3 + 3 * mt];
      kend = p.K;
    }
    const int n0 = nt * BN;

    // K-contiguous operand row pointers (already offset by the thread's chunk).
    const bf16_t* pa[4];
    const bf16_t* pb[4];
    if constexpr (A_KC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int r = row0 + rbase + 32 * i;
        if (r >= row1) r = row1 - 1;  // ragged tile: any valid row, never stored
        pa[i] = p.a + (long)r * p.lda + kc * 8;
      }
    }
    if constexpr (KIND == K_GATEUP_FWD) {
      // Tile rows interleave 32 gate rows and 32 up rows so each wave's two
      // N blocks are the gate and up values of the same 32 columns of h.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = nt * 64 + (i >> 1) * 32 + rbase;
        const bf16_t* base = (i & 1) ? p.b1 : p.b0;
        pb[i] = base + e * p.b_group_stride + (long)col * p.ldb + kc * 8;
      }
    } else if constexpr (KIND == K_DOWN_FWD) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int n = n0 + rbase + 32 * i;
        if (n >= p.N) n = p.N - 1;
        pb[i] = p.b0 + e * p.b_group_stride + (long)n * p.ldb + kc * 8;
      }
    }

    // ------------------------------------------------------------ staging
    uint4 ra[4], rb[4], rt[8];
    auto load_stage = [&](int k0) {
      if constexpr (A_KC) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const uint4*>(pa[i] + k0);
      }
      if constexpr (B_KC) {
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[i] = *reinterpret_cast<const uint4*>(pb[i] + k0);
      }
      if constexpr (KIND == K_DOWN_DGRAD || KIND == K_GATEUP_DGRAD) {
        if (tid < 128) {
          int mn = n0 + mb * 8;
          if (mn > p.N - 8) mn = p.N - 8;
          const int k = k0 + kb * 8;
          const bf16_t* src;
          if constexpr (KIND == K_DOWN_DGRAD)
            src = p.b0 + e * p.b_group_stride + (long)k * p.ldb + mn;
          else
            src = (k < p.I ? p.b0 + e * p.b_group_stride + (long)k * p.ldb
                           : p.b1 + e * p.b_group_stride + (long)(k - p.I) * p.ldb) + mn;
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) rt[ii] = *reinterpret_cast<const uint4*>(src + ii * p.ldb);
        }
      }
      if constexpr (KIND == K_WGRAD) {
        const bool isA = tid < 128;
        int mn = (isA ? m0 : n0) + mb * 8;
        const int lim = isA ? p.M : p.N;
        if (mn > lim - 8) mn = lim - 8;
        const bf16_t* base = isA ? p.a : p.b0;
        const long ld = isA ? p.lda : p.ldb;
        const int k = kbeg + k0 + kb * 8;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii)
          rt[ii] = (k + ii < kend) ? *reinterpret_cast<const uint4*>(base + (long)(k + ii) * ld + mn)
                                   : make_uint4(0u, 0u, 0u, 0u);
      }
    };
    auto store_stage = [&](int buf) {
      if constexpr (A_KC) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint4*>(&sA[buf][lds_idx(rbase + 32 * i, kc)]) = ra[i];
      }
      if constexpr (B_KC) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint4*>(&sB[buf][lds_idx(rbase + 32 * i, kc)]) = rb[i];
      }
      if constexpr (!B_KC) {
        bf16_t* dst = nullptr;
        if constexpr (KIND == K_WGRAD)
          dst = tid < 128 ? sA[buf] : sB[buf];
        else
          dst = tid < 128 ? sB[buf] : nullptr;
        if (dst != nullptr) {
          uint4 o[8];
          transpose8x8(rt, o);
#pragma unroll
          for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(&dst[lds_idx(mb * 8 + j, kb)]) = o[j];
        }
      }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16_t{};

    const int nk = (kend - kbeg + BK - 1) / BK;
    if (nk > 0) {
      load_stage(0);
      store_stage(0);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_stage((kt + 1) * BK);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int ch = 2 * s + (lane >> 5);
          bf16x8_t af[2], bfg[2];
#pragma unroll
          for (int mi = 0; mi < 2; ++mi)
            af[mi] = *reinterpret_cast<const bf16x8_t*>(
                &sA[cur][lds_idx(wm * 64 + mi * 32 + (lane & 31), ch)]);
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            bfg[ni] = *reinterpret_cast<const bf16x8_t*>(
                &sB[cur][lds_idx(wn * 64 + ni * 32 + (lane & 31), ch)]);
#pragma unroll
          for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
              acc[mi][ni] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfg[ni], acc[mi][ni], 0, 0, 0);
        }
        if (kt + 1 < nk) store_stage(cur ^ 1);
        __syncthreads();
      }
    }

    // ------------------------------------------------------------ epilogue
    // acc[mi][ni][q] sits at tile row wm*64 + mi*32 + 8*(q/4) + 4*(lane/32) + q%4
    // and tile column wn*64 + ni*32 + lane%32.
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rl = wm * 64 + mi * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if constexpr (KIND == K_GATEUP_FWD) {
          const long r = row0 + rl;
          if (r >= row1) continue;
          const int col = nt * 64 + wn * 32 + (lane & 31);
          const float g = acc[mi][0][q], u = acc[mi][1][q];
          const float h = g / (1.f + __expf(-g)) * u;
          p.c0[r * p.ldc + col] = f2bf(h);
          if (p.c1 != nullptr) {
            p.c1[r * 2 * p.I + col] = f2bf(g);
            p.c1[r * 2 * p.I + p.I + col] = f2bf(u);
          }
        } else if constexpr (KIND == K_DOWN_FWD || KIND == K_GATEUP_DGRAD) {
          const long r = row0 + rl;
          if (r >= row1) continue;
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            const int n = n0 + wn * 64 + ni * 32 + (lane & 31);
            if (n < p.N) p.c0[r * p.ldc + n] = f2bf(acc[mi][ni][q]);
          }
        } else if constexpr (KIND == K_DOWN_DGRAD) {
          const long r = row0 + rl;
          if (r >= row1) continue;
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            const int col = n0 + wn * 64 + ni * 32 + (lane & 31);
            if (col >= p.N) continue;
            const float dh = acc[mi][ni][q];
            const float g = bf2f(p.gu[r * 2 * p.I + col]);
            const float u = bf2f(p.gu[r * 2 * p.I + p.I + col]);
            const float sg = 1.f / (1.f + __expf(-g));
            const float dg = dh * u * sg * (1.f + g * (1.f - sg));
            const float du = dh * g * sg;
            p.c0[r * 2 * p.I + col] = f2bf(dg);
            p.c0[r * 2 * p.I + p.I + col] = f2bf(du);
          }
        } else {  // K_WGRAD
          const int m = m0 + rl;
          if (m >= p.M) continue;
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            const int n = n0 + wn * 64 + ni * 32 + (lane & 31);
            if (n >= p.N) continue;
            float* dst = (m < p.m_split)
                             ? p.f0 + e * p.f_group_stride + (long)m * p.ldc + n
                             : p.f1 + e * p.f_group_stride + (long)(m - p.m_split) * p.ldc + n;
            if (p.accumulate)
              *dst += acc[mi][ni][q];
            else
              *dst = acc[mi][ni][q];
          }
        }
      }
    }
  }
}

// Tile table of the M-grouped products: for every expert with rows, one entry
// (expert, first row, end row) per BM rows.  sched[0] = number of entries.
__global__ __launch_bounds__(kMaxE) void ffn_sched_kernel(const int32_t* __restrict__ offsets,
                                                          int E_l, int32_t* __restrict__ sched) {
  __shared__ int s[kMaxE + 1];
  const int e = threadIdx.x;
  const int n = (e < E_l) ? offsets[e + 1] - offsets[e] : 0;
  const int tiles = (n + BM - 1) / BM;
  s[e + 1] = tiles;
  if (e == 0) s[0] = 0;
  __syncthreads();
  for (int o = 1; o <= kMaxE; o <<= 1) {  // inclusive scan of s[1..kMaxE]
    const int v = (e + 1 - o >= 1) ? s[e + 1 - o] : 0;
    __syncthreads();
    s[e + 1] += v;
    __syncthreads();
  }
  const int count = s[E_l];
  if (e == 0) sched[0] = count;
  for (int i = e; i < count; i += kMaxE) {
    int lo = 0, hi = E_l - 1;  // largest g with s[g] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int r0 = offsets[lo] + (i - s[lo]) * BM;
    sched[1 + 3 * i] = lo;
    sched[2 + 3 * i] = r0;
    sched[3 + 3 * i] = offsets[lo + 1];
  }
}

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t ffn_sched_bytes(int R_cap, int E_l) {
  const size_t entries = (size_t)R_cap / BM + E_l + 1;
  return align256((1 + 3 * entries) * sizeof(int32_t));
}

template <int KIND>
static hipError_t launch_gemm(const GemmArgs& a, int work_upper, int kernel_id, hipStream_t s) {
  if (work_upper <= 0) return hipSuccess;
  int grid = std::min(work_upper, kPersistentBlocks);
  ProfScope ps(kernel_id, s);
  gemm_kernel<KIND><<<grid, NTH, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_ffn_fwd_bf16(const bf16_t* x_perm, const int32_t* offsets, int E_l, int R_cap,
                               int H, int I, const bf16_t* w_gate, const bf16_t* w_up,
                               const bf16_t* w_down, bf16_t* gu, bf16_t* h_perm, bf16_t* y_perm,
                               void* ws, hipStream_t s) {
  int32_t* sched = (int32_t*)ws;
  ffn_sched_kernel<<<1, kMaxE, 0, s>>>(offsets, E_l, sched);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int mt_upper = R_cap / BM + E_l;

  GemmArgs g{};
  g.a = x_perm;
  g.lda = H;
  g.b0 = w_gate;
  g.b1 = w_up;
  g.ldb = H;
  g.b_group_stride = (long)I * H;
  g.sched = sched;
  g.K = H;
  g.N = I;
  g.I = I;
  g.n_ntiles = I / 64;
  g.c0 = h_perm;
  g.ldc = I;
  g.c1 = gu;
  err = launch_gemm<K_GATEUP_FWD>(g, mt_upper * g.n_ntiles, MOE_KERNEL_FFN_GATEUP, s);
  if (err != hipSuccess) return err;

  GemmArgs d{};
  d.a = h_perm;
  d.lda = I;
  d.b0 = w_down;
  d.ldb = I;
  d.b_group_stride = (long)H * I;
  d.sched = sched;
  d.K = I;
  d.N = H;
  d.I = I;
  d.n_ntiles = (H + BN - 1) / BN;
  d.c0 = y_perm;
  d.ldc = H;
  return launch_gemm<K_DOWN_FWD>(d, mt_upper * d.n_ntiles, MOE_KERNEL_FFN_DOWN, s);
}

hipError_t launch_ffn_bwd_bf16(const bf16_t* dy_perm, const bf16_t* x_perm, const bf16_t* gu,
                               const bf16_t* h_perm, const int32_t* offsets, int E_l, int R_cap,
                               int H, int I, const bf16_t* w_gate, const bf16_t* w_up,
                               const bf16_t* w_down, bf16_t* dx_perm, float* dw_gate,
                               float* dw_up, float* dw_down, bool accumulate, void* ws,
                               hipStream_t s) {
  int32_t* sched = (int32_t*)ws;
  bf16_t* dgu = (bf16_t*)((char*)ws + ffn_sched_bytes(R_cap, E_l));
  ffn_sched_kernel<<<1, kMaxE, 0, s>>>(offsets, E_l, sched);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int mt_upper = R_cap / BM + E_l;

  // dh = dY_e W_down[e]  ->  [dG dU] through the SiLU' epilogue.
  GemmArgs a{};
  a.a = dy_perm;
  a.lda = H;
  a.b0 = w_down;
  a.ldb = I;
  a.b_group_stride = (long)H * I;
  a.sched = sched;
  a.K = H;
  a.N = I;
  a.I = I;
  a.n_ntiles = (I + BN - 1) / BN;
  a.gu = gu;
  a.c0 = dgu;
  err = launch_gemm<K_DOWN_DGRAD>(a, mt_upper * a.n_ntiles, MOE_KERNEL_FFN_DOWN_DGRAD, s);
  if (err != hipSuccess) return err;

  // dW_down[e] = dY_e^T h_e
  GemmArgs b{};
  b.a = dy_perm;
  b.lda = H;
  b.M = H;
  b.b0 = h_perm;
  b.ldb = I;
  b.N = I;
  b.offsets = offsets;
  b.groups = E_l;
  b.n_mtiles = (H + BM - 1) / BM;
  b.n_ntiles = (I + BN - 1) / BN;
  b.f0 = dw_down;
  b.m_split = H;
  b.ldc = I;
  b.f_group_stride = (long)H * I;
  b.accumulate = accumulate ? 1 : 0;
  err = launch_gemm<K_WGRAD>(b, E_l * b.n_mtiles * b.n_ntiles, MOE_KERNEL_FFN_DOWN_WGRAD, s);
  if (err != hipSuccess) return err;

  // dX_e = dG W_gate[e] + dU W_up[e]
  GemmArgs c{};
  c.a = dgu;
  c.lda = 2 * I;
  c.b0 = w_gate;
  c.b1 = w_up;
  c.ldb = H;
  c.b_group_stride = (long)I * H;
  c.sched = sched;
  c.K = 2 * I;
  c.N = H;
  c.I = I;
  c.n_ntiles = (H + BN - 1) / BN;
  c.c0 = dx_perm;
  c.ldc = H;
  err = launch_gemm<K_GATEUP_DGRAD>(c, mt_upper * c.n_ntiles, MOE_KERNEL_FFN_GATEUP_DGRAD, s);
  if (err != hipSuccess) return err;

  // dW_gate[e] = dG_e^T X_e, dW_up[e] = dU_e^T X_e (one product with M = 2I).
  GemmArgs w{};
  w.a = dgu;
  w.lda = 2 * I;
  w.M = 2 * I;
  w.b0 = x_perm;
  w.ldb = H;
  w.N = H;
  w.offsets = offsets;
  w.groups = E_l;
  w.n_mtiles = (2 * I + BM - 1) / BM;
  w.n_ntiles = (H + BN - 1) / BN;
  w.f0 = dw_gate;
  w.f1 = dw_up;
  w.m_split = I;
  w.ldc = H;
  w.f_group_stride = (long)I * H;
  w.accumulate = accumulate ? 1 : 0;
  return launch_gemm<K_WGRAD>(w, E_l * w.n_mtiles * w.n_ntiles, MOE_KERNEL_FFN_GATEUP_WGRAD, s);
}

hipError_t launch_dw_router_bf16(const bf16_t* x, const bf16_t* dz_hilo, int T, int H, int E,
                                 int nsplit, int32_t* /*split_offsets*/, float* partials,
                                 hipStream_t s) {
  GemmArgs w{};
  w.a = x;
  w.lda = H;
  w.M = H;
  w.b0 = dz_hilo;
  w.ldb = 2 * E;
  w.N = 2 * E;
  w.offsets = nullptr;
  w.groups = nsplit;
  w.split_rows = (T + nsplit - 1) / nsplit;
  w.ktot = T;
  w.n_mtiles = (H + BM - 1) / BM;
  w.n_ntiles = (2 * E + BN - 1) / BN;
  w.f0 = partials;
  w.m_split = H;
  w.ldc = 2 * E;
  w.f_group_stride = (long)H * 2 * E;
  w.accumulate = 0;
  return launch_gemm<K_WGRAD>(w, nsplit * w.n_mtiles * w.n_ntiles, MOE_KERNEL_ROUTE_BWD_DW, s);
}

}  // namespace moe
