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
// and a tile table (built on the device from the offsets) maps M tiles to
// experts.  "K-grouped": the reduction runs over an expert's rows.
//
// Tiling: 256 threads = 4 waves in a 2x2 grid, block tile 128 x 256, K step 64,
// each wave a 64 x 128 sub-tile of 2 x 4 MFMA 32x32x16 bf16 blocks with fp32
// accumulators.  Operand tiles stream into a 3-stage LDS ring (144 KB, one
// workgroup per CU) by buffer->LDS DMA (buffer_load_dwordx4 ... lds): no
// staging registers, and the buffer range check turns every row outside the
// tile's valid range into zeros, which handles ragged expert groups.  The DMA
// of K step k+2 is in flight while step k computes; waits are explicit
// (s_waitcnt vmcnt / lgkmcnt and s_barrier).
//   K-contiguous operands ("KC": activations in the forward, A of the data
//   gradients) are stored as rows of 64 bf16 with the 16-byte chunks
//   XOR-swizzled by row and read as MFMA fragments with ds_read_b128.
//   MN-contiguous operands ("MC": weights in the data gradients, both operands
//   of the weight gradients) are stored untransposed (rows = k) with 16-byte
//   chunks XOR-swizzled by 2 * (k & 3), and each MFMA fragment is assembled
//   from two transposing reads (ds_read_b64_tr_b16): within each 16-lane
//   group, lane i points at row kb + i/4, column c0 + 4 * (i % 4), and lane l
//   receives the four consecutive-k values of column c0 + l.
#include "common.h"

#include <algorithm>

namespace moe {

constexpr int BM = 128, BN = 256, BK = 64, NST = 3, NTH = 256;
constexpr int kPersistentBlocks = 256;  // one 144 KB workgroup per CU
constexpr int kStageA = BM * BK;        // bf16 elements per A stage
constexpr int kStageB = BN * BK;        // bf16 elements per B stage
constexpr int NIA = BM / 32;            // DMA instructions per wave per stage, A
constexpr int NIB = BN / 32;            // ... B

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

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef int rsrc_t __attribute__((ext_vector_type(4)));  // buffer descriptor (4 SGPRs)

template <int KIND> struct Traits {
  static constexpr bool A_KC = KIND != K_WGRAD;
  static constexpr bool B_KC = KIND == K_GATEUP_FWD || KIND == K_DOWN_FWD;
};

// ---------------------------------------------------------------------------
// LDS layouts
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kc_swz(int r) { return (r ^ (r >> 3)) & 7; }
// KC tile [rows][64]: first element of logical 16-byte chunk `chunk` of row r.
__device__ __forceinline__ int kc_idx(int r, int chunk) { return r * BK + ((chunk ^ kc_swz(r)) << 3); }
// MC tile [64][W]: LDS position of logical 16-byte chunk c of row k (and back).
__device__ __forceinline__ int mc_chunk(int k, int c) { return c ^ ((k & 3) << 1); }

// ---------------------------------------------------------------------------
// buffer -> LDS DMA and explicit synchronisation
// ---------------------------------------------------------------------------
// Raw buffer descriptor: 48-bit base, stride 0, byte range nbytes, word 3 =
// 0x00020000 (32-bit untyped data); byte offsets >= nbytes read as zero.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  rsrc_t r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)((b >> 32) & 0xffffu);
  r[2] = (int)nbytes;
  r[3] = 0x00020000;
  return r;
}

// LDS byte address of a __shared__ pointer (wave-uniform by construction).
__device__ __forceinline__ uint32_t lds_addr(const bf16_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)p);
}

// 64 lanes x 16 bytes into LDS at lds + 16 * lane.  Issued through inline asm:
// the compiler then keeps no counter for these loads and adds no waits of its
// own; the ring's explicit vmcnt waits and barriers order every access.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(r) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One operand of one tile: buffer resource(s) and, per DMA instruction of this
// lane, the byte offset at k = 0.
template <int NI>
struct Operand {
  rsrc_t rsrc;
  rsrc_t rsrc2;      // second tensor (gate/up split), if any
  uint32_t voff[NI];
  uint32_t kstep;    // byte step per unit of k (KC: 2, MC: row pitch in bytes)
};

// KC operand: DMA instruction u of wave w covers 16-byte LDS chunks
// p = (w*NI + u)*64 + lane, i.e. tile row p/8, LDS chunk p%8, which holds the
// logical k chunk (p%8) ^ swz(row).
template <int NI>
__device__ __forceinline__ void kc_rows(int wave, int lane, int u, int& row, int& chunk) {
  const int p = (wave * NI + u) * 64 + lane;
  row = p >> 3;
  chunk = (p & 7) ^ kc_swz(row);
}

// MC operand of width W: chunk p -> k row p / (W/8), LDS chunk p % (W/8),
// holding logical chunk mc_chunk(row, p % (W/8)).
template <int NI, int W>
__device__ __forceinline__ void mc_rows(int wave, int lane, int u, int& row, int& chunk) {
  const int p = (wave * NI + u) * 64 + lane;
  row = p / (W / 8);
  chunk = mc_chunk(row, p % (W / 8));
}

// ---------------------------------------------------------------------------
// MFMA fragments from LDS
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8_t frag_kc(const bf16_t* tile, int r, int chunk) {
  return *reinterpret_cast<const bf16x8_t*>(&tile[kc_idx(r, chunk)]);
}

// Lane l gets column c0 + l % 32, k = kbase + 8 * (l / 32) + 0..7.
template <int W>
__device__ __forceinline__ bf16x8_t frag_mc(const bf16_t* tile, int kbase, int c0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int k = kbase + 8 * (g >> 1) + (i >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (i & 3);
  const int e0 = k * W + (mc_chunk(k, col >> 3) << 3) + (col & 7);
  const int e1 = (k + 4) * W + (mc_chunk(k + 4, col >> 3) << 3) + (col & 7);
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tile + e0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tile + e1));
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// DMA of one K step (k0 = first k) into the wave's part of a ring slot
// (la, lb: LDS byte addresses).
template <int KIND>
__device__ __forceinline__ void issue_stage(const GemmArgs& p, const Operand<NIA>& opA,
                                            const Operand<NIB>& opB, uint32_t la, uint32_t lb,
                                            int k0) {
#pragma unroll
  for (int u = 0; u < NIA; ++u) dma16(opA.rsrc, opA.voff[u] + (uint32_t)k0 * opA.kstep, la + u * 1024);
  if constexpr (KIND == K_GATEUP_FWD) {
#pragma unroll
    for (int u = 0; u < NIB; ++u)  // instructions with (u >> 2) & 1 == 1 carry up rows
      dma16(((u >> 2) & 1) ? opB.rsrc2 : opB.rsrc, opB.voff[u] + (uint32_t)k0 * 2, lb + u * 1024);
  } else if constexpr (KIND == K_GATEUP_DGRAD) {
    const bool up = k0 >= p.I;
    const uint32_t kk = (uint32_t)(up ? k0 - p.I : k0);
#pragma unroll
    for (int u = 0; u < NIB; ++u)
      dma16(up ? opB.rsrc2 : opB.rsrc, opB.voff[u] + kk * opB.kstep, lb + u * 1024);
  } else {
#pragma unroll
    for (int u = 0; u < NIB; ++u) dma16(opB.rsrc, opB.voff[u] + (uint32_t)k0 * opB.kstep, lb + u * 1024);
  }
}

// ---------------------------------------------------------------------------
// The LDS ring: one array per slot and operand.  Distinct objects let the
// compiler see that the DMA into slot k+2 cannot touch slot k, so it adds no
// wait of its own before the fragment reads (the explicit waits below order
// the ring).
// ---------------------------------------------------------------------------
__shared__ __attribute__((aligned(1024))) bf16_t g_sA0[kStageA];
__shared__ __attribute__((aligned(1024))) bf16_t g_sA1[kStageA];
__shared__ __attribute__((aligned(1024))) bf16_t g_sA2[kStageA];
__shared__ __attribute__((aligned(1024))) bf16_t g_sB0[kStageB];
__shared__ __attribute__((aligned(1024))) bf16_t g_sB1[kStageB];
__shared__ __attribute__((aligned(1024))) bf16_t g_sB2[kStageB];

template <int S> __device__ __forceinline__ bf16_t* slot_a() {
  if constexpr (S == 0) return g_sA0;
  else if constexpr (S == 1) return g_sA1;
  else return g_sA2;
}
template <int S> __device__ __forceinline__ bf16_t* slot_b() {
  if constexpr (S == 0) return g_sB0;
  else if constexpr (S == 1) return g_sB1;
  else return g_sB2;
}

// MFMA fragments of one k = 16 sub-step of a wave's 64 x 128 sub-tile.
struct Frags {
  bf16x8_t a[2];
  bf16x8_t b[4];
};

template <int KIND, int S>
__device__ __forceinline__ void load_frags(Frags& f, int s, int wave, int lane) {
  using Tr = Traits<KIND>;
  const int wm = wave >> 1, wn = wave & 1;
  const bf16_t* ta = slot_a<S>();
  const bf16_t* tb = slot_b<S>();
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    if constexpr (Tr::A_KC)
      f.a[mi] = frag_kc(ta, wm * 64 + mi * 32 + (lane & 31), 2 * s + (lane >> 5));
    else
      f.a[mi] = frag_mc<BM>(ta, 16 * s, wm * 64 + mi * 32, lane);
  }
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    if constexpr (Tr::B_KC)
      f.b[ni] = frag_kc(tb, wn * 128 + ni * 32 + (lane & 31), 2 * s + (lane >> 5));
    else
      f.b[ni] = frag_mc<BN>(tb, 16 * s, wn * 128 + ni * 32, lane);
  }
}

__device__ __forceinline__ void mma(f32x16_t (&acc)[2][4], const Frags& f) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
}

// One K step on ring slot S, software pipelined: on entry `cur` holds the
// fragments of sub-step 0; the fragments of sub-step s + 1 are read while the
// MFMAs of sub-step s run.  Before the MFMAs of the last sub-step the wave
// waits for step kt + 1 to land (barrier), starts the DMA of step kt + 3 into
// this slot (every wave has finished reading it) and reads the next step's
// first fragments, so that the barrier and LDS latency hide behind MFMAs.
template <int KIND, int S>
__device__ __forceinline__ void k_step(const GemmArgs& p, const Operand<NIA>& opA,
                                       const Operand<NIB>& opB, f32x16_t (&acc)[2][4],
                                       Frags& cur, int kt, int nk, int wave, int lane) {
  Frags nxt;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    load_frags<KIND, S>(nxt, s + 1, wave, lane);
    mma(acc, cur);
    cur = nxt;
  }
  if (kt + 1 < nk) {
    // Step kt + 1 has landed when at most one newer step (NIA + NIB loads) is in flight.
    if (kt + 2 < nk)
      wait_vm<NIA + NIB>();
    else
      wait_vm<0>();
    lds_barrier();  // every wave: step kt + 1 landed, slot S fully read
    if (kt + 3 < nk)
      issue_stage<KIND>(p, opA, opB, lds_addr(slot_a<S>()) + wave * NIA * 1024,
                        lds_addr(slot_b<S>()) + wave * NIB * 1024, (kt + 3) * BK);
    load_frags<KIND, (S + 1) % NST>(nxt, 0, wave, lane);
  }
  mma(acc, cur);
  cur = nxt;
}

// ---------------------------------------------------------------------------
// Epilogue: the accumulators go through LDS so that global stores are 16-byte
// row segments.  Each wave stages one 32 x 128 fp32 half of its 64 x 128
// sub-tile at a time into its own 16 KB of a B ring slot (16-byte chunks
// XOR-swizzled so the row pairs written by one MFMA output register hit
// different banks), then every lane handles 8 consecutive columns of a row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float* stage_area(int wave) {
  return reinterpret_cast<float*>(wave < 2 ? g_sB0 : g_sB1) + (wave & 1) * 4096;
}
// fp32 element (row r < 32, col c < 128) of a wave's staging area
__device__ __forceinline__ int stage_idx(int r, int c) { return r * 128 + (c ^ (((r >> 2) & 1) << 5)); }

__device__ __forceinline__ void stage_half(float* st, const f32x16_t (&acc)[2][4], int mi, int lane) {
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      st[stage_idx(r, ni * 32 + (lane & 31))] = acc[mi][ni][q];
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// 8 consecutive staged values (c % 8 == 0): 16-byte chunks never straddle the swizzle.
__device__ __forceinline__ void load8(const float* st, int r, int c, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(&st[stage_idx(r, c)]);
  const float4 b = *reinterpret_cast<const float4*>(&st[stage_idx(r, c + 4)]);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <int KIND>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const f32x16_t (&acc)[2][4], int e,
                                         int nt, int n0, int m0, int row0, int row1, int wave,
                                         int lane) {
  const int wm = wave >> 1, wn = wave & 1;
  float* st = stage_area(wave);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    stage_half(st, acc, mi, lane);
    if constexpr (KIND == K_GATEUP_FWD) {
      // staged columns: [g 32 | u 32 | g 32 | u 32] for h columns nt*128 + wn*64 + 0..63
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3);
        const int hc = (lane & 7) * 8;           // 0..56: h column within the wave
        const int sc = (hc >> 5) * 64 + (hc & 31);  // staged gate column
        const long row = row0 + wm * 64 + mi * 32 + r;
        const int col = nt * 128 + wn * 64 + hc;
        if (row >= row1 || col >= p.I) continue;
        float g[8], u[8], h[8];
        load8(st, r, sc, g);
        load8(st, r, sc + 32, u);
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = g[j] * fast_rcp(1.f + __expf(-g[j])) * u[j];
        *reinterpret_cast<uint4*>(p.c0 + row * p.ldc + col) = pack8(h);
        if (p.c1 != nullptr) {
          *reinterpret_cast<uint4*>(p.c1 + row * 2 * p.I + col) = pack8(g);
          *reinterpret_cast<uint4*>(p.c1 + row * 2 * p.I + p.I + col) = pack8(u);
        }
      }
    } else if constexpr (KIND == K_WGRAD) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = it * 4 + (lane >> 4);
        const int c = (lane & 15) * 8;
        const int m = m0 + wm * 64 + mi * 32 + r;
        const int n = n0 + wn * 128 + c;
        if (m >= p.M || n >= p.N) continue;
        float v[8];
        load8(st, r, c, v);
        float* dst = (m < p.m_split) ? p.f0 + e * p.f_group_stride + (long)m * p.ldc + n
                                     : p.f1 + e * p.f_group_stride + (long)(m - p.m_split) * p.ldc + n;
        float4* d4 = reinterpret_cast<float4*>(dst);
        if (p.accumulate) {
          const float4 o0 = d4[0], o1 = d4[1];
          d4[0] = make_float4(o0.x + v[0], o0.y + v[1], o0.z + v[2], o0.w + v[3]);
          d4[1] = make_float4(o1.x + v[4], o1.y + v[5], o1.z + v[6], o1.w + v[7]);
        } else {
          d4[0] = make_float4(v[0], v[1], v[2], v[3]);
          d4[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
      }
    } else {  // DOWN_FWD, GATEUP_DGRAD, DOWN_DGRAD: rows of the grouped buffer
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = it * 4 + (lane >> 4);
        const int c = (lane & 15) * 8;
        const long row = row0 + wm * 64 + mi * 32 + r;
        const int n = n0 + wn * 128 + c;
        if (row >= row1 || n >= p.N) continue;
        float v[8];
        load8(st, r, c, v);
        if constexpr (KIND == K_DOWN_DGRAD) {
          // v = dh; dG = dh * u * s * (1 + g (1 - s)), dU = dh * SiLU(g), s = sigmoid(g)
          float g[8], u[8], dg[8], du[8];
          unpack8(*reinterpret_cast<const uint4*>(p.gu + row * 2 * p.I + n), g);
          unpack8(*reinterpret_cast<const uint4*>(p.gu + row * 2 * p.I + p.I + n), u);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float sg = fast_rcp(1.f + __expf(-g[j]));
            dg[j] = v[j] * u[j] * sg * (1.f + g[j] * (1.f - sg));
            du[j] = v[j] * g[j] * sg;
          }
          *reinterpret_cast<uint4*>(p.c0 + row * 2 * p.I + n) = pack8(dg);
          *reinterpret_cast<uint4*>(p.c0 + row * 2 * p.I + p.I + n) = pack8(du);
        } else {
          *reinterpret_cast<uint4*>(p.c0 + row * p.ldc + n) = pack8(v);
        }
      }
    }
    // the other half reuses the staging area
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(NTH) void gemm_kernel(const GemmArgs p) {
  using Tr = Traits<KIND>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int total;
  if constexpr (KIND == K_WGRAD)
    total = p.groups * p.n_mtiles * p.n_ntiles;
  else
    total = p.sched[0] * p.n_ntiles;

  for (int work = xcd_remap(blockIdx.x, gridDim.x); work < total; work += gridDim.x) {
    // ---------------------------------------------------------------- tile
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
    // Tile scalars are wave-uniform; saying so keeps buffer descriptors and
    // DMA addresses in SGPRs (no per-lane waterfall loops).
    e = __builtin_amdgcn_readfirstlane(e);
    nt = __builtin_amdgcn_readfirstlane(nt);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    row1 = __builtin_amdgcn_readfirstlane(row1);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    kbeg = __builtin_amdgcn_readfirstlane(kbeg);
    kend = __builtin_amdgcn_readfirstlane(kend);
    const int n0 = nt * BN;

    // ------------------------------------------------------ operand setup
    Operand<NIA> opA;
    Operand<NIB> opB;
    if constexpr (Tr::A_KC) {
      // the tile's rows [row0, row1) of A; rows past row1 read as zero
      opA.rsrc = make_rsrc(p.a + (long)row0 * p.lda, (uint32_t)((row1 - row0) * p.lda * 2));
      opA.kstep = 2;
#pragma unroll
      for (int u = 0; u < NIA; ++u) {
        int r, c;
        kc_rows<NIA>(wave, lane, u, r, c);
        opA.voff[u] = (uint32_t)(r * p.lda * 2 + c * 16);
      }
    } else {  // WGRAD: A[k = row of the group][m]; rows past the group read as zero
      opA.rsrc = make_rsrc(p.a + (long)kbeg * p.lda, (uint32_t)((kend - kbeg) * p.lda * 2));
      opA.kstep = (uint32_t)(p.lda * 2);
#pragma unroll
      for (int u = 0; u < NIA; ++u) {
        int r, c;
        mc_rows<NIA, BM>(wave, lane, u, r, c);
        const int col = min(m0 + c * 8, p.M - 8);  // tail columns: any in-row data, never stored
        opA.voff[u] = (uint32_t)(r * p.lda * 2 + col * 2);
      }
    }
    if constexpr (KIND == K_GATEUP_FWD) {
      // Tile rows interleave 32 gate rows and 32 up rows, so each wave's N
      // blocks (g, u, g, u) pair gate and up values of the same h columns.
      const long est = (long)e * p.b_group_stride;
      opB.rsrc = make_rsrc(p.b0 + est, (uint32_t)(p.I * p.ldb * 2));
      opB.rsrc2 = make_rsrc(p.b1 + est, (uint32_t)(p.I * p.ldb * 2));
      opB.kstep = 2;
#pragma unroll
      for (int u = 0; u < NIB; ++u) {
        int r, c;
        kc_rows<NIB>(wave, lane, u, r, c);
        const int col = nt * 128 + (r >> 6) * 32 + (r & 31);
        opB.voff[u] = (uint32_t)(col * p.ldb * 2 + c * 16);
      }
    } else if constexpr (KIND == K_DOWN_FWD) {
      opB.rsrc = make_rsrc(p.b0 + (long)e * p.b_group_stride, (uint32_t)(p.N * p.ldb * 2));
      opB.kstep = 2;
#pragma unroll
      for (int u = 0; u < NIB; ++u) {
        int r, c;
        kc_rows<NIB>(wave, lane, u, r, c);
        opB.voff[u] = (uint32_t)((n0 + r) * p.ldb * 2 + c * 16);
      }
    } else if constexpr (KIND == K_DOWN_DGRAD || KIND == K_GATEUP_DGRAD) {
      // B[k][n] = weight row k, column n (MN-contiguous), whole expert matrix
      const long est = (long)e * p.b_group_stride;
      const uint32_t rows = (KIND == K_DOWN_DGRAD) ? (uint32_t)p.K : (uint32_t)p.I;
      opB.rsrc = make_rsrc(p.b0 + est, rows * (uint32_t)p.ldb * 2);
      if constexpr (KIND == K_GATEUP_DGRAD) opB.rsrc2 = make_rsrc(p.b1 + est, rows * (uint32_t)p.ldb * 2);
      opB.kstep = (uint32_t)(p.ldb * 2);
#pragma unroll
      for (int u = 0; u < NIB; ++u) {
        int r, c;
        mc_rows<NIB, BN>(wave, lane, u, r, c);
        const int col = min(n0 + c * 8, p.N - 8);
        opB.voff[u] = (uint32_t)(r * p.ldb * 2 + col * 2);
      }
    } else {  // WGRAD B
      opB.rsrc = make_rsrc(p.b0 + (long)kbeg * p.ldb, (uint32_t)((kend - kbeg) * p.ldb * 2));
      opB.kstep = (uint32_t)(p.ldb * 2);
#pragma unroll
      for (int u = 0; u < NIB; ++u) {
        int r, c;
        mc_rows<NIB, BN>(wave, lane, u, r, c);
        const int col = min(n0 + c * 8, p.N - 8);
        opB.voff[u] = (uint32_t)(r * p.ldb * 2 + col * 2);
      }
    }

    f32x16_t acc[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x16_t{};

    const int nk = (kend - kbeg + BK - 1) / BK;
    if (nk > 0) {
      // three steps in flight, then step 0's first fragments
      issue_stage<KIND>(p, opA, opB, lds_addr(slot_a<0>()) + wave * NIA * 1024,
                        lds_addr(slot_b<0>()) + wave * NIB * 1024, 0);
      if (nk > 1)
        issue_stage<KIND>(p, opA, opB, lds_addr(slot_a<1>()) + wave * NIA * 1024,
                          lds_addr(slot_b<1>()) + wave * NIB * 1024, BK);
      if (nk > 2)
        issue_stage<KIND>(p, opA, opB, lds_addr(slot_a<2>()) + wave * NIA * 1024,
                          lds_addr(slot_b<2>()) + wave * NIB * 1024, 2 * BK);
      if (nk > 2)
        wait_vm<2 * (NIA + NIB)>();
      else if (nk > 1)
        wait_vm<NIA + NIB>();
      else
        wait_vm<0>();
      lds_barrier();
      Frags cur;
      load_frags<KIND, 0>(cur, 0, wave, lane);
      for (int kt = 0; kt < nk; kt += NST) {
        k_step<KIND, 0>(p, opA, opB, acc, cur, kt, nk, wave, lane);
        if (kt + 1 >= nk) break;
        k_step<KIND, 1>(p, opA, opB, acc, cur, kt + 1, nk, wave, lane);
        if (kt + 2 >= nk) break;
        k_step<KIND, 2>(p, opA, opB, acc, cur, kt + 2, nk, wave, lane);
      }
      // Every wave is done with the ring before the epilogue stages into it.
      lds_barrier();
    }

    // ------------------------------------------------------------ epilogue
    epilogue<KIND>(p, acc, e, nt, n0, m0, row0, row1, wave, lane);
    // The next tile's first DMA overwrites the epilogue's staging area.
    lds_barrier();
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
    sched[3 + 3 * i] = min(r0 + BM, offsets[lo + 1]);
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
  g.n_ntiles = (I + 127) / 128;
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
