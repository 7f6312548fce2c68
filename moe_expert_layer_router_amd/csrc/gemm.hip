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
//   ROUTER_DX    dx_router = [dz_hi dz_lo] [W_r W_r]^T      one group of T rows, fp32 out
// and, with FP8 = true, the two forward products on E4M3 codes (below).
// "M-grouped": each expert owns a contiguous row range of the grouped buffer
// and a tile table (built on the device from the offsets) maps M tiles to
// experts.  "K-grouped": the reduction runs over an expert's rows.
//
// Tiling: 256 threads = 4 waves in a 2x2 grid, block tile BM x 256, each wave
// a BM/2 x 128 sub-tile of (BM/64) x 4 MFMA 32x32x16 bf16 blocks with fp32
// accumulators.  Two block heights:
//   BM = 256: 128 x 128 wave tiles (256 accumulator registers, one wave per
//     SIMD), 128 KB of ring plus a 32 KB staging area, one workgroup per CU.
//     Per k16 sub-step a wave reads 8 KB of fragments for 16 MFMAs, which
//     keeps the LDS traffic per MFMA well inside the CU's LDS bandwidth.
//   BM = 128: 64 x 128 wave tiles (128 accumulators), 3-stage ring of 72 KB,
//     two workgroups per CU: twice the LDS traffic per MFMA, but half the tile
//     height (less padding of ragged expert groups, more tiles to spread over
//     256 CUs) and a second workgroup whose MFMAs fill the gaps of the other's
//     barriers, prologue and epilogue.
// Two rings (Cfg):
//   narrow: K steps of 32, NST slots; the DMA of step k + NST - 1 is in
//     flight while step k computes.
//   wide (the bf16 M-grouped products): K blocks of 64 in five 32 KB regions
//     (the fifth doubles as the staging area); blocks j + 1 and j + 2 are in
//     flight while block j computes.  A K-contiguous row of a block is one
//     whole 128-byte line, where a narrow step reads half lines: on gfx950 the
//     buffer->LDS path moves about twice the bytes per cycle for whole lines.
// Operand tiles stream into the ring by buffer->LDS DMA
// (buffer_load_dwordx4 ... lds): no staging registers, and the buffer range
// check turns every row outside the tile's valid range into zeros, which
// handles ragged expert groups.  Waits are explicit (s_waitcnt vmcnt /
// lgkmcnt and s_barrier).
//   K-contiguous operands ("KC": activations in the forward, A of the data
//   gradients) are stored as rows of 32 or 64 bf16 with the 16-byte chunks
//   XOR-swizzled by row and read as MFMA fragments with ds_read_b128.
//   MN-contiguous operands ("MC": weights in the data gradients, both operands
//   of the weight gradients) are stored untransposed (rows = k) with 16-byte
//   chunks XOR-swizzled by 4 * (k & 3), and each MFMA fragment is assembled
//   from two transposing reads (ds_read_b64_tr_b16): within each 16-lane
//   group, lane i points at row kb + i/4, column c0 + 4 * (i % 4), and lane l
//   receives the four consecutive-k values of column c0 + l.
//
// FP8 forward (FP8 = true, GATEUP_FWD and DOWN_FWD): operands are E4M3 codes
// with one power-of-two scale per row (activation rows, weight output
// channels).  At the byte level a row of K codes is a row of K / 2 bf16 slots,
// so the launcher passes K / 2 and row pitches / 2 and the DMA ring, the
// swizzles and the fragment reads run unchanged: a 64-byte K step holds 64
// codes.  Per K step each (mi, ni) block takes one v_mfma_scale_f32_32x32x64
// _f8f6f4 (unit block scales) whose 32 operand bytes per lane are the two
// 16-byte fragments the bf16 path reads for its two k16 sub-steps (a
// permutation of K applied to both operands, so the sum is the same); on the
// wide ring a 128-code block is two such steps.  The epilogue multiplies each
// accumulator by its row scale times its column scale (both powers of two:
// exact) before the SwiGLU.
#include "common.h"
#include "lds_layout.h"

#include <algorithm>
#include <mutex>

namespace moe {

constexpr int BN = 256, NTH = 256;  // BK, KCH: lds_layout.h
constexpr int kMaxDevices = 64;  // per-device objects the launchers keep
constexpr int kTileCtrs = 4;             // dynamic tile counters in the FFN workspace
constexpr int WN = 128;                  // wave sub-tile width
constexpr int NI = WN / 32;              // MFMA blocks per wave along N

// Block-height and ring dependent parameters.  Two rings:
//   narrow (WIDE = false): K steps of BK = 32, NST slots of A then NST slots
//     of B.  A K-contiguous row of a step is 64 bytes: every DMA instruction
//     reads 16 half cache lines.
//   wide (WIDE = true, BM = 256 only): K blocks of 64, five 32 KiB regions;
//     load i of a tile (A of block j = load 2j, B of block j = load 2j + 1)
//     goes to region i % 5.  A K-contiguous row of a block is a whole 128-byte
//     line, and each DMA instruction reads 8 whole lines: the texture path
//     moves about twice the bytes per cycle (a probe of the two patterns over
//     L2-resident data: 123 against 66 GB/s per CU).  Region 4 is also the
//     epilogue's staging area.
template <int BM_, bool WIDE_ = false>
struct Cfg {
  static constexpr int BM = BM_;
  static constexpr bool WIDE = WIDE_;
  static constexpr int BKX = WIDE ? 64 : BK;           // K per ring stage (bf16)
  static constexpr int KSUB = BKX / 16;                // k16 sub-steps per stage
  static constexpr int WM = BM / 2;                    // wave sub-tile height
  static constexpr int MI = WM / 32;                   // MFMA blocks per wave along M
  static constexpr int NST = BM == 256 ? 4 : 3;        // narrow ring: stages
  static constexpr int kStageA = BM * BKX;             // bf16 elements per A stage
  static constexpr int kStageB = BN * BKX;             // bf16 elements per B stage
  static constexpr int NIA = kStageA * 2 / 1024 / 4;   // DMA instructions (1 KB) per wave per stage, A
  static constexpr int NIB = kStageB * 2 / 1024 / 4;   // and B
  static constexpr int kSlotA = kStageA * 2;           // bytes
  static constexpr int kSlotB = kStageB * 2;
  static constexpr int kRegion = 32768;                // wide ring: region bytes
  static constexpr int kOffB = WIDE ? 0 : NST * kSlotA;  // narrow: B slots start here
  // wide: regions 0..3 (region 4 is the staging area below)
  static constexpr int kRingBytes = WIDE ? 4 * kRegion : NST * (kSlotA + kSlotB);
  static constexpr int kWavesPerSimd = BM == 256 ? 1 : 2;  // = workgroups per CU
  // The epilogue stages 16 x 128 fp32 (8 KB) per wave.  256-row tiles keep
  // that area after the ring, so the next tile's first K steps are loaded
  // during the epilogue; 128-row tiles (two workgroups per CU) stage in the
  // ring and start the next tile's loads after it.  (A fifth ring slot with
  // the staging area laid over it, four K steps in flight instead of three,
  // measured no faster on the training step or the 128-expert forward.)
  static constexpr bool kSepStage = BM == 256;
  static constexpr int kStageBytes = 4 * 8192;
  static constexpr int kStageOff = kSepStage ? kRingBytes : 0;
  static constexpr int kLdsBytes = kSepStage ? kRingBytes + kStageBytes : kRingBytes;
  static_assert(kLdsBytes * kWavesPerSimd <= 160 * 1024, "LDS per CU");
  static_assert(kSepStage || kRingBytes >= kStageBytes, "staging area inside the ring");
  static_assert(!WIDE || (BM == 256 && kSlotA == kRegion && kSlotB == kRegion && kStageBytes == kRegion &&
                          kStageOff == 4 * kRegion),
                "wide ring: five equal regions, the fifth is the staging area");
};
// Tile heights in use: 256 for every product (chosen by measurement: the
// larger tile's lower L2 and LDS traffic per MFMA wins over the finer tiling
// of 128; the down-projection weight gradient, whose K = expert rows is
// short, ran faster with 128 on the narrow ring and about even, slightly
// ahead, with 256 on the wide one).  The 128-row configuration stays
// available.
constexpr int kBmGrouped = 256;
// The bf16 products with 256-row tiles run on the wide ring: the M-grouped
// ones (their K, H or I or 2I, is a multiple of 64, so no K block straddles a
// row's end) and the weight gradients with 256-row tiles (their K tail is a
// row range, dropped by the descriptors like any ragged group; their
// MN-contiguous 512-byte rows read whole lines either way, and the wide ring
// measured even with the narrow one there).  The FP8 weight gradient keeps
// the narrow ring.
constexpr bool kWideGrouped = true;
constexpr bool kWideWgrad = true;
// The FP8 M-grouped products (the forward and both data gradients; their K in
// 16-bit slots, H / 2, I / 2 or I, is a multiple of 64 since the FP8 entry
// points need H and I multiples of 128) run on it too.
constexpr bool kWideF8 = true;
constexpr int kBmWgrad = 256;
constexpr int kBmWgradDown = 256;

enum GemmKind {
  K_GATEUP_FWD = 0, K_DOWN_FWD = 1, K_DOWN_DGRAD = 2, K_GATEUP_DGRAD = 3, K_WGRAD = 4,
  K_WGRAD8 = 5,   // FP8 weight gradient: K-grouped, both operands K-contiguous codes
  K_ROUTER_DX = 6  // router input gradient: T token rows, K = 2E, B = W_r read twice
};
constexpr bool k_grouped(int kind) { return kind == K_WGRAD || kind == K_WGRAD8; }

struct GemmArgs {
  const bf16_t* a;
  long lda;
  // M-grouped products with a K-contiguous A: null = A row r is row r of a;
  // else A row r is row a_rows[r] of a, which has a_nrows rows (the grouped
  // FFN forward reading the token rows in place of their permuted copy)
  const int32_t* a_rows;
  int a_nrows;
  const bf16_t* b0;  // B operand (gate / the only one)
  const bf16_t* b1;  // second B tensor (up), or null
  long ldb;
  long b_group_stride;      // elements between experts in b0 / b1
  const int32_t* offsets;   // group row offsets [groups + 1], or null for even splits
                            // (WGRAD8: padded code offsets, multiples of 64)
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
  int fold;                 // WGRAD: F > 0 stores column c + column F + c (c < F), 0 = plain
  // FP8 forward: row scales of A (grouped-row order) and column scales of the
  // B tensors ([groups][N] floats, sb_group_stride apart)
  const float* sa;
  const float* sb0;
  const float* sb1;
  long sb_group_stride;
  long sa_group_stride;     // WGRAD8: per-group row scales of A ([groups][M] floats)
  // Dynamic tile order: null = static (workgroup g takes tiles g, g + grid,
  // ...); else a zeroed counter from which workgroups draw their tiles after
  // the first (tile grid + ticket), so that kernels running side by side
  // share CUs as they free up.
  int* tile_ctr;
  // K-grouped FFN weight gradients: the K-chunk plan (null: one chunk per
  // group, the offsets' row ranges) and the fp32 partial slots [slots][M][N]
  // of the chunks after a split group's first
  const int32_t* kplan;
  float* fpart;
};

// Load balance of the K-grouped weight gradients.  Their reduction runs over an
// expert's rows, so one hot expert makes n_mtiles x n_ntiles tiles whose K
// loops are as long as its row count, while the rest of the chip idles.  An
// expert whose rows exceed W = max(kSplitMinRows, ceil(R tiles / CUs)) (R the
// routed rows, tiles its tiles per expert: beyond W one of its tiles alone is
// more than a CU's average share) is cut into S = min(kSplitMaxChunks,
// ceil(rows / W)) chunks of a multiple of 64 rows.  Chunk 0 writes the
// expert's weight gradient as an unsplit expert would (overwriting or adding);
// chunks 1 .. S - 1 write fp32 partial slots, which wgrad_split_reduce_kernel
// then adds in chunk order (a fixed order: the result does not depend on
// timing).  Since S - 1 < rows / W for a split expert, the slots of one
// product never exceed R / W <= kCUs / tiles.
constexpr int kSplitMaxChunks = 8;
constexpr int kSplitMinRows = 1024;
// Plan of one product (int32): [0] chunks, [1] split experts, then per chunk
// (expert, first row, end row, partial slot or -1), in the order the tiles are
// handed out (largest experts first), then per split expert (expert, chunks,
// first slot) from word 2 + 4 (E_l + slots).
struct WgradPlan {
  int32_t* t[2];  // gate/up product, down product (null: no plans)
  int tiles[2];   // tiles per expert
  int slots[2];   // partial slots available
};
__host__ __device__ constexpr int wgrad_plan_ints(int E_l, int slots) {
  return 2 + 4 * (E_l + slots) + 3 * (E_l < slots ? E_l : slots);
}

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

template <int KIND> struct Traits {
  static constexpr bool A_KC = KIND != K_WGRAD;
  static constexpr bool B_KC =
      KIND == K_GATEUP_FWD || KIND == K_DOWN_FWD || KIND == K_WGRAD8 || KIND == K_ROUTER_DX;
};

// LDS layouts of the tiles (swizzles, DMA placement, fragment offsets):
// lds_layout.h.

// ---------------------------------------------------------------------------
// DMA operands (the buffer -> LDS helpers are in common.h)
// ---------------------------------------------------------------------------
// One operand of one tile: buffer resource(s) and, per DMA instruction of this
// lane, the byte offset at k = 0.
template <int NI>
struct Operand {
  rsrc_t rsrc;
  rsrc_t rsrc2;      // second tensor (gate/up split), if any
  uint32_t voff[NI];
  uint32_t kstep;    // byte step per unit of k (KC: 2, MC: row pitch in bytes)
};

// ---------------------------------------------------------------------------
// MFMA fragments from LDS
// ---------------------------------------------------------------------------
// GATEUP_FWD B tile rows interleave 32 gate rows and 32 up rows; DMA
// instruction u of a wave fills tile rows R (w NIB + u) .. + R - 1, R = 512 /
// BKX rows per instruction (w NIB R a multiple of 64), so whether it carries
// up rows depends on u alone.
template <class C>
__device__ __forceinline__ bool gateup_is_up(int u) { return ((u * (512 / C::BKX)) >> 5) & 1; }

// DMA of one K step (k0 = first k) into the wave's part of a ring slot
// (la, lb: LDS byte addresses).
// DMA instruction u of one K step (k0 = first k) into the wave's part of a
// ring slot (la, lb: LDS byte addresses); u < NIA: A, else B.  u is a
// compile-time constant at every call (unrolled loops).  The K loop issues
// every stage unconditionally, also the ones past the end of K, so that it
// has no branches (a branch between MFMAs costs the matrix core about 40% of
// its rate): for those `kill` = 2^31 moves the offset beyond every operand's
// buffer range (all below 2 GiB), the hardware drops the read and writes
// zeros into a slot that is not read again.

template <int KIND, class C>
__device__ __forceinline__ void dma_piece(const GemmArgs& p, const Operand<C::NIA>& opA,
                                          const Operand<C::NIB>& opB, uint32_t la, uint32_t lb,
                                          int k0, uint32_t kill, int u) {
  constexpr int NIA = C::NIA;
  if (u < NIA) {
    dma16(opA.rsrc, (opA.voff[u] + (uint32_t)k0 * opA.kstep) | kill, la + u * 1024);
    return;
  }
  const int v = u - NIA;
  if constexpr (KIND == K_GATEUP_FWD) {
    // each instruction fills 16 rows of one gate or up block
    dma16(gateup_is_up<C>(v) ? opB.rsrc2 : opB.rsrc, (opB.voff[v] + (uint32_t)k0 * 2) | kill, lb + v * 1024);
  } else if constexpr (KIND == K_GATEUP_DGRAD) {
    const bool up = k0 >= p.I;
    const uint32_t kk = (uint32_t)(up ? k0 - p.I : k0);
    dma16(up ? opB.rsrc2 : opB.rsrc, (opB.voff[v] + kk * opB.kstep) | kill, lb + v * 1024);
  } else if constexpr (KIND == K_ROUTER_DX) {
    // columns k and E + k of the product both read W_r's column k (p.I = E)
    const uint32_t kk = (uint32_t)(k0 >= p.I ? k0 - p.I : k0);
    dma16(opB.rsrc, (opB.voff[v] + kk * 2) | kill, lb + v * 1024);
  } else {
    dma16(opB.rsrc, (opB.voff[v] + (uint32_t)k0 * opB.kstep) | kill, lb + v * 1024);
  }
}

// ---------------------------------------------------------------------------
// The LDS ring (dynamic LDS of Cfg::kLdsBytes): NST slots of A, then NST slots
// of B.  Slots are addressed with a wave-uniform byte offset, so one per-lane
// base register serves every slot (the DMA is inline asm, so the compiler adds
// no waits of its own between the DMA and the fragment reads; the explicit
// waits below order the ring).
// ---------------------------------------------------------------------------
extern __shared__ bf16_t g_lds[];
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

__device__ __forceinline__ lds_char_t* lds_ptr(uint32_t byte) {
  return (lds_char_t*)((lds_void_t*)g_lds) + byte;
}

// Per-lane byte offsets of the MFMA fragments inside a tile slot, fixed for the
// kernel's life; everything else in a fragment address is wave-uniform or a
// compile-time constant.
//   KC (rows of BKX bf16): lane l reads row l % 32 of a 32-row block, logical
//   chunk 2 s + l / 32; the block's first row (a multiple of 16) does not
//   change the swizzle, so kc[s] is the offset for block row 0.
//   MC (transposing reads, width W): with g = l / 16, i = l % 16 the lane reads
//   k = 16 s + 8 (g / 2) + i / 4 and column 32 M + 16 (g % 2) + 4 (i % 4) of the
//   slot row, M the absolute 32-column block (wave base plus fragment index),
//   i.e. logical chunk 4 M + x, x = 2 (g % 2) + (i % 4) / 2, which sits at
//   chunk 4 (M ^ (k % 4)) + x.  The four k rows one half-wave reads (k % 4 =
//   0..3) thus fall in four different 64-byte quarters of the 256-byte bank
//   line: the 32 lanes cover all 64 banks once.  mc[j] is the whole offset of
//   fragment j (wave base included; the k sub-step is added per read).
template <class C>
struct FragLanes {
  uint32_t kc[C::KSUB];
  uint32_t mc_a[4];
  uint32_t mc_b[NI];
};

template <int W, int N>
__device__ __forceinline__ void mc_lane_offsets(int lane, int mb, uint32_t (&mc)[N], int n) {
#pragma unroll
  for (int j = 0; j < N; ++j) mc[j] = j < n ? mc_lane_offset<W>(lane, mb + j) : 0u;
}

template <class C>
__device__ __forceinline__ FragLanes<C> frag_lanes(int lane, int wave) {
  FragLanes<C> L;
#pragma unroll
  for (int s = 0; s < C::KSUB; ++s) L.kc[s] = kc_lane_offset<C::BKX>(lane, s);
  mc_lane_offsets<C::BM>(lane, (wave >> 1) * (C::WM / 32), L.mc_a, C::MI);
  mc_lane_offsets<BN>(lane, (wave & 1) * (WN / 32), L.mc_b, NI);
  return L;
}

// KC fragment: block of 32 rows starting at byte `blk` of the slot.
__device__ __forceinline__ bf16x8_t frag_kc(uint32_t slot, uint32_t lane_off, int blk) {
  return *(const lds_bf16x8_t*)(lds_ptr(slot + lane_off) + blk);
}

// MC fragment: lane l gets column c0 + l % 32, k = 16 s + 8 (l / 32) + 0..7,
// from two transposing reads (rows k and k + 4 of each 16-lane group).
template <int W>
__device__ __forceinline__ bf16x8_t frag_mc(uint32_t slot, uint32_t lane_off, int cst) {
  lds_char_t* q = lds_ptr(slot + lane_off) + cst;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)q);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(q + 8 * W));
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// MFMA fragments of one k = 16 sub-step of a wave's sub-tile.
template <class C>
struct Frags {
  bf16x8_t a[C::MI];
  bf16x8_t b[NI];
};

// sa / sb: byte offsets of the A / B slot plus the wave's block base
// (KC: first row * BKX * 2; MC: first column * 2).
// Fragment j of a sub-step, in the order the MFMAs of the next sub-step need
// them: A0, B0, B1, B2, B3, A1, A2, ... (MFMAs run mi-major).
template <class C>
__host__ __device__ constexpr int frag_order(int j) {
  return j == 0 ? 0 : j <= NI ? C::MI + j - 1 : j - NI;
}

template <int KIND, class C>
__device__ __forceinline__ void load_frag(Frags<C>& f, int j, int s, uint32_t sa, uint32_t sb,
                                          const FragLanes<C>& L) {
  using Tr = Traits<KIND>;
  constexpr int MI = C::MI, BM = C::BM;
  const int q = frag_order<C>(j);
  if (q < MI) {
    const int mi = q;
    if constexpr (Tr::A_KC)
      f.a[mi] = frag_kc(sa, L.kc[s], mi * 32 * C::BKX * 2);
    else
      f.a[mi] = frag_mc<BM>(sa, L.mc_a[mi], 2 * (16 * s * BM));
  } else {
    const int ni = q - MI;
    if constexpr (Tr::B_KC)
      f.b[ni] = frag_kc(sb, L.kc[s], ni * 32 * C::BKX * 2);
    else
      f.b[ni] = frag_mc<BN>(sb, L.mc_b[ni], 2 * (16 * s * BN));
  }
}

template <int KIND, class C>
__device__ __forceinline__ void load_frags(Frags<C>& f, int s, uint32_t sa, uint32_t sb,
                                           const FragLanes<C>& L) {
#pragma unroll
  for (int j = 0; j < C::MI + NI; ++j) load_frag<KIND, C>(f, j, s, sa, sb, L);
}

__device__ __forceinline__ void mfma1(f32x16_t& acc, bf16x8_t a, bf16x8_t b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

template <class C>
__device__ __forceinline__ void mma(f32x16_t (&acc)[C::MI][NI], const Frags<C>& f) {
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) mfma1(acc[mi][ni], f.a[mi], f.b[ni]);
}

// FP8: a (mi, ni) block's operands for one 64-code K step: bytes 0..15 of the
// lane's 32 are the fragment of bf16 sub-step 0, bytes 16..31 that of
// sub-step 1 (on the wide ring the block's second step takes sub-steps 2
// and 3).
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
template <class C>
struct Frags8 {
  i32x8_t a[C::MI];
  i32x8_t b[NI];
};

__device__ __forceinline__ void mfma_f8(f32x16_t& acc, const i32x8_t& a, const i32x8_t& b) {
  // format 0 = E4M3 for both operands; scale 127 = 2^0 for every 32-code block
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

template <class C>
__device__ __forceinline__ void read_a8(Frags8<C>& f, int mi, int s, uint32_t sa, const FragLanes<C>& L) {
  const i32x4_t v = __builtin_bit_cast(i32x4_t, frag_kc(sa, L.kc[s], mi * 32 * C::BKX * 2));
  if ((s & 1) == 0) f.a[mi].lo = v; else f.a[mi].hi = v;
}
template <class C>
__device__ __forceinline__ void read_b8(Frags8<C>& f, int ni, int s, uint32_t sb, const FragLanes<C>& L) {
  const i32x4_t v = __builtin_bit_cast(i32x4_t, frag_kc(sb, L.kc[s], ni * 32 * C::BKX * 2));
  if ((s & 1) == 0) f.b[ni].lo = v; else f.b[ni].hi = v;
}

// A stall in a wave's instruction stream idles its matrix core unless another
// wave has MFMAs ready, and a wave runs at most about one MFMA ahead of the
// pipe.  So the other work of a K step is spread between the MFMAs, one or
// two instructions after each (the scheduling barriers keep this order), and
// the K loop has no branches (a branch between MFMAs costs the matrix core
// about 40% of its rate).  A step's DMA is issued in two halves, each spread
// evenly over the MFMAs of one sub-step (every DSTR-th MFMA): four waves'
// DMA instructions bunched together outrun the texture unit and stall the
// issuing waves.
//   sub-step 0: MFMA j, then fragment j of the next sub-step (j < MI + NI)
//               and the second half of the DMA of step kt + NST - 1;
//   sub-step 1: MFMA j, then the first half of the DMA of step kt + NST and
//               fragment j - (MI NI - MI - NI) of the next step's sub-step 0
//               (the reads end with the last MFMA).
template <class C>
struct DmaSplit {
  static constexpr int ND = C::NIA + C::NIB;  // DMA instructions per wave per step
  static constexpr int NH = ND / 2;        // per half
  static constexpr int DSTR = C::MI * NI / NH;
  static_assert(ND % 2 == 0 && DSTR >= 1, "DMA halves");
};

template <int KIND, class C>
__device__ __forceinline__ void mma_read_next(f32x16_t (&acc)[C::MI][NI], const Frags<C>& cur,
                                              Frags<C>& nxt, int s_next, uint32_t sa, uint32_t sb,
                                              const FragLanes<C>& L, const GemmArgs& p,
                                              const Operand<C::NIA>& opA, const Operand<C::NIB>& opB,
                                              uint32_t la, uint32_t lb, int k0, uint32_t kill) {
  constexpr int NM = C::MI * NI, NR = C::MI + NI;
  using D = DmaSplit<C>;
  static_assert(NR <= NM, "interleave pattern");
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    mfma1(acc[j / NI][j % NI], cur.a[j / NI], cur.b[j % NI]);
    if (j < NR) load_frag<KIND, C>(nxt, j, s_next, sa, sb, L);
    if (j % D::DSTR == 0 && j / D::DSTR < D::NH)
      dma_piece<KIND, C>(p, opA, opB, la, lb, k0, kill, D::NH + j / D::DSTR);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int KIND, class C>
__device__ __forceinline__ void mma_dma_read(f32x16_t (&acc)[C::MI][NI], const Frags<C>& cur,
                                             Frags<C>& nxt, uint32_t sa, uint32_t sb,
                                             const FragLanes<C>& L, const GemmArgs& p,
                                             const Operand<C::NIA>& opA, const Operand<C::NIB>& opB,
                                             uint32_t la, uint32_t lb, int k0, uint32_t kill) {
  constexpr int NM = C::MI * NI, NR = C::MI + NI;
  using D = DmaSplit<C>;
  static_assert(NR <= NM, "interleave pattern");
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    mfma1(acc[j / NI][j % NI], cur.a[j / NI], cur.b[j % NI]);
    if (j % D::DSTR == 0 && j / D::DSTR < D::NH)
      dma_piece<KIND, C>(p, opA, opB, la, lb, k0, kill, j / D::DSTR);
    if (j >= NM - NR) load_frag<KIND, C>(nxt, j - (NM - NR), 0, sa, sb, L);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// Epilogue: the accumulators go through LDS so that global stores are 16-byte
// row segments.  Each wave stages 16 rows x 128 fp32 of its sub-tile at a time
// (half of a 32-row MFMA block row: output registers q = 8 h .. 8 h + 7) into
// its own 8 KB (16-byte chunks XOR-swizzled so the row pairs written by one
// MFMA output register hit different banks), then every lane handles 8
// consecutive columns of a row.
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ float* stage_area(int wave) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(g_lds) + C::kStageOff) + wave * 2048;
}

template <int MI>
__device__ __forceinline__ void stage_half(float* st, const f32x16_t (&acc)[MI][NI], int mi, int h,
                                           int lane) {
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int q8 = 0; q8 < 8; ++q8) {
      const int q = 8 * h + q8;
      const int r = 8 * (q8 >> 2) + 4 * (lane >> 5) + (q & 3);  // row within the half
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

// Output descriptors of the M-grouped products cover exactly the tile's rows
// [row0, row1) of a buffer: the hardware range check drops stores of rows past
// the tile (and any offset at or past kOutKill), so the stores are issued
// unconditionally and the compiler counts them exactly (no branch-forced
// drains of the memory counter).  A null buffer gets an empty range.
typedef __amdgpu_buffer_rsrc_t out_rsrc_t;
constexpr uint32_t kOutKill = 0x80000000u;
__device__ __forceinline__ out_rsrc_t out_rsrc(const bf16_t* base, long row0, long row1, long ld) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base) + (base ? row0 * ld : 0), 0,
                                           base ? (int)((row1 - row0) * ld * 2) : 0, 0x00020000);
}
__device__ __forceinline__ void store16(out_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, off, 0, 0);
}
// The same with the non-temporal cache policy (gfx950 cache-policy bit NT):
// for outputs that the next kernels do not read.
constexpr int kCpolNT = 2;
__device__ __forceinline__ void store16_nt(out_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, off, 0, kCpolNT);
}

// FP8 epilogue scales of one tile, loaded after the previous tile's epilogue
// (so that no wait for them lands behind this tile's DMAs): the lane's row
// scales in the order the epilogue visits its rows, and its 8 columns' scales
// (GATEUP_FWD: gate then up).
template <int KIND, class C>
struct Scales {
  static constexpr int NR = KIND == K_GATEUP_FWD ? 4 * C::MI : 8 * C::MI;
  static constexpr int NC = KIND == K_GATEUP_FWD ? 16 : 8;
  float row[NR];
  float col[NC];
};

template <int KIND, class C>
__device__ __forceinline__ void load_scales(const GemmArgs& p, int e, int nt, int n0, int row0,
                                            int row1, int wave, int lane, Scales<KIND, C>& S) {
  constexpr int MI = C::MI, WM = C::WM;
  const int wm = wave >> 1, wn = wave & 1;
  if constexpr (KIND == K_WGRAD8) {
    // row0 = the tile's first output row m0: the group's A scales of the rows
    // the epilogue visits (past M: zero, never stored), and the B scales of
    // the lane's columns 4 (lane % 16) .. + 3 and 64 more
    const out_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.sa) + (long)e * p.sa_group_stride + row0, 0, (p.M - row0) * 4, 0x00020000);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int lrow = wm * WM + mi * 32 + 16 * h + it * 4 + (lane >> 4);
          S.row[(mi * 2 + h) * 4 + it] =
              __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, lrow * 4, 0, 0));
        }
    const int n = n0 + wn * WN + (lane & 15) * 4;
    const out_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.sb0) + (long)e * p.sb_group_stride, 0, p.N * 4, 0x00020000);
    const u32x4_t c0 = __builtin_amdgcn_raw_buffer_load_b128(rc, n < p.N ? (uint32_t)n * 4 : kOutKill, 0, 0);
    const u32x4_t c1 =
        __builtin_amdgcn_raw_buffer_load_b128(rc, n + 64 < p.N ? (uint32_t)(n + 64) * 4 : kOutKill, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S.col[i] = __uint_as_float(c0[i]);
      S.col[4 + i] = __uint_as_float(c1[i]);
    }
    return;
  }
  // rows [row0, row1) of the row scales; the ones past row1 read as zero
  const out_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.sa) + row0, 0,
                                                          (row1 - row0) * 4, 0x00020000);
  const float* cb = p.sb0 + (long)e * p.sb_group_stride;
  if constexpr (KIND == K_GATEUP_FWD) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int lrow = wm * WM + mi * 32 + 16 * h + it * 8 + (lane >> 3);
          S.row[(mi * 2 + h) * 2 + it] =
              __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, lrow * 4, 0, 0));
        }
    const int col = nt * 128 + wn * 64 + (lane & 7) * 8;
    const uint32_t o = col < p.I ? (uint32_t)col * 4 : kOutKill;
    const out_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(cb), 0, p.I * 4, 0x00020000);
    const out_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.sb1 + (long)e * p.sb_group_stride), 0, p.I * 4, 0x00020000);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4_t g = __builtin_amdgcn_raw_buffer_load_b128(rg, o + 16 * q, 0, 0);
      const u32x4_t u = __builtin_amdgcn_raw_buffer_load_b128(ru, o + 16 * q, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        S.col[4 * q + i] = __uint_as_float(g[i]);
        S.col[8 + 4 * q + i] = __uint_as_float(u[i]);
      }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int lrow = wm * WM + mi * 32 + 16 * h + it * 4 + (lane >> 4);
          S.row[(mi * 2 + h) * 4 + it] =
              __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, lrow * 4, 0, 0));
        }
    const int n = n0 + wn * WN + (lane & 15) * 8;
    const uint32_t o = n < p.N ? (uint32_t)n * 4 : kOutKill;
    const out_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(cb), 0, p.N * 4, 0x00020000);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4_t c = __builtin_amdgcn_raw_buffer_load_b128(rc, o + 16 * q, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) S.col[4 * q + i] = __uint_as_float(c[i]);
    }
  }
}

// The scale registers are ready (called after the K loop has drained the
// memory counter, so the compiler's wait for them costs nothing there).
template <int KIND, class C>
__device__ __forceinline__ void touch_scales(const Scales<KIND, C>& S) {
#pragma unroll
  for (int i = 0; i < Scales<KIND, C>::NR; ++i) asm volatile("" ::"v"(S.row[i]));
#pragma unroll
  for (int i = 0; i < Scales<KIND, C>::NC; ++i) asm volatile("" ::"v"(S.col[i]));
}

template <int KIND, class C, bool F8 = false>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const f32x16_t (&acc)[C::MI][NI], int e,
                                         int nt, int n0, int m0, int row0, int row1, int wave,
                                         int lane,
                                         const Scales<KIND, C>& S, int slot = -1) {
  constexpr int MI = C::MI, WM = C::WM;
  const int wm = wave >> 1, wn = wave & 1;
  float* st = stage_area<C>(wave);
  if constexpr (KIND == K_WGRAD) {
    if (p.fold > 0) {  // uniform: the whole workgroup takes this path
      // Output column c (< F) is the sum of tile columns c and F + c, which
      // may belong to the other wave of the row pair: all four waves stage a
      // half block row, then every thread adds pairs of 8 columns.
      const int F = p.fold;
      const int tasks = 2 * 16 * (F / 8);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          stage_half(st, acc, mi, h, lane);
          __syncthreads();
          for (int q = threadIdx.x; q < tasks; q += NTH) {
            const int c = (q % (F / 8)) * 8;
            const int r = (q / (F / 8)) % 16;
            const int pw = q / (F / 8) / 16;  // wave row of the pair
            const int m = m0 + pw * WM + mi * 32 + 16 * h + r;
            if (m >= p.M) continue;
            float lo[8], hi[8];
            load8(stage_area<C>(pw * 2 + c / WN), r, c % WN, lo);
            load8(stage_area<C>(pw * 2 + (F + c) / WN), r, (F + c) % WN, hi);
            float* dst = p.f0 + e * p.f_group_stride + (long)m * p.ldc + c;
            float4* d4 = reinterpret_cast<float4*>(dst);
            d4[0] = make_float4(lo[0] + hi[0], lo[1] + hi[1], lo[2] + hi[2], lo[3] + hi[3]);
            d4[1] = make_float4(lo[4] + hi[4], lo[5] + hi[5], lo[6] + hi[6], lo[7] + hi[7]);
          }
          __syncthreads();
        }
      return;
    }
    if (p.accumulate == 0 || slot >= 0) {  // uniform
      // Overwrite: unconditional buffer stores whose descriptor covers the
      // output rows of this 16-row pass (rows past M dropped by the range
      // check, columns past N by the kill offset), so their number is static
      // (epilogue_vmem_ops) and the next tile's K loop waits for its own DMA,
      // not for these stores.  Each store instruction writes 256 contiguous
      // bytes of a row (lane l: columns 4 (l % 16) .. + 3 and 64 more), and the
      // non-temporal policy keeps the fp32 result out of L2 (read only by the
      // optimizer).
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          stage_half(st, acc, mi, h, lane);
          // first output row of the pass; a pass never straddles m_split
          // (a multiple of 64 rows)
          const int mb = m0 + wm * WM + mi * 32 + 16 * h;
          // a split chunk's partial slot is one [M][N] block (no gate/up split)
          const bool part = slot >= 0;
          const bool first = part || mb < p.m_split || p.f1 == nullptr;
          float* base = part ? p.fpart + (long)slot * p.M * p.ldc
                             : (first ? p.f0 : p.f1) + e * p.f_group_stride;
          const int mrel = (part || first) ? mb : mb - p.m_split;
          const int nrows = (part ? p.M : first ? min(p.m_split, p.M) : p.M - p.m_split) - mrel;
          const out_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
              base + (long)max(mrel, 0) * p.ldc, 0, nrows > 0 ? (int)(nrows * p.ldc * 4) : 0, 0x00020000);
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int r = it * 4 + (lane >> 4);
            const int c = (lane & 15) * 4;
            const int n = n0 + wn * WN + c;
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&st[stage_idx(r, c)]);
            const f32x4_t b = *reinterpret_cast<const f32x4_t*>(&st[stage_idx(r, c + 64)]);
            const uint32_t oa = n < p.N ? (uint32_t)((r * p.ldc + n) * 4) : kOutKill;
            const uint32_t ob = n + 64 < p.N ? (uint32_t)((r * p.ldc + n + 64) * 4) : kOutKill;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, a), ro, oa, 0, kCpolNT);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, b), ro, ob, 0, kCpolNT);
          }
          // the next half reuses the staging area
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
      return;
    }
    // Accumulate: read, add, write back (memory operations depend on the
    // data; the next tile's K loop then waits for them all).
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        stage_half(st, acc, mi, h, lane);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int r = it * 4 + (lane >> 4);
          const int c = (lane & 15) * 8;
          const int m = m0 + wm * WM + mi * 32 + 16 * h + r;
          const int n = n0 + wn * WN + c;
          if (m >= p.M || n >= p.N) continue;
          float v[8];
          load8(st, r, c, v);
          float* dst = (m < p.m_split) ? p.f0 + e * p.f_group_stride + (long)m * p.ldc + n
                                       : p.f1 + e * p.f_group_stride + (long)(m - p.m_split) * p.ldc + n;
          float4* d4 = reinterpret_cast<float4*>(dst);
          const float4 o0 = d4[0], o1 = d4[1];
          d4[0] = make_float4(o0.x + v[0], o0.y + v[1], o0.z + v[2], o0.w + v[3]);
          d4[1] = make_float4(o1.x + v[4], o1.y + v[5], o1.z + v[6], o1.w + v[7]);
        }
        // the next half reuses the staging area
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
  } else if constexpr (KIND == K_WGRAD8) {
    // FP8 weight gradient: the sum of the code products times the group's row
    // scale of A and column scale of B (powers of two: exact), then the same
    // stores as the bf16 overwrite above (rows past M dropped by the range
    // check, columns past N by the kill offset); accumulate reads the old
    // value through the same descriptor and adds it first.
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        stage_half(st, acc, mi, h, lane);
        const int mb = m0 + wm * WM + mi * 32 + 16 * h;
        // a split chunk's partial slot is one [M][N] block, overwritten
        const bool part = slot >= 0;
        const bool first = part || mb < p.m_split || p.f1 == nullptr;
        float* base = part ? p.fpart + (long)slot * p.M * p.ldc
                           : (first ? p.f0 : p.f1) + e * p.f_group_stride;
        const int mrel = (part || first) ? mb : mb - p.m_split;
        const int nrows = (part ? p.M : first ? min(p.m_split, p.M) : p.M - p.m_split) - mrel;
        const out_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            base + (long)max(mrel, 0) * p.ldc, 0, nrows > 0 ? (int)(nrows * p.ldc * 4) : 0, 0x00020000);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int r = it * 4 + (lane >> 4);
          const int c = (lane & 15) * 4;
          const int n = n0 + wn * WN + c;
          f32x4_t a = *reinterpret_cast<const f32x4_t*>(&st[stage_idx(r, c)]);
          f32x4_t b = *reinterpret_cast<const f32x4_t*>(&st[stage_idx(r, c + 64)]);
          const float sr = S.row[(mi * 2 + h) * 4 + it];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a[j] *= sr * S.col[j];
            b[j] *= sr * S.col[4 + j];
          }
          const uint32_t oa = n < p.N ? (uint32_t)((r * p.ldc + n) * 4) : kOutKill;
          const uint32_t ob = n + 64 < p.N ? (uint32_t)((r * p.ldc + n + 64) * 4) : kOutKill;
          if (p.accumulate != 0 && !part) {  // uniform
            a = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, oa, 0, 0)) + a;
            b = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, ob, 0, 0)) + b;
          }
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, a), ro, oa, 0, kCpolNT);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, b), ro, ob, 0, kCpolNT);
        }
        // the next half reuses the staging area
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
  } else if constexpr (KIND == K_ROUTER_DX) {
    // fp32 rows [row0, row1) of dx_router: as the weight gradients' overwriting
    // epilogue, each store instruction writes 256 contiguous bytes of a row
    // (lane l: columns 4 (l % 16) .. + 3 and 64 more); rows past the tile fall
    // outside the descriptor's range, columns past N take the kill offset.
    const out_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(p.f0 + (long)row0 * p.ldc, 0,
                                                            (int)((row1 - row0) * p.ldc * 4), 0x00020000);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        stage_half(st, acc, mi, h, lane);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int r = it * 4 + (lane >> 4);
          const int lrow = wm * WM + mi * 32 + 16 * h + r;
          const int c = (lane & 15) * 4;
          const int n = n0 + wn * WN + c;
          const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&st[stage_idx(r, c)]);
          const f32x4_t b = *reinterpret_cast<const f32x4_t*>(&st[stage_idx(r, c + 64)]);
          const uint32_t oa = n < p.N ? (uint32_t)((lrow * p.ldc + n) * 4) : kOutKill;
          const uint32_t ob = n + 64 < p.N ? (uint32_t)((lrow * p.ldc + n + 64) * 4) : kOutKill;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, a), ro, oa, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, b), ro, ob, 0, 0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
  } else if constexpr (KIND == K_GATEUP_FWD) {
    // staged columns: [g 32 | u 32 | g 32 | u 32] for h columns nt*128 + wn*64 + 0..63
    const out_rsrc_t rh = out_rsrc(p.c0, row0, row1, p.ldc);
    const out_rsrc_t rgu = out_rsrc(p.c1, row0, row1, 2L * p.I);
    const int hc = (lane & 7) * 8;              // 0..56: h column within the wave
    const int sc = (hc >> 5) * 64 + (hc & 31);  // staged gate column
    const int col = nt * 128 + wn * 64 + hc;
    const bool col_ok = col < p.I;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        stage_half(st, acc, mi, h, lane);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int r = it * 8 + (lane >> 3);
          const int lrow = wm * WM + mi * 32 + 16 * h + r;  // row within the tile
          float g[8], u[8], hv[8];
          load8(st, r, sc, g);
          load8(st, r, sc + 32, u);
          if constexpr (F8) {
            const float sr = S.row[(mi * 2 + h) * 2 + it];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              g[j] *= sr * S.col[j];
              u[j] *= sr * S.col[8 + j];
            }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) hv[j] = g[j] * fast_rcp(1.f + __expf(-g[j])) * u[j];
          const uint32_t oh = col_ok ? (uint32_t)((lrow * p.ldc + col) * 2) : kOutKill;
          const uint32_t og = col_ok ? (uint32_t)((lrow * 2 * p.I + col) * 2) : kOutKill;
          store16(rh, oh, pack8(hv));
          // g and u are read again only by the backward
          store16_nt(rgu, og, pack8(g));
          store16_nt(rgu, og + (col_ok ? p.I * 2 : 0), pack8(u));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
  } else {  // DOWN_FWD, GATEUP_DGRAD, DOWN_DGRAD: rows of the grouped buffer
    const int c = (lane & 15) * 8;
    const int n = n0 + wn * WN + c;
    const bool col_ok = n < p.N;
    const long ldo = (KIND == K_DOWN_DGRAD) ? 2L * p.I : p.ldc;
    const out_rsrc_t ro = out_rsrc(p.c0, row0, row1, ldo);
    // DOWN_DGRAD reads the saved g / u of its rows through the same kind of
    // descriptor (rows past the tile read as zero).  The loads of half pass
    // q + 1 are issued before half pass q's math and stores, so their latency
    // hides behind a pass.
    constexpr int NP = 2 * MI;  // half passes
    out_rsrc_t rg;
    u32x4_t graw[2][4], uraw[2][4];
    if constexpr (KIND == K_DOWN_DGRAD) rg = out_rsrc(p.gu, row0, row1, 2L * p.I);
    // Columns past N take the kill bit OR'd into distinct offsets: with a
    // select between an offset and one shared kill offset, the compiler merged
    // the g and u loads of the killed lanes and branched around them, and the
    // branch's join waited for every outstanding memory operation (vmcnt(0)),
    // the next tile's prefetched DMA included.
    const uint32_t gu_kill = (uint32_t)(!col_ok) << 31;
    auto load_gu = [&](int pq, int b) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int lrow = wm * WM + (pq >> 1) * 32 + 16 * (pq & 1) + it * 4 + (lane >> 4);
        const uint32_t o = (uint32_t)((lrow * 2 * p.I + n) * 2);
        graw[b][it] = __builtin_amdgcn_raw_buffer_load_b128(rg, o | gu_kill, 0, 0);
        uraw[b][it] = __builtin_amdgcn_raw_buffer_load_b128(rg, (o + p.I * 2) | gu_kill, 0, 0);
      }
    };
    if constexpr (KIND == K_DOWN_DGRAD) load_gu(0, 0);
#pragma unroll
    for (int pq = 0; pq < NP; ++pq) {
      const int mi = pq >> 1, h = pq & 1;
      if constexpr (KIND == K_DOWN_DGRAD)
        if (pq + 1 < NP) load_gu(pq + 1, (pq + 1) & 1);
      stage_half(st, acc, mi, h, lane);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 4 + (lane >> 4);
        const int lrow = wm * WM + mi * 32 + 16 * h + r;
        float v[8];
        load8(st, r, c, v);
        if constexpr (F8) {
          const float sr = S.row[pq * 4 + it];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] *= sr * S.col[j];
        }
        const uint32_t o = col_ok ? (uint32_t)((lrow * ldo + n) * 2) : kOutKill;
        if constexpr (KIND == K_DOWN_DGRAD) {
          // v = dh; dG = dh * u * s * (1 + g (1 - s)), dU = dh * SiLU(g), s = sigmoid(g)
          float g[8], u[8], dg[8], du[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4_t& gw = graw[pq & 1][it];
            const u32x4_t& uw = uraw[pq & 1][it];
            g[2 * q] = __uint_as_float(gw[q] << 16);
            g[2 * q + 1] = __uint_as_float(gw[q] & 0xffff0000u);
            u[2 * q] = __uint_as_float(uw[q] << 16);
            u[2 * q + 1] = __uint_as_float(uw[q] & 0xffff0000u);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float sg = fast_rcp(1.f + __expf(-g[j]));
            dg[j] = v[j] * u[j] * sg * (1.f + g[j] * (1.f - sg));
            du[j] = v[j] * g[j] * sg;
          }
          store16(ro, o, pack8(dg));
          store16(ro, o + (col_ok ? p.I * 2 : 0), pack8(du));
        } else {
          store16(ro, o, pack8(v));
        }
      }
      // the next half reuses the staging area
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
// The K steps of one tile (the ring holds steps 0 .. NST - 2 and half of step
// NST - 1 when it starts; f0 holds step 0's sub-step 0 fragments).
// One K step per iteration on ring slot `slot`, software pipelined: the
// fragments of sub-step 1 are read during the first MFMAs of sub-step 0,
// together with the second half of the DMA of step kt + NST - 1 into the
// previous slot (every wave finished reading it before the previous barrier).
// Before the MFMAs of sub-step 1 the wave waits for step kt + 1 to land
// (barrier); between those MFMAs it starts the first half of the DMA of step
// kt + NST into this slot (every wave has finished reading it) and reads the
// next step's sub-step 0 fragments.
template <int KIND, class C>
__device__ __forceinline__ void k_steps(f32x16_t (&acc)[C::MI][NI], Frags<C>& f0, Frags<C>& f1,
                                        const FragLanes<C>& L, const GemmArgs& p,
                                        const Operand<C::NIA>& opA, const Operand<C::NIB>& opB,
                                        uint32_t dma_a, uint32_t dma_b, uint32_t wa, uint32_t wb,
                                        int nk) {
  constexpr int NST = C::NST, NIA = C::NIA, NIB = C::NIB, kSlotA = C::kSlotA, kSlotB = C::kSlotB;
  constexpr int kOffB = C::kOffB, BK = C::BKX;
  static_assert(!C::WIDE, "narrow ring");
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const uint32_t sa = slot * kSlotA + wa, sb = kOffB + slot * kSlotB + wb;
    const int pslot = slot == 0 ? NST - 1 : slot - 1;
    mma_read_next<KIND, C>(acc, f0, f1, 1, sa, sb, L, p, opA, opB, dma_a + pslot * kSlotA,
                           dma_b + pslot * kSlotB, (kt + NST - 1) * BK,
                           kt + NST - 1 < nk ? 0u : kDmaKill);
    const int nslot = slot + 1 == NST ? 0 : slot + 1;
    // Steps kt + 1 .. kt + NST - 1 are in flight; step kt + 1 has landed
    // when only the newer ones (NIA + NIB loads each) remain.
    wait_vm<(NST - 2) * (NIA + NIB)>();
    lds_barrier();  // every wave: step kt + 1 landed, slot `slot` fully read
    mma_dma_read<KIND, C>(acc, f1, f0, nslot * kSlotA + wa, kOffB + nslot * kSlotB + wb, L, p,
                          opA, opB, dma_a + slot * kSlotA, dma_b + slot * kSlotB, (kt + NST) * BK,
                          kt + NST < nk ? 0u : kDmaKill);
    slot = nslot;
  }
}

// The K blocks of one tile on the wide ring.  Block j sits in regions
// (2j) % 5 (A) and (2j + 1) % 5 (B); on entry the regions hold blocks 0 and 1
// (landed or in flight) and f0 holds block 0's sub-step 0 fragments.
//   s0: MFMAs of sub-step 0 (f0), sub-step 1's fragments into f1;
//   s1, s2: MFMAs (f1, then f0), the next sub-step's fragments, and spread
//       between the MFMAs the DMA of block j + 2's A (load 2j + 4, region
//       (2j + 4) % 5 = block j - 1's B, read before the previous barrier);
//   wait until block j + 1 has landed (only block j + 2's A may remain in
//       flight), barrier: every wave has also finished reading block j;
//   s3: MFMAs (f1), the DMA of block j + 2's B (load 2j + 5, region (2j) % 5 =
//       block j's A) and block j + 1's sub-step 0 fragments into f0.
// Block j + 2's B thus has three sub-steps to land, its A about one block.
// MIA < MI: the wave's rows end inside the tile, and only its first MIA
// 32-row blocks are multiplied (the accumulators of the others stay zero; the
// loads, waits and barriers are those of the full form).
template <int KIND, class C, int MIA = C::MI>
__device__ __forceinline__ void k_blocks(f32x16_t (&acc)[C::MI][NI], Frags<C>& f0, Frags<C>& f1,
                                         const FragLanes<C>& L, const GemmArgs& p,
                                         const Operand<C::NIA>& opA, const Operand<C::NIB>& opB,
                                         uint32_t dma_w, uint32_t wa, uint32_t wb, int nk) {
  constexpr int R = C::kRegion, NIA = C::NIA, NIB = C::NIB, MI = C::MI;
  constexpr int NM = MI * NI, NR = MI + NI;
  static_assert(C::WIDE && C::KSUB == 4, "wide ring");
  static_assert(NR <= NM && NIA % 2 == 0 && NM % (NIA / 2) == 0 && NM % NIB == 0, "interleave pattern");
  constexpr int SA = NM / (NIA / 2);  // one A piece every SA MFMAs of s1 and s2
  constexpr int SB = NM / NIB;        // one B piece every SB MFMAs of s3
  int ra = 0;                         // (2j) % 5
  for (int j = 0; j < nk; ++j) {
    const int rb = ra == 4 ? 0 : ra + 1;    // (2j + 1) % 5
    const int rn = rb == 4 ? 0 : rb + 1;    // (2j + 2) % 5: block j + 1's A
    const int rnb = rn == 4 ? 0 : rn + 1;   // (2j + 3) % 5: block j + 1's B
    const int rq = rnb == 4 ? 0 : rnb + 1;  // (2j + 4) % 5: block j + 2's A
    const uint32_t sa = ra * R + wa, sb = rb * R + wb;
    const uint32_t kill = j + 2 < nk ? 0u : kDmaKill;
    const int k2 = (j + 2) * C::BKX;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m / NI < MIA) mfma1(acc[m / NI][m % NI], f0.a[m / NI], f0.b[m % NI]);
      if (m < NR) load_frag<KIND, C>(f1, m, 1, sa, sb, L);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m / NI < MIA) mfma1(acc[m / NI][m % NI], f1.a[m / NI], f1.b[m % NI]);
      if (m < NR) load_frag<KIND, C>(f0, m, 2, sa, sb, L);
      if (m % SA == 0) dma_piece<KIND, C>(p, opA, opB, dma_w + rq * R, 0u, k2, kill, m / SA);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m / NI < MIA) mfma1(acc[m / NI][m % NI], f0.a[m / NI], f0.b[m % NI]);
      if (m < NR) load_frag<KIND, C>(f1, m, 3, sa, sb, L);
      if (m % SA == 0) dma_piece<KIND, C>(p, opA, opB, dma_w + rq * R, 0u, k2, kill, NIA / 2 + m / SA);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm<NIA>();
    lds_barrier();  // every wave: block j + 1 landed, block j fully read
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m / NI < MIA) mfma1(acc[m / NI][m % NI], f1.a[m / NI], f1.b[m % NI]);
      if (m % SB == 0) dma_piece<KIND, C>(p, opA, opB, 0u, dma_w + ra * R, k2, kill, NIA + m / SB);
      if (m >= NM - NR) load_frag<KIND, C>(f0, m - (NM - NR), 0, rn * R + wa, rnb * R + wb, L);
      __builtin_amdgcn_sched_barrier(0);
    }
    ra = rn;
  }
}

// FP8 K loop, on the same ring and DMA schedule as k_steps.  On entry f holds
// the A blocks mi < MI / 2 and every B block of step 0.  Per step:
//   phase 1: MFMAs of the blocks mi < MI / 2; between them the A blocks
//            mi >= MI / 2 of this step are read and the second half of the
//            DMA of step kt + NST - 1 is issued;
//   wait for step kt + 1, barrier;
//   phase 2: MFMAs of the blocks mi >= MI / 2 (ni-major); after the last use
//            of B block ni it is read for step kt + 1, the A blocks
//            mi < MI / 2 of step kt + 1 are read in between, and the first
//            half of the DMA of step kt + NST is issued.
template <int KIND, class C>
__device__ __forceinline__ void k_steps_f8(f32x16_t (&acc)[C::MI][NI], Frags8<C>& f,
                                           const FragLanes<C>& L, const GemmArgs& p,
                                           const Operand<C::NIA>& opA, const Operand<C::NIB>& opB,
                                           uint32_t dma_a, uint32_t dma_b, uint32_t wa, uint32_t wb,
                                           int nk) {
  constexpr int NST = C::NST, NIA = C::NIA, NIB = C::NIB, kSlotA = C::kSlotA, kSlotB = C::kSlotB;
  constexpr int kOffB = C::kOffB, MI = C::MI, BK = C::BKX;
  static_assert(!C::WIDE, "narrow ring");
  constexpr int MH = MI / 2, NP = MH * NI;  // MFMAs per phase
  using D = DmaSplit<C>;
  constexpr int STR = NP / D::NH;           // one DMA piece every STR MFMAs
  static_assert(MI % 2 == 0 && NP % D::NH == 0 && STR >= 1, "FP8 phase split");
  static_assert(2 * MH <= NP, "A reads of phase 1");
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const uint32_t sa = slot * kSlotA + wa, sb = kOffB + slot * kSlotB + wb;
    const int pslot = slot == 0 ? NST - 1 : slot - 1;
    const uint32_t kill1 = kt + NST - 1 < nk ? 0u : kDmaKill;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      mfma_f8(acc[j / NI][j % NI], f.a[j / NI], f.b[j % NI]);
      if (j < 2 * MH) read_a8<C>(f, MH + j / 2, j % 2, sa, L);
      if (j % STR == 0)
        dma_piece<KIND, C>(p, opA, opB, dma_a + pslot * kSlotA, dma_b + pslot * kSlotB,
                           (kt + NST - 1) * BK, kill1, D::NH + j / STR);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int nslot = slot + 1 == NST ? 0 : slot + 1;
    wait_vm<(NST - 2) * (NIA + NIB)>();
    lds_barrier();  // every wave: step kt + 1 landed, slot `slot` fully read
    const uint32_t na = nslot * kSlotA + wa, nb = kOffB + nslot * kSlotB + wb;
    const uint32_t kill2 = kt + NST < nk ? 0u : kDmaKill;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int ni = j / MH, mi = MH + j % MH;
      mfma_f8(acc[mi][ni], f.a[mi], f.b[ni]);
      if (j % MH == MH - 1) {  // last use of B block ni in this step
        read_b8<C>(f, ni, 0, nb, L);
        read_b8<C>(f, ni, 1, nb, L);
      }
      if (j < 2 * MH) read_a8<C>(f, j / 2, j % 2, na, L);
      if (j % STR == 0)
        dma_piece<KIND, C>(p, opA, opB, dma_a + slot * kSlotA, dma_b + slot * kSlotB,
                           (kt + NST) * BK, kill2, j / STR);
      __builtin_amdgcn_sched_barrier(0);
    }
    slot = nslot;
  }
}

// FP8 K blocks on the wide ring: a block holds 128 codes per row, two E4M3
// MFMA steps (step 0 on the fragments of bf16 sub-steps 0 and 1, step 1 on
// sub-steps 2 and 3).  One fragment set, as in k_steps_f8: on entry f holds
// step 0's A blocks mi < MI / 2 and all its B blocks.  Per block j:
//   1a: MFMAs of step 0, blocks mi < MI / 2; step 0's A blocks mi >= MI / 2
//       are read;
//   2a: MFMAs of step 0, mi >= MI / 2 (ni-major); B block ni of step 1 is
//       read after its last use in step 0, step 1's A blocks mi < MI / 2 in
//       between, and half of block j + 2's A DMA is issued;
//   1b: MFMAs of step 1, mi < MI / 2; step 1's A blocks mi >= MI / 2 read and
//       the other half of block j + 2's A DMA issued;
//   wait until block j + 1 has landed (only block j + 2's A in flight),
//       barrier: every wave has also finished reading block j;
//   2b: MFMAs of step 1, mi >= MI / 2; block j + 1's step-0 B blocks read
//       after their last use and its A blocks mi < MI / 2 in between; block
//       j + 2's B DMA issued into block j's A region.
// Regions as in k_blocks: block j in (2j) % 5 (A) and (2j + 1) % 5 (B).
template <int KIND, class C>
__device__ __forceinline__ void k_blocks_f8(f32x16_t (&acc)[C::MI][NI], Frags8<C>& f,
                                            const FragLanes<C>& L, const GemmArgs& p,
                                            const Operand<C::NIA>& opA, const Operand<C::NIB>& opB,
                                            uint32_t dma_w, uint32_t wa, uint32_t wb, int nk) {
  constexpr int R = C::kRegion, NIA = C::NIA, NIB = C::NIB, MI = C::MI;
  constexpr int MH = MI / 2, NP = MH * NI;  // MFMAs per phase
  static_assert(C::WIDE && C::KSUB == 4 && MI % 2 == 0 && 2 * MH <= NP, "wide FP8 ring");
  static_assert(NIA % 2 == 0 && NP % (NIA / 2) == 0 && NP % NIB == 0, "DMA spread");
  constexpr int SA = NP / (NIA / 2);  // one A piece every SA MFMAs of phases 2a and 1b
  constexpr int SB = NP / NIB;        // one B piece every SB MFMAs of phase 2b
  int ra = 0;                         // (2j) % 5
  for (int j = 0; j < nk; ++j) {
    const int rb = ra == 4 ? 0 : ra + 1;    // (2j + 1) % 5
    const int rn = rb == 4 ? 0 : rb + 1;    // (2j + 2) % 5: block j + 1's A
    const int rnb = rn == 4 ? 0 : rn + 1;   // (2j + 3) % 5: block j + 1's B
    const int rq = rnb == 4 ? 0 : rnb + 1;  // (2j + 4) % 5: block j + 2's A
    const uint32_t sa = ra * R + wa, sb = rb * R + wb;
    const uint32_t kill = j + 2 < nk ? 0u : kDmaKill;
    const int k2 = (j + 2) * C::BKX;
#pragma unroll
    for (int m = 0; m < NP; ++m) {  // 1a
      mfma_f8(acc[m / NI][m % NI], f.a[m / NI], f.b[m % NI]);
      if (m < 2 * MH) read_a8<C>(f, MH + m / 2, m % 2, sa, L);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < NP; ++m) {  // 2a
      const int ni = m / MH, mi = MH + m % MH;
      mfma_f8(acc[mi][ni], f.a[mi], f.b[ni]);
      if (m % MH == MH - 1) {
        read_b8<C>(f, ni, 2, sb, L);
        read_b8<C>(f, ni, 3, sb, L);
      }
      if (m < 2 * MH) read_a8<C>(f, m / 2, 2 + m % 2, sa, L);
      if (m % SA == 0) dma_piece<KIND, C>(p, opA, opB, dma_w + rq * R, 0u, k2, kill, m / SA);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < NP; ++m) {  // 1b
      mfma_f8(acc[m / NI][m % NI], f.a[m / NI], f.b[m % NI]);
      if (m < 2 * MH) read_a8<C>(f, MH + m / 2, 2 + m % 2, sa, L);
      if (m % SA == 0) dma_piece<KIND, C>(p, opA, opB, dma_w + rq * R, 0u, k2, kill, NIA / 2 + m / SA);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm<NIA>();
    lds_barrier();  // every wave: block j + 1 landed, block j fully read
    const uint32_t na = rn * R + wa, nb = rnb * R + wb;
#pragma unroll
    for (int m = 0; m < NP; ++m) {  // 2b
      const int ni = m / MH, mi = MH + m % MH;
      mfma_f8(acc[mi][ni], f.a[mi], f.b[ni]);
      if (m % MH == MH - 1) {
        read_b8<C>(f, ni, 0, nb, L);
        read_b8<C>(f, ni, 1, nb, L);
      }
      if (m < 2 * MH) read_a8<C>(f, m / 2, m % 2, na, L);
      if (m % SB == 0) dma_piece<KIND, C>(p, opA, opB, 0u, dma_w + ra * R, k2, kill, NIA + m / SB);
      __builtin_amdgcn_sched_barrier(0);
    }
    ra = rn;
  }
}

// Vector memory instructions each lane issues in the epilogue of a product
// (the buffer stores and loads there are unconditional: the range checks drop
// the ones outside the tile; WGRAD: its overwriting epilogue, the accumulating
// and folding ones depend on the data and take the plain wait).  A K loop that
// starts after the previous tile's epilogue (its first DMAs issued before that
// epilogue) waits past exactly these.
template <int KIND, class C, bool F8 = false>
__host__ __device__ constexpr int epilogue_vmem_ops() {
  // WGRAD8: not counted (the plain wait)
  if (KIND == K_WGRAD8) return -1;
  // FP8: the next tile's scale loads follow the epilogue (rows, then columns
  // four at a time)
  return (F8 ? Scales<KIND, C>::NR + Scales<KIND, C>::NC / 4 : 0) +
         (KIND == K_GATEUP_FWD   ? 12 * C::MI   // 3 stores x 2 rows x 2 halves per block row
          : KIND == K_DOWN_DGRAD ? 32 * C::MI   // 2 loads + 2 stores x 4 rows x 2 halves
          : KIND == K_WGRAD      ? 16 * C::MI   // overwrite: 2 stores x 4 rows x 2 halves
          : KIND == K_ROUTER_DX  ? 16 * C::MI   // 2 stores x 4 rows x 2 halves
                                 : 8 * C::MI);  // 1 store x 4 rows x 2 halves
}

// One output tile: expert / group e, N tile nt and its first column n0; the
// M-grouped products' rows [row0, row1), the K-grouped products' first output
// row m0 and rows [kbeg, kend) of the reduction; nk K steps.
struct Tile {
  int e, nt, n0, row0, row1, m0, kbeg, kend, nk;
  int slot;  // K-grouped with a plan: the chunk's partial slot, or -1 (the weight gradient itself)
};

template <int KIND, class C>
__device__ __forceinline__ Tile decode_tile(const GemmArgs& p, int work) {
  constexpr int BM = C::BM;
  int e, nt, row0 = 0, row1 = 0, m0 = 0, kbeg = 0, kend = 0, slot = -1;
  if constexpr (KIND == K_WGRAD8) {
    // K = the group's padded code columns [offsets[e], offsets[e + 1]), two
    // codes per bf16 slot; row0 carries m0 for the scale loads
    e = work / (p.n_mtiles * p.n_ntiles);
    const int rem = work - e * p.n_mtiles * p.n_ntiles;
    m0 = (rem / p.n_ntiles) * BM;
    nt = rem % p.n_ntiles;
    if (p.kplan != nullptr) {  // chunk `e` of the plan (code columns, multiples of 64)
      const int32_t* c = p.kplan + 2 + 4 * e;
      slot = c[3];
      kbeg = c[1] >> 1;
      kend = c[2] >> 1;
      e = c[0];
    } else {
      kbeg = p.offsets[e] >> 1;
      kend = p.offsets[e + 1] >> 1;
    }
    row0 = m0;
  } else if constexpr (KIND == K_WGRAD) {
    e = work / (p.n_mtiles * p.n_ntiles);
    const int rem = work - e * p.n_mtiles * p.n_ntiles;
    m0 = (rem / p.n_ntiles) * BM;
    nt = rem % p.n_ntiles;
    if (p.kplan != nullptr) {  // chunk `e` of the plan
      const int32_t* c = p.kplan + 2 + 4 * e;
      slot = c[3];
      kbeg = c[1];
      kend = c[2];
      e = c[0];
    } else if (p.offsets != nullptr) {
      kbeg = p.offsets[e];
      kend = p.offsets[e + 1];
    } else {
      kbeg = min(e * p.split_rows, p.ktot);
      kend = min(kbeg + p.split_rows, p.ktot);
    }
  } else if constexpr (KIND == K_ROUTER_DX) {
    // one group: tiles of BM consecutive rows
    const int mt = work / p.n_ntiles;
    nt = work - mt * p.n_ntiles;
    e = 0;
    row0 = mt * BM;
    row1 = min(row0 + BM, p.M);
    kend = p.K;
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
  slot = __builtin_amdgcn_readfirstlane(slot);

  Tile t;
  t.e = e;
  t.nt = nt;
  t.n0 = nt * BN;
  t.row0 = row0;
  t.row1 = row1;
  t.m0 = m0;
  t.kbeg = kbeg;
  t.kend = kend;
  t.nk = (kend - kbeg + C::BKX - 1) / C::BKX;
  t.slot = slot;
  return t;
}

// Buffer descriptors and per-lane DMA offsets of a tile's operands.
template <int KIND, class C>
__device__ __forceinline__ void setup_operands(const GemmArgs& p, const Tile& t, int wave, int lane,
                                               Operand<C::NIA>& opA, Operand<C::NIB>& opB) {
  using Tr = Traits<KIND>;
  constexpr int BM = C::BM, NIA = C::NIA, NIB = C::NIB, BKX = C::BKX;
  const int e = t.e, nt = t.nt, n0 = t.n0, row0 = t.row0, row1 = t.row1, m0 = t.m0;
  const int kbeg = t.kbeg, kend = t.kend;
  if constexpr (KIND == K_WGRAD8) {
    // A: code rows m0 .. of [M][lda slots], B: code rows n0 .. of [N][ldb],
    // both from slot kbeg on (the group's padded columns, zeros past its
    // rows); rows past M / N lie past the ranges and read as zero
    opA.rsrc = make_rsrc(p.a + (long)m0 * p.lda + kbeg, (uint32_t)(((long)(p.M - m0) * p.lda - kbeg) * 2));
    opA.kstep = 2;
#pragma unroll
    for (int u = 0; u < NIA; ++u) {
      int r, c;
      kc_rows<NIA, BKX>(wave, lane, u, r, c);
      opA.voff[u] = (uint32_t)(r * p.lda * 2 + c * 16);
    }
    opB.rsrc = make_rsrc(p.b0 + (long)n0 * p.ldb + kbeg, (uint32_t)(((long)(p.N - n0) * p.ldb - kbeg) * 2));
    opB.kstep = 2;
#pragma unroll
    for (int u = 0; u < NIB; ++u) {
      int r, c;
      kc_rows<NIB, BKX>(wave, lane, u, r, c);
      opB.voff[u] = (uint32_t)(r * p.ldb * 2 + c * 16);
    }
    return;
  }
  if constexpr (Tr::A_KC) {
    opA.kstep = 2;
    if (!k_grouped(KIND) && p.a_rows != nullptr) {  // uniform
      // the tile's rows gathered: DMA row r reads row a_rows[row0 + r] of a;
      // rows past row1 take the kill offset and read as zero.  (The K loop
      // of the previous tile has drained the memory counter, so these index
      // loads are the only memory operations in flight here.)
      opA.rsrc = make_rsrc(p.a, (uint32_t)((long)p.a_nrows * p.lda * 2));
      // every index load first (rows clamped into the tile, no branch), then
      // one wait for all of them
      int g[NIA];
#pragma unroll
      for (int u = 0; u < NIA; ++u) {
        int r, c;
        kc_rows<NIA, BKX>(wave, lane, u, r, c);
        g[u] = p.a_rows[min(row0 + r, row1 - 1)];
      }
#pragma unroll
      for (int u = 0; u < NIA; ++u) {
        int r, c;
        kc_rows<NIA, BKX>(wave, lane, u, r, c);
        const uint32_t o = (uint32_t)(g[u] * (uint32_t)p.lda * 2u + (uint32_t)c * 16u);
        opA.voff[u] = row0 + r < row1 ? o : kDmaKill;
      }
    } else {
      // the tile's rows [row0, row1) of A; rows past row1 read as zero
      opA.rsrc = make_rsrc(p.a + (long)row0 * p.lda, (uint32_t)((row1 - row0) * p.lda * 2));
#pragma unroll
      for (int u = 0; u < NIA; ++u) {
        int r, c;
        kc_rows<NIA, BKX>(wave, lane, u, r, c);
        opA.voff[u] = (uint32_t)(r * p.lda * 2 + c * 16);
      }
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
      kc_rows<NIB, BKX>(wave, lane, u, r, c);
      const int col = nt * 128 + (r >> 6) * 32 + (r & 31);
      opB.voff[u] = (uint32_t)(col * p.ldb * 2 + c * 16);
    }
  } else if constexpr (KIND == K_DOWN_FWD) {
    opB.rsrc = make_rsrc(p.b0 + (long)e * p.b_group_stride, (uint32_t)(p.N * p.ldb * 2));
    opB.kstep = 2;
#pragma unroll
    for (int u = 0; u < NIB; ++u) {
      int r, c;
      kc_rows<NIB, BKX>(wave, lane, u, r, c);
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
  } else if constexpr (KIND == K_ROUTER_DX) {
    // B[n][k] = W_r[n][k mod E]: rows of W_r [N][E], K-contiguous
    opB.rsrc = make_rsrc(p.b0, (uint32_t)(p.N * p.ldb * 2));
    opB.kstep = 2;
#pragma unroll
    for (int u = 0; u < NIB; ++u) {
      int r, c;
      kc_rows<NIB, BKX>(wave, lane, u, r, c);
      opB.voff[u] = (uint32_t)((n0 + r) * p.ldb * 2 + c * 16);
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
}

// Narrow ring: steps 0 .. NST - 2 and the first half of step NST - 1 of a
// tile.  Wide ring: loads 0 .. 3 (A and B of blocks 0 and 1) into regions
// 0 .. 3.  The ones past K are dropped.
template <int KIND, class C>
__device__ __forceinline__ void issue_prologue(const GemmArgs& p, const Operand<C::NIA>& opA,
                                               const Operand<C::NIB>& opB, uint32_t dma_a,
                                               uint32_t dma_b, int nk) {
  constexpr int NIA = C::NIA, ND = C::NIA + C::NIB;
  if constexpr (C::WIDE) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const uint32_t kill = blk < nk ? 0u : kDmaKill;
#pragma unroll
      for (int u = 0; u < ND; ++u)
        dma_piece<KIND, C>(p, opA, opB, dma_a + 2 * blk * C::kRegion, dma_b + (2 * blk + 1) * C::kRegion,
                           blk * C::BKX, kill, u);
    }
  } else {
    constexpr int NST = C::NST;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const uint32_t kill = st < nk ? 0u : kDmaKill;
#pragma unroll
      for (int u = 0; u < (st < NST - 1 ? ND : ND / 2); ++u)
        dma_piece<KIND, C>(p, opA, opB, dma_a + st * C::kSlotA, dma_b + st * C::kSlotB, st * C::BKX, kill,
                           u);
    }
  }
}

template <int KIND, int BM_, bool F8 = false, bool WIDE = false>
__global__ __launch_bounds__(NTH)
__attribute__((amdgpu_waves_per_eu(Cfg<BM_, WIDE>::kWavesPerSimd, Cfg<BM_, WIDE>::kWavesPerSimd)))
void gemm_kernel(const GemmArgs p) {
  static_assert(!F8 || KIND == K_GATEUP_FWD || KIND == K_DOWN_FWD || KIND == K_WGRAD8,
                "FP8: K-contiguous products only");
  static_assert(KIND != K_WGRAD8 || F8, "WGRAD8 runs on E4M3 codes");
  // (the FP8 weight gradient's groups are padded to 64 codes, half a wide block)
  static_assert(!(WIDE && KIND == K_WGRAD8), "the FP8 weight gradient runs on the narrow ring");
  static_assert(KIND != K_ROUTER_DX || (WIDE && !F8), "the router product runs on the wide ring");
  using Tr = Traits<KIND>;
  using C = Cfg<BM_, WIDE>;
  constexpr int WM = C::WM, MI = C::MI, NST = C::NST, NIA = C::NIA, NIB = C::NIB;
  constexpr int kOffB = C::kOffB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const FragLanes<C> L = frag_lanes<C>(lane, wave);

  int total;
  if constexpr (KIND == K_WGRAD || KIND == K_WGRAD8)
    total = (p.kplan != nullptr ? p.kplan[0] : p.groups) * p.n_mtiles * p.n_ntiles;
  else if constexpr (k_grouped(KIND))
    total = p.groups * p.n_mtiles * p.n_ntiles;
  else if constexpr (KIND == K_ROUTER_DX)
    total = p.n_mtiles * p.n_ntiles;
  else
    total = p.sched[0] * p.n_ntiles;

  int work = xcd_remap(blockIdx.x, gridDim.x);
  if (work >= total) return;
  // Dynamic order: thread 0 holds the ticket of the tile after next; it is
  // read only after a K loop has drained the memory counter.
  int ticket = 0;
  if (p.tile_ctr != nullptr && tid == 0) ticket = atomicAdd(p.tile_ctr, 1);
  const uint32_t dma_a = lds_addr(g_lds) + wave * NIA * 1024;  // this wave's DMA area
  const uint32_t dma_b = lds_addr(g_lds) + kOffB + wave * NIB * 1024;
  // wave block bases inside a slot or region
  // (MC fragment offsets hold the wave's columns themselves)
  const uint32_t wa = Tr::A_KC ? (uint32_t)(wm * WM * C::BKX * 2) : 0u;
  const uint32_t wb = Tr::B_KC ? (uint32_t)(wn * WN * C::BKX * 2) : 0u;
  constexpr int ND = NIA + NIB;

  Tile t = decode_tile<KIND, C>(p, work);
  Operand<NIA> opA;
  Operand<NIB> opB;
  setup_operands<KIND, C>(p, t, wave, lane, opA, opB);
  if (t.nk > 0) issue_prologue<KIND, C>(p, opA, opB, dma_a, dma_b, t.nk);
  Scales<KIND, C> S;
  if constexpr (F8) load_scales<KIND, C>(p, t.e, t.nt, t.n0, t.row0, t.row1, wave, lane, S);
  // Whether the previous tile's epilogue (a known number of memory
  // operations) was issued after this tile's first DMAs.
  bool after_epi = false;

  for (;;) {
    f32x16_t acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16_t{};

    if (t.nk > 0) {
      // Step (block) 0 has landed when only the newer DMAs remain (memory
      // operations retire in order).  After an epilogue of a known size the
      // wait also lets those newer operations stay in flight (up to the
      // counter's 63); otherwise the epilogue's operations only make the wait
      // stronger.
      constexpr int kFirst = C::WIDE ? ND : (NST - 2) * ND + ND / 2;
      constexpr int kEpi = epilogue_vmem_ops<KIND, C, F8>();
      constexpr int kAfter = kEpi < 0 ? kFirst : (kFirst + kEpi > 63 ? 63 : kFirst + kEpi);
      if (C::kSepStage && after_epi && (KIND != K_WGRAD || (p.accumulate == 0 && p.fold == 0)))
        wait_vm<kAfter>();
      else
        wait_vm<kFirst>();
      lds_barrier();
      // Two fragment sets, no copies between them: f0 holds sub-step 0 (read
      // at the end of the previous step), f1 sub-step 1 (wide ring: f0 and f1
      // alternate over the four sub-steps).
      if constexpr (F8) {
        // step 0's A blocks mi < MI / 2 and B blocks (B: narrow ring slot 0,
        // wide ring region 1)
        const uint32_t b0 = C::WIDE ? C::kRegion + wb : kOffB + wb;
        Frags8<C> f;
#pragma unroll
        for (int mi = 0; mi < MI / 2; ++mi) {
          read_a8<C>(f, mi, 0, wa, L);
          read_a8<C>(f, mi, 1, wa, L);
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          read_b8<C>(f, ni, 0, b0, L);
          read_b8<C>(f, ni, 1, b0, L);
        }
        if constexpr (C::WIDE) {
          k_blocks_f8<KIND, C>(acc, f, L, p, opA, opB, dma_a, wa, wb, t.nk);
        } else {
          static_assert(C::KSUB == 2, "the narrow FP8 pipeline reads two 16-byte halves per K step");
          k_steps_f8<KIND, C>(acc, f, L, p, opA, opB, dma_a, dma_b, wa, wb, t.nk);
        }
      } else if constexpr (C::WIDE) {
        Frags<C> f0, f1;
        load_frags<KIND, C>(f0, 0, wa, C::kRegion + wb, L);
        if constexpr (!k_grouped(KIND)) {
          // an expert's last row tile (or the router product's last token
          // tile) may end inside this wave's rows: MFMAs only for its 32-row
          // blocks that hold rows
          const int mi_act = __builtin_amdgcn_readfirstlane(
              min(MI, max(0, (t.row1 - t.row0 - wm * WM + 31) / 32)));
          static_assert(MI == 4, "the short forms below assume four 32-row blocks per wave");
          if (mi_act > 2)
            k_blocks<KIND, C>(acc, f0, f1, L, p, opA, opB, dma_a, wa, wb, t.nk);
          else if (mi_act > 0)
            k_blocks<KIND, C, 2>(acc, f0, f1, L, p, opA, opB, dma_a, wa, wb, t.nk);
          else
            k_blocks<KIND, C, 0>(acc, f0, f1, L, p, opA, opB, dma_a, wa, wb, t.nk);
        } else {
          k_blocks<KIND, C>(acc, f0, f1, L, p, opA, opB, dma_a, wa, wb, t.nk);
        }
      } else {
        static_assert(C::KSUB == 2, "the fragment pipeline below assumes two k16 sub-steps");
        Frags<C> f0, f1;
        load_frags<KIND, C>(f0, 0, wa, kOffB + wb, L);
        k_steps<KIND, C>(acc, f0, f1, L, p, opA, opB, dma_a, dma_b, wa, wb, t.nk);
      }
      // Every wave is done with the ring, and every DMA (also the dropped
      // ones, which write zeros) has landed, before the ring is reused.
      wait_vm<0>();
      lds_barrier();
    }
    if constexpr (F8) touch_scales<KIND, C>(S);

    // ------------------------------------------------------------ epilogue
    int next = work + gridDim.x;
    if (p.tile_ctr != nullptr) {  // uniform
      // hand thread 0's ticket to the workgroup through the first word of
      // the ring (idle here: this tile's K loop is done, the next tile's DMA
      // is not issued yet), and draw the next ticket
      // an LDS-address-space pointer: a generic one made this a flat store,
      // which the compiler follows with a wait for all memory operations
      typedef __attribute__((address_space(3))) volatile int lds_int_t;
      lds_int_t* slot0 = reinterpret_cast<lds_int_t*>(lds_ptr(0));
      if (tid == 0) {
        slot0[0] = (int)gridDim.x + ticket;
        ticket = atomicAdd(p.tile_ctr, 1);
      }
      lds_barrier();
      next = __builtin_amdgcn_readfirstlane(slot0[0]);
      lds_barrier();  // every wave has it before the ring is written again
    }
    const bool more = next < total;
    Tile tn = t;
    if constexpr (C::kSepStage) {
      // the next tile's first steps load during this tile's epilogue
      if (more) {
        tn = decode_tile<KIND, C>(p, next);
        setup_operands<KIND, C>(p, tn, wave, lane, opA, opB);
        if (tn.nk > 0) issue_prologue<KIND, C>(p, opA, opB, dma_a, dma_b, tn.nk);
      }
    }
    after_epi = C::kSepStage;
    epilogue<KIND, C, F8>(p, acc, t.e, t.nt, t.n0, t.m0, t.row0, t.row1, wave, lane, S, t.slot);
    // The staging area is reused by the next epilogue (and, for tiles staged
    // in the ring, overwritten by the next tile's first DMA).
    lds_barrier();
    if (!more) break;
    if constexpr (F8) load_scales<KIND, C>(p, tn.e, tn.nt, tn.n0, tn.row0, tn.row1, wave, lane, S);
    if constexpr (!C::kSepStage) {
      tn = decode_tile<KIND, C>(p, next);
      setup_operands<KIND, C>(p, tn, wave, lane, opA, opB);
      if (tn.nk > 0) issue_prologue<KIND, C>(p, opA, opB, dma_a, dma_b, tn.nk);
    }
    t = tn;
    work = next;
  }
}

// The weight gradients' K-chunk plans (one workgroup of kMaxE threads; thread
// e holds expert e's offsets o0, o1; s_off the offsets in LDS, complete).
// When no expert exceeds its product's split threshold (balanced loads), each
// expert is one chunk in expert order, written by its own thread.  Otherwise
// experts go in order of rows, largest first (ties: lower id first); each
// thread sizes its own expert's chunks, and scans over the ranking give its
// first chunk and first slot.
__device__ void build_wgrad_plans(const int* s_off, int E_l, int o0, int o1, int e, int lane, int w,
                                  int* s_wave, const WgradPlan& plan) {
  const long R = (long)s_off[E_l] - s_off[0];
  bool any = false;
  for (int q = 0; q < 2; ++q) {
    const long Wl = (R * plan.tiles[q] + kCUs - 1) / kCUs;
    const int W = (int)(Wl > kSplitMinRows ? Wl : kSplitMinRows);
    any = any || (e < E_l && o1 - o0 > W && plan.slots[q] > 0);
  }
  if (!__syncthreads_or(any)) {
    for (int q = 0; q < 2; ++q) {
      int32_t* t = plan.t[q];
      if (e < E_l) {
        t[2 + 4 * e] = e;
        t[3 + 4 * e] = o0;
        t[4 + 4 * e] = o1;
        t[5 + 4 * e] = -1;
      }
      if (e == 0) {
        t[0] = E_l;
        t[1] = 0;
      }
    }
    return;
  }
  int rank = 0;
  if (e < E_l) {
    const int re = o1 - o0;
    for (int q = 0; q < E_l; ++q) {
      const int rq = s_off[q + 1] - s_off[q];
      rank += (rq > re || (rq == re && q < e)) ? 1 : 0;
    }
  }
  __shared__ int s_scan[kMaxE];
  for (int q = 0; q < 2; ++q) {
    int32_t* t = plan.t[q];
    const int P = plan.slots[q];
    const long Wl = (R * plan.tiles[q] + kCUs - 1) / kCUs;
    const int W = (int)(Wl > kSplitMinRows ? Wl : kSplitMinRows);
    const int n = o1 - o0;
    int S = 1, len = n;
    if (e < E_l && n > W && P > 0) {
      S = min(kSplitMaxChunks, (n + W - 1) / W);
      len = (((n + S - 1) / S) + 63) & ~63;  // rows per chunk, a multiple of 64
      S = (n + len - 1) / len;
    }
    if (e >= E_l) S = 0;
    // exclusive scans in rank order of the chunk counts (low 16 bits) and the
    // partial slots (high 16 bits; both below 2^15 here)
    __syncthreads();
    if (e < E_l) s_scan[rank] = S + ((S > 1 ? S - 1 : 0) << 16);
    if (e >= E_l && e < kMaxE) s_scan[e] = 0;
    __syncthreads();
    int v = s_scan[e];
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int u = __shfl_up(v, d, kWave);
      if (lane >= d) v += u;
    }
    if (lane == kWave - 1) s_wave[w] = v;
    __syncthreads();
    for (int qq = 0; qq < w; ++qq) v += s_wave[qq];
    const int incl = v;  // inclusive, at position e of the rank order
    __syncthreads();
    s_scan[e] = incl;
    __syncthreads();
    const int total = s_scan[kMaxE - 1];
    const int chunks = total & 0xffff, slots = total >> 16;
    // the slot bound holds by construction (S - 1 < rows / W); should it ever
    // fail, no expert is split
    const bool ok = slots <= P;
    int c0 = 0, slot0 = 0, nsplit_before = 0;
    if (e < E_l) {
      const int ex = rank > 0 ? s_scan[rank - 1] : 0;
      c0 = ex & 0xffff;
      slot0 = ex >> 16;
    }
    // split experts before this one in rank order: a third scan, over (S > 1)
    __syncthreads();
    if (e < E_l) s_scan[rank] = (ok && S > 1) ? 1 : 0;
    if (e >= E_l) s_scan[e] = 0;
    __syncthreads();
    v = s_scan[e];
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int u = __shfl_up(v, d, kWave);
      if (lane >= d) v += u;
    }
    if (lane == kWave - 1) s_wave[w] = v;
    __syncthreads();
    for (int qq = 0; qq < w; ++qq) v += s_wave[qq];
    __syncthreads();
    s_scan[e] = v;
    __syncthreads();
    const int nsplit = s_scan[kMaxE - 1];
    if (e < E_l) nsplit_before = rank > 0 ? s_scan[rank - 1] : 0;
    if (e < E_l) {
      if (ok) {
        for (int j = 0; j < S; ++j) {
          const int kb = o0 + j * len, c = c0 + j;
          t[2 + 4 * c] = e;
          t[3 + 4 * c] = kb;
          t[4 + 4 * c] = min(kb + len, o1);
          t[5 + 4 * c] = j == 0 ? -1 : slot0 + j - 1;
        }
        if (S > 1) {
          int32_t* split = t + 2 + 4 * (E_l + P) + 3 * nsplit_before;
          split[0] = e;
          split[1] = S;
          split[2] = slot0;
        }
      } else {  // one chunk per expert, in rank order
        t[2 + 4 * rank] = e;
        t[3 + 4 * rank] = o0;
        t[4 + 4 * rank] = o1;
        t[5 + 4 * rank] = -1;
      }
    }
    if (e == 0) {
      t[0] = ok ? chunks : E_l;
      t[1] = ok ? nsplit : 0;
    }
  }
}

// Tile table of the M-grouped products: for every expert with rows, one entry
// (expert, first row, end row) per `rows` rows.  sched[0] = number of entries.
__global__ __launch_bounds__(kMaxE) void ffn_sched_kernel(const int32_t* __restrict__ offsets,
                                                          int E_l, int rows,
                                                          int32_t* __restrict__ sched,
                                                          int32_t* __restrict__ ctrs,
                                                          WgradPlan plan = WgradPlan{}) {
  // the dynamic tile counters of the products that follow start at zero
  if (ctrs != nullptr && threadIdx.x < kTileCtrs) ctrs[threadIdx.x] = 0;
  __shared__ int s[kMaxE + 1];      // s[g] = tiles of experts < g
  __shared__ int s_off[kMaxE + 1];  // the offsets, in LDS for the tile loop
  __shared__ int s_wave[kMaxE / kWave];
  const int e = threadIdx.x, lane = e & (kWave - 1), w = e / kWave;
  const int o0 = (e < E_l) ? offsets[e] : 0;
  const int o1 = (e < E_l) ? offsets[e + 1] : 0;
  // Only the owners write: s_off[E_l] comes from thread E_l - 1 alone (thread
  // E_l, in another wave when E_l % 64 == 0, must not store its zero there).
  if (e < E_l) s_off[e] = o0;
  if (e == E_l - 1) s_off[E_l] = o1;
  int v = (o1 - o0 + rows - 1) / rows;  // this expert's tiles
  // inclusive scan: within each wave by shuffles, then the waves' totals
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int t = __shfl_up(v, d, kWave);
    if (lane >= d) v += t;
  }
  if (lane == kWave - 1) s_wave[w] = v;
  __syncthreads();
  for (int q = 0; q < w; ++q) v += s_wave[q];
  s[e + 1] = v;
  if (e == 0) s[0] = 0;
  __syncthreads();
  const int count = s[E_l];
  if (e == 0) sched[0] = count;
  for (int i = e; i < count; i += kMaxE) {
    int lo = 0, hi = E_l - 1;  // largest g with s[g] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int r0 = s_off[lo] + (i - s[lo]) * rows;
    sched[1 + 3 * i] = lo;
    sched[2 + 3 * i] = r0;
    sched[3 + 3 * i] = min(r0 + rows, s_off[lo + 1]);
  }
  if (plan.t[0] == nullptr) return;
  __syncthreads();
  build_wgrad_plans(s_off, E_l, o0, o1, e, lane, w, s_wave, plan);
}

// The plans alone, from a given offsets array (the FP8 weight gradient's
// padded code offsets).
__global__ __launch_bounds__(kMaxE) void wgrad_plan_kernel(const int32_t* __restrict__ offsets, int E_l,
                                                           WgradPlan plan) {
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_wave[kMaxE / kWave];
  const int e = threadIdx.x, lane = e & (kWave - 1), w = e / kWave;
  const int o0 = (e < E_l) ? offsets[e] : 0;
  const int o1 = (e < E_l) ? offsets[e + 1] : 0;
  if (e < E_l) s_off[e] = o0;
  if (e == E_l - 1) s_off[E_l] = o1;
  __syncthreads();
  build_wgrad_plans(s_off, E_l, o0, o1, e, lane, w, s_wave, plan);
}

// The split experts' partial slots added to their weight gradients in chunk
// order: out += part[slot0] + ... (chunk 0 wrote out itself).  Both products in
// one launch; elements in float4s, grid-strided.  Nothing to do (the usual
// case) returns at once.
struct WgradReduce {
  const int32_t* plan[2];
  const float* part[2];
  float* out0[2];   // rows below m_split (gate; down: all rows)
  float* out1[2];   // rows from m_split on (up), or null
  int M[2], N[2], m_split[2];
  long group_stride[2];
  int E_l, slots[2];
};

__global__ __launch_bounds__(256) void wgrad_split_reduce_kernel(const WgradReduce a) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const int stride = gridDim.x * blockDim.x;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int32_t* pl = a.plan[q];
    const int ns = pl[1];
    const int32_t* split = pl + 2 + 4 * (a.E_l + a.slots[q]);
    const int N = a.N[q], mn4 = a.M[q] * N / 4;  // M N < 2^31 (checked by the entry point)
    for (int i = 0; i < ns; ++i) {
      const int g = split[3 * i], S = split[3 * i + 1], slot0 = split[3 * i + 2];
      const float* part = a.part[q] + (long)slot0 * a.M[q] * N;
      for (int x = tid; x < mn4; x += stride) {
        const int el = 4 * x;
        const int m = el / N, n = el - m * N;
        const bool up = a.out1[q] != nullptr && m >= a.m_split[q];
        float* dst = (up ? a.out1[q] : a.out0[q]) + g * a.group_stride[q] +
                     (long)(up ? m - a.m_split[q] : m) * N + n;
        // every partial loaded first, then added in chunk order
        f32x4_t pv[kSplitMaxChunks - 1];
#pragma unroll
        for (int j = 0; j < kSplitMaxChunks - 1; ++j)
          pv[j] = j < S - 1 ? *reinterpret_cast<const f32x4_t*>(part + (long)j * a.M[q] * N + el)
                            : f32x4_t{};
        f32x4_t v = *reinterpret_cast<const f32x4_t*>(dst);
#pragma unroll
        for (int j = 0; j < kSplitMaxChunks - 1; ++j)
          if (j < S - 1) v += pv[j];
        *reinterpret_cast<f32x4_t*>(dst) = v;
      }
    }
  }
}

static constexpr size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

int gemm_tiles(int M, int N) { return ((M + kBmWgrad - 1) / kBmWgrad) * ((N + BN - 1) / BN); }

bool dw_router_folds(int E) { return E % 8 == 0 && 2 * E <= BN; }

// Tile table, then kTileCtrs dynamic tile counters (256 bytes).
static size_t ffn_sched_table_bytes(int R_cap, int E_l) {
  const size_t entries = (size_t)R_cap / kBmGrouped + E_l + 1;
  return align256((1 + 3 * entries) * sizeof(int32_t));
}
size_t ffn_sched_bytes(int R_cap, int E_l) { return ffn_sched_table_bytes(R_cap, E_l) + 256; }

// The weight gradients' split plans and partial slots (after dgu in the FFN
// backward workspace): gate/up product (M = 2I, N = H), then down (M = H, N = I).
static int wgrad_split_slots(int E_l, int tiles) {
  return std::min(E_l * (kSplitMaxChunks - 1), kCUs / tiles);
}
struct WgradSplitLayout {
  int tiles[2], slots[2];
  size_t plan_off[2], part_off[2], bytes;
};
static WgradSplitLayout wgrad_split_layout(int E_l, int H, int I) {
  WgradSplitLayout L{};
  L.tiles[0] = gemm_tiles(2 * I, H);
  L.tiles[1] = gemm_tiles(H, I);
  size_t o = 0;
  for (int q = 0; q < 2; ++q) {
    L.slots[q] = wgrad_split_slots(E_l, L.tiles[q]);
    L.plan_off[q] = o;
    o += align256((size_t)wgrad_plan_ints(E_l, L.slots[q]) * sizeof(int32_t));
  }
  const size_t mn[2] = {(size_t)2 * I * H, (size_t)H * I};
  for (int q = 0; q < 2; ++q) {
    L.part_off[q] = o;
    o += align256((size_t)L.slots[q] * mn[q] * sizeof(float));
  }
  L.bytes = o;
  return L;
}
size_t ffn_wgrad_split_bytes(int E_l, int H, int I) { return wgrad_split_layout(E_l, H, I).bytes; }

// The split experts' partial slots added in chunk order, for both products.
static hipError_t launch_wgrad_split_reduce(const WgradPlan& plan, float* const (&part)[2],
                                            const WgradSplitLayout& SL, int E_l, int H, int I,
                                            float* dw_gate, float* dw_up, float* dw_down, hipStream_t s) {
  WgradReduce r{};
  for (int q = 0; q < 2; ++q) {
    r.plan[q] = plan.t[q];
    r.part[q] = part[q];
    r.slots[q] = SL.slots[q];
  }
  r.out0[0] = dw_gate;
  r.out1[0] = dw_up;
  r.M[0] = 2 * I;
  r.N[0] = H;
  r.m_split[0] = I;
  r.group_stride[0] = (long)I * H;
  r.out0[1] = dw_down;
  r.out1[1] = nullptr;
  r.M[1] = H;
  r.N[1] = I;
  r.m_split[1] = H;
  r.group_stride[1] = (long)H * I;
  r.E_l = E_l;
  ProfScope ps(MOE_KERNEL_FFN_WGRAD_REDUCE, s);
  wgrad_split_reduce_kernel<<<kCUs * 2, 256, 0, s>>>(r);
  return hipGetLastError();
}
static int32_t* ffn_tile_ctrs(void* ws, int R_cap, int E_l) {
  return (int32_t*)((char*)ws + ffn_sched_table_bytes(R_cap, E_l));
}

template <int KIND, int BM_, bool F8 = false, bool WIDE = false>
static hipError_t launch_gemm(const GemmArgs& a, int work_upper, int kernel_id, hipStream_t s) {
  using C = Cfg<BM_, WIDE>;
  if (work_upper <= 0) return hipSuccess;
  const int grid = std::min(work_upper, kCUs * C::kWavesPerSimd);  // persistent
  ProfScope ps(kernel_id, s);
  gemm_kernel<KIND, BM_, F8, WIDE><<<grid, NTH, C::kLdsBytes, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_ffn_fwd_bf16(const bf16_t* x_perm, const int32_t* offsets, int E_l, int R_cap,
                               int H, int I, const bf16_t* w_gate, const bf16_t* w_up,
                               const bf16_t* w_down, bf16_t* gu, bf16_t* h_perm, bf16_t* y_perm,
                               void* ws, hipStream_t s, const int32_t* x_rows, int T) {
  int32_t* sched = (int32_t*)ws;
  ffn_sched_kernel<<<1, kMaxE, 0, s>>>(offsets, E_l, kBmGrouped, sched, nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int mt_upper = R_cap / kBmGrouped + E_l;

  GemmArgs g{};
  g.a = x_perm;
  g.lda = H;
  g.a_rows = x_rows;  // null: x_perm holds the grouped rows; else x = the token rows
  g.a_nrows = T;
  g.b0 = w_gate;
  g.b1 = w_up;
  g.ldb = H;
  g.b_group_stride = (long)I * H;
  g.sched = sched;
  g.K = H;
  g.N = I;
  g.I = I;
  g.n_ntiles = (I + BN / 2 - 1) / (BN / 2);  // BN / 2 h columns (gate + up) per tile
  g.c0 = h_perm;
  g.ldc = I;
  g.c1 = gu;
  err = launch_gemm<K_GATEUP_FWD, kBmGrouped, false, kWideGrouped>(g, mt_upper * g.n_ntiles, MOE_KERNEL_FFN_GATEUP, s);
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
  return launch_gemm<K_DOWN_FWD, kBmGrouped, false, kWideGrouped>(d, mt_upper * d.n_ntiles, MOE_KERNEL_FFN_DOWN, s);
}

// ---------------------------------------------------------------------------
// The forward without a workspace (moe_grouped_ffn_fwd_noalloc): its only
// scratch, the tile table, lives in a static device array of fixed size, one
// copy per GPU, held until the process ends.  On the host the array's name is
// not a device address: the launcher uses only the address hipGetSymbolAddress
// returns, looked up once per device with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = 64 * 1024;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static_assert(align256((1 + 3 * ((size_t)kNoAllocMaxRows / kBmGrouped + kMaxE + 1)) * sizeof(int32_t)) <=
                  kNoAllocScratchBytes,
              "the tile table of the largest no-workspace forward fits the static scratch");

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_ffn_fwd_bf16_noalloc(const bf16_t* x_perm, const int32_t* offsets, int E_l,
                                       int R_cap, int H, int I, const bf16_t* w_gate,
                                       const bf16_t* w_up, const bf16_t* w_down, bf16_t* gu,
                                       bf16_t* h_perm, bf16_t* y_perm, hipStream_t s) {
  if (R_cap > kNoAllocMaxRows) return hipErrorInvalidValue;  // the ABI refuses these first
  void* table = nullptr;
  hipError_t e = noalloc_scratch(&table);
  if (e != hipSuccess) return e;
  // the tile-table kernel writes every entry the products read (count first),
  // so nothing in the array needs clearing
  return launch_ffn_fwd_bf16(x_perm, offsets, E_l, R_cap, H, I, w_gate, w_up, w_down, gu, h_perm,
                             y_perm, table, s);
}

// Row scales of the permuted activations: sxp[r] = sx[src_row[r]] for the
// R = offsets[E_l] rows in use.
__global__ __launch_bounds__(256) void gather_row_scales_kernel(const float* __restrict__ sx,
                                                                const int32_t* __restrict__ src_row,
                                                                const int32_t* __restrict__ offsets,
                                                                int E_l, int R_cap,
                                                                float* __restrict__ sxp) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R_cap || r >= offsets[E_l]) return;
  sxp[r] = sx[src_row[r]];
}

size_t ffn_fwd_fp8_ws_bytes(int R_cap, int E_l, int I) {
  return ffn_sched_bytes(R_cap, E_l) + align256((size_t)R_cap * 4) + align256((size_t)R_cap * I) +
         align256((size_t)R_cap * 4);
}

hipError_t launch_ffn_fwd_fp8(const uint8_t* x_q, const float* x_scale, const int32_t* src_row,
                              const int32_t* offsets, int E_l, int R_cap, int H, int I,
                              const uint8_t* wg_q, const float* wg_s, const uint8_t* wu_q,
                              const float* wu_s, const uint8_t* wd_q, const float* wd_s,
                              bf16_t* gu, bf16_t* h_perm, bf16_t* y_perm, void* ws,
                              hipStream_t s, int gather_T) {
  char* w = (char*)ws;
  int32_t* sched = (int32_t*)w;
  w += ffn_sched_bytes(R_cap, E_l);
  float* sxp = (float*)w;
  w += align256((size_t)R_cap * 4);
  uint8_t* hq = (uint8_t*)w;
  w += align256((size_t)R_cap * I);
  float* sh = (float*)w;
  ffn_sched_kernel<<<1, kMaxE, 0, s>>>(offsets, E_l, kBmGrouped, sched, nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  gather_row_scales_kernel<<<(R_cap + 255) / 256, 256, 0, s>>>(x_scale, src_row, offsets, E_l,
                                                               R_cap, sxp);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int mt_upper = R_cap / kBmGrouped + E_l;

  // E4M3 rows of K codes run through the ring as rows of K / 2 bf16 slots.
  GemmArgs g{};
  g.a = (const bf16_t*)x_q;
  g.lda = H / 2;
  if (gather_T >= 0) {  // token code rows, grouped row r = row src_row[r]
    g.a_rows = src_row;
    g.a_nrows = gather_T;
  }
  g.b0 = (const bf16_t*)wg_q;
  g.b1 = (const bf16_t*)wu_q;
  g.ldb = H / 2;
  g.b_group_stride = (long)I * H / 2;
  g.sched = sched;
  g.K = H / 2;
  g.N = I;
  g.I = I;
  g.n_ntiles = (I + BN / 2 - 1) / (BN / 2);
  g.c0 = h_perm;
  g.ldc = I;
  g.c1 = gu;
  g.sa = sxp;
  g.sb0 = wg_s;
  g.sb1 = wu_s;
  g.sb_group_stride = I;
  err = launch_gemm<K_GATEUP_FWD, kBmGrouped, true, kWideF8>(g, mt_upper * g.n_ntiles, MOE_KERNEL_FFN_GATEUP, s);
  if (err != hipSuccess) return err;

  err = launch_quantize_fp8(h_perm, R_cap, I, true, offsets + E_l, hq, sh, s);
  if (err != hipSuccess) return err;

  GemmArgs d{};
  d.a = (const bf16_t*)hq;
  d.lda = I / 2;
  d.b0 = (const bf16_t*)wd_q;
  d.ldb = I / 2;
  d.b_group_stride = (long)H * I / 2;
  d.sched = sched;
  d.K = I / 2;
  d.N = H;
  d.I = I;
  d.n_ntiles = (H + BN - 1) / BN;
  d.c0 = y_perm;
  d.ldc = H;
  d.sa = sh;
  d.sb0 = wd_s;
  d.sb_group_stride = H;
  return launch_gemm<K_DOWN_FWD, kBmGrouped, true, kWideF8>(d, mt_upper * d.n_ntiles, MOE_KERNEL_FFN_DOWN, s);
}

// FP8 data gradients of the expert FFN.  Both products are the FP8 down
// kernel (A and B K-contiguous, row x column scales): dh [R, I] = dy codes x
// rows of W_down^T (N = I, K = H), then, after the SiLU derivative and the row
// quantization of [dg | du], dx [R, H] = [dg | du] codes x rows of
// [W_gate^T | W_up^T] (N = H, K = 2I).
size_t ffn_dgrad_fp8_ws_bytes(int R_cap, int E_l, int I) {
  return ffn_sched_bytes(R_cap, E_l) + align256((size_t)R_cap * I * 2) +
         align256((size_t)R_cap * 2 * I) + align256((size_t)R_cap * 4);
}

hipError_t launch_ffn_dgrad_fp8(const uint8_t* dy_q, const float* dy_scale, const bf16_t* gu,
                                const int32_t* offsets, int E_l, int R_cap, int H, int I,
                                const uint8_t* wdt_q, const float* wdt_s, const uint8_t* wgut_q,
                                const float* wgut_s, bf16_t* dgu, bf16_t* dx_perm, void* ws,
                                hipStream_t s) {
  char* w = (char*)ws;
  int32_t* sched = (int32_t*)w;
  w += ffn_sched_bytes(R_cap, E_l);
  bf16_t* dh = (bf16_t*)w;
  w += align256((size_t)R_cap * I * 2);
  uint8_t* dguq = (uint8_t*)w;
  w += align256((size_t)R_cap * 2 * I);
  float* sdgu = (float*)w;
  ffn_sched_kernel<<<1, kMaxE, 0, s>>>(offsets, E_l, kBmGrouped, sched, nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int mt_upper = R_cap / kBmGrouped + E_l;

  // E4M3 rows of K codes run through the ring as rows of K / 2 bf16 slots.
  GemmArgs d{};
  d.a = (const bf16_t*)dy_q;
  d.lda = H / 2;
  d.b0 = (const bf16_t*)wdt_q;
  d.ldb = H / 2;
  d.b_group_stride = (long)I * H / 2;
  d.sched = sched;
  d.K = H / 2;
  d.N = I;
  d.I = I;
  d.n_ntiles = (I + BN - 1) / BN;
  d.c0 = dh;
  d.ldc = I;
  d.sa = dy_scale;
  d.sb0 = wdt_s;
  d.sb_group_stride = I;
  err = launch_gemm<K_DOWN_FWD, kBmGrouped, true, kWideF8>(d, mt_upper * d.n_ntiles, MOE_KERNEL_FFN_DOWN_DGRAD, s);
  if (err != hipSuccess) return err;

  err = launch_swiglu_bwd_fp8(dh, gu, R_cap, I, offsets + E_l, dgu, dguq, sdgu, s);
  if (err != hipSuccess) return err;

  GemmArgs x{};
  x.a = (const bf16_t*)dguq;
  x.lda = I;  // 2I codes
  x.b0 = (const bf16_t*)wgut_q;
  x.ldb = I;
  x.b_group_stride = (long)H * I;
  x.sched = sched;
  x.K = I;
  x.N = H;
  x.I = I;
  x.n_ntiles = (H + BN - 1) / BN;
  x.c0 = dx_perm;
  x.ldc = H;
  x.sa = sdgu;
  x.sb0 = wgut_s;
  x.sb_group_stride = H;
  return launch_gemm<K_DOWN_FWD, kBmGrouped, true, kWideF8>(x, mt_upper * x.n_ntiles, MOE_KERNEL_FFN_GATEUP_DGRAD, s);
}

// FP8 weight gradients of the expert FFN: the four operands' columns are
// quantized per (expert, column) into transposed code matrices whose rows
// hold each expert's rows at a padded offset (a multiple of 64 codes, zeros
// past its rows), so that both operands of every product are K-contiguous
// and each expert's K range is whole 64-code steps:
//   dW_gate | dW_up  [2I, H] per expert = codes of [dg | du]^T x codes of x^T
//   dW_down          [H, I]  per expert = codes of dy^T x codes of h^T
int wgrad_fp8_pitch(int R_cap, int E_l) { return ((R_cap + 63) & ~63) + 64 * E_l; }

static size_t wgrad_fp8_codes_bytes(int R_cap, int E_l, int C) {
  return align256((size_t)wgrad_fp8_pitch(R_cap, E_l) * C);
}

size_t ffn_wgrad_fp8_ws_bytes(int R_cap, int E_l, int H, int I) {
  return wgrad_fp8_codes_bytes(R_cap, E_l, 2 * I) + 2 * wgrad_fp8_codes_bytes(R_cap, E_l, H) +
         wgrad_fp8_codes_bytes(R_cap, E_l, I) + align256((size_t)E_l * (3 * I + 2 * H) * 4) +
         align256((size_t)(E_l + 1) * 4) + 256 + ffn_wgrad_split_bytes(E_l, H, I);
}

// The FP8 weight-gradient workspace: the four operands' transposed codes and
// per-(expert, column) scales, the padded offsets, the two products' tile
// counters, the K-chunk plans and the partial slots.
struct Wgrad8Ws {
  int Kp;
  uint8_t *q_gu, *q_x, *q_dy, *q_h;
  float *s_gu, *s_x, *s_dy, *s_h;
  int32_t* poff;
  int32_t* ctrs;
  WgradSplitLayout SL;
  WgradPlan plan;
  float* part[2];
};

static Wgrad8Ws wgrad8_ws(void* ws, int R_cap, int E_l, int H, int I) {
  Wgrad8Ws L{};
  L.Kp = wgrad_fp8_pitch(R_cap, E_l);
  char* w = (char*)ws;
  L.q_gu = (uint8_t*)w;
  w += wgrad_fp8_codes_bytes(R_cap, E_l, 2 * I);
  L.q_x = (uint8_t*)w;
  w += wgrad_fp8_codes_bytes(R_cap, E_l, H);
  L.q_dy = (uint8_t*)w;
  w += wgrad_fp8_codes_bytes(R_cap, E_l, H);
  L.q_h = (uint8_t*)w;
  w += wgrad_fp8_codes_bytes(R_cap, E_l, I);
  L.s_gu = (float*)w;
  L.s_x = L.s_gu + (size_t)E_l * 2 * I;
  L.s_dy = L.s_x + (size_t)E_l * H;
  L.s_h = L.s_dy + (size_t)E_l * H;
  w += align256((size_t)E_l * (3 * I + 2 * H) * 4);
  L.poff = (int32_t*)w;
  w += align256((size_t)(E_l + 1) * 4);
  L.ctrs = (int32_t*)w;
  w += 256;
  // the K-chunk plans over the padded code columns and the partial slots
  L.SL = wgrad_split_layout(E_l, H, I);
  for (int q = 0; q < 2; ++q) {
    L.plan.t[q] = (int32_t*)(w + L.SL.plan_off[q]);
    L.plan.tiles[q] = L.SL.tiles[q];
    L.plan.slots[q] = L.SL.slots[q];
    L.part[q] = (float*)(w + L.SL.part_off[q]);
  }
  return L;
}

// First half: the columns of x (through src_row), dy_perm and h quantized,
// both products' tile counters zeroed, the K-chunk plans built, then dW_down
// (its split experts' partial sums are added by the second half).
hipError_t launch_ffn_wgrad_fp8_begin(const bf16_t* x, const int32_t* src_row,
                                      const bf16_t* h_perm, const bf16_t* dy_perm,
                                      const int32_t* offsets, int E_l, int R_cap, int H, int I,
                                      float* dw_down, bool accumulate, void* ws, hipStream_t s) {
  const Wgrad8Ws L = wgrad8_ws(ws, R_cap, E_l, H, I);
  QuantGroupT q{};
  q.t[0] = {x, src_row, (long)H, H, L.q_x, L.s_x};
  q.t[1] = {dy_perm, nullptr, (long)H, H, L.q_dy, L.s_dy};
  q.t[2] = {h_perm, nullptr, (long)I, I, L.q_h, L.s_h};
  q.nt = 3;
  q.offsets = offsets;
  q.E_l = E_l;
  q.max_rows = R_cap;
  q.Kp = L.Kp;
  q.poff = L.poff;
  q.ctrs = L.ctrs;
  q.nctrs = 2;
  hipError_t err = launch_quantize_group_t_fp8(q, s);
  if (err != hipSuccess) return err;
  wgrad_plan_kernel<<<1, kMaxE, 0, s>>>(L.poff, E_l, L.plan);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  // E4M3 rows of Kp codes run through the ring as rows of Kp / 2 bf16 slots.
  GemmArgs d{};
  d.a = (const bf16_t*)L.q_dy;
  d.lda = L.Kp / 2;
  d.b0 = (const bf16_t*)L.q_h;
  d.ldb = L.Kp / 2;
  d.offsets = L.poff;
  d.groups = E_l;
  d.M = H;
  d.N = I;
  d.n_mtiles = (H + kBmWgrad - 1) / kBmWgrad;
  d.n_ntiles = (I + BN - 1) / BN;
  d.f0 = dw_down;
  d.m_split = H;
  d.ldc = I;
  d.f_group_stride = (long)H * I;
  d.accumulate = accumulate ? 1 : 0;
  d.sa = L.s_dy;
  d.sa_group_stride = H;
  d.sb0 = L.s_h;
  d.sb_group_stride = I;
  d.tile_ctr = L.ctrs + 1;
  d.kplan = L.plan.t[1];
  d.fpart = L.part[1];
  return launch_gemm<K_WGRAD8, kBmWgrad, true>(d, (E_l + L.SL.slots[1]) * d.n_mtiles * d.n_ntiles,
                                               MOE_KERNEL_FFN_DOWN_WGRAD, s);
}

// Second half, after the first on the same workspace: the columns of
// [dg | du] quantized, [dW_gate; dW_up], then the ordered sums of both
// products' split experts.
hipError_t launch_ffn_wgrad_fp8_end(const bf16_t* dgu, const int32_t* offsets, int E_l, int R_cap,
                                    int H, int I, float* dw_gate, float* dw_up, float* dw_down,
                                    bool accumulate, void* ws, hipStream_t s) {
  const Wgrad8Ws L = wgrad8_ws(ws, R_cap, E_l, H, I);
  QuantGroupT q{};
  q.t[0] = {dgu, nullptr, 2L * I, 2 * I, L.q_gu, L.s_gu};
  q.nt = 1;
  q.offsets = offsets;
  q.E_l = E_l;
  q.max_rows = R_cap;
  q.Kp = L.Kp;
  q.poff = L.poff;  // rewritten with the values the first half wrote
  hipError_t err = launch_quantize_group_t_fp8(q, s);
  if (err != hipSuccess) return err;

  GemmArgs g{};
  g.a = (const bf16_t*)L.q_gu;
  g.lda = L.Kp / 2;
  g.b0 = (const bf16_t*)L.q_x;
  g.ldb = L.Kp / 2;
  g.offsets = L.poff;
  g.groups = E_l;
  g.M = 2 * I;
  g.N = H;
  g.n_mtiles = (2 * I + kBmWgrad - 1) / kBmWgrad;
  g.n_ntiles = (H + BN - 1) / BN;
  g.f0 = dw_gate;
  g.f1 = dw_up;
  g.m_split = I;
  g.ldc = H;
  g.f_group_stride = (long)I * H;
  g.accumulate = accumulate ? 1 : 0;
  g.sa = L.s_gu;
  g.sa_group_stride = 2 * I;
  g.sb0 = L.s_x;
  g.sb_group_stride = H;
  g.tile_ctr = L.ctrs;
  g.kplan = L.plan.t[0];
  g.fpart = L.part[0];
  err = launch_gemm<K_WGRAD8, kBmWgrad, true>(g, (E_l + L.SL.slots[0]) * g.n_mtiles * g.n_ntiles,
                                              MOE_KERNEL_FFN_GATEUP_WGRAD, s);
  if (err != hipSuccess) return err;
  WgradPlan plan = L.plan;
  float* part[2] = {L.part[0], L.part[1]};
  return launch_wgrad_split_reduce(plan, part, L.SL, E_l, H, I, dw_gate, dw_up, dw_down, s);
}

hipError_t launch_ffn_wgrad_fp8(const bf16_t* x, const int32_t* src_row, const bf16_t* dgu,
                                const bf16_t* h_perm, const bf16_t* dy_perm,
                                const int32_t* offsets, int E_l, int R_cap, int H, int I,
                                float* dw_gate, float* dw_up, float* dw_down, bool accumulate,
                                void* ws, hipStream_t s) {
  hipError_t err = launch_ffn_wgrad_fp8_begin(x, src_row, h_perm, dy_perm, offsets, E_l, R_cap, H,
                                              I, dw_down, accumulate, ws, s);
  if (err != hipSuccess) return err;
  return launch_ffn_wgrad_fp8_end(dgu, offsets, E_l, R_cap, H, I, dw_gate, dw_up, dw_down,
                                  accumulate, ws, s);
}

// A second stream of the calling device for products that may run beside
// others, and the events that fork it from and join it back to the caller's
// stream.  One set per calling thread and device (created on first use,
// default priority, held until the process ends), so that calls from several
// host threads never record or wait on each other's events.  Within one
// thread, each call records an event and enqueues the waits on it before it
// returns, so a later call's record does not move an earlier call's wait.
// Null when it cannot be created: everything then runs on the caller's stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, mid = nullptr, join = nullptr;
};

static SideStream* side_stream() {
  thread_local SideStream per_dev[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& ss = per_dev[dev];
  if (ss.s == nullptr) {
    hipStream_t st = nullptr;
    hipEvent_t e[3] = {nullptr, nullptr, nullptr};
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    for (int i = 0; i < 3; ++i)
      if (hipEventCreateWithFlags(&e[i], hipEventDisableTiming) != hipSuccess) return nullptr;
    ss.fork = e[0];
    ss.mid = e[1];
    ss.join = e[2];
    ss.s = st;
  }
  return &ss;
}

// waiter runs the rest of its work after everything enqueued on s so far.
hipError_t order_after(hipStream_t s, hipStream_t waiter) {
  SideStream* side = side_stream();
  if (side == nullptr) return hipErrorNotInitialized;
  hipError_t e = hipEventRecord(side->join, s);
  return e == hipSuccess ? hipStreamWaitEvent(waiter, side->join, 0) : e;
}

hipError_t launch_ffn_bwd_bf16(const bf16_t* dy_perm, const bf16_t* x_perm, const bf16_t* gu,
                               const bf16_t* h_perm, const int32_t* offsets, int E_l, int R_cap,
                               int H, int I, const bf16_t* w_gate, const bf16_t* w_up,
                               const bf16_t* w_down, bf16_t* dx_perm, float* dw_gate,
                               float* dw_up, float* dw_down, bool accumulate, void* ws,
                               hipStream_t s, hipStream_t wgrad_stream) {
  int32_t* sched = (int32_t*)ws;
  bf16_t* dgu = (bf16_t*)((char*)ws + ffn_sched_bytes(R_cap, E_l));
  int32_t* ctrs = ffn_tile_ctrs(ws, R_cap, E_l);
  // the weight gradients' K-chunk plans and partial slots, after dgu
  char* split_base = (char*)dgu + align256((size_t)R_cap * 2 * I * 2);
  const WgradSplitLayout SL = wgrad_split_layout(E_l, H, I);
  WgradPlan plan{};
  float* part[2];
  for (int q = 0; q < 2; ++q) {
    plan.t[q] = (int32_t*)(split_base + SL.plan_off[q]);
    plan.tiles[q] = SL.tiles[q];
    plan.slots[q] = SL.slots[q];
    part[q] = (float*)(split_base + SL.part_off[q]);
  }
  ffn_sched_kernel<<<1, kMaxE, 0, s>>>(offsets, E_l, kBmGrouped, sched, ctrs, plan);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int mt_upper = R_cap / kBmGrouped + E_l;
  // The weight gradients run on a side stream beside the data gradients:
  //   s:  DOWN_DGRAD -> (mid) -> GATEUP_DGRAD -> wait(join)
  //   s2: wait(fork) -> DOWN_WGRAD -> wait(mid) -> GATEUP_WGRAD -> (join)
  // The data-gradient products leave CUs idle on this layer's shapes (few N
  // tiles, a short last round), which the weight-gradient tiles then use.
  // wgrad_stream (a caller's stream, not joined here) takes the place of the
  // side stream when given.
  SideStream* side = side_stream();
  hipStream_t s2 = s;
  if (side != nullptr) {
    s2 = wgrad_stream != nullptr ? wgrad_stream : side->s;
    if ((err = hipEventRecord(side->fork, s)) != hipSuccess) return err;
    if ((err = hipStreamWaitEvent(s2, side->fork, 0)) != hipSuccess) return err;
  }

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
  a.tile_ctr = ctrs + 0;
  err = launch_gemm<K_DOWN_DGRAD, kBmGrouped, false, kWideGrouped>(a, mt_upper * a.n_ntiles, MOE_KERNEL_FFN_DOWN_DGRAD, s);
  if (err != hipSuccess) return err;
  if (side != nullptr && (err = hipEventRecord(side->mid, s)) != hipSuccess) return err;

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
  b.n_mtiles = (H + kBmWgradDown - 1) / kBmWgradDown;
  b.n_ntiles = (I + BN - 1) / BN;
  b.f0 = dw_down;
  b.m_split = H;
  b.ldc = I;
  b.f_group_stride = (long)H * I;
  b.accumulate = accumulate ? 1 : 0;
  b.tile_ctr = ctrs + 1;
  b.kplan = plan.t[1];
  b.fpart = part[1];
  err = launch_gemm<K_WGRAD, kBmWgradDown, false, kWideWgrad>(b, (E_l + SL.slots[1]) * b.n_mtiles * b.n_ntiles,
                                                             MOE_KERNEL_FFN_DOWN_WGRAD, s2);
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
  c.tile_ctr = ctrs + 2;
  err = launch_gemm<K_GATEUP_DGRAD, kBmGrouped, false, kWideGrouped>(c, mt_upper * c.n_ntiles, MOE_KERNEL_FFN_GATEUP_DGRAD, s);
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
  w.n_mtiles = (2 * I + kBmWgrad - 1) / kBmWgrad;
  w.n_ntiles = (H + BN - 1) / BN;
  w.f0 = dw_gate;
  w.f1 = dw_up;
  w.m_split = I;
  w.ldc = H;
  w.f_group_stride = (long)I * H;
  w.accumulate = accumulate ? 1 : 0;
  w.tile_ctr = ctrs + 3;
  w.kplan = plan.t[0];
  w.fpart = part[0];
  if (side != nullptr && (err = hipStreamWaitEvent(s2, side->mid, 0)) != hipSuccess) return err;
  err = launch_gemm<K_WGRAD, kBmWgrad, false, kWideWgrad>(w, (E_l + SL.slots[0]) * w.n_mtiles * w.n_ntiles,
                                                         MOE_KERNEL_FFN_GATEUP_WGRAD, s2);
  if (err != hipSuccess) return err;
  // the split experts' partial slots, added in chunk order (both products)
  if ((err = launch_wgrad_split_reduce(plan, part, SL, E_l, H, I, dw_gate, dw_up, dw_down, s2)) != hipSuccess)
    return err;
  if (side != nullptr && wgrad_stream == nullptr) {
    if ((err = hipEventRecord(side->join, s2)) != hipSuccess) return err;
    if ((err = hipStreamWaitEvent(s, side->join, 0)) != hipSuccess) return err;
  }
  return hipSuccess;
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
  w.n_mtiles = (H + kBmWgrad - 1) / kBmWgrad;
  w.n_ntiles = (2 * E + BN - 1) / BN;
  w.f0 = partials;
  w.m_split = H;
  const int F = dw_router_folds(E) ? E : 0;  // one N tile: hi in columns 0..E-1, lo in E..2E-1
  w.fold = F;
  w.ldc = F > 0 ? E : 2 * E;
  w.f_group_stride = (long)H * w.ldc;
  w.accumulate = 0;
  return launch_gemm<K_WGRAD, kBmWgrad, false, kWideWgrad>(w, nsplit * w.n_mtiles * w.n_ntiles,
                                                           MOE_KERNEL_ROUTE_BWD_DW, s);
}

bool router_dx_mfma_ok(int H, int E) { return H % 64 == 0 && E > 0 && E % 64 == 0; }

hipError_t launch_router_dx(const bf16_t* dz_hilo, const bf16_t* w_router, int T, int H, int E,
                            float* dx_router, hipStream_t s) {
  if (!router_dx_mfma_ok(H, E)) return hipErrorInvalidValue;
  GemmArgs a{};
  a.a = dz_hilo;     // [T][2E]: high halves, then low halves
  a.lda = 2 * E;
  a.b0 = w_router;   // [H][E]
  a.b1 = w_router;
  a.ldb = E;
  a.M = T;
  a.N = H;
  a.K = 2 * E;       // a multiple of 64, and a K block never straddles E
  a.I = E;
  a.n_mtiles = (T + kBmGrouped - 1) / kBmGrouped;
  a.n_ntiles = (H + BN - 1) / BN;
  a.f0 = dx_router;  // [T][H]
  a.ldc = H;
  a.tile_ctr = nullptr;
  return launch_gemm<K_ROUTER_DX, kBmGrouped, false, true>(a, a.n_mtiles * a.n_ntiles,
                                                           MOE_KERNEL_ROUTE_BWD_DX, s);
}

}  // namespace moe
