// Router GEMM + top-k softmax gating for gfx950.
//
// The pages leave the router open; the layer uses the plain top-k router:
// logits z = x . W_r (+ bias), the k largest logits per token (equal logits go
// to the lower expert id, slot order = logit descending then id ascending),
// gate weights = softmax over the kept logits (identical to a softmax over all
// experts renormalised over the kept ones).
//
// bf16, E % 8 == 0 and E <= 128: one launch.  A workgroup of eight waves
// takes 32 tokens and all of W_r, each wave one eighth of H, streamed through
// a private LDS ring by DMA (no barrier in the K loop); bf16 32x32x16 MFMAs
// with W_r as the A operand leave each lane four consecutive experts of one
// token.  The waves' fp32 partial logits meet in LDS, are added in wave order
// (+ bias), and one 16-lane group per token takes the top k: each lane sorts
// its eight (logit, id) keys once, then k rounds take the group maximum of
// the lanes' first keys.  Nothing but logits and the selection leaves the chip.
//
// Other bf16 shapes, two launches.  (1) A workgroup of four waves takes 128
// tokens and one slice of HS rows of W_r (all E experts), copied once into
// LDS; each wave multiplies its 32 tokens' x fragments by the slice and
// stores fp32 partial logits.  (2) One half wave per token adds the slices'
// partials in slice order (+ bias), stores the logits and takes the top k
// with k rounds of a branch-free arg-max over unique (logit, id) keys.
//
// Every sum runs in a fixed order, so logits are deterministic.
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

int route_nb(int E) { return E <= 32 ? 1 : E <= 64 ? 2 : E <= 128 ? 4 : 8; }

// ---------------------------------------------------------------------------
// bf16: sliced router GEMM (partial logits), then sum + top-k
// ---------------------------------------------------------------------------
constexpr int kRtTokens = 128;  // tokens per workgroup: 4 waves x 32
constexpr int kRtMaxRows = 512;  // rows of W_r per slice at most (x fragments held in registers)

// Slice count S (slice HS = H / S rows, a multiple of 64): the fewest slices
// whose W_r copy fits 128 KB of LDS and whose x fragments fit the registers,
// then more while the grid has fewer workgroups than CUs.
int route_slices(int T, int H, int E) {
  const int EP = 32 * route_nb(E);
  const int units = H / 64;
  const int tiles = (T + kRtTokens - 1) / kRtTokens;
  int S = units;
  for (int d = 1; d <= units; ++d) {
    const int HS = H / d;
    if (units % d == 0 && HS <= kRtMaxRows && (size_t)HS * EP * 2 <= 128 * 1024) {
      S = d;
      break;
    }
  }
  for (int d = S + 1; d <= units && tiles * S < kCUs; ++d)
    if (units % d == 0) S = d;
  return S;
}
bool route_fused(int H, int E);
size_t route_ws_bytes(int T, int H, int E) {
  return route_fused(H, E) ? 0 : (size_t)route_slices(T, H, E) * T * E * sizeof(float);
}

// LDS copy of a W_r slice: row h (= k of the product) holds EP bf16 (experts,
// zero past E) as 16-byte chunks; logical chunk c sits at c ^ swz(h), which
// spreads the four rows a transposing read touches over the bank line.
template <int NB>
__device__ __forceinline__ int rt_swz(int h) { return ((h & 3) << 2) & (4 * NB - 1); }

// B fragment of k16-step j, expert block nb: lane l gets expert 32 nb + l % 32,
// k = 16 j + 8 (l / 32) + 0..7, from two transposing reads (rows k and k + 4
// of each 16-lane group): within a group, lane i points at row
// 16 j + 8 (g / 2) + i / 4 and column 32 nb + 16 (g % 2) + 4 (i % 4).
template <int NB>
__device__ __forceinline__ bf16x8_t rt_frag(const bf16_t* s_w, int j, int nb, int lane) {
  constexpr int EP = 32 * NB;
  const int g = lane >> 4, i = lane & 15;
  const int h = 16 * j + 8 * (g >> 1) + (i >> 2);  // h % 4 == (i >> 2) % 4, also for h + 4
  const int c = (4 * nb + 2 * (g & 1) + ((i & 3) >> 1)) ^ rt_swz<NB>(h);
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const auto* q = (const __attribute__((address_space(3))) char*)(
      (const __attribute__((address_space(3))) void*)s_w) + (h * EP + c * 8 + 4 * (i & 1)) * 2;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)q);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 4 * EP * 2));
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// part[(s T + t) E + e] = sum over h in slice s (ascending, in MFMA k-steps) of x[t][h] W_r[h][e].
template <int NB, int NSMAX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void route_part_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int T, int H,
                       int E, int HS, float* __restrict__ part) {
  constexpr int EP = 32 * NB;
  constexpr int CPR = EP / 8;  // 16-byte chunks per LDS row
  extern __shared__ __align__(16) bf16_t s_w[];  // [HS][EP]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int sl = blockIdx.y, h0 = sl * HS;
  const int nstep = HS / 16;
  const int t0 = blockIdx.x * kRtTokens + wave * 32;

  // Load order: this thread's chunks of the W_r slice (at most 32: the slice
  // is at most 128 KB), then the x fragments of the whole slice, all in
  // flight together; the LDS stores of the slice wait only for the W_r loads
  // (older in the in-order memory counter), and each MFMA step only for its
  // own x fragment, so the MFMAs overlap the x stream.
  //   x: lane row t0 + l % 32 (clamped into range; rows past T are computed but
  //   never stored), k = 16 j + 8 (l / 32) + 0..7.
  const int nchunk = HS * CPR;
  constexpr int kMaxChunks = 128 * 1024 / 16 / 256;
  const bool vec = E % 8 == 0;
  u32x4_t wv[kMaxChunks];
  if (vec) {
#pragma unroll
    for (int u = 0; u < kMaxChunks; ++u) {
      const int c = threadIdx.x + u * 256;
      const int h = c / CPR, ch = c % CPR;
      wv[u] = (c < nchunk && ch * 8 < E)
                  ? *reinterpret_cast<const u32x4_t*>(w + (size_t)(h0 + h) * E + ch * 8)
                  : u32x4_t{};
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  int trow = min(t0 + (lane & 31), T - 1);
  const bf16_t* xa = x + (size_t)trow * H + h0 + (lane >> 5) * 8;
  bf16x8_t a[NSMAX];
#pragma unroll
  for (int j = 0; j < NSMAX; ++j) a[j] = *reinterpret_cast<const bf16x8_t*>(xa + 16 * min(j, nstep - 1));
  __builtin_amdgcn_sched_barrier(0);

  // W_r[h0 .. h0 + HS) -> s_w
  if (vec) {
#pragma unroll
    for (int u = 0; u < kMaxChunks; ++u) {
      const int c = threadIdx.x + u * 256;
      if (c >= nchunk) break;
      const int h = c / CPR, ch = c % CPR;
      *reinterpret_cast<u32x4_t*>(s_w + h * EP + ((ch ^ rt_swz<NB>(h)) * 8)) = wv[u];
    }
  } else {
    for (int i = threadIdx.x; i < HS * EP; i += 256) {
      const int h = i / EP, e = i % EP;
      s_w[h * EP + (((e >> 3) ^ rt_swz<NB>(h)) << 3) + (e & 7)] =
          e < E ? w[(size_t)(h0 + h) * E + e] : bf16_t(0);
    }
  }
  __syncthreads();

  f32x16_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16_t{};
#pragma unroll
  for (int j = 0; j < NSMAX; ++j) {
    // steps past the slice multiply zeros (by a fragment of step 0)
    const bool on = j < nstep;
    const bf16x8_t av = on ? a[j] : bf16x8_t{};
    const int js = on ? j : 0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, rt_frag<NB>(s_w, js, nb, lane), acc[nb], 0,
                                                        0, 0);
  }
  float* ps = part + (size_t)sl * T * E;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int t = t0 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      const int e = nb * 32 + (lane & 31);
      if (t < T && e < E) ps[(size_t)t * E + e] = acc[nb][q];
    }
}

// Logits z[t][e] = sum over slices s (ascending) of part[s][t][e] (+ bias[e]),
// then the top-k.  Two tokens per wave, one per half.
template <int NB>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ part, int S,
                                                         int T, int E, int k,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (2 * pair >= T) return;
  const int t = 2 * pair + ((threadIdx.x >> 5) & 1);
  const bool active = t < T;
  const int tr = active ? t : T - 1;
  const int h32 = lane_id() & 31;
  float v[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) v[i] = 0.f;
  // four slices' loads in flight at a time, added in slice order
  for (int s0 = 0; s0 < S; s0 += 4) {
    float pv[4][NB];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* ps = part + ((size_t)min(s0 + u, S - 1) * T + tr) * E;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int e = h32 + 32 * i;
        pv[u][i] = (e < E) ? ps[e] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + u < S) {
#pragma unroll
        for (int i = 0; i < NB; ++i) v[i] += pv[u][i];
      }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int e = h32 + 32 * i;
    if (e < E) {
      if (bias != nullptr) v[i] += bias[e];
      if (logits != nullptr && active) logits[(size_t)t * E + e] = v[i];
    }
  }
  topk_softmax_half<NB>(v, E, k, active, topk_idx + (size_t)tr * k, topk_w + (size_t)tr * k);
}

// ---------------------------------------------------------------------------
// bf16, one launch: a workgroup of eight waves multiplies 32 tokens by all of
// W_r, the waves splitting H into eight ranges; the waves' partial logits are
// added through LDS and the same workgroup takes the top k.
// ---------------------------------------------------------------------------
// Each wave streams its own H range through a private LDS ring, so the K loop
// has no barrier.  A step is 16 rows of H (one MFMA k-step): W_r[h .. h+16)
// [0 .. EP), DMA'd into the swizzled rows of the sliced kernel and read back
// with transposing reads, DW steps ahead.  x comes in stages of 64 columns
// (four steps): x[32 tokens][h .. h+64), whole 128-byte rows per 8 lanes, so
// every request is a full cache line, DXQ stages ahead; the 16-byte chunks of
// a row are XOR-swizzled by (row / 2) % 8 so that the fragment reads (32 rows
// of one chunk) spread over all banks.  Every load is a DMA with explicit
// counter waits.  Expert columns past E and token rows past T are read as
// zeros (outside the buffer range), as are the stages past a wave's range,
// which keeps the loop free of branches.
constexpr int kRfWaves = 8;

template <int NB>
struct RfCfg {
  static constexpr int EP = 32 * NB;
  static constexpr int CPR = EP / 8;                  // 16-byte chunks per W_r row
  static constexpr int DW = NB == 4 ? 3 : 4;          // W_r stages (16 rows) in the ring
  static constexpr int DXQ = 2;                       // x stages (64 columns) in the ring
  static constexpr int WST = 16 * EP * 2;             // bytes of one W_r stage
  static constexpr int XST = 32 * 64 * 2;             // bytes of one x stage
  static constexpr int RING = DW * WST + DXQ * XST;   // one wave's ring
  static constexpr int NJ = EP > 64 ? EP / 64 : 1;   // 4-expert groups per lane in the top-k
  static constexpr int NV = 4 * NJ;                   // logits per lane in the top-k
  static constexpr int RLD = 64 * NJ + 4;             // fp32 pitch of a reduction row
  static constexpr int RED = kRfWaves * 32 * RLD * 4;
  static constexpr int LDS = kRfWaves * RING > RED ? kRfWaves * RING : RED;
  static_assert(LDS <= 160 * 1024 && 4 * DXQ >= DW && DW >= 3, "router ring");
  // Issue order: after step i, the W_r stage of step i + DW; after the last
  // step of x stage q, also x stage q + DXQ.  The fragments of step i are
  // read while step i - 1 multiplies, i.e. before the issue that follows step
  // i - 1 (lag 1; lag 0 for step 0).  The wait leaves in flight the DMA
  // instructions issued after the later of the two stages step i reads.
  static constexpr int vm_wait(int s, int lag) {
    const int i = 400 + s;
    const int ew = i - DW, ex = (i - s) - 4 * DXQ + 3;
    const int later = ew > ex ? ew : ex;
    int n = 0;
    for (int j = later; j < i - lag; ++j) {
      const int nx = (j % 4 == 3) ? 4 : 0;
      n += (j == later) ? (later == ex ? 0 : nx) : NB + nx;
    }
    return n;
  }
  static constexpr int NR = 1 + 2 * NB;  // LDS reads of one step's fragments
};

template <int NB, int S, int LAG>
__device__ __forceinline__ void rf_wait() {
  constexpr int n = RfCfg<NB>::vm_wait(S, LAG);
  static_assert(n < 64, "vmcnt");
  wait_vm<n>();
}

// 16-lane group reductions (xor 1, xor 2, i <-> 7 - i, i <-> 15 - i): every
// lane of the group ends with the group's result.
__device__ __forceinline__ float sum16_f32(float v) {
  v += __uint_as_float(dpp32<kDppXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<kDppXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<kDppHalfMirror>(__float_as_uint(v)));
  return v + __uint_as_float(dpp32<kDppMirror>(__float_as_uint(v)));
}
// Sorting networks (descending) on the selection keys of one lane.
template <int NV>
struct SortNet;
template <>
struct SortNet<4> {
  static constexpr int n = 5;
  static constexpr int a[5] = {0, 2, 0, 1, 1}, b[5] = {1, 3, 2, 3, 2};
};
template <>
struct SortNet<8> {
  static constexpr int n = 19;
  static constexpr int a[19] = {0, 1, 4, 5, 0, 1, 2, 3, 0, 2, 4, 6, 2, 3, 1, 3, 1, 3, 5};
  static constexpr int b[19] = {2, 3, 6, 7, 4, 5, 6, 7, 1, 3, 5, 7, 4, 5, 4, 6, 2, 4, 6};
};

__device__ __forceinline__ uint64_t max16_u64(uint64_t k) {
  k = max_u64(k, dpp64<kDppXor1>(k));
  k = max_u64(k, dpp64<kDppXor2>(k));
  k = max_u64(k, dpp64<kDppHalfMirror>(k));
  return max_u64(k, dpp64<kDppMirror>(k));
}

// k-round selection + softmax of one token held by a 16-lane group: key[i]
// is the selection key of expert ids[i] (0 for none).  The lane's keys are
// sorted once; a round then takes the group maximum of the lanes' first keys
// (keys are unique, so one lane holds it) and that lane drops its first key.
// Lane h keeps rounds h and h + 16 and writes those slots.
template <int NV>
__device__ __forceinline__ void topk_softmax_16(uint64_t (&key)[NV], int k, bool active,
                                                int32_t* idx_out, float* w_out) {
  const int h = lane_id() & 15;
#pragma unroll
  for (int c = 0; c < SortNet<NV>::n; ++c) {
    const int a = SortNet<NV>::a[c], b = SortNet<NV>::b[c];
    const uint64_t hi = max_u64(key[a], key[b]), lo = key[a] ^ key[b] ^ hi;
    key[a] = hi;
    key[b] = lo;
  }
  uint64_t mine0 = 0, mine1 = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t best = max16_u64(key[0]);
    // the winning lane drops its first key (a mask, not a select: a select
    // between neighbours becomes an indexed access over the whole array)
    const uint64_t m = 0ull - (uint64_t)(key[0] == best);
#pragma unroll
    for (int i = 0; i + 1 < NV; ++i) key[i] = (key[i + 1] & m) | (key[i] & ~m);
    key[NV - 1] &= ~m;
    mine0 = (j == h) ? best : mine0;
    mine1 = (j == h + 16) ? best : mine1;
  }
  const float z0 = key_value(mine0), z1 = key_value(mine1);
  const float zmax = __shfl(z0, lane_id() & ~15, kWave);  // slot 0 of this group
  const float ex0 = h < k ? expf(z0 - zmax) : 0.f;
  const float ex1 = h + 16 < k ? expf(z1 - zmax) : 0.f;
  const float sum = sum16_f32(ex0 + ex1);
  if (active) {
    if (h < k) {
      idx_out[h] = key_expert(mine0);
      w_out[h] = ex0 / sum;
    }
    if (h + 16 < k) {
      idx_out[h + 16] = key_expert(mine1);
      w_out[h + 16] = ex1 / sum;
    }
  }
}

template <int NB>
__global__ __launch_bounds__(512) void route_fused_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ w,
                                                          const float* __restrict__ bias, int T,
                                                          int H, int E, int k,
                                                          float* __restrict__ logits,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w) {
  using C = RfCfg<NB>;
  extern __shared__ __align__(16) bf16_t s_rf[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tok0 = blockIdx.x * 32;
  const int nq = H / 64;
  const int q0 = wave * nq / kRfWaves;
  const int nqw = (wave + 1) * nq / kRfWaves - q0;  // this wave's x stages (may be 0)
  const int ns = 4 * nqw;

  const rsrc_t rw = make_rsrc(w, (uint32_t)H * E * 2);
  const int rows = min(T - tok0, 32);
  const rsrc_t rx = make_rsrc(x + (size_t)tok0 * H, (uint32_t)rows * H * 2);
  const uint32_t ring = lds_addr(s_rf) + wave * C::RING;
  const uint32_t xring = ring + C::DW * C::WST;
  // byte offsets at this wave's first step / stage.  W_r: DMA instruction u
  // fills LDS chunk p = 64 u + lane = row p / CPR, logical chunk
  // (p % CPR) ^ swz(row).  x: instruction u fills rows 8 u + lane / 8, LDS
  // chunk lane % 8 = logical chunk (lane % 8) ^ ((row / 2) % 8).
  uint32_t wo[NB], xo[4];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int p = u * 64 + lane, r = p / C::CPR;
    const int c = (p % C::CPR) ^ rt_swz<NB>(r);
    wo[u] = 8 * c < E ? (uint32_t)(((64 * q0 + r) * E + 8 * c) * 2) : kDmaKill;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 8 * u + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    xo[u] = (uint32_t)((r * H + 64 * q0 + 8 * c) * 2);
  }
  const uint32_t wstep = 32u * (uint32_t)E;  // bytes of 16 rows of W_r

  auto issue_w = [&](int i) {
    const uint32_t kill = i < ns ? 0u : kDmaKill;
    const uint32_t dst = ring + (uint32_t)(i % C::DW) * C::WST;
#pragma unroll
    for (int u = 0; u < NB; ++u) dma16(rw, (wo[u] + (uint32_t)i * wstep) | kill, dst + u * 1024);
  };
  auto issue_x = [&](int q) {
    const uint32_t kill = q < nqw ? 0u : kDmaKill;
    const uint32_t dst = xring + (uint32_t)(q % C::DXQ) * C::XST;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma16(rx, (xo[u] + 128u * (uint32_t)q) | kill, dst + u * 1024);
  };
  // prologue: the steady state's issue order for the steps before step 0
#pragma unroll
  for (int j = -(4 * C::DXQ > C::DW ? 4 * C::DXQ : C::DW); j < 0; ++j) {
    if (j + C::DW >= 0) issue_w(j + C::DW);
    if ((j & 3) == 3 && (j >> 2) + C::DXQ >= 0) issue_x((j >> 2) + C::DXQ);
  }

  // fragments of step i: x from stage i / 4 (lane: token row lane % 32,
  // logical chunk 2 (i % 4) + lane / 32), W_r from ring slot i % DW
  const int arow = lane & 31;
  const bf16_t* xbase = s_rf + (wave * C::RING + C::DW * C::WST) / 2 + arow * 64;
  auto read_frags = [&](int i, bf16x8_t& a, bf16x8_t (&b)[NB]) {
    const int c = (2 * (i & 3) + (lane >> 5)) ^ ((arow >> 1) & 7);
    a = *reinterpret_cast<const bf16x8_t*>(xbase + ((i >> 2) % C::DXQ) * (C::XST / 2) + c * 8);
    const bf16_t* sw = s_rf + (wave * C::RING + (i % C::DW) * C::WST) / 2;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[nb] = rt_frag<NB>(sw, 0, nb, lane);
  };

  f32x16_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16_t{};
  bf16x8_t a, b[NB];
  rf_wait<NB, 0, 0>();
  read_frags(0, a, b);
  for (int q = 0; q < nqw; ++q) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int i = 4 * q + s4;
      // step i + 1's fragments (past the wave's range: zeros, unused) are read
      // while step i multiplies
      if (s4 == 0) rf_wait<NB, 1, 1>();
      else if (s4 == 1) rf_wait<NB, 2, 1>();
      else if (s4 == 2) rf_wait<NB, 3, 1>();
      else rf_wait<NB, 0, 1>();
      bf16x8_t an, bn[NB];
      read_frags(i + 1, an, bn);
      // the compiler keeps this order (reads of step i + 1, then the MFMAs of
      // step i, then the refill): left free, it moves the MFMAs behind reads
      // they do not need and waits for those too
      __builtin_amdgcn_sched_barrier(0);
      // W_r fragment as A (experts are the rows of the product), x as B
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[nb], a, acc[nb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      // step i's slots are refilled next: its reads (older than step i + 1's)
      // must have returned
      asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(C::NR) : "memory");
      issue_w(i + C::DW);
      if (s4 == 3) issue_x(q + C::DXQ);
      a = an;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) b[nb] = bn[nb];
    }
  }
  wait_vm<0>();  // the trailing (zero-filling) stages land before LDS is reused
  __syncthreads();

  // acc[nb][q] = partial logit of expert 32 nb + 8 (q / 4) + 4 (lane / 32) + q % 4
  // for token lane % 32: four consecutive experts per 16-byte LDS store.
  float* red = reinterpret_cast<float*>(s_rf);  // [wave][token][RLD]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<f32x4_t*>(red + (wave * 32 + (lane & 31)) * C::RLD + 32 * nb + 8 * g +
                                  4 * (lane >> 5)) =
          f32x4_t{acc[nb][4 * g], acc[nb][4 * g + 1], acc[nb][4 * g + 2], acc[nb][4 * g + 3]};
  __syncthreads();
  // wave w: token rows 4 w .. 4 w + 3, one per 16-lane group; lane h of a
  // group holds experts 4 h + 64 j + 0..3.  Logit = sum over waves (H ranges
  // ascending) + bias.
  const int r = 4 * wave + (lane >> 4), h = lane & 15;
  const int t = tok0 + r;
  const bool active = t < T;
  const bool vec = ((uintptr_t)logits & 15) == 0 && ((uintptr_t)bias & 15) == 0;
  uint64_t key[C::NV];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    const int e0 = 4 * h + 64 * j;
    f32x4_t z = f32x4_t{};
#pragma unroll
    for (int wv = 0; wv < kRfWaves; ++wv)
      z += *reinterpret_cast<const f32x4_t*>(red + (wv * 32 + r) * C::RLD + e0);
    if (e0 < E) {  // E % 8 == 0: the four experts are all valid
      if (bias != nullptr) {
        if (vec) {
          z += *reinterpret_cast<const f32x4_t*>(bias + e0);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) z[c] += bias[e0 + c];
        }
      }
      if (logits != nullptr && active) {
        if (vec) {
          *reinterpret_cast<f32x4_t*>(logits + (size_t)t * E + e0) = z;
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) logits[(size_t)t * E + e0 + c] = z[c];
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) key[4 * j + c] = e0 < E ? topk_key(z[c], e0 + c) : 0ull;
  }
  const int tr = active ? t : T - 1;
  topk_softmax_16<C::NV>(key, k, active, topk_idx + (size_t)tr * k, topk_w + (size_t)tr * k);
}

// Shapes the one-launch router takes (else the sliced two-launch path).
bool route_fused(int H, int E) {
  return E % 8 == 0 && E <= 128 && H % 64 == 0 && (size_t)H * E * 2 < (1u << 31) &&
         (size_t)32 * H * 2 < (1u << 31);
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
                             float* part_ws, hipStream_t s) {
  const int nb = route_nb(E);
  if (route_fused(H, E)) {
    ProfScope ps(MOE_KERNEL_ROUTE, s);
    const int grid = (T + 31) / 32;
    if (nb == 1)
      route_fused_kernel<1><<<grid, 512, RfCfg<1>::LDS, s>>>(x, w_router, bias, T, H, E, k, logits, topk_idx, topk_w);
    else if (nb == 2)
      route_fused_kernel<2><<<grid, 512, RfCfg<2>::LDS, s>>>(x, w_router, bias, T, H, E, k, logits, topk_idx, topk_w);
    else
      route_fused_kernel<4><<<grid, 512, RfCfg<4>::LDS, s>>>(x, w_router, bias, T, H, E, k, logits, topk_idx, topk_w);
    return hipGetLastError();
  }
  const int S = route_slices(T, H, E);
  const int HS = H / S;
  const dim3 grid((T + kRtTokens - 1) / kRtTokens, S);
  const size_t lds = (size_t)HS * 32 * nb * sizeof(bf16_t);
  ProfScope ps(MOE_KERNEL_ROUTE, s);
#define MOE_RT_CASE(NB)                                                                        \
  do {                                                                                         \
    if (HS <= 256)                                                                             \
      route_part_kernel<NB, 16><<<grid, 256, lds, s>>>(x, w_router, T, H, E, HS, part_ws);     \
    else                                                                                       \
      route_part_kernel<NB, 32><<<grid, 256, lds, s>>>(x, w_router, T, H, E, HS, part_ws);     \
    route_topk_kernel<NB><<<(T + 7) / 8, 256, 0, s>>>(part_ws, S, T, E, k, bias, logits,       \
                                                      topk_idx, topk_w);                      \
  } while (0)
  if (nb == 1) MOE_RT_CASE(1);
  else if (nb == 2) MOE_RT_CASE(2);
  else if (nb == 4) MOE_RT_CASE(4);
  else MOE_RT_CASE(8);
#undef MOE_RT_CASE
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
