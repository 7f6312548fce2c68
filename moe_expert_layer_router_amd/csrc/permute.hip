// Permute: group routed token rows by expert (the "permute" op of the
// dispatcher table on the page "FSDPTurbo EP/EFSDP and LlamaFactory FSDP2/CP
// Design", section 3).  Rows of one expert keep ascending token order (the
// order a stable sort by expert gives), so the result is unique and the
// kernels are bit-exact against a plain definition.
//
// Three launches, no host synchronisation:
//  1. hist_rank: each block of 256 tokens builds, in LDS, one 256-bit token
//     mask per local expert with atomicOr (order independent), then reads off
//     per-expert block counts and each slot's rank among earlier tokens of the
//     block (popcount of the mask bits below it).  A block in which a token
//     lists one local expert twice ranks its slots by a walk in (token, slot)
//     order instead.
//  2. scan: one workgroup turns block counts into counts, offsets and the base
//     row of every (block, expert) pair.
//  3. scatter: one wave per token computes its k destination rows and, if
//     any slot is local, copies the token row once from HBM into its grouped
//     rows with 16-byte vectors (or, without a grouped buffer, writes the
//     maps alone).
#include "common.h"

namespace moe {

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t permute_ws_bytes(int T, int k, int E_l) {
  const size_t nblk = (size_t)(T + kPermBlock - 1) / kPermBlock;
  return 2 * align256(nblk * E_l * sizeof(int32_t)) + align256((size_t)T * k * sizeof(int32_t));
}

__global__ __launch_bounds__(kPermBlock) void hist_rank_kernel(const int32_t* __restrict__ idx,
                                                               int T, int k, int e_lo, int E_l,
                                                               int32_t* __restrict__ block_counts,
                                                               int32_t* __restrict__ rank) {
  constexpr int NW = kPermBlock / 32;  // mask words per expert
  __shared__ uint32_t mask[kMaxE][NW];
  __shared__ int16_t s_e[kPermBlock * kMaxK];  // local expert of each slot of the block, or -1
  __shared__ int32_t s_pre[kMaxE][NW];         // set bits of mask[e] in words before w
  __shared__ int s_dup;                        // some token repeats a local expert
  const int tid = threadIdx.x;
  if (tid == 0) s_dup = 0;
  const int t0 = blockIdx.x * kPermBlock;
  const int nt = min(kPermBlock, T - t0);
  const int nslot = nt * k;
  for (int i = tid; i < E_l * NW; i += kPermBlock) (&mask[0][0])[i] = 0u;
  // Coalesced copy of the block's [nt, k] slice of idx, four loads in flight
  // per thread before any is used.
  const int32_t* src = idx + (size_t)t0 * k;
  for (int i0 = 0; i0 < nslot; i0 += 4 * kPermBlock) {
    int v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kPermBlock + tid;
      v[u] = i < nslot ? src[i] - e_lo : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kPermBlock + tid;
      if (i < nslot) s_e[i] = (v[u] >= 0 && v[u] < E_l) ? (int16_t)v[u] : (int16_t)-1;
    }
  }
  __syncthreads();
  const int word = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  if (tid < nt) {
    bool dup = false;
    for (int j = 0; j < k; ++j) {
      const int e = s_e[tid * k + j];
      // only this thread sets this token's bit, so a bit already set means the
      // token lists expert e in an earlier slot
      if (e >= 0) dup |= (atomicOr(&mask[e][word], bit) & bit) != 0u;
    }
    if (dup) s_dup = 1;
  }
  __syncthreads();
  if (s_dup != 0) {
    // A token of this block lists one local expert in several slots (top-k
    // never does; a caller's own lists may).  One bit per (expert, token)
    // cannot count those slots, so each expert's thread walks the block's
    // slots in (token, slot) order instead: the slots of one expert get
    // consecutive ranks in that order, as the plain definition orders them.
    for (int e = tid; e < E_l; e += kPermBlock) {
      int c = 0;
      for (int i = 0; i < nslot; ++i)
        if (s_e[i] == e) rank[(size_t)t0 * k + i] = c++;
      block_counts[(size_t)blockIdx.x * E_l + e] = c;
    }
    for (int i = tid; i < nslot; i += kPermBlock)
      if (s_e[i] < 0) rank[(size_t)t0 * k + i] = -1;
    return;
  }
  for (int e = tid; e < E_l; e += kPermBlock) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      s_pre[e][w] = c;
      c += __popc(mask[e][w]);
    }
    block_counts[(size_t)blockIdx.x * E_l + e] = c;
  }
  __syncthreads();
  if (tid < nt) {
    for (int j = 0; j < k; ++j) {
      const int e = s_e[tid * k + j];
      rank[(size_t)(t0 + tid) * k + j] =
          e >= 0 ? s_pre[e][word] + __popc(mask[e][word] & (bit - 1u)) : -1;
    }
  }
}

// One workgroup of kMaxE threads; thread e owns local expert e.  Block counts
// are read 64 blocks at a time with all loads in flight together (one round
// trip up to 16384 tokens).
__global__ __launch_bounds__(kMaxE) void scan_kernel(const int32_t* __restrict__ block_counts,
                                                     int nblk, int E_l,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ base) {
  constexpr int CH = 64;
  __shared__ int s[kMaxE / kWave];
  const int e = threadIdx.x;
  const bool own = e < E_l;
  int total = 0;
  int v[CH];
  for (int b0 = 0; b0 < nblk; b0 += CH) {
#pragma unroll
    for (int u = 0; u < CH; ++u)
      v[u] = (own && b0 + u < nblk) ? block_counts[(size_t)(b0 + u) * E_l + e] : 0;
#pragma unroll
    for (int u = 0; u < CH; ++u) total += v[u];
  }
  // inclusive scan of the totals: within each wave by shuffles, then the
  // waves' sums
  const int lane = e & (kWave - 1), w = e / kWave;
  int incl = total;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int t = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += t;
  }
  if (lane == kWave - 1) s[w] = incl;
  __syncthreads();
  for (int q = 0; q < w; ++q) incl += s[q];
  const int excl = incl - total;
  if (!own) return;
  counts[e] = total;
  offsets[e] = excl;
  if (e == E_l - 1) offsets[E_l] = excl + total;
  int run = excl;
  for (int b0 = 0; b0 < nblk; b0 += CH) {
    if (nblk > CH) {  // the values of this chunk are no longer in registers
#pragma unroll
      for (int u = 0; u < CH; ++u)
        v[u] = b0 + u < nblk ? block_counts[(size_t)(b0 + u) * E_l + e] : 0;
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (b0 + u < nblk) base[(size_t)(b0 + u) * E_l + e] = run;
      run += v[u];
    }
  }
}

// One wave per token: destination rows, inverse map, and the row copy.  The
// token row is read only when at least one of its slots is local, together
// with the slots' ranks and block bases.  COPY = false writes the two maps
// only (a caller whose grouped FFN reads the token rows through src_row).
template <bool COPY>
__global__ __launch_bounds__(256) void scatter_kernel(const u32x4_t* __restrict__ x,
                                                      const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ base, int T,
                                                      int k, int e_lo, int E_l, int nvec,
                                                      int32_t* __restrict__ dest_row,
                                                      int32_t* __restrict__ src_row,
                                                      u32x4_t* __restrict__ x_perm) {
  constexpr int CU = 4;  // 16-byte vectors per lane in flight
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const int b = t / kPermBlock;
  int e = -1;
  if (lane < k) {
    e = idx[(size_t)t * k + lane] - e_lo;
    if (e >= E_l) e = -1;
  }
  const uint64_t m = __ballot(e >= 0);
  if (m == 0) {
    if (lane < k) dest_row[(size_t)t * k + lane] = -1;
    return;
  }
  int dest = -1;
  if (e >= 0) dest = base[(size_t)b * E_l + e] + rank[(size_t)t * k + lane];
  if constexpr (!COPY) {
    if (lane < k) {
      dest_row[(size_t)t * k + lane] = dest;
      if (dest >= 0) src_row[dest] = t;
    }
    return;
  }
  const u32x4_t* xs = x + (size_t)t * nvec;
  u32x4_t r[CU];
  int v0 = lane;
#pragma unroll
  for (int u = 0; u < CU; ++u) r[u] = (v0 + u * kWave < nvec) ? xs[v0 + u * kWave] : u32x4_t{};
  if (lane < k) {
    dest_row[(size_t)t * k + lane] = dest;
    if (dest >= 0) src_row[dest] = t;
  }
  // Wave-uniform trip counts: every lane joins every shuffle.
  for (;;) {
    for (uint64_t mm = m; mm != 0; mm &= mm - 1) {
      const int d = __shfl(dest, __ffsll((long long)mm) - 1, kWave);
      u32x4_t* xd = x_perm + (size_t)d * nvec;
#pragma unroll
      for (int u = 0; u < CU; ++u)
        if (v0 + u * kWave < nvec) xd[v0 + u * kWave] = r[u];
    }
    v0 += CU * kWave;
    if (v0 - lane >= nvec) break;
#pragma unroll
    for (int u = 0; u < CU; ++u) r[u] = (v0 + u * kWave < nvec) ? xs[v0 + u * kWave] : u32x4_t{};
  }
}

hipError_t launch_permute(const void* x, const int32_t* topk_idx, int T, int H, int k, int e_lo,
                          int e_hi, int elem_bytes, int32_t* counts, int32_t* offsets,
                          int32_t* dest_row, int32_t* src_row, void* x_perm, void* ws,
                          hipStream_t s) {
  const int E_l = e_hi - e_lo;
  const int nblk = (T + kPermBlock - 1) / kPermBlock;
  char* w = (char*)ws;
  int32_t* block_counts = (int32_t*)w;
  w += align256((size_t)nblk * E_l * sizeof(int32_t));
  int32_t* base = (int32_t*)w;
  w += align256((size_t)nblk * E_l * sizeof(int32_t));
  int32_t* rank = (int32_t*)w;

  hipError_t err;
  if (nblk > 0) {
    ProfScope ps(MOE_KERNEL_PERMUTE_HIST, s);
    hist_rank_kernel<<<nblk, kPermBlock, 0, s>>>(topk_idx, T, k, e_lo, E_l, block_counts, rank);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // Runs for T == 0 too: counts and offsets are then all zero.
  {
    ProfScope ps(MOE_KERNEL_PERMUTE_SCAN, s);
    scan_kernel<<<1, kMaxE, 0, s>>>(block_counts, nblk, E_l, counts, offsets, base);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (T == 0) return hipSuccess;
  const int nvec = H * elem_bytes / 16;
  ProfScope ps(MOE_KERNEL_PERMUTE_SCATTER, s);
  if (x_perm != nullptr)
    scatter_kernel<true><<<(T + 3) / 4, 256, 0, s>>>((const u32x4_t*)x, topk_idx, rank, base, T, k,
                                                    e_lo, E_l, nvec, dest_row, src_row,
                                                    (u32x4_t*)x_perm);
  else
    scatter_kernel<false><<<(T + 3) / 4, 256, 0, s>>>(nullptr, topk_idx, rank, base, T, k, e_lo, E_l,
                                                     nvec, dest_row, src_row, nullptr);
  return hipGetLastError();
}

}  // namespace moe
