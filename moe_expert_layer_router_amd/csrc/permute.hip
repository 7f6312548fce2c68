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
//     block (popcount of the mask bits below it).
//  2. scan: one workgroup turns block counts into counts, offsets and the base
//     row of every (block, expert) pair.
//  3. scatter: one wave per token computes its k destination rows and copies
//     the token row once from HBM into k grouped rows with 16-byte vectors.
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
  __shared__ uint32_t mask[kMaxE][kPermBlock / 32];
  const int tid = threadIdx.x;
  const int t = blockIdx.x * kPermBlock + tid;
  for (int i = tid; i < E_l * (kPermBlock / 32); i += kPermBlock) (&mask[0][0])[i] = 0u;
  __syncthreads();
  const int word = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j] - e_lo;
      if (e >= 0 && e < E_l) atomicOr(&mask[e][word], bit);
    }
  }
  __syncthreads();
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j] - e_lo;
      int r = -1;
      if (e >= 0 && e < E_l) {
        r = __popc(mask[e][word] & (bit - 1u));
        for (int w = 0; w < word; ++w) r += __popc(mask[e][w]);
      }
      rank[(size_t)t * k + j] = r;
    }
  }
  for (int e = tid; e < E_l; e += kPermBlock) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kPermBlock / 32; ++w) c += __popc(mask[e][w]);
    block_counts[(size_t)blockIdx.x * E_l + e] = c;
  }
}

// One workgroup of kMaxE threads; thread e owns local expert e.
__global__ __launch_bounds__(kMaxE) void scan_kernel(const int32_t* __restrict__ block_counts,
                                                     int nblk, int E_l,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ base) {
  __shared__ int s[kMaxE];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E_l)
    for (int b = 0; b < nblk; ++b) total += block_counts[(size_t)b * E_l + e];
  s[e] = total;
  __syncthreads();
  // Hillis-Steele inclusive scan over the kMaxE entries.
  for (int o = 1; o < kMaxE; o <<= 1) {
    const int v = (e >= o) ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  const int excl = s[e] - total;
  if (e < E_l) {
    counts[e] = total;
    offsets[e] = excl;
    if (e == E_l - 1) offsets[E_l] = excl + total;
    int run = excl;
    for (int b = 0; b < nblk; ++b) {
      base[(size_t)b * E_l + e] = run;
      run += block_counts[(size_t)b * E_l + e];
    }
  }
}

// One wave per token: destination rows, inverse map, and the row copy.
__global__ __launch_bounds__(256) void scatter_kernel(const uint4* __restrict__ x,
                                                      const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ base, int T,
                                                      int k, int e_lo, int E_l, int nvec,
                                                      int32_t* __restrict__ dest_row,
                                                      int32_t* __restrict__ src_row,
                                                      uint4* __restrict__ x_perm) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const int b = t / kPermBlock;
  int dest = -1;
  if (lane < k) {
    const int e = idx[(size_t)t * k + lane] - e_lo;
    if (e >= 0 && e < E_l) {
      dest = base[(size_t)b * E_l + e] + rank[(size_t)t * k + lane];
      src_row[dest] = t;
    }
    dest_row[(size_t)t * k + lane] = dest;
  }
  const uint4* xs = x + (size_t)t * nvec;
  // Wave-uniform trip count: every lane joins every shuffle.
  for (int v00 = 0; v00 < nvec; v00 += 4 * kWave) {
    const int v0 = v00 + lane;
    uint4 r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (v0 + u * kWave < nvec) r[u] = xs[v0 + u * kWave];
    for (int j = 0; j < k; ++j) {
      const int d = __shfl(dest, j, kWave);
      if (d < 0) continue;
      uint4* xd = x_perm + (size_t)d * nvec;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (v0 + u * kWave < nvec) xd[v0 + u * kWave] = r[u];
    }
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
  scatter_kernel<<<(T + 3) / 4, 256, 0, s>>>((const uint4*)x, topk_idx, rank, base, T, k, e_lo,
                                              E_l, nvec, dest_row, src_row, (uint4*)x_perm);
  return hipGetLastError();
}

}  // namespace moe
