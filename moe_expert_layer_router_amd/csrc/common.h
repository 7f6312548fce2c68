// Shared device helpers and internal launch declarations of the gfx950 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// 16 bytes as a native vector: staging values stay in registers (the
// union-based HIP uint4 is not always split into registers by the compiler).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kMaxE = 256;
constexpr int kMaxK = 32;
constexpr int kCUs = 256;  // compute units of one MI355X

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round to nearest, ties to even, with the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32); NaN stays NaN, infinities pass.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 1 / x with the hardware reciprocal (about 1 ulp).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Unpack 8 bf16 held in a uint4 into fp32.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]),
                    pack_bf2(f[6], f[7]));
}

// ---------------------------------------------------------------------------
// Wave-level reductions (64 lanes, fixed butterfly order => deterministic)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Workgroup barrier that orders LDS only: global loads stay in flight and
// stores are not waited for (__syncthreads waits for every memory operation).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Logical workgroup id with consecutive ids on the same XCD.  The hardware
// hands workgroup i to XCD i % 8; remapping makes each XCD own a contiguous
// slice of the logical range, so neighbouring tiles share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks / 8;
  if (bid >= per * 8) return bid;  // ragged tail keeps its id
  return (bid % 8) * per + bid / 8;
}

// ---------------------------------------------------------------------------
// buffer -> LDS DMA and explicit synchronisation
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef int rsrc_t __attribute__((ext_vector_type(4)));  // buffer descriptor (4 SGPRs)

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

// Offset that moves a DMA beyond every buffer range used here (all below
// 2 GiB): the hardware drops the read and writes zeros into LDS.
constexpr uint32_t kDmaKill = 0x80000000u;

}  // namespace moe

// ---------------------------------------------------------------------------
// Optional event recording around one kernel's launches (see moe_profile_kernel).
// ---------------------------------------------------------------------------
namespace moe {
struct ProfScope {
  ProfScope(int kernel_id, hipStream_t s);
  ~ProfScope();
  int slot;
  hipStream_t stream;
};
}  // namespace moe

// ---------------------------------------------------------------------------
// Internal launchers (host side).  Arguments were validated by the C ABI.
// Each returns hipSuccess or the launch error.
// ---------------------------------------------------------------------------
namespace moe {

// route.hip
int route_nb(int E);                      // 32-expert column blocks of the bf16 router
size_t route_ws_bytes(int T, int H, int E);  // partial logits of the bf16 router
hipError_t launch_route_bf16(const bf16_t* x, const bf16_t* w_router, const float* bias, int T,
                             int H, int E, int k, float* logits, int32_t* topk_idx, float* topk_w,
                             float* part_ws, hipStream_t s);
hipError_t launch_route_f32(const float* x, const float* w_router, const float* bias, int T, int H,
                            int E, int k, float* logits, int32_t* topk_idx, float* topk_w,
                            hipStream_t s);
hipError_t launch_route_from_logits(const float* logits, int T, int E, int k, int32_t* topk_idx,
                                    float* topk_w, hipStream_t s);
hipError_t launch_transpose(const void* src, void* dst, int rows, int cols, int elem_bytes,
                            hipStream_t s);

// permute.hip
constexpr int kPermBlock = 256;  // tokens per histogram block
size_t permute_ws_bytes(int T, int k, int E_l);
hipError_t launch_permute(const void* x, const int32_t* topk_idx, int T, int H, int k, int e_lo,
                          int e_hi, int elem_bytes, int32_t* counts, int32_t* offsets,
                          int32_t* dest_row, int32_t* src_row, void* x_perm, void* ws,
                          hipStream_t s);

// combine.hip
hipError_t launch_combine(const void* y_perm, const float* topk_w, const int32_t* dest_row,
                          const float* addend, int T, int H, int k, bool bf16, void* y,
                          hipStream_t s);
hipError_t launch_combine_bwd(const void* dy, const void* y_perm, const float* topk_w,
                              const int32_t* dest_row, int T, int H, int k, bool bf16,
                              void* dy_perm, float* d_topk_w, hipStream_t s);
hipError_t launch_combine_dx(const void* dx_perm, const int32_t* dest_row, const float* d_topk_w,
                             const float* topk_w, const int32_t* topk_idx, const void* w_router_t,
                             int T, int H, int k, bool bf16, void* dx, hipStream_t s);
hipError_t launch_route_bwd_dz(const float* d_topk_w, const float* topk_w,
                               const int32_t* topk_idx, const void* w_router_t, int T, int H, int E,
                               int k, bool bf16, float* d_logits, float* dx_router,
                               bf16_t* dz_hilo, hipStream_t s);
hipError_t launch_dw_router_f32(const float* x, const float* d_logits, int T, int H, int E,
                                float* dw_router, hipStream_t s);
hipError_t launch_dw_router_reduce(const float* partials, int nsplit, int H, int E, bool folded,
                                   float* dw_router, hipStream_t s);

// gemm.hip (bf16 MFMA grouped GEMMs)
int gemm_tiles(int M, int N);  // output tiles of one M x N product
// Whether the router weight gradient's split products add their hi and lo
// halves before storing ([nsplit, H, E] partials instead of [nsplit, H, 2E]).
bool dw_router_folds(int E);
size_t ffn_sched_bytes(int R_cap, int E_l);
// The weight gradients' split plans and partial slots (FFN backward workspace).
size_t ffn_wgrad_split_bytes(int E_l, int H, int I);
// x_rows null: x_perm holds the grouped rows; else x_perm is the token matrix
// x [T, H] and grouped row r is its row x_rows[r] (the permutation's src_row)
hipError_t launch_ffn_fwd_bf16(const bf16_t* x_perm, const int32_t* offsets, int E_l, int R_cap,
                               int H, int I, const bf16_t* w_gate, const bf16_t* w_up,
                               const bf16_t* w_down, bf16_t* gu, bf16_t* h_perm, bf16_t* y_perm,
                               void* ws, hipStream_t s, const int32_t* x_rows = nullptr, int T = 0);
// The same with the tile table in the library's static per-GPU scratch (no
// workspace argument); R_cap <= kNoAllocMaxRows.
constexpr int kNoAllocMaxRows = 1 << 20;
hipError_t launch_ffn_fwd_bf16_noalloc(const bf16_t* x_perm, const int32_t* offsets, int E_l,
                                       int R_cap, int H, int I, const bf16_t* w_gate,
                                       const bf16_t* w_up, const bf16_t* w_down, bf16_t* gu,
                                       bf16_t* h_perm, bf16_t* y_perm, hipStream_t s);
// FP8 forward (gemm.hip) and E4M3 row quantization (fp8.hip)
size_t ffn_fwd_fp8_ws_bytes(int R_cap, int E_l, int I);
hipError_t launch_ffn_fwd_fp8(const uint8_t* x_q, const float* x_scale, const int32_t* src_row,
                              const int32_t* offsets, int E_l, int R_cap, int H, int I,
                              const uint8_t* wg_q, const float* wg_s, const uint8_t* wu_q,
                              const float* wu_s, const uint8_t* wd_q, const float* wd_s,
                              bf16_t* gu, bf16_t* h_perm, bf16_t* y_perm, void* ws, hipStream_t s,
                              int gather_T = -1);  // >= 0: x_q holds the T token rows, read through src_row
hipError_t launch_quantize_fp8(const void* src, int rows, int cols, bool bf16,
                               const int32_t* nrows, uint8_t* q, float* scale, hipStream_t s);
// per-input-channel (transposed) weight codes and the SiLU derivative + row
// quantization of the FP8 data gradients (fp8.hip)
hipError_t launch_quantize_t_fp8(const bf16_t* src0, const bf16_t* src1, int batch, int N, int K,
                                 uint8_t* q, float* scale, hipStream_t s);
hipError_t launch_swiglu_bwd_fp8(const bf16_t* dh, const bf16_t* gu, int rows, int I,
                                 const int32_t* nrows, bf16_t* dgu, uint8_t* q, float* scale,
                                 hipStream_t s);
size_t ffn_dgrad_fp8_ws_bytes(int R_cap, int E_l, int I);
hipError_t launch_ffn_dgrad_fp8(const uint8_t* dy_q, const float* dy_scale, const bf16_t* gu,
                                const int32_t* offsets, int E_l, int R_cap, int H, int I,
                                const uint8_t* wdt_q, const float* wdt_s, const uint8_t* wgut_q,
                                const float* wgut_s, bf16_t* dgu, bf16_t* dx_perm, void* ws,
                                hipStream_t s);
// FP8 weight gradients: columns of grouped rows quantized per (group, column)
// into transposed code rows, each group at a padded offset (fp8.hip), and the
// two K-grouped products on them (gemm.hip).
struct QuantGroupTensor {
  const bf16_t* src;     // [rows][ld] bf16
  const int32_t* rows;   // logical row r reads src row rows[r] (null: row r)
  long ld;
  int C;                 // columns (multiple of 64)
  uint8_t* q;            // [C][Kp] codes
  float* scale;          // [groups][C]
};
constexpr int kQuantGroupTensors = 4;
struct QuantGroupT {
  QuantGroupTensor t[kQuantGroupTensors];
  int nt;
  const int32_t* offsets;  // [groups + 1] row offsets (device)
  int E_l;
  int max_rows;            // bound on offsets[E_l] (sizes the grid)
  int Kp;                  // code row pitch
  int32_t* poff;           // out: [groups + 1] padded offsets (multiples of 64)
  int32_t* ctrs;           // counters zeroed for the products that follow, or null
  int nctrs;
};
hipError_t launch_quantize_group_t_fp8(const QuantGroupT& q, hipStream_t s);
// both code layouts of expert weights (rows; per input channel, transposed)
size_t quantize_w_fp8_ws_bytes(int batch, int N, int K, int nsrc);
hipError_t launch_quantize_w_fp8(const bf16_t* w0, const bf16_t* w1, int batch, int N, int K,
                                 uint8_t* q0, float* s0, uint8_t* q1, float* s1, uint8_t* qt,
                                 float* st, void* ws, hipStream_t s);
int wgrad_fp8_pitch(int R_cap, int E_l);
size_t ffn_wgrad_fp8_ws_bytes(int R_cap, int E_l, int H, int I);
hipError_t launch_ffn_wgrad_fp8(const bf16_t* x, const int32_t* src_row, const bf16_t* dgu,
                                const bf16_t* h_perm, const bf16_t* dy_perm,
                                const int32_t* offsets, int E_l, int R_cap, int H, int I,
                                float* dw_gate, float* dw_up, float* dw_down, bool accumulate,
                                void* ws, hipStream_t s);
hipError_t launch_ffn_wgrad_fp8_begin(const bf16_t* x, const int32_t* src_row,
                                      const bf16_t* h_perm, const bf16_t* dy_perm,
                                      const int32_t* offsets, int E_l, int R_cap, int H, int I,
                                      float* dw_down, bool accumulate, void* ws, hipStream_t s);
hipError_t launch_ffn_wgrad_fp8_end(const bf16_t* dgu, const int32_t* offsets, int E_l, int R_cap,
                                    int H, int I, float* dw_gate, float* dw_up, float* dw_down,
                                    bool accumulate, void* ws, hipStream_t s);
hipError_t order_after(hipStream_t s, hipStream_t waiter);
hipError_t launch_ffn_bwd_bf16(const bf16_t* dy_perm, const bf16_t* x_perm, const bf16_t* gu,
                               const bf16_t* h_perm, const int32_t* offsets, int E_l, int R_cap,
                               int H, int I, const bf16_t* w_gate, const bf16_t* w_up,
                               const bf16_t* w_down, bf16_t* dx_perm, float* dw_gate,
                               float* dw_up, float* dw_down, bool accumulate, void* ws,
                               hipStream_t s,
                               hipStream_t wgrad_stream = nullptr);
// X^T . [dz_hi | dz_lo] split over token chunks: partials [nsplit][H][2E] fp32.
hipError_t launch_dw_router_bf16(const bf16_t* x, const bf16_t* dz_hilo, int T, int H, int E,
                                 int nsplit, int32_t* split_offsets, float* partials,
                                 hipStream_t s);
// dx_router [T][H] fp32 = [dz_hi | dz_lo] . [W_r | W_r]^T on the matrix cores
// (dz_hilo [T][2E], W_r [H][E] bf16); needs router_dx_mfma_ok(H, E).
bool router_dx_mfma_ok(int H, int E);
hipError_t launch_router_dx(const bf16_t* dz_hilo, const bf16_t* w_router, int T, int H, int E,
                            float* dx_router, hipStream_t s);

// gemm_f32.hip (plain fp32 kernels for the fp32 path)
hipError_t launch_ffn_fwd_f32(const float* x_perm, const int32_t* offsets, int E_l, int R_cap,
                              int H, int I, const float* w_gate, const float* w_up,
                              const float* w_down, float* gu, float* h_perm, float* y_perm,
                              hipStream_t s);
hipError_t launch_ffn_bwd_f32(const float* dy_perm, const float* x_perm, const float* gu,
                              const float* h_perm, const int32_t* offsets, int E_l, int R_cap,
                              int H, int I, const float* w_gate, const float* w_up,
                              const float* w_down, float* dx_perm, float* dw_gate, float* dw_up,
                              float* dw_down, bool accumulate, float* dgu_ws, hipStream_t s);

}  // namespace moe
