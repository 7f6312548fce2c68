// C ABI of the gfx950 MoE expert layer: argument validation (host only, before
// any HIP call), workspace layout and dispatch to the kernels.  Declarations
// and the contract of every entry point are in include/moe.h.
#include "../../include/moe.h"

#include <stdarg.h>
#include <stdio.h>

#include <algorithm>

#include "common.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

// Entry points launch only after their arguments validated.  The launchers
// report hipGetLastError(), which is sticky per thread: clear an error left
// by some earlier, unrelated HIP call first, so that only this call's own
// launch errors are reported.
hipStream_t begin_launch(void* stream) {
  (void)hipGetLastError();
  return (hipStream_t)stream;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline int elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : dtype == MOE_FP8 ? 1 : 4; }

int check_dtype(int dtype, const char* fn) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return fail(MOE_EINVAL, "%s: unknown dtype %d", fn, dtype);
  return MOE_OK;
}

int check_row_width(int H, int dtype, const char* fn) {
  if (H <= 0) return fail(MOE_EINVAL, "%s: H must be positive (got %d)", fn, H);
  const int q = dtype == MOE_BF16 ? 8 : dtype == MOE_FP8 ? 16 : 4;
  if (H % q != 0) return fail(MOE_EINVAL, "%s: H=%d must be a multiple of %d for this dtype", fn, H, q);
  return MOE_OK;
}

int check_routing_shape(int T, int E, int k, const char* fn) {
  if (T < 0) return fail(MOE_EINVAL, "%s: T must be >= 0 (got %d)", fn, T);
  if (E < 1 || E > kMaxE) return fail(MOE_EINVAL, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (k < 1 || k > E || k > kMaxK)
    return fail(MOE_EINVAL, "%s: k=%d outside [1, min(E=%d, %d)]", fn, k, E, kMaxK);
  if ((long long)T * k > 0x7fffffffLL) return fail(MOE_EINVAL, "%s: T*k overflows int32", fn);
  return MOE_OK;
}

int check_ptr(const void* p, const char* name, const char* fn, bool need16 = false) {
  if (p == nullptr) return fail(MOE_EINVAL, "%s: %s must not be NULL", fn, name);
  if (need16 && !aligned16(p)) return fail(MOE_EINVAL, "%s: %s must be 16-byte aligned", fn, name);
  return MOE_OK;
}

int check_ws(const void* ws, size_t have, size_t need, const char* fn) {
  if (need == 0) return MOE_OK;
  if (ws == nullptr || have < need)
    return fail(MOE_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                ws == nullptr ? (size_t)0 : have);
  if (((uintptr_t)ws & 255u) != 0) return fail(MOE_EINVAL, "%s: ws must be 256-byte aligned", fn);
  return MOE_OK;
}

// K splits of the router weight gradient x^T . dz: enough workgroups for one
// per CU, each split at least 256 token rows, at most 32 (every split writes an
// fp32 partial that a second pass sums).
int route_bwd_splits(int T, int H, int E) {
  const int tiles = gemm_tiles(H, 2 * E);
  const int want = (kCUs + tiles - 1) / tiles;
  return std::max(1, std::min(std::min(32, want), (T + 255) / 256));
}

size_t ws_route(int T, int H, int E, int dtype) {
  return dtype == MOE_BF16 ? align256(route_ws_bytes(T, H, E)) : 0;
}
size_t ws_ffn_fwd(int R_cap, int E_l, int dtype) {
  return dtype == MOE_BF16 ? ffn_sched_bytes(R_cap, E_l) : 0;
}
size_t ws_ffn_bwd(int R_cap, int E_l, int H, int I, int dtype) {
  if (dtype == MOE_BF16)
    return ffn_sched_bytes(R_cap, E_l) + align256((size_t)R_cap * 2 * I * 2) + ffn_wgrad_split_bytes(E_l, H, I);
  return align256((size_t)R_cap * 2 * I * 4);
}
size_t ws_route_bwd(int T, int H, int E, int dtype) {
  const size_t wt = align256((size_t)E * H * elem_bytes(dtype));
  if (dtype != MOE_BF16) return wt;
  return wt + align256((size_t)T * 2 * E * 2) +
         align256((size_t)route_bwd_splits(T, H, E) * H * (dw_router_folds(E) ? 1 : 2) * E *
                  sizeof(float));
}

// The MFMA kernels address their operands through buffer descriptors with
// 32-bit byte ranges, and move the DMA of K steps past the end to offset 2^31
// (where the hardware drops it): every range they read or write must stay
// below 2 GiB.
constexpr int64_t kMaxRangeBytes = (int64_t)1 << 31;

int check_range(int64_t bytes, const char* what, const char* fn) {
  if (bytes >= kMaxRangeBytes)
    return fail(MOE_EUNSUPPORTED, "%s: %s spans %lld bytes; the MFMA kernels need every operand "
                "below 2 GiB", fn, what, (long long)bytes);
  return MOE_OK;
}

int check_ffn_shape(int E_l, int R_cap, int H, int I, int dtype, const char* fn) {
  if (E_l < 1 || E_l > kMaxE) return fail(MOE_EINVAL, "%s: E_l=%d outside [1, %d]", fn, E_l, kMaxE);
  if (R_cap < 0) return fail(MOE_EINVAL, "%s: R_cap must be >= 0", fn);
  if (I <= 0) return fail(MOE_EINVAL, "%s: I must be positive", fn);
  if (int rc = check_row_width(H, dtype, fn)) return rc;
  if (dtype == MOE_BF16 && (H % 64 != 0 || I % 64 != 0))
    return fail(MOE_EUNSUPPORTED, "%s: bf16 expert GEMMs need H %% 64 == 0 and I %% 64 == 0 (H=%d, I=%d)",
                fn, H, I);
  if (dtype != MOE_F32) {  // the fp32 kernels index with 64-bit offsets
    const int64_t eb = elem_bytes(dtype);
    if (int rc = check_range((int64_t)R_cap * std::max(H, 2 * I) * eb, "a grouped-row buffer", fn)) return rc;
    if (int rc = check_range((int64_t)2 * I * H * eb, "one expert's gate and up weights", fn)) return rc;
  }
  return MOE_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// kernel timing hook
// ---------------------------------------------------------------------------
// Per calling thread: only launches made by the thread that armed the hook
// are recorded.
namespace {
thread_local int g_prof_id = -1;
thread_local void** g_prof_start = nullptr;
thread_local void** g_prof_stop = nullptr;
thread_local int g_prof_n = 0;
thread_local int g_prof_next = 0;
}  // namespace

namespace moe {
ProfScope::ProfScope(int kernel_id, hipStream_t s) : slot(-1), stream(s) {
  if (kernel_id == g_prof_id && g_prof_next < g_prof_n) {
    slot = g_prof_next++;
    (void)hipEventRecord((hipEvent_t)g_prof_start[slot], s);
  }
}
ProfScope::~ProfScope() {
  if (slot >= 0) (void)hipEventRecord((hipEvent_t)g_prof_stop[slot], stream);
}
}  // namespace moe

extern "C" {

int moe_profile_kernel(int kernel_id, void** start_events, void** stop_events, int n) {
  if (kernel_id >= MOE_KERNEL_COUNT) return fail(MOE_EINVAL, "moe_profile_kernel: unknown kernel %d", kernel_id);
  if (kernel_id >= 0 && (n < 0 || (n > 0 && (start_events == nullptr || stop_events == nullptr))))
    return fail(MOE_EINVAL, "moe_profile_kernel: need n >= 0 and event arrays");
  g_prof_id = kernel_id < 0 ? -1 : kernel_id;
  g_prof_start = start_events;
  g_prof_stop = stop_events;
  g_prof_n = kernel_id < 0 ? 0 : n;
  g_prof_next = 0;
  return MOE_OK;
}

int moe_profile_recorded(void) { return g_prof_next; }


int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err; }

int64_t moe_workspace_bytes(int op, int T, int H, int I, int E, int k, int e_lo, int e_hi,
                            int dtype) {
  const char* fn = "moe_workspace_bytes";
  if (dtype == MOE_FP8) {
    if (op != MOE_OP_PERMUTE && op != MOE_OP_FFN_FWD_FP8 && op != MOE_OP_FFN_DGRAD_FP8 &&
        op != MOE_OP_FFN_WGRAD_FP8 && op != MOE_OP_QUANTIZE_W_FP8)
      return fail(MOE_EINVAL, "%s: MOE_FP8 applies to MOE_OP_PERMUTE and the FP8 FFN ops only", fn);
  } else if (int rc = check_dtype(dtype, fn)) {
    return rc;
  }
  if (int rc = check_routing_shape(T, E, k, fn)) return rc;
  if (int rc = check_row_width(H, dtype, fn)) return rc;
  const int R_cap = T * k;
  switch (op) {
    case MOE_OP_ROUTE:
      return (int64_t)ws_route(T, H, E, dtype);
    case MOE_OP_ROUTE_BWD:
      return (int64_t)ws_route_bwd(T, H, E, dtype);
    case MOE_OP_COMBINE_DX:
      return (int64_t)align256((size_t)E * H * elem_bytes(dtype));
    case MOE_OP_QUANTIZE_W_FP8: {
      if (e_lo < 0 || e_hi > E || e_lo >= e_hi)
        return fail(MOE_EINVAL, "%s: need 0 <= e_lo < e_hi <= E", fn);
      if (I <= 0 || I % 128 != 0 || H % 128 != 0)
        return fail(MOE_EINVAL, "%s: need I > 0 and H, I multiples of 128", fn);
      return (int64_t)quantize_w_fp8_ws_bytes(e_hi - e_lo, I, H, 2);
    }
    case MOE_OP_FFN_FWD_FP8:
    case MOE_OP_FFN_DGRAD_FP8:
    case MOE_OP_FFN_WGRAD_FP8: {
      if (e_lo < 0 || e_hi > E || e_lo >= e_hi)
        return fail(MOE_EINVAL, "%s: need 0 <= e_lo < e_hi <= E", fn);
      if (I <= 0) return fail(MOE_EINVAL, "%s: I must be positive", fn);
      const int E_l = e_hi - e_lo;
      if (op == MOE_OP_FFN_WGRAD_FP8) return (int64_t)ffn_wgrad_fp8_ws_bytes(R_cap, E_l, H, I);
      return (int64_t)(op == MOE_OP_FFN_FWD_FP8 ? ffn_fwd_fp8_ws_bytes(R_cap, E_l, I)
                                                : ffn_dgrad_fp8_ws_bytes(R_cap, E_l, I));
    }
    case MOE_OP_PERMUTE:
    case MOE_OP_FFN_FWD:
    case MOE_OP_FFN_BWD: {
      if (e_lo < 0 || e_hi > E || e_lo >= e_hi)
        return fail(MOE_EINVAL, "%s: need 0 <= e_lo < e_hi <= E", fn);
      const int E_l = e_hi - e_lo;
      if (op == MOE_OP_PERMUTE) return (int64_t)permute_ws_bytes(T, k, E_l);
      if (I <= 0) return fail(MOE_EINVAL, "%s: I must be positive", fn);
      if (op == MOE_OP_FFN_FWD) return (int64_t)ws_ffn_fwd(R_cap, E_l, dtype);
      return (int64_t)ws_ffn_bwd(R_cap, E_l, H, I, dtype);
    }
    default:
      return fail(MOE_EINVAL, "%s: unknown op %d", fn, op);
  }
}

int moe_route(const void* x, const void* w_router, const float* bias, int T, int H, int E, int k,
              int dtype, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
              size_t ws_bytes, void* stream) {
  const char* fn = "moe_route";
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (int rc = check_routing_shape(T, E, k, fn)) return rc;
  if (int rc = check_row_width(H, dtype, fn)) return rc;
  if (dtype == MOE_BF16 && H % 64 != 0)
    return fail(MOE_EUNSUPPORTED, "%s: the bf16 router needs H %% 64 == 0 (H=%d)", fn, H);
  if (int rc = check_ptr(x, "x", fn, true)) return rc;
  if (int rc = check_ptr(w_router, "w_router", fn, true)) return rc;
  if (int rc = check_ptr(topk_idx, "topk_idx", fn)) return rc;
  if (int rc = check_ptr(topk_w, "topk_w", fn)) return rc;
  if (int rc = check_ws(ws, ws_bytes, ws_route(T, H, E, dtype), fn)) return rc;
  if (T == 0) return MOE_OK;
  hipStream_t s = begin_launch(stream);
  hipError_t e;
  if (dtype == MOE_BF16)
    e = launch_route_bf16((const bf16_t*)x, (const bf16_t*)w_router, bias, T, H, E, k, logits,
                          topk_idx, topk_w, (float*)ws, s);
  else
    e = launch_route_f32((const float*)x, (const float*)w_router, bias, T, H, E, k, logits,
                         topk_idx, topk_w, s);
  return hip_status(e, fn);
}

int moe_route_from_logits(const float* logits, int T, int E, int k, int32_t* topk_idx,
                          float* topk_w, void* stream) {
  const char* fn = "moe_route_from_logits";
  if (int rc = check_routing_shape(T, E, k, fn)) return rc;
  if (int rc = check_ptr(logits, "logits", fn)) return rc;
  if (int rc = check_ptr(topk_idx, "topk_idx", fn)) return rc;
  if (int rc = check_ptr(topk_w, "topk_w", fn)) return rc;
  if (T == 0) return MOE_OK;
  return hip_status(launch_route_from_logits(logits, T, E, k, topk_idx, topk_w, begin_launch(stream)),
                    fn);
}

int moe_permute(const void* x, const int32_t* topk_idx, int T, int H, int E, int k, int e_lo,
                int e_hi, int dtype, int32_t* counts, int32_t* offsets, int32_t* dest_row,
                int32_t* src_row, void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_permute";
  if (dtype != MOE_FP8)
    if (int rc = check_dtype(dtype, fn)) return rc;
  if (int rc = check_routing_shape(T, E, k, fn)) return rc;
  if (int rc = check_row_width(H, dtype, fn)) return rc;
  if (e_lo < 0 || e_hi > E || e_lo >= e_hi)
    return fail(MOE_EINVAL, "%s: need 0 <= e_lo < e_hi <= E (got %d, %d, E=%d)", fn, e_lo, e_hi, E);
  if (int rc = check_ptr(counts, "counts", fn)) return rc;
  if (int rc = check_ptr(offsets, "offsets", fn)) return rc;
  if (T > 0) {
    if (int rc = check_ptr(topk_idx, "topk_idx", fn)) return rc;
    if (int rc = check_ptr(dest_row, "dest_row", fn)) return rc;
    if (int rc = check_ptr(src_row, "src_row", fn)) return rc;
    if (x_perm != nullptr) {  // NULL: the maps alone
      if (int rc = check_ptr(x, "x", fn, true)) return rc;
      if (int rc = check_ptr(x_perm, "x_perm", fn, true)) return rc;
    }
  }
  const int E_l = e_hi - e_lo;
  if (int rc = check_ws(ws, ws_bytes, permute_ws_bytes(T, k, E_l), fn)) return rc;
  return hip_status(launch_permute(x, topk_idx, T, H, k, e_lo, e_hi, elem_bytes(dtype), counts,
                                   offsets, dest_row, src_row, x_perm, ws, begin_launch(stream)),
                    fn);
}

int moe_grouped_ffn_fwd(const void* x_perm, const int32_t* offsets, int E_l, int R_cap, int H,
                        int I, const void* w_gate, const void* w_up, const void* w_down, int dtype,
                        void* gu_saved, void* h_perm, void* y_perm, void* ws, size_t ws_bytes,
                        void* stream) {
  const char* fn = "moe_grouped_ffn_fwd";
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (int rc = check_ffn_shape(E_l, R_cap, H, I, dtype, fn)) return rc;
  if (int rc = check_ptr(offsets, "offsets", fn)) return rc;
  if (int rc = check_ptr(w_gate, "w_gate", fn, true)) return rc;
  if (int rc = check_ptr(w_up, "w_up", fn, true)) return rc;
  if (int rc = check_ptr(w_down, "w_down", fn, true)) return rc;
  if (R_cap > 0) {
    if (int rc = check_ptr(x_perm, "x_perm", fn, true)) return rc;
    if (int rc = check_ptr(h_perm, "h_perm", fn, true)) return rc;
    if (int rc = check_ptr(y_perm, "y_perm", fn, true)) return rc;
  }
  if (int rc = check_ws(ws, ws_bytes, ws_ffn_fwd(R_cap, E_l, dtype), fn)) return rc;
  if (R_cap == 0) return MOE_OK;
  hipStream_t s = begin_launch(stream);
  hipError_t e;
  if (dtype == MOE_BF16)
    e = launch_ffn_fwd_bf16((const bf16_t*)x_perm, offsets, E_l, R_cap, H, I,
                            (const bf16_t*)w_gate, (const bf16_t*)w_up, (const bf16_t*)w_down,
                            (bf16_t*)gu_saved, (bf16_t*)h_perm, (bf16_t*)y_perm, ws, s);
  else
    e = launch_ffn_fwd_f32((const float*)x_perm, offsets, E_l, R_cap, H, I, (const float*)w_gate,
                           (const float*)w_up, (const float*)w_down, (float*)gu_saved,
                           (float*)h_perm, (float*)y_perm, s);
  return hip_status(e, fn);
}

int moe_grouped_ffn_fwd_gather(const void* x, const int32_t* src_row, const int32_t* offsets,
                               int E_l, int R_cap, int T, int H, int I, const void* w_gate,
                               const void* w_up, const void* w_down, int dtype, void* gu_saved,
                               void* h_perm, void* y_perm, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_grouped_ffn_fwd_gather";
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "%s: bf16 only", fn);
  if (int rc = check_ffn_shape(E_l, R_cap, H, I, dtype, fn)) return rc;
  if (T < 0) return fail(MOE_EINVAL, "%s: T must be >= 0 (got %d)", fn, T);
  if (int rc = check_range((int64_t)T * H * 2, "x", fn)) return rc;
  if (int rc = check_ptr(offsets, "offsets", fn)) return rc;
  if (int rc = check_ptr(w_gate, "w_gate", fn, true)) return rc;
  if (int rc = check_ptr(w_up, "w_up", fn, true)) return rc;
  if (int rc = check_ptr(w_down, "w_down", fn, true)) return rc;
  if (R_cap > 0) {
    if (int rc = check_ptr(x, "x", fn, true)) return rc;
    if (int rc = check_ptr(src_row, "src_row", fn)) return rc;
    if (int rc = check_ptr(h_perm, "h_perm", fn, true)) return rc;
    if (int rc = check_ptr(y_perm, "y_perm", fn, true)) return rc;
  }
  if (int rc = check_ws(ws, ws_bytes, ws_ffn_fwd(R_cap, E_l, dtype), fn)) return rc;
  if (R_cap == 0) return MOE_OK;
  return hip_status(launch_ffn_fwd_bf16((const bf16_t*)x, offsets, E_l, R_cap, H, I,
                                        (const bf16_t*)w_gate, (const bf16_t*)w_up,
                                        (const bf16_t*)w_down, (bf16_t*)gu_saved, (bf16_t*)h_perm,
                                        (bf16_t*)y_perm, ws, begin_launch(stream), src_row, T),
                    fn);
}

int moe_grouped_ffn_fwd_noalloc(const void* x_perm, const int32_t* offsets, int E_l, int R_cap,
                                int H, int I, const void* w_gate, const void* w_up,
                                const void* w_down, int dtype, void* gu_saved, void* h_perm,
                                void* y_perm, void* stream) {
  const char* fn = "moe_grouped_ffn_fwd_noalloc";
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (int rc = check_ffn_shape(E_l, R_cap, H, I, dtype, fn)) return rc;
  if (R_cap > kNoAllocMaxRows)
    return fail(MOE_EUNSUPPORTED, "%s: R_cap=%d exceeds the %d rows the library's static scratch "
                "holds a tile table for; use moe_grouped_ffn_fwd with a workspace", fn, R_cap,
                kNoAllocMaxRows);
  if (int rc = check_ptr(offsets, "offsets", fn)) return rc;
  if (int rc = check_ptr(w_gate, "w_gate", fn, true)) return rc;
  if (int rc = check_ptr(w_up, "w_up", fn, true)) return rc;
  if (int rc = check_ptr(w_down, "w_down", fn, true)) return rc;
  if (R_cap > 0) {
    if (int rc = check_ptr(x_perm, "x_perm", fn, true)) return rc;
    if (int rc = check_ptr(h_perm, "h_perm", fn, true)) return rc;
    if (int rc = check_ptr(y_perm, "y_perm", fn, true)) return rc;
  }
  if (gu_saved != nullptr && !aligned16(gu_saved))
    return fail(MOE_EINVAL, "%s: gu_saved must be 16-byte aligned", fn);
  if (R_cap == 0) return MOE_OK;
  hipStream_t s = begin_launch(stream);
  hipError_t e;
  if (dtype == MOE_BF16)
    e = launch_ffn_fwd_bf16_noalloc((const bf16_t*)x_perm, offsets, E_l, R_cap, H, I,
                                    (const bf16_t*)w_gate, (const bf16_t*)w_up,
                                    (const bf16_t*)w_down, (bf16_t*)gu_saved, (bf16_t*)h_perm,
                                    (bf16_t*)y_perm, s);
  else  // the fp32 kernels use no scratch
    e = launch_ffn_fwd_f32((const float*)x_perm, offsets, E_l, R_cap, H, I, (const float*)w_gate,
                           (const float*)w_up, (const float*)w_down, (float*)gu_saved,
                           (float*)h_perm, (float*)y_perm, s);
  return hip_status(e, fn);
}

int moe_quantize_fp8(const void* src, int rows, int cols, int dtype, const int32_t* nrows,
                     uint8_t* q, float* scale, void* stream) {
  const char* fn = "moe_quantize_fp8";
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (rows < 0) return fail(MOE_EINVAL, "%s: rows must be >= 0", fn);
  if (cols <= 0 || cols % 16 != 0) return fail(MOE_EINVAL, "%s: cols=%d must be a positive multiple of 16", fn, cols);
  if (rows == 0) return MOE_OK;
  if (int rc = check_ptr(src, "src", fn, true)) return rc;
  if (int rc = check_ptr(q, "q", fn, true)) return rc;
  if (int rc = check_ptr(scale, "scale", fn)) return rc;
  return hip_status(launch_quantize_fp8(src, rows, cols, dtype == MOE_BF16, nrows, q, scale,
                                        begin_launch(stream)),
                    fn);
}

int moe_grouped_ffn_fwd_fp8(const uint8_t* x_q, const float* x_scale, const int32_t* src_row,
                            const int32_t* offsets, int E_l, int R_cap, int H, int I,
                            const uint8_t* wg_q, const float* wg_scale, const uint8_t* wu_q,
                            const float* wu_scale, const uint8_t* wd_q, const float* wd_scale,
                            void* gu_saved, void* h_perm, void* y_perm, void* ws, size_t ws_bytes,
                            void* stream) {
  const char* fn = "moe_grouped_ffn_fwd_fp8";
  if (int rc = check_ffn_shape(E_l, R_cap, H, I, MOE_FP8, fn)) return rc;
  if (H % 128 != 0 || I % 128 != 0)
    return fail(MOE_EUNSUPPORTED, "%s: needs H %% 128 == 0 and I %% 128 == 0 (H=%d, I=%d)", fn, H, I);
  if (int rc = check_ptr(offsets, "offsets", fn)) return rc;
  if (int rc = check_ptr(wg_q, "wg_q", fn, true)) return rc;
  if (int rc = check_ptr(wu_q, "wu_q", fn, true)) return rc;
  if (int rc = check_ptr(wd_q, "wd_q", fn, true)) return rc;
  if (int rc = check_ptr(wg_scale, "wg_scale", fn, true)) return rc;
  if (int rc = check_ptr(wu_scale, "wu_scale", fn, true)) return rc;
  if (int rc = check_ptr(wd_scale, "wd_scale", fn, true)) return rc;
  if (R_cap > 0) {
    if (int rc = check_ptr(x_q, "x_q", fn, true)) return rc;
    if (int rc = check_ptr(x_scale, "x_scale", fn)) return rc;
    if (int rc = check_ptr(src_row, "src_row", fn)) return rc;
    if (int rc = check_ptr(h_perm, "h_perm", fn, true)) return rc;
    if (int rc = check_ptr(y_perm, "y_perm", fn, true)) return rc;
  }
  if (gu_saved != nullptr && !aligned16(gu_saved)) return fail(MOE_EINVAL, "%s: gu_saved must be 16-byte aligned", fn);
  if (int rc = check_ws(ws, ws_bytes, ffn_fwd_fp8_ws_bytes(R_cap, E_l, I), fn)) return rc;
  if (R_cap == 0) return MOE_OK;
  return hip_status(launch_ffn_fwd_fp8(x_q, x_scale, src_row, offsets, E_l, R_cap, H, I, wg_q,
                                       wg_scale, wu_q, wu_scale, wd_q, wd_scale, (bf16_t*)gu_saved,
                                       (bf16_t*)h_perm, (bf16_t*)y_perm, ws, begin_launch(stream)),
                    fn);
}

int moe_grouped_ffn_fwd_fp8_gather(const uint8_t* x_q, const float* x_scale, const int32_t* src_row,
                                   const int32_t* offsets, int E_l, int R_cap, int T, int H, int I,
                                   const uint8_t* wg_q, const float* wg_scale, const uint8_t* wu_q,
                                   const float* wu_scale, const uint8_t* wd_q, const float* wd_scale,
                                   void* gu_saved, void* h_perm, void* y_perm, void* ws,
                                   size_t ws_bytes, void* stream) {
  const char* fn = "moe_grouped_ffn_fwd_fp8_gather";
  if (int rc = check_ffn_shape(E_l, R_cap, H, I, MOE_FP8, fn)) return rc;
  if (H % 128 != 0 || I % 128 != 0)
    return fail(MOE_EUNSUPPORTED, "%s: needs H %% 128 == 0 and I %% 128 == 0 (H=%d, I=%d)", fn, H, I);
  if (T < 0) return fail(MOE_EINVAL, "%s: T must be >= 0 (got %d)", fn, T);
  if (int rc = check_range((int64_t)T * H, "x_q", fn)) return rc;
  if (int rc = check_ptr(offsets, "offsets", fn)) return rc;
  if (int rc = check_ptr(wg_q, "wg_q", fn, true)) return rc;
  if (int rc = check_ptr(wu_q, "wu_q", fn, true)) return rc;
  if (int rc = check_ptr(wd_q, "wd_q", fn, true)) return rc;
  if (int rc = check_ptr(wg_scale, "wg_scale", fn, true)) return rc;
  if (int rc = check_ptr(wu_scale, "wu_scale", fn, true)) return rc;
  if (int rc = check_ptr(wd_scale, "wd_scale", fn, true)) return rc;
  if (R_cap > 0) {
    if (int rc = check_ptr(x_q, "x_q", fn, true)) return rc;
    if (int rc = check_ptr(x_scale, "x_scale", fn)) return rc;
    if (int rc = check_ptr(src_row, "src_row", fn)) return rc;
    if (int rc = check_ptr(h_perm, "h_perm", fn, true)) return rc;
    if (int rc = check_ptr(y_perm, "y_perm", fn, true)) return rc;
  }
  if (gu_saved != nullptr && !aligned16(gu_saved)) return fail(MOE_EINVAL, "%s: gu_saved must be 16-byte aligned", fn);
  if (int rc = check_ws(ws, ws_bytes, ffn_fwd_fp8_ws_bytes(R_cap, E_l, I), fn)) return rc;
  if (R_cap == 0) return MOE_OK;
  return hip_status(launch_ffn_fwd_fp8(x_q, x_scale, src_row, offsets, E_l, R_cap, H, I, wg_q,
                                       wg_scale, wu_q, wu_scale, wd_q, wd_scale, (bf16_t*)gu_saved,
                                       (bf16_t*)h_perm, (bf16_t*)y_perm, ws, begin_launch(stream), T),
                    fn);
}

int moe_quantize_fp8_t(const void* src0, const void* src1, int batch, int N, int K, int dtype,
                       uint8_t* q, float* scale, void* stream) {
  const char* fn = "moe_quantize_fp8_t";
  if (dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "%s: needs MOE_BF16 weights", fn);
  if (batch < 0 || N <= 0 || K <= 0)
    return fail(MOE_EINVAL, "%s: need batch >= 0, N > 0, K > 0 (batch=%d, N=%d, K=%d)", fn, batch, N, K);
  if (N % 64 != 0 || K % 64 != 0)
    return fail(MOE_EUNSUPPORTED, "%s: needs N %% 64 == 0 and K %% 64 == 0 (N=%d, K=%d)", fn, N, K);
  if (batch == 0) return MOE_OK;
  if (int rc = check_ptr(src0, "src0", fn, true)) return rc;
  if (src1 != nullptr && !aligned16(src1)) return fail(MOE_EINVAL, "%s: src1 must be 16-byte aligned", fn);
  if (int rc = check_ptr(q, "q", fn, true)) return rc;
  if (int rc = check_ptr(scale, "scale", fn)) return rc;
  return hip_status(launch_quantize_t_fp8((const bf16_t*)src0, (const bf16_t*)src1, batch, N, K, q,
                                          scale, begin_launch(stream)),
                    fn);
}

int moe_quantize_fp8_w(const void* w0, const void* w1, int batch, int N, int K, int dtype,
                       uint8_t* q0, float* s0, uint8_t* q1, float* s1, uint8_t* qt, float* st,
                       void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_quantize_fp8_w";
  if (dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "%s: needs MOE_BF16 weights", fn);
  if (batch < 0 || N <= 0 || K <= 0)
    return fail(MOE_EINVAL, "%s: need batch >= 0, N > 0, K > 0 (batch=%d, N=%d, K=%d)", fn, batch, N, K);
  if (N % 128 != 0 || K % 128 != 0)
    return fail(MOE_EUNSUPPORTED, "%s: needs N %% 128 == 0 and K %% 128 == 0 (N=%d, K=%d)", fn, N, K);
  if (batch == 0) return MOE_OK;
  if (int rc = check_ptr(w0, "w0", fn, true)) return rc;
  if (int rc = check_ptr(q0, "q0", fn, true)) return rc;
  if (int rc = check_ptr(s0, "s0", fn)) return rc;
  if (w1 != nullptr) {
    if (int rc = check_ptr(w1, "w1", fn, true)) return rc;
    if (int rc = check_ptr(q1, "q1", fn, true)) return rc;
    if (int rc = check_ptr(s1, "s1", fn)) return rc;
  }
  if (qt != nullptr) {
    if (!aligned16(qt)) return fail(MOE_EINVAL, "%s: qt must be 16-byte aligned", fn);
    if (int rc = check_ptr(st, "st", fn)) return rc;
  }
  if (int rc = check_ws(ws, ws_bytes, quantize_w_fp8_ws_bytes(batch, N, K, w1 != nullptr ? 2 : 1), fn))
    return rc;
  return hip_status(launch_quantize_w_fp8((const bf16_t*)w0, (const bf16_t*)w1, batch, N, K, q0, s0,
                                          q1, s1, qt, st, ws, begin_launch(stream)),
                    fn);
}

int moe_grouped_ffn_dgrad_fp8(const uint8_t* dy_q, const float* dy_scale, const void* gu_saved,
                              const int32_t* offsets, int E_l, int R_cap, int H, int I,
                              const uint8_t* wdt_q, const float* wdt_scale, const uint8_t* wgut_q,
                              const float* wgut_scale, void* dgu, void* dx_perm, void* ws,
                              size_t ws_bytes, void* stream) {
  const char* fn = "moe_grouped_ffn_dgrad_fp8";
  if (int rc = check_ffn_shape(E_l, R_cap, H, I, MOE_FP8, fn)) return rc;
  if (H % 128 != 0 || I % 128 != 0 || I > 2048)
    return fail(MOE_EUNSUPPORTED, "%s: needs H %% 128 == 0, I %% 128 == 0 and I <= 2048 (H=%d, I=%d)", fn, H, I);
  if (int rc = check_ptr(offsets, "offsets", fn)) return rc;
  if (int rc = check_ptr(wdt_q, "wdt_q", fn, true)) return rc;
  if (int rc = check_ptr(wgut_q, "wgut_q", fn, true)) return rc;
  if (int rc = check_ptr(wdt_scale, "wdt_scale", fn, true)) return rc;
  if (int rc = check_ptr(wgut_scale, "wgut_scale", fn, true)) return rc;
  if (R_cap > 0) {
    if (int rc = check_ptr(dy_q, "dy_q", fn, true)) return rc;
    if (int rc = check_ptr(dy_scale, "dy_scale", fn)) return rc;
    if (int rc = check_ptr(gu_saved, "gu_saved", fn, true)) return rc;
    if (int rc = check_ptr(dgu, "dgu", fn, true)) return rc;
    if (int rc = check_ptr(dx_perm, "dx_perm", fn, true)) return rc;
  }
  if (int rc = check_ws(ws, ws_bytes, ffn_dgrad_fp8_ws_bytes(R_cap, E_l, I), fn)) return rc;
  if (R_cap == 0) return MOE_OK;
  return hip_status(launch_ffn_dgrad_fp8(dy_q, dy_scale, (const bf16_t*)gu_saved, offsets, E_l,
                                         R_cap, H, I, wdt_q, wdt_scale, wgut_q, wgut_scale,
                                         (bf16_t*)dgu, (bf16_t*)dx_perm, ws, begin_launch(stream)),
                    fn);
}

int moe_quantize_fp8_group_t(const void* src, const int32_t* src_row, int C,
                             const int32_t* offsets, int E_l, int R_cap, uint8_t* q, int q_pitch,
                             float* scale, int32_t* poff, void* stream) {
  const char* fn = "moe_quantize_fp8_group_t";
  if (E_l < 1 || E_l > kMaxE) return fail(MOE_EINVAL, "%s: E_l=%d outside [1, %d]", fn, E_l, kMaxE);
  if (R_cap < 0) return fail(MOE_EINVAL, "%s: R_cap must be >= 0", fn);
  if (C <= 0 || C % 64 != 0) return fail(MOE_EINVAL, "%s: C=%d must be a positive multiple of 64", fn, C);
  const int64_t need = (((int64_t)R_cap + 63) & ~(int64_t)63) + 64 * (int64_t)E_l;
  if (q_pitch % 64 != 0 || q_pitch < need)
    return fail(MOE_EINVAL, "%s: q_pitch=%d must be a multiple of 64 and >= %lld", fn, q_pitch,
                (long long)need);
  if (int rc = check_ptr(offsets, "offsets", fn)) return rc;
  if (int rc = check_ptr(q, "q", fn, true)) return rc;
  if (int rc = check_ptr(scale, "scale", fn)) return rc;
  if (int rc = check_ptr(poff, "poff", fn)) return rc;
  if (R_cap > 0)
    if (int rc = check_ptr(src, "src", fn, true)) return rc;
  QuantGroupT a{};
  a.t[0] = {(const bf16_t*)src, src_row, (long)C, C, q, scale};
  a.nt = 1;
  a.offsets = offsets;
  a.E_l = E_l;
  a.max_rows = R_cap;
  a.Kp = q_pitch;
  a.poff = poff;
  return hip_status(launch_quantize_group_t_fp8(a, begin_launch(stream)), fn);
}

// the shape, workspace and pointer checks of the FP8 weight gradients
static int check_wgrad_fp8(int E_l, int R_cap, int H, int I, const int32_t* offsets,
                           const void* ws, size_t ws_bytes, const char* fn) {
  if (int rc = check_ffn_shape(E_l, R_cap, H, I, MOE_FP8, fn)) return rc;
  if (H % 128 != 0 || I % 128 != 0)
    return fail(MOE_EUNSUPPORTED, "%s: needs H %% 128 == 0 and I %% 128 == 0 (H=%d, I=%d)", fn, H, I);
  // the transposed code matrices: max(2I, H) rows of the padded pitch
  const int64_t pitch = (((int64_t)R_cap + 63) & ~(int64_t)63) + 64 * (int64_t)E_l;
  if (int rc = check_range(pitch * std::max(2 * I, H), "a transposed code matrix", fn)) return rc;
  if (int rc = check_ptr(offsets, "offsets", fn)) return rc;
  return check_ws(ws, ws_bytes, ffn_wgrad_fp8_ws_bytes(R_cap, E_l, H, I), fn);
}

int moe_grouped_ffn_wgrad_fp8_begin(const void* x, const int32_t* src_row, const void* h_perm,
                                    const void* dy_perm, const int32_t* offsets, int E_l,
                                    int R_cap, int H, int I, float* dw_down, int accumulate,
                                    void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_grouped_ffn_wgrad_fp8_begin";
  if (int rc = check_wgrad_fp8(E_l, R_cap, H, I, offsets, ws, ws_bytes, fn)) return rc;
  if (int rc = check_ptr(dw_down, "dw_down", fn, true)) return rc;
  if (R_cap > 0) {
    if (int rc = check_ptr(x, "x", fn, true)) return rc;
    if (int rc = check_ptr(h_perm, "h_perm", fn, true)) return rc;
    if (int rc = check_ptr(dy_perm, "dy_perm", fn, true)) return rc;
  }
  return hip_status(launch_ffn_wgrad_fp8_begin((const bf16_t*)x, src_row, (const bf16_t*)h_perm,
                                               (const bf16_t*)dy_perm, offsets, E_l, R_cap, H, I,
                                               dw_down, accumulate != 0, ws, begin_launch(stream)),
                    fn);
}

int moe_grouped_ffn_wgrad_fp8_end(const void* dgu, const int32_t* offsets, int E_l, int R_cap,
                                  int H, int I, float* dw_gate, float* dw_up, float* dw_down,
                                  int accumulate, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_grouped_ffn_wgrad_fp8_end";
  if (int rc = check_wgrad_fp8(E_l, R_cap, H, I, offsets, ws, ws_bytes, fn)) return rc;
  if (int rc = check_ptr(dw_gate, "dw_gate", fn, true)) return rc;
  if (int rc = check_ptr(dw_up, "dw_up", fn, true)) return rc;
  if (int rc = check_ptr(dw_down, "dw_down", fn, true)) return rc;
  if (R_cap > 0)
    if (int rc = check_ptr(dgu, "dgu", fn, true)) return rc;
  return hip_status(launch_ffn_wgrad_fp8_end((const bf16_t*)dgu, offsets, E_l, R_cap, H, I,
                                             dw_gate, dw_up, dw_down, accumulate != 0, ws,
                                             begin_launch(stream)),
                    fn);
}

int moe_grouped_ffn_wgrad_fp8(const void* x, const int32_t* src_row, const void* dgu,
                              const void* h_perm, const void* dy_perm, const int32_t* offsets,
                              int E_l, int R_cap, int H, int I, float* dw_gate, float* dw_up,
                              float* dw_down, int accumulate, void* ws, size_t ws_bytes,
                              void* stream) {
  const char* fn = "moe_grouped_ffn_wgrad_fp8";
  if (int rc = check_wgrad_fp8(E_l, R_cap, H, I, offsets, ws, ws_bytes, fn)) return rc;
  if (int rc = check_ptr(dw_gate, "dw_gate", fn, true)) return rc;
  if (int rc = check_ptr(dw_up, "dw_up", fn, true)) return rc;
  if (int rc = check_ptr(dw_down, "dw_down", fn, true)) return rc;
  if (R_cap > 0) {
    if (int rc = check_ptr(x, "x", fn, true)) return rc;
    if (int rc = check_ptr(dgu, "dgu", fn, true)) return rc;
    if (int rc = check_ptr(h_perm, "h_perm", fn, true)) return rc;
    if (int rc = check_ptr(dy_perm, "dy_perm", fn, true)) return rc;
  }
  return hip_status(launch_ffn_wgrad_fp8((const bf16_t*)x, src_row, (const bf16_t*)dgu,
                                         (const bf16_t*)h_perm, (const bf16_t*)dy_perm, offsets,
                                         E_l, R_cap, H, I, dw_gate, dw_up, dw_down,
                                         accumulate != 0, ws, begin_launch(stream)),
                    fn);
}

int moe_combine(const void* y_perm, const float* topk_w, const int32_t* dest_row,
                const float* addend, int T, int H, int k, int dtype, void* y, void* stream) {
  const char* fn = "moe_combine";
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (T < 0) return fail(MOE_EINVAL, "%s: T must be >= 0", fn);
  if (k < 1 || k > kMaxK) return fail(MOE_EINVAL, "%s: k=%d outside [1, %d]", fn, k, kMaxK);
  if (int rc = check_row_width(H, dtype, fn)) return rc;
  if (T == 0) return MOE_OK;
  if (int rc = check_ptr(y_perm, "y_perm", fn, true)) return rc;
  if (int rc = check_ptr(dest_row, "dest_row", fn)) return rc;
  if (int rc = check_ptr(y, "y", fn, true)) return rc;
  if (addend != nullptr && !aligned16(addend)) return fail(MOE_EINVAL, "%s: addend must be 16-byte aligned", fn);
  return hip_status(launch_combine(y_perm, topk_w, dest_row, addend, T, H, k, dtype == MOE_BF16, y,
                                   begin_launch(stream)),
                    fn);
}

// Argument checks shared by the two forms of the fused input gradient (the
// router weight as given, [H,E], or already transposed, [E,H]).
static int check_combine_dx(const void* dx_perm, const int32_t* dest_row, const float* d_topk_w,
                            const float* topk_w, const int32_t* topk_idx, const void* w_router,
                            const char* w_name, int T, int H, int E, int k, int dtype, void* dx,
                            const char* fn) {
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (int rc = check_routing_shape(T, E, k, fn)) return rc;
  if (int rc = check_row_width(H, dtype, fn)) return rc;
  if (T == 0) return MOE_OK;
  if (int rc = check_ptr(dx_perm, "dx_perm", fn, true)) return rc;
  if (int rc = check_ptr(dest_row, "dest_row", fn)) return rc;
  if (int rc = check_ptr(d_topk_w, "d_topk_w", fn)) return rc;
  if (int rc = check_ptr(topk_w, "topk_w", fn)) return rc;
  if (int rc = check_ptr(topk_idx, "topk_idx", fn)) return rc;
  if (int rc = check_ptr(w_router, w_name, fn, true)) return rc;
  if (int rc = check_ptr(dx, "dx", fn, true)) return rc;
  return MOE_OK;
}

int moe_combine_dx(const void* dx_perm, const int32_t* dest_row, const float* d_topk_w,
                   const float* topk_w, const int32_t* topk_idx, const void* w_router, int T,
                   int H, int E, int k, int dtype, void* dx, void* ws, size_t ws_bytes,
                   void* stream) {
  const char* fn = "moe_combine_dx";
  if (int rc = check_combine_dx(dx_perm, dest_row, d_topk_w, topk_w, topk_idx, w_router,
                                "w_router", T, H, E, k, dtype, dx, fn))
    return rc;
  if (int rc = check_ws(ws, ws_bytes, align256((size_t)E * H * elem_bytes(dtype)), fn)) return rc;
  if (T == 0) return MOE_OK;
  hipStream_t s = begin_launch(stream);
  hipError_t e = launch_transpose(w_router, ws, H, E, elem_bytes(dtype), s);
  if (e == hipSuccess)
    e = launch_combine_dx(dx_perm, dest_row, d_topk_w, topk_w, topk_idx, ws, T, H, k,
                          dtype == MOE_BF16, dx, s);
  return hip_status(e, fn);
}

int moe_combine_dx_t(const void* dx_perm, const int32_t* dest_row, const float* d_topk_w,
                     const float* topk_w, const int32_t* topk_idx, const void* w_router_t, int T,
                     int H, int E, int k, int dtype, void* dx, void* stream) {
  const char* fn = "moe_combine_dx_t";
  if (int rc = check_combine_dx(dx_perm, dest_row, d_topk_w, topk_w, topk_idx, w_router_t,
                                "w_router_t", T, H, E, k, dtype, dx, fn))
    return rc;
  if (T == 0) return MOE_OK;
  hipStream_t s = begin_launch(stream);
  return hip_status(launch_combine_dx(dx_perm, dest_row, d_topk_w, topk_w, topk_idx, w_router_t,
                                      T, H, k, dtype == MOE_BF16, dx, s),
                    fn);
}

int moe_router_weight_t(const void* w_router, int H, int E, int dtype, void* w_router_t,
                        void* stream) {
  const char* fn = "moe_router_weight_t";
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (H < 0 || H > (1 << 20) || E < 0 || E > (1 << 20))
    return fail(MOE_EINVAL, "%s: H=%d and E=%d must lie in [0, 2^20]", fn, H, E);
  if ((long long)H * E == 0) return MOE_OK;
  if (int rc = check_ptr(w_router, "w_router", fn)) return rc;
  if (int rc = check_ptr(w_router_t, "w_router_t", fn)) return rc;
  hipStream_t s = begin_launch(stream);
  return hip_status(launch_transpose(w_router, w_router_t, H, E, elem_bytes(dtype), s), fn);
}

int moe_combine_bwd(const void* dy, const void* y_perm, const float* topk_w,
                    const int32_t* dest_row, int T, int H, int k, int dtype, void* dy_perm,
                    float* d_topk_w, void* stream) {
  const char* fn = "moe_combine_bwd";
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (T < 0) return fail(MOE_EINVAL, "%s: T must be >= 0", fn);
  if (k < 1 || k > kMaxK) return fail(MOE_EINVAL, "%s: k=%d outside [1, %d]", fn, k, kMaxK);
  if (int rc = check_row_width(H, dtype, fn)) return rc;
  if (T == 0) return MOE_OK;
  if (int rc = check_ptr(dy, "dy", fn, true)) return rc;
  if (int rc = check_ptr(y_perm, "y_perm", fn, true)) return rc;
  if (int rc = check_ptr(topk_w, "topk_w", fn)) return rc;
  if (int rc = check_ptr(dest_row, "dest_row", fn)) return rc;
  if (int rc = check_ptr(dy_perm, "dy_perm", fn, true)) return rc;
  if (int rc = check_ptr(d_topk_w, "d_topk_w", fn)) return rc;
  return hip_status(launch_combine_bwd(dy, y_perm, topk_w, dest_row, T, H, k, dtype == MOE_BF16,
                                       dy_perm, d_topk_w, begin_launch(stream)),
                    fn);
}

namespace {
int ffn_bwd(const char* fn, const void* dy_perm, const void* x_perm, const void* gu_saved,
            const void* h_perm, const int32_t* offsets, int E_l, int R_cap, int H, int I,
            const void* w_gate, const void* w_up, const void* w_down, int dtype, void* dx_perm,
            float* dw_gate, float* dw_up, float* dw_down, int accumulate, void* ws,
            size_t ws_bytes, void* stream, void* wgrad_stream) {
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (int rc = check_ffn_shape(E_l, R_cap, H, I, dtype, fn)) return rc;
  if (accumulate != 0 && accumulate != 1) return fail(MOE_EINVAL, "%s: accumulate must be 0 or 1", fn);
  if (int rc = check_ptr(offsets, "offsets", fn)) return rc;
  if (int rc = check_ptr(w_gate, "w_gate", fn, true)) return rc;
  if (int rc = check_ptr(w_up, "w_up", fn, true)) return rc;
  if (int rc = check_ptr(w_down, "w_down", fn, true)) return rc;
  if (int rc = check_ptr(dw_gate, "dw_gate", fn)) return rc;
  if (int rc = check_ptr(dw_up, "dw_up", fn)) return rc;
  if (int rc = check_ptr(dw_down, "dw_down", fn)) return rc;
  if (R_cap > 0) {
    if (int rc = check_ptr(dy_perm, "dy_perm", fn, true)) return rc;
    if (int rc = check_ptr(x_perm, "x_perm", fn, true)) return rc;
    if (int rc = check_ptr(gu_saved, "gu_saved", fn, true)) return rc;
    if (int rc = check_ptr(h_perm, "h_perm", fn, true)) return rc;
    if (int rc = check_ptr(dx_perm, "dx_perm", fn, true)) return rc;
  }
  if (int rc = check_ws(ws, ws_bytes, ws_ffn_bwd(R_cap, E_l, H, I, dtype), fn)) return rc;
  hipStream_t s = begin_launch(stream);
  hipError_t e;
  if (dtype == MOE_BF16)
    e = launch_ffn_bwd_bf16((const bf16_t*)dy_perm, (const bf16_t*)x_perm,
                            (const bf16_t*)gu_saved, (const bf16_t*)h_perm, offsets, E_l, R_cap, H,
                            I, (const bf16_t*)w_gate, (const bf16_t*)w_up, (const bf16_t*)w_down,
                            (bf16_t*)dx_perm, dw_gate, dw_up, dw_down, accumulate != 0, ws, s,
                            (hipStream_t)wgrad_stream);
  else
    e = launch_ffn_bwd_f32((const float*)dy_perm, (const float*)x_perm, (const float*)gu_saved,
                           (const float*)h_perm, offsets, E_l, R_cap, H, I, (const float*)w_gate,
                           (const float*)w_up, (const float*)w_down, (float*)dx_perm, dw_gate,
                           dw_up, dw_down, accumulate != 0, (float*)ws, s);
  if (e == hipSuccess && wgrad_stream != nullptr && dtype != MOE_BF16)
    e = order_after(s, (hipStream_t)wgrad_stream);  // weight gradients in wgrad_stream's order
  return hip_status(e, fn);
}
}  // namespace

int moe_grouped_ffn_bwd(const void* dy_perm, const void* x_perm, const void* gu_saved,
                        const void* h_perm, const int32_t* offsets, int E_l, int R_cap, int H,
                        int I, const void* w_gate, const void* w_up, const void* w_down,
                        int dtype, void* dx_perm, float* dw_gate, float* dw_up, float* dw_down,
                        int accumulate, void* ws, size_t ws_bytes, void* stream) {
  return ffn_bwd("moe_grouped_ffn_bwd", dy_perm, x_perm, gu_saved, h_perm, offsets, E_l, R_cap, H,
                 I, w_gate, w_up, w_down, dtype, dx_perm, dw_gate, dw_up, dw_down, accumulate, ws,
                 ws_bytes, stream, nullptr);
}

int moe_grouped_ffn_bwd_split(const void* dy_perm, const void* x_perm, const void* gu_saved,
                              const void* h_perm, const int32_t* offsets, int E_l, int R_cap,
                              int H, int I, const void* w_gate, const void* w_up,
                              const void* w_down, int dtype, void* dx_perm, float* dw_gate,
                              float* dw_up, float* dw_down, int accumulate, void* ws,
                              size_t ws_bytes, void* stream, void* wgrad_stream) {
  if (wgrad_stream == nullptr || wgrad_stream == stream)
    return fail(MOE_EINVAL, "moe_grouped_ffn_bwd_split: wgrad_stream must be a second stream");
  return ffn_bwd("moe_grouped_ffn_bwd_split", dy_perm, x_perm, gu_saved, h_perm, offsets, E_l,
                 R_cap, H, I, w_gate, w_up, w_down, dtype, dx_perm, dw_gate, dw_up, dw_down,
                 accumulate, ws, ws_bytes, stream, wgrad_stream);
}

int moe_route_bwd(const float* d_topk_w, const float* topk_w, const int32_t* topk_idx,
                  const void* x, const void* w_router, int T, int H, int E, int k, int dtype,
                  float* d_logits, float* dx_router, float* dw_router, void* ws, size_t ws_bytes,
                  void* stream) {
  const char* fn = "moe_route_bwd";
  if (int rc = check_dtype(dtype, fn)) return rc;
  if (int rc = check_routing_shape(T, E, k, fn)) return rc;
  if (int rc = check_row_width(H, dtype, fn)) return rc;
  if (dtype == MOE_BF16 && (H % 64 != 0 || E % 4 != 0))
    return fail(MOE_EUNSUPPORTED,
                "%s: the bf16 router backward needs H %% 64 == 0 and E %% 4 == 0 (H=%d, E=%d)", fn, H, E);
  if (dtype == MOE_BF16 && dw_router != nullptr) {  // x^T . dz runs on the MFMA kernel
    if (int rc = check_range((int64_t)T * H * 2, "x", fn)) return rc;
    if (int rc = check_range((int64_t)T * 4 * E, "the split logit gradient", fn)) return rc;
  }
  if (int rc = check_ptr(w_router, "w_router", fn, true)) return rc;
  if (int rc = check_ptr(d_logits, "d_logits", fn)) return rc;
  if (dx_router != nullptr && !aligned16(dx_router))
    return fail(MOE_EINVAL, "%s: dx_router must be 16-byte aligned", fn);
  if (T > 0) {
    if (int rc = check_ptr(d_topk_w, "d_topk_w", fn)) return rc;
    if (int rc = check_ptr(topk_w, "topk_w", fn)) return rc;
    if (int rc = check_ptr(topk_idx, "topk_idx", fn)) return rc;
    if (dw_router != nullptr)
      if (int rc = check_ptr(x, "x", fn, true)) return rc;
  }
  if (int rc = check_ws(ws, ws_bytes, ws_route_bwd(T, H, E, dtype), fn)) return rc;
  hipStream_t s = begin_launch(stream);
  const bool bf16 = dtype == MOE_BF16;
  char* w = (char*)ws;
  void* wt = w;
  w += align256((size_t)E * H * elem_bytes(dtype));
  bf16_t* dz_hilo = nullptr;
  float* partials = nullptr;
  const int nsplit = route_bwd_splits(T, H, E);
  if (bf16) {
    dz_hilo = (bf16_t*)w;
    w += align256((size_t)T * 2 * E * 2);
    partials = (float*)w;
  }
  hipError_t e = hipSuccess;
  // bf16 with E % 64 == 0: dx_router as an MFMA product of the split logit
  // gradient with W_r itself (no transpose, no per-token gather)
  const bool dx_mfma = bf16 && dx_router != nullptr && router_dx_mfma_ok(H, E);
  if (T > 0 && dx_router != nullptr && !dx_mfma)
    e = launch_transpose(w_router, wt, H, E, elem_bytes(dtype), s);
  if (e == hipSuccess && T > 0)
    e = launch_route_bwd_dz(d_topk_w, topk_w, topk_idx, wt, T, H, E, k, bf16, d_logits,
                            dx_mfma ? nullptr : dx_router,
                            (bf16 && (dw_router != nullptr || dx_mfma)) ? dz_hilo : nullptr, s);
  if (e == hipSuccess && T > 0 && dx_mfma)
    e = launch_router_dx(dz_hilo, (const bf16_t*)w_router, T, H, E, dx_router, s);
  if (e == hipSuccess && dw_router != nullptr) {
    if (bf16) {
      if (T > 0) {
        e = launch_dw_router_bf16((const bf16_t*)x, dz_hilo, T, H, E, nsplit, nullptr, partials, s);
        if (e == hipSuccess)
          e = launch_dw_router_reduce(partials, nsplit, H, E, dw_router_folds(E), dw_router, s);
      } else {
        e = launch_dw_router_reduce(partials, 0, H, E, false, dw_router, s);  // writes zeros
      }
    } else {
      e = launch_dw_router_f32((const float*)x, d_logits, T, H, E, dw_router, s);
    }
  }
  return hip_status(e, fn);
}

}  // extern "C"
