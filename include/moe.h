/*
 * moe.h - C ABI of the per-GPU MoE expert layer for AMD Instinct MI355X (gfx950).
 *
 * The layer is the local part of an expert-parallel MoE block: router GEMM,
 * softmax/top-k gating, permutation of routed token rows into contiguous
 * per-expert groups, a grouped SwiGLU expert FFN and the weighted
 * unpermute/combine, plus the backward of each step.  The op split follows
 * the local expert computation named on the page "FSDPTurbo EP/EFSDP and
 * LlamaFactory FSDP2/CP Design" (section 3, dispatcher table: permute,
 * unpermute and grouped matmul between the two all-to-alls; empty experts
 * are legal).  Expert tensor shapes follow the page
 * "Qwen3-MoE-30B-A3B模型EP+FSDP2并行方案" (section "Qwen3-MoE-30B-A3B模型":
 * gate/up [E, I, H], down [E, H, I]; section "完整并行流程": one EP rank of
 * eight holds a 16-expert slice along dim 0, passed here as plain local
 * tensors).
 *
 * Conventions (all entry points)
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major,
 *     dense.  Activations and weights are bf16 (MOE_BF16) or fp32 (MOE_F32);
 *     indices are int32; gate weights, logits and weight gradients are fp32.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *     null stream).  No call synchronises, allocates device memory or passes
 *     data from one call to the next.  Scratch memory is the caller's `ws`
 *     buffer, sized by moe_workspace_bytes() and aligned to 256 bytes.  The
 *     only objects the library keeps are, per calling thread and device, the
 *     second stream and three events of moe_grouped_ffn_bwd (and the events of
 *     moe_grouped_ffn_bwd_split), created on first use and held until the
 *     process ends; calls from different host threads share none of them.
 *   - Arguments are validated on the host before any HIP call.  On error the
 *     call enqueues nothing and returns a negative moe_status; moe_last_error()
 *     returns a per-thread message.  MOE_EHIP reports a failed launch.
 *   - T = 0 is legal and enqueues nothing.
 *   - Routed-row buffers have capacity R_cap = T*k rows.  The routed row
 *     count R = offsets[E_l] stays on the device; rows >= R of capacity
 *     buffers are never written and never read for a result.
 *   - All results are deterministic: identical inputs give bitwise identical
 *     outputs (no floating-point atomics anywhere).
 *   - Shape limits: 1 <= k <= min(E, 32), E <= 256, H % 8 == 0 (bf16) or
 *     H % 4 == 0 (fp32).  The bf16 router and expert GEMMs additionally need
 *     H % 64 == 0 and I % 64 == 0 (else MOE_EUNSUPPORTED).  Pointers to
 *     row data must be 16-byte aligned.
 *   - The bf16 and FP8 matrix-core kernels address operands with 32-bit byte
 *     ranges: R_cap * max(H, 2I) * elem, 2 * I * H * elem (one expert's gate
 *     and up weights) and, for the bf16 router weight gradient, T * H * 2
 *     must each stay below 2^31 bytes (else MOE_EUNSUPPORTED).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 10

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad argument: null pointer, shape or range */
  MOE_EUNSUPPORTED = -2,  /* legal request the library does not implement */
  MOE_EWORKSPACE = -3,    /* ws_bytes smaller than moe_workspace_bytes() */
  MOE_EHIP = -4           /* a HIP launch failed; see moe_last_error() */
} moe_status;

/* MOE_FP8: one byte per value (E4M3 codes); accepted by moe_permute only. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8 = 2 } moe_dtype;

typedef enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_FFN_FWD = 2,
  MOE_OP_FFN_BWD = 3,
  MOE_OP_ROUTE_BWD = 4,
  MOE_OP_COMBINE_DX = 5,
  MOE_OP_FFN_FWD_FP8 = 6,
  MOE_OP_FFN_DGRAD_FP8 = 7,
  MOE_OP_FFN_WGRAD_FP8 = 8,
  MOE_OP_QUANTIZE_W_FP8 = 9
} moe_op;

/* Returns MOE_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  The string
 * is owned by the library and valid until the next call on this thread. */
const char* moe_last_error(void);

/* Bytes of workspace the op needs for these sizes (0 if none), or a negative
 * moe_status for invalid sizes.  I is ignored by ROUTE/PERMUTE/ROUTE_BWD;
 * e_lo/e_hi are ignored by ROUTE/ROUTE_BWD. */
int64_t moe_workspace_bytes(int op, int T, int H, int I, int E, int k, int e_lo, int e_hi,
                            int dtype);

/* Router GEMM and top-k gating.
 *   z[t,e]   = sum_h x[t,h] * w_router[h,e] (+ bias[e]), fp32 accumulation
 *   topk_idx[t,j] = the k experts with the largest z[t,:], slot j in order of
 *             (logit descending, expert id ascending): equal logits go to
 *             the lower expert id
 *   topk_w[t,j]   = softmax over all E, restricted to the k kept experts and
 *             renormalised (equal to exp(z_j - z_max) / sum over kept)
 * The pages do not state the router; this is the plain top-k-then-renormalise
 * router, selecting on logits.
 *   x        [T,H] dtype          w_router [H,E] dtype      bias [E] fp32 or NULL
 *   logits   [T,E] fp32 or NULL (written when given)
 *   topk_idx [T,k] int32          topk_w   [T,k] fp32
 *   ws       MOE_OP_ROUTE workspace: none for fp32 and for bf16 with E % 8 == 0
 *            and E <= 128 (one launch); other bf16 shapes hold the fp32
 *            partial logits of S slices of H, S*T*E*4 bytes with S = 1..H/64
 *            chosen from T, H, E */
int moe_route(const void* x, const void* w_router, const float* bias, int T, int H, int E, int k,
              int dtype, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
              size_t ws_bytes, void* stream);

/* The selection and gating half of moe_route on given fp32 logits [T,E]. */
int moe_route_from_logits(const float* logits, int T, int E, int k, int32_t* topk_idx,
                          float* topk_w, void* stream);

/* Permutation of routed rows into contiguous per-expert groups (the
 * "permute" of the dispatcher table).  Only experts in [e_lo, e_hi) are kept
 * (E_l = e_hi - e_lo local experts of one EP rank; the full layer uses
 * [0, E)).  Rows of one expert are in ascending token order.
 *   counts   [E_l]   int32: routed rows per local expert (0 is legal)
 *   offsets  [E_l+1] int32: exclusive prefix sum, offsets[E_l] = R
 *   dest_row [T*k]   int32: grouped row of slot (t,j), or -1 if not local
 *   src_row  [T*k]   int32: token of grouped row r, for r < R
 *   x_perm   [T*k,H] dtype: x_perm[dest_row[t*k+j]] = x[t], bitwise; or NULL:
 *            the maps alone (for moe_grouped_ffn_fwd_gather, which reads the
 *            token rows through src_row); x may then be NULL too
 *   ws       MOE_OP_PERMUTE workspace
 * dtype MOE_FP8 moves rows of H one-byte codes (H % 16 == 0).
 * A row of topk_idx may name one expert in several slots (moe_route never
 * does): each such slot gets its own grouped row, the slots of one token in
 * slot order, and counts count slots. */
int moe_permute(const void* x, const int32_t* topk_idx, int T, int H, int E, int k, int e_lo,
                int e_hi, int dtype, int32_t* counts, int32_t* offsets, int32_t* dest_row,
                int32_t* src_row, void* x_perm, void* ws, size_t ws_bytes, void* stream);

/* Grouped SwiGLU expert FFN (the "grouped matmul"), forward.  For each local
 * expert e and each of its rows r in [offsets[e], offsets[e+1]):
 *   g = x_perm[r] . w_gate[e]^T, u = x_perm[r] . w_up[e]^T     (fp32 accumulate)
 *   h_perm[r] = SiLU(g) * u,  SiLU(a) = a * sigmoid(a)          (fp32, stored as dtype)
 *   y_perm[r] = h_perm[r] . w_down[e]^T                         (fp32 accumulate)
 *   x_perm [R_cap,H], w_gate/w_up [E_l,I,H], w_down [E_l,H,I]  dtype
 *   gu_saved [R_cap,2I] dtype or NULL: g in columns [0,I), u in [I,2I)
 *   h_perm [R_cap,I], y_perm [R_cap,H]  dtype
 *   ws       MOE_OP_FFN_FWD workspace (the tile schedule) */
int moe_grouped_ffn_fwd(const void* x_perm, const int32_t* offsets, int E_l, int R_cap, int H,
                        int I, const void* w_gate, const void* w_up, const void* w_down, int dtype,
                        void* gu_saved, void* h_perm, void* y_perm, void* ws, size_t ws_bytes,
                        void* stream);

/* moe_grouped_ffn_fwd with the permutation folded into the first product:
 * grouped row r is token row x[src_row[r]] (src_row from moe_permute, which
 * then needs no x_perm), read by the gate/up product's operand loads in place
 * of a permuted copy; everything else, results and rounding included, is
 * moe_grouped_ffn_fwd's (the same products over the same rows: the same
 * bits).  The permute then moves no rows, and the product reads the T token
 * rows instead of T*k routed copies.
 *   x [T,H] bf16, src_row [R_cap] int32 (entries below offsets[E_l] in [0,T))
 *   other arguments as in moe_grouped_ffn_fwd (ws: MOE_OP_FFN_FWD)
 * bf16 only (MOE_EUNSUPPORTED otherwise); T*H*2 < 2^31. */
int moe_grouped_ffn_fwd_gather(const void* x, const int32_t* src_row, const int32_t* offsets,
                               int E_l, int R_cap, int T, int H, int I, const void* w_gate,
                               const void* w_up, const void* w_down, int dtype, void* gu_saved,
                               void* h_perm, void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* moe_grouped_ffn_fwd without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments, results and rounding are those of
 * moe_grouped_ffn_fwd (the same kernels, so the same bits).  The tile schedule
 * goes to a static scratch array in the library, 64 KiB per GPU, allocated
 * when the library is loaded and held until the process ends; it serves
 * R_cap <= 1048576 (2^20) routed-row capacity for any E_l <= 256, and larger
 * R_cap returns MOE_EUNSUPPORTED before anything is enqueued.  Every call on
 * one GPU uses that GPU's single array: calls that overlap on one GPU (two
 * streams, or two host threads, without an order between the calls) race on
 * it and must not be issued.  The call itself allocates nothing. */
int moe_grouped_ffn_fwd_noalloc(const void* x_perm, const int32_t* offsets, int E_l, int R_cap,
                                int H, int I, const void* w_gate, const void* w_up,
                                const void* w_down, int dtype, void* gu_saved, void* h_perm,
                                void* y_perm, void* stream);

/* FP8 recipe of the expert FFN.  The pages name FP8 as their only
 * kernel-level speed lever (page "TorchTitan FSDP2 完全指南", section
 * "性能表现", H100 benchmark table, row FSDP + compile + FP8) and fix no
 * format or scaling; this library's
 * reading: OCP E4M3 codes (largest finite 448, subnormals down to 2^-9), one
 * power-of-two scale per row (token row of the activations, output channel of
 * a weight matrix, row of h).
 *
 * Row quantization: for each row i < rows (and i < *nrows when nrows is not
 * NULL; nrows is a DEVICE pointer, e.g. offsets + E_l), scale[i] = 2^e with e
 * the smallest integer such that max_c |src[i,c]| <= 448 * 2^e (e = 0 for a
 * zero row), and q[i,c] = the E4M3 code nearest to src[i,c] / scale[i], ties
 * to even (the division is exact).  Rows >= *nrows are not written.
 *   src [rows,cols] MOE_BF16 or MOE_F32, q [rows,cols] uint8, scale [rows] fp32
 *   cols % 16 == 0; src and q 16-byte aligned. */
int moe_quantize_fp8(const void* src, int rows, int cols, int dtype, const int32_t* nrows,
                     uint8_t* q, float* scale, void* stream);

/* Grouped SwiGLU expert FFN, forward, on E4M3 codes.  With x_q the permuted
 * code rows (moe_permute with MOE_FP8 of moe_quantize_fp8's token rows) and
 * x_scale the per-TOKEN scales (row r uses x_scale[src_row[r]]):
 *   g[r,n] = x_scale[src_row[r]] * wg_scale[e,n] * sum_c code(x_q[r,c]) code(wg_q[e,n,c])
 *   (u likewise with wu), h_perm[r] = bf16(SiLU(g) * u),
 *   h's rows quantized as moe_quantize_fp8 does (codes and scales in ws),
 *   y_perm[r,m] = sh[r] * wd_scale[e,m] * sum_i code(hq[r,i]) code(wd_q[e,m,i])
 * Code products are exact and summed in fp32; outputs are rounded once.
 *   x_q [R_cap,H] uint8, x_scale [T] fp32, src_row [R_cap] int32,
 *   wg_q / wu_q [E_l,I,H] uint8 with wg_scale / wu_scale [E_l,I] fp32,
 *   wd_q [E_l,H,I] uint8 with wd_scale [E_l,H] fp32,
 *   gu_saved [R_cap,2I] bf16 or NULL (g, u as in moe_grouped_ffn_fwd),
 *   h_perm [R_cap,I] bf16, y_perm [R_cap,H] bf16
 *   ws       MOE_OP_FFN_FWD_FP8 workspace (schedule, row scales, codes of h)
 * Needs H % 128 == 0 and I % 128 == 0 (else MOE_EUNSUPPORTED). */
int moe_grouped_ffn_fwd_fp8(const uint8_t* x_q, const float* x_scale, const int32_t* src_row,
                            const int32_t* offsets, int E_l, int R_cap, int H, int I,
                            const uint8_t* wg_q, const float* wg_scale, const uint8_t* wu_q,
                            const float* wu_scale, const uint8_t* wd_q, const float* wd_scale,
                            void* gu_saved, void* h_perm, void* y_perm, void* ws, size_t ws_bytes,
                            void* stream);

/* moe_grouped_ffn_fwd_fp8 with the permutation folded into the gate/up
 * product's operand loads (as moe_grouped_ffn_fwd_gather does in bf16): x_q
 * holds the T token code rows [T,H] of moe_quantize_fp8 and grouped row r is
 * x_q[src_row[r]], so moe_permute (MOE_FP8) needs no x_perm.  Results, rounding
 * and workspace are moe_grouped_ffn_fwd_fp8's: the same products over the
 * same code rows, the same bits.  T*H < 2^31. */
int moe_grouped_ffn_fwd_fp8_gather(const uint8_t* x_q, const float* x_scale, const int32_t* src_row,
                                   const int32_t* offsets, int E_l, int R_cap, int T, int H, int I,
                                   const uint8_t* wg_q, const float* wg_scale, const uint8_t* wu_q,
                                   const float* wu_scale, const uint8_t* wd_q, const float* wd_scale,
                                   void* gu_saved, void* h_perm, void* y_perm, void* ws,
                                   size_t ws_bytes, void* stream);

/* Per-input-channel E4M3 codes of expert weights, for the FP8 data
 * gradients (same scale rule as moe_quantize_fp8, applied to the columns):
 * with src0 (and src1, or NULL) [batch,N,K] bf16, row k of batch b of the
 * output is column k of src0[b] followed by column k of src1[b]:
 *   q [batch,K,n*N] uint8 (n = 1 or 2), scale [batch,K] fp32.
 * W_down [E_l,H,I] gives the rows of W_down^T ([E_l,I,H]); W_gate and W_up
 * [E_l,I,H] give the rows of [W_gate^T | W_up^T] ([E_l,H,2I]).
 * N % 64 == 0 and K % 64 == 0 (else MOE_EUNSUPPORTED); pointers 16-byte
 * aligned. */
int moe_quantize_fp8_t(const void* src0, const void* src1, int batch, int N, int K, int dtype,
                       uint8_t* q, float* scale, void* stream);

/* Both FP8 code layouts of expert weights from one pair of passes: with w0
 * (and w1, or NULL) [batch,N,K] bf16,
 *   q0 / s0 (q1 / s1): the rows of w0 (w1) quantized as moe_quantize_fp8 does
 *                      ([batch,N,K] codes, [batch,N] scales; forward operands),
 *   qt / st          : the rows of [w0^T | w1^T] quantized as moe_quantize_fp8_t
 *                      does ([batch,K,n*N] codes, [batch,K] scales; operands of
 *                      the data gradients), skipped when qt is NULL;
 * bit for bit the results of those two calls.  ws: MOE_OP_QUANTIZE_W_FP8
 * workspace (the per-tile maxima), sized for the gate/up pair (batch = E_l,
 * N = I, K = H, two sources), which also covers W_down alone.
 * N % 128 == 0 and K % 128 == 0 (else MOE_EUNSUPPORTED); dtype MOE_BF16;
 * pointers 16-byte aligned. */
int moe_quantize_fp8_w(const void* w0, const void* w1, int batch, int N, int K, int dtype,
                       uint8_t* q0, float* s0, uint8_t* q1, float* s1, uint8_t* qt, float* st,
                       void* ws, size_t ws_bytes, void* stream);

/* Data gradients of the grouped SwiGLU FFN on E4M3 codes (the weight
 * gradients: moe_grouped_ffn_wgrad_fp8, or moe_grouped_ffn_bwd in bf16).  With dy_q / dy_scale the
 * rows of dy_perm quantized by moe_quantize_fp8, wdt_* the codes of W_down^T
 * and wgut_* those of [W_gate^T | W_up^T] from moe_quantize_fp8_t:
 *   dh[r,i]  = bf16(dy_scale[r] * wdt_scale[e,i] * sum_h code(dy_q[r,h]) code(wdt_q[e,i,h]))
 *   dg, du   = SiLU derivative of the saved g, u (as moe_grouped_ffn_bwd);
 *   dgu[r]   = bf16([dg | du]), its row quantized as moe_quantize_fp8 does
 *   dx_perm[r,m] = bf16(sdgu[r] * wgut_scale[e,m] * sum_c code(dguq[r,c]) code(wgut_q[e,m,c]))
 * Code products are exact and summed in fp32.
 *   dy_q [R_cap,H] uint8, dy_scale [R_cap] fp32, gu_saved [R_cap,2I] bf16,
 *   wdt_q [E_l,I,H] uint8 / wdt_scale [E_l,I], wgut_q [E_l,H,2I] uint8 /
 *   wgut_scale [E_l,H], dgu [R_cap,2I] bf16 (out), dx_perm [R_cap,H] bf16 (out)
 *   ws       MOE_OP_FFN_DGRAD_FP8 workspace (schedule, dh, codes of [dg | du])
 * Needs H % 128 == 0, I % 128 == 0 and I <= 2048 (else MOE_EUNSUPPORTED). */
int moe_grouped_ffn_dgrad_fp8(const uint8_t* dy_q, const float* dy_scale, const void* gu_saved,
                              const int32_t* offsets, int E_l, int R_cap, int H, int I,
                              const uint8_t* wdt_q, const float* wdt_scale, const uint8_t* wgut_q,
                              const float* wgut_scale, void* dgu, void* dx_perm, void* ws,
                              size_t ws_bytes, void* stream);

/* Column quantization of grouped rows for the FP8 weight gradients, which
 * sum over each expert's rows, so a scale must hold along them: for group g
 * (rows offsets[g] .. offsets[g+1]-1 of the logical matrix, row r being
 * src[src_row[r]] when src_row is not NULL, else src[r]) and column c,
 *   scale[g,c] = 2^e, e the smallest integer with max_r |src[r,c]| <= 448 * 2^e
 *                over the group's rows (e = 0 for an empty group or a zero column),
 *   q[c, poff[g] + i] = the E4M3 code nearest to src[offsets[g]+i, c] / scale[g,c]
 *                (ties to even) for i < n_g, and code 0 for n_g <= i < round64(n_g),
 *   poff[g]  = sum over g' < g of round64(n_g'), poff[E_l] the total (out).
 * Columns poff[E_l] .. q_pitch-1 of q are not written.
 *   src [rows,C] bf16 (row pitch C), src_row [R_cap] int32 or NULL, offsets
 *   [E_l+1] int32 (device), q [C,q_pitch] uint8, scale [E_l,C] fp32, poff
 *   [E_l+1] int32.  C % 64 == 0 and q_pitch % 64 == 0 with
 *   q_pitch >= round64(R_cap) + 64 * E_l (else MOE_EINVAL); src and q 16-byte
 *   aligned.  Reading of the FP8 recipe (page "TorchTitan FSDP2 完全指南",
 *   section "性能表现", row FSDP + compile + FP8, which fixes no scaling). */
int moe_quantize_fp8_group_t(const void* src, const int32_t* src_row, int C,
                             const int32_t* offsets, int E_l, int R_cap, uint8_t* q, int q_pitch,
                             float* scale, int32_t* poff, void* stream);

/* Weight gradients of the grouped SwiGLU FFN on E4M3 codes (same FP8
 * reading).  Each operand is column-quantized per expert as
 * moe_quantize_fp8_group_t does (codes and scales in ws), then, for every
 * local expert e with rows r in its group (r < R = offsets[E_l]):
 *   [dW_gate; dW_up][e][i,h] = s_gu[e,i] * s_x[e,h] * sum_r code(dgu[r,i]) code(x_r[h])
 *   dW_down[e][h,i]          = s_dy[e,h] * s_h[e,i] * sum_r code(dy_perm[r,h]) code(h_perm[r,i])
 * (rows i < I of the first product are dW_gate, the rest dW_up), with x_r the
 * grouped token row: x[src_row[r]] if src_row is not NULL, else x[r].
 * Code products are exact and summed in fp32; accumulate != 0 adds to the
 * fp32 outputs instead of overwriting them.  An expert without rows gets 0.
 *   x [T,H] (with src_row [R_cap]) or [R_cap,H] bf16, dgu [R_cap,2I] bf16
 *   (moe_grouped_ffn_dgrad_fp8's dgu), h_perm [R_cap,I] bf16, dy_perm
 *   [R_cap,H] bf16, dw_gate / dw_up [E_l,I,H] fp32, dw_down [E_l,H,I] fp32
 *   ws       MOE_OP_FFN_WGRAD_FP8 workspace (codes, scales, padded offsets)
 * Needs H % 128 == 0 and I % 128 == 0 (else MOE_EUNSUPPORTED). */
int moe_grouped_ffn_wgrad_fp8(const void* x, const int32_t* src_row, const void* dgu,
                              const void* h_perm, const void* dy_perm, const int32_t* offsets,
                              int E_l, int R_cap, int H, int I, float* dw_gate, float* dw_up,
                              float* dw_down, int accumulate, void* ws, size_t ws_bytes,
                              void* stream);

/* moe_grouped_ffn_wgrad_fp8 in two halves, so that a caller can start the
 * part that does not need dgu (the output of the SiLU' pass of the data
 * gradients) as soon as x, h_perm and dy_perm exist, e.g. on a second stream
 * beside the data gradients.  Same FP8 reading and arguments as
 * moe_grouped_ffn_wgrad_fp8; begin then end on one workspace compute exactly
 * (bit for bit) what that call computes.
 *   begin: quantizes the columns of x (through src_row), dy_perm and h_perm
 *          per expert into ws, builds the K-chunk plans and writes dW_down
 *          (overwrite, or added to with accumulate != 0).  An expert whose
 *          rows are split into K chunks gets its chunks after the first as
 *          fp32 partials in ws: dw_down is complete only after end.
 *   end:   quantizes the columns of dgu, writes dW_gate and dW_up, then adds
 *          the partials of both products' split experts in chunk order.
 * end must run after begin (same stream, or ordered after it by an event),
 * with the same ws, offsets, E_l, R_cap, H, I and accumulate, and dw_down the
 * pointer begin wrote; nothing else may use ws in between.  Errors as
 * moe_grouped_ffn_wgrad_fp8. */
int moe_grouped_ffn_wgrad_fp8_begin(const void* x, const int32_t* src_row, const void* h_perm,
                                    const void* dy_perm, const int32_t* offsets, int E_l,
                                    int R_cap, int H, int I, float* dw_down, int accumulate,
                                    void* ws, size_t ws_bytes, void* stream);
int moe_grouped_ffn_wgrad_fp8_end(const void* dgu, const int32_t* offsets, int E_l, int R_cap,
                                  int H, int I, float* dw_gate, float* dw_up, float* dw_down,
                                  int accumulate, void* ws, size_t ws_bytes, void* stream);

/* Weighted unpermute ("combine"): for every token, in slot order j = 0..k-1,
 *   y[t] = sum_{j: dest_row[t*k+j] >= 0} topk_w[t,j] * y_perm[dest_row[t*k+j]]  (+ addend[t])
 * accumulated in fp32 and rounded once to dtype.  topk_w == NULL means
 * weight 1 (the unweighted unpermute-reduce of the backward).  A token with
 * no local slot gets addend[t] (or 0).
 *   y_perm [R_cap,H] dtype, topk_w [T,k] fp32 or NULL, dest_row [T*k] int32,
 *   addend [T,H] fp32 or NULL, y [T,H] dtype */
int moe_combine(const void* y_perm, const float* topk_w, const int32_t* dest_row,
                const float* addend, int T, int H, int k, int dtype, void* y, void* stream);

/* Backward of moe_combine for upstream gradient dy [T,H] (dtype):
 *   dy_perm[dest_row[t*k+j]] = topk_w[t,j] * dy[t]           (stored as dtype)
 *   d_topk_w[t,j] = <dy[t], y_perm[dest_row[t*k+j]]>         (fp32; 0 for non-local slots) */
int moe_combine_bwd(const void* dy, const void* y_perm, const float* topk_w,
                    const int32_t* dest_row, int T, int H, int k, int dtype, void* dy_perm,
                    float* d_topk_w, void* stream);

/* The layer's input gradient in one pass: the unweighted unpermute-reduce of
 * the experts' input gradient plus the router's input gradient, for every
 * token
 *   dx[t] = sum_{j: dest_row[t*k+j] >= 0} dx_perm[dest_row[t*k+j]]
 *         + sum_j dz_j * w_router[:, topk_idx[t,j]],
 *   dz_j = w_j (dw_j - sum_l w_l dw_l),   w = topk_w[t,:], dw = d_topk_w[t,:]
 * accumulated in fp32 (local rows in slot order, then the router term in slot
 * order) and rounded once to dtype.  It equals moe_combine(dx_perm, NULL,
 * dest_row, dx_router) with dx_router from moe_route_bwd, without that
 * [T,H] fp32 intermediate.
 *   dx_perm [R_cap,H] dtype, dest_row [T*k] int32, d_topk_w, topk_w [T,k]
 *   fp32, topk_idx [T,k] int32, w_router [H,E] dtype, dx [T,H] dtype
 *   ws       MOE_OP_COMBINE_DX workspace (the transposed router weight) */
int moe_combine_dx(const void* dx_perm, const int32_t* dest_row, const float* d_topk_w,
                   const float* topk_w, const int32_t* topk_idx, const void* w_router, int T,
                   int H, int E, int k, int dtype, void* dx, void* ws, size_t ws_bytes,
                   void* stream);

/* moe_combine_dx with the router weight already transposed,
 *   w_router_t [E,H] dtype (w_router_t[e,h] = w_router[h,e], 16-byte aligned),
 * e.g. from moe_router_weight_t; the other arguments, the result and the
 * accumulation order are those of moe_combine_dx, and no workspace is used.
 * Lets a caller make the transpose where the chip is idle (before the
 * backward's concurrent products) instead of in front of the gather. */
int moe_combine_dx_t(const void* dx_perm, const int32_t* dest_row, const float* d_topk_w,
                     const float* topk_w, const int32_t* topk_idx, const void* w_router_t, int T,
                     int H, int E, int k, int dtype, void* dx, void* stream);

/* Transpose of the router weight, the operand of the router's input
 * gradient (dx_router = dz . w_router^T, the router product's backward):
 *   w_router [H,E] dtype -> w_router_t [E,H] dtype, a bit copy.
 * H and E in [0, 2^20]; nothing is launched when H*E = 0.  Caller-owned
 * device buffers, which must not overlap. */
int moe_router_weight_t(const void* w_router, int H, int E, int dtype, void* w_router_t,
                        void* stream);

/* Backward of the grouped FFN, given dy_perm [R_cap,H] and the forward's
 * x_perm, gu_saved (required) and h_perm:
 *   dx_perm [R_cap,H] dtype   gradient wrt x_perm
 *   dw_gate, dw_up [E_l,I,H] fp32, dw_down [E_l,H,I] fp32: overwritten
 *   (accumulate == 0) or added to (accumulate == 1); an expert with no rows
 *   gets exact zeros (or is left unchanged when accumulating).  In bf16 an
 *   expert with far more rows than the rest (more than max(1024, R*tiles/256),
 *   tiles = its weight-gradient tiles) has its row range cut into up to 8
 *   chunks whose fp32 sums are added in chunk order: the result is the same
 *   for every run, but its summation order differs from an unsplit one.
 *   ws       MOE_OP_FFN_BWD workspace (schedule, the [R_cap,2I] gradient of
 *            g and u, the weight gradients' chunk plans and partial sums) */
int moe_grouped_ffn_bwd(const void* dy_perm, const void* x_perm, const void* gu_saved,
                        const void* h_perm, const int32_t* offsets, int E_l, int R_cap, int H,
                        int I, const void* w_gate, const void* w_up, const void* w_down,
                        int dtype, void* dx_perm, float* dw_gate, float* dw_up, float* dw_down,
                        int accumulate, void* ws, size_t ws_bytes, void* stream);

/* moe_grouped_ffn_bwd with the weight gradients left on a second stream, so
 * that the caller can overlap them with later work (e.g. moe_combine_dx).
 * dx_perm is complete in `stream` order; dw_gate, dw_up and dw_down are
 * complete in `wgrad_stream` order (which this call makes wait for the data it
 * reads).  ws must not be reused by any work until both streams have passed
 * this call.  wgrad_stream must differ from stream (else MOE_EINVAL). */
int moe_grouped_ffn_bwd_split(const void* dy_perm, const void* x_perm, const void* gu_saved,
                              const void* h_perm, const int32_t* offsets, int E_l, int R_cap,
                              int H, int I, const void* w_gate, const void* w_up,
                              const void* w_down, int dtype, void* dx_perm, float* dw_gate,
                              float* dw_up, float* dw_down, int accumulate, void* ws,
                              size_t ws_bytes, void* stream, void* wgrad_stream);

/* Backward of moe_route, given the gradient d_topk_w [T,k] of the gate weights:
 *   d_logits[t, topk_idx[t,j]] = w_j * (dw_j - sum_l w_l dw_l), 0 elsewhere  [T,E] fp32
 *   dx_router[t] = sum_e d_logits[t,e] * w_router[:,e]      [T,H] fp32 or NULL
 *   dw_router    = x^T . d_logits                           [H,E] fp32 or NULL (overwritten)
 *   ws       MOE_OP_ROUTE_BWD workspace
 * The bf16 path also needs E % 4 == 0 (else MOE_EUNSUPPORTED).  In bf16 with
 * E % 64 == 0, dx_router is a dense MFMA product over all E columns, with each
 * d_logits value entering as two bf16 halves (about 16 bits) and fp32 sums in
 * the matrix core's order; otherwise it is gathered from the k kept experts in
 * slot order.  Both agree with the exact sum to within 2^-14 of the sum of
 * absolute terms. */
int moe_route_bwd(const float* d_topk_w, const float* topk_w, const int32_t* topk_idx,
                  const void* x, const void* w_router, int T, int H, int E, int k, int dtype,
                  float* d_logits, float* dx_router, float* dw_router, void* ws, size_t ws_bytes,
                  void* stream);

/* Kernel timing hook (benchmarks and profilers).  After this call the library
 * records start_events[i] and stop_events[i] (each a hipEvent_t created by
 * the caller) on the launch stream immediately before and after the i-th
 * launch of kernel `kernel_id`, for i < n; later launches are not recorded.
 * kernel_id < 0 switches recording off.  The arrays must stay valid while
 * recording is on.  The hook is per calling thread: it records launches made
 * by the thread that armed it, and other threads' calls are not affected.
 * Returns MOE_OK or MOE_EINVAL. */
typedef enum {
  MOE_KERNEL_ROUTE = 0,           /* router GEMM + top-k */
  MOE_KERNEL_PERMUTE_HIST = 1,
  MOE_KERNEL_PERMUTE_SCAN = 2,
  MOE_KERNEL_PERMUTE_SCATTER = 3,
  MOE_KERNEL_FFN_GATEUP = 4,      /* gate/up GEMM + SiLU*up */
  MOE_KERNEL_FFN_DOWN = 5,
  MOE_KERNEL_COMBINE = 6,
  MOE_KERNEL_COMBINE_BWD = 7,
  MOE_KERNEL_ROUTE_BWD_DZ = 8,
  MOE_KERNEL_ROUTE_BWD_DW = 9,
  MOE_KERNEL_FFN_DOWN_DGRAD = 10,
  MOE_KERNEL_FFN_DOWN_WGRAD = 11,
  MOE_KERNEL_FFN_GATEUP_DGRAD = 12,
  MOE_KERNEL_FFN_GATEUP_WGRAD = 13,
  MOE_KERNEL_COMBINE_DX = 14,     /* fused input gradient (moe_combine_dx) */
  MOE_KERNEL_ROUTE_BWD_DX = 15,   /* router input gradient as an MFMA product (moe_route_bwd) */
  MOE_KERNEL_COMBINE_ADD = 16,    /* moe_combine with an addend (an input gradient's unpermute-reduce) */
  MOE_KERNEL_FFN_WGRAD_REDUCE = 17, /* split experts' weight-gradient partials added (moe_grouped_ffn_bwd) */
  MOE_KERNEL_COUNT = 18
} moe_kernel;

int moe_profile_kernel(int kernel_id, void** start_events, void** stop_events, int n);

/* Number of launches recorded since the calling thread's last
 * moe_profile_kernel() call. */
int moe_profile_recorded(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
