/*
 * nvfp4moe.h -- C ABI of libnvfp4moe.so, the NVFP4 block-scaled mixture-of-experts
 * hot path for AMD Instinct MI355X (gfx950).
 *
 * The layer this library computes, one call per stage:
 *
 *   logits --moe_route_permute--> top-k ids/weights, per-expert row offsets, permutation
 *   x      --moe_grouped_gemm_nvfp4(EPI_SWIGLU)--> h = silu(x W_gate^T) * (x W_up^T)  per expert
 *   h      --moe_grouped_gemm_nvfp4(EPI_NONE)  --> Y = h W_down^T                    per expert
 *   Y      --moe_unpermute_reduce--> out[t] = sum_j w[t,j] * Y[row of slot (t,j)]
 *
 * plus nvfp4_quantize (weights offline; W4A4 activations and h per forward) and
 * act_fp8_e4m3_roundtrip (FP8 E4M3 activations dequantized to bf16); and the MXFP4 variant
 * (mxfp4_quantize, mxfp4_weights_tile, moe_grouped_gemm_mxfp4 and
 * moe_grouped_gemm_mxfp4_swiglu_q: group-32 UE8M0 scales, W4A4 on the scaled FP4 matrix cores).
 *
 * Sources for what is computed (web pages; section names):
 *   [P1] "Native FP4 Is Slower Than Emulated FP4: A Kernel-Maturity Measurement on
 *        First-Generation Workstation Blackwell", section 1 (512 experts, 22 active;
 *        NVFP4 = FP4 weights with FP8 activations).
 *   [P2] "The Benchmark That Confirmed the Ceiling: NVFP4 Cutlass on sm_120",
 *        section "The NVFP4 Pivot" (NVFP4 = FP4 values, one E4M3 scale per 16;
 *        W4A16 = dequantize FP4 to 16-bit and multiply; W4A4 = FP4 x FP4) and
 *        section "Roofline Awareness" (half a byte per FP4 parameter).
 *   [P3] "The 2x Gap: Diagnosing Suboptimal FP4 GEMM Kernels on Blackwell SM120",
 *        sections "The Investigation So Far" (256 experts, top-8, ~16 tokens per
 *        expert at decode) and "Discovering the sgl_kernel Alternative" (a scaled
 *        FP4 GEMM takes two FP4-packed operands, their block scales, an alpha and an
 *        output dtype; a fused MoE gathers tokens to experts and scatters them back).
 *   [P4] "The 24% Ceiling: Diagnosing the Limits of NVFP4 Quantization on Blackwell
 *        SM120 GPUs", sections "The Core Insight" and "The Decision" (W4A16 versus
 *        true W4A4 grouped GEMM for the MoE).
 *
 * NVFP4 storage of a matrix [R, C] (groups of 16 along C, the GEMM's K):
 *   packed  uint8 [R, C/2]   E2M1 codes, element 2i in the LOW nibble of byte i
 *   scales  uint8 [R, C/16]  OCP E4M3FN codes (bias 7, NaN = 0x7F/0xFF, max 448)
 *   g       float32          per-tensor scale; value = E2M1[q] * E4M3[s] * g
 * A batch of B matrices is stored back to back ([B, R, C/2], [B, R, C/16], g[B]).
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is DEVICE memory owned by the caller; the library
 *     allocates nothing. Scratch memory comes in through (ws, ws_bytes); its size
 *     is given by the matching *_workspace_size query and it need not be zeroed.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream) and
 *     never synchronize the device. Outputs are valid once the stream reaches them.
 *   - Arguments are validated on the host before any HIP call. A bad argument
 *     returns NVFP4MOE_ERR_INVALID_ARG (a too-small workspace NVFP4MOE_ERR_WORKSPACE)
 *     and launches nothing; a failed launch returns NVFP4MOE_ERR_HIP. The message is
 *     available from nvfp4moe_last_error() on the calling thread. There is no
 *     fallback path: a call either runs its kernels or reports why not.
 *   - Results are deterministic: the same inputs give the same bytes (no
 *     order-dependent floating-point atomics anywhere).
 *   - Data-dependent sizes (rows per expert, active experts) stay on the device;
 *     the host passes only upper bounds.
 *   - The library keeps no state besides the thread-local error message and the
 *     last dispatch code; concurrent calls on different streams are safe.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4MOE_OK = 0,
  NVFP4MOE_ERR_INVALID_ARG = 1,
  NVFP4MOE_ERR_UNSUPPORTED = 2,
  NVFP4MOE_ERR_WORKSPACE = 3,
  NVFP4MOE_ERR_HIP = 4
} nvfp4moe_status;

/* [P2] "The NVFP4 Pivot", [P4] "The Decision": weight-only FP4 with 16-bit
 * activations, or FP4 weights and FP4 activations. W4A16_PREPARED: W4A16 with the token rows
 * already prepared by moe_dispatch_w4a16. */
typedef enum { NVFP4MOE_W4A16 = 0, NVFP4MOE_W4A4 = 1, NVFP4MOE_W4A16_PREPARED = 2 } nvfp4moe_mode;

typedef enum { NVFP4MOE_EPI_NONE = 0, NVFP4MOE_EPI_SWIGLU = 1 } nvfp4moe_epilogue;

typedef enum { NVFP4MOE_F32 = 0, NVFP4MOE_BF16 = 1 } nvfp4moe_dtype;

/* Kernel family chosen by the last moe_grouped_gemm_nvfp4 call on this thread. */
typedef enum {
  NVFP4MOE_PATH_NONE = 0,
  NVFP4MOE_PATH_STREAM = 1, /* small-M weight-streaming kernel (HBM-bound regime)   */
  NVFP4MOE_PATH_MFMA = 2    /* large-M LDS-tiled MFMA kernel (compute-bound regime) */
} nvfp4moe_path;

/* Byte order of quantized codes and scales: the row-major storage above, or the tiled
 * storage the grouped GEMM reads (described at nvfp4_weights_tile). */
typedef enum { NVFP4MOE_LAYOUT_ROW_MAJOR = 0, NVFP4MOE_LAYOUT_TILED = 1 } nvfp4moe_layout;

/* ---------------------------------------------------------------------------
 * nvfp4_quantize -- quantize B float matrices [R, C] to NVFP4.  [P2] "The NVFP4 Pivot".
 *
 *   x        device, x_dtype (F32 or BF16), [B, R, C] row-major.
 *   B, R, C  1 <= B <= 65535, R >= 1, C >= 32 and C % 32 == 0; x 16-byte aligned,
 *            packed 16-byte aligned, scales 2-byte aligned.
 *   g_in     device float[B] or NULL. If given, used as the global scales.
 *   amax_in  device float[B] or NULL. If g_in is NULL and amax_in is given,
 *            g[b] = amax_in[b] / 2688 (or 1 when amax_in[b] == 0); amax_in must be
 *            the max |x| over the finite entries of matrix b.
 *            If both are NULL, the amax is computed on the device.
 *   layout   NVFP4MOE_LAYOUT_ROW_MAJOR: packed [B, R, C/2] and scales [B, R, C/16] as above.
 *            NVFP4MOE_LAYOUT_TILED: the same codes and scales written straight into the
 *            tiled storage moe_grouped_gemm_nvfp4 reads (bytes identical to nvfp4_weights_tile
 *            of the row-major result, padding zeros included): packed [B *
 *            nvfp4_tiled_codes_bytes(R, C)], scales [B * nvfp4_tiled_scales_bytes(R, C)], both
 *            16-byte aligned; needs R % 16 == 0 and B * R * C / 2 < 2^40. So one call turns a
 *            weight matrix into the GEMM's operand.
 *   packed   device uint8 (output), codes in `layout`.
 *   scales   device uint8 (output), E4M3 scales in `layout`.
 *   g_out    device float[B]           (output) the global scales used.
 *   ws       workspace of nvfp4_quantize_workspace_size(B, R, C) bytes.
 *
 * Rule, in float32 with round-to-nearest-even (all steps on the device):
 *   g = amax / 2688 (2688 = 6 * 448; 1 if amax == 0);
 *   per 16-group: a NaN/Inf in the group -> scale 0x7F and codes 0;
 *                 amax_g == 0 -> scale 0, codes +-0;
 *                 else s = E4M3(min(amax_g / (6 g), 448)), S = E4M3[s] * g,
 *                      q_i = E2M1(w_i / S) saturating at 6, sign bit from w_i.
 * ------------------------------------------------------------------------- */
nvfp4moe_status nvfp4_quantize(const void* x, nvfp4moe_dtype x_dtype, int64_t B, int64_t R,
                               int64_t C, const float* g_in, const float* amax_in,
                               nvfp4moe_layout layout, uint8_t* packed, uint8_t* scales,
                               float* g_out, void* ws, size_t ws_bytes, void* stream);
size_t nvfp4_quantize_workspace_size(int64_t B, int64_t R, int64_t C);

/* ---------------------------------------------------------------------------
 * nvfp4_quantize_noalloc -- nvfp4_quantize for callers that cannot allocate memory: code
 * under HIP graph capture, tight serving loops that quantize activations every forward,
 * harnesses that forbid allocation. Same arguments, rule and outputs as nvfp4_quantize
 * (bit for bit), without (ws, ws_bytes); the call allocates nothing.
 *
 *   The amax pass (g_in and amax_in both NULL) keeps its partial maxima in a scratch array
 *   of 64 KiB that the library holds on each GPU it runs on until the process ends:
 *   B * (amax workgroups per matrix) floats, i.e. nvfp4_quantize_workspace_size(B, R, C)
 *   bytes, must not exceed 65536 (any single matrix fits; a larger batch returns
 *   NVFP4MOE_ERR_WORKSPACE and launches nothing). Every entry the call reads is written by
 *   the same call, so nothing needs clearing between calls.
 *   All calls on one GPU share that GPU's scratch: calls that may overlap on one GPU (on
 *   different streams, or from different threads without ordering) race and must not be
 *   issued. stream must belong to the current device (else NVFP4MOE_ERR_INVALID_ARG).
 * ------------------------------------------------------------------------- */
nvfp4moe_status nvfp4_quantize_noalloc(const void* x, nvfp4moe_dtype x_dtype, int64_t B, int64_t R,
                                       int64_t C, const float* g_in, const float* amax_in,
                                       nvfp4moe_layout layout, uint8_t* packed, uint8_t* scales,
                                       float* g_out, void* stream);

/* ---------------------------------------------------------------------------
 * nvfp4_weights_tile -- reorder NVFP4 weight matrices (the row-major storage above) into
 * the tiled storage that moe_grouped_gemm_nvfp4 reads. A pure permutation of the bytes
 * plus zero padding (no value changes); run once per weight set, like the quantization.
 * The format is the pages' ([P2] "The NVFP4 Pivot"); only the byte order differs.
 *
 *   packed, scales  device uint8 [B, R, C/2] and [B, R, C/16] as written by nvfp4_quantize;
 *                   packed 16-byte aligned, scales 2-byte aligned.
 *   B, R, C         1 <= B <= 65535, R >= 16, R % 16 == 0, C >= 32, C % 32 == 0,
 *                   B * R * C / 2 < 2^40.
 *   tiled_codes     device uint8 [B * nvfp4_tiled_codes_bytes(R, C)]  (output), 16-byte aligned
 *   tiled_scales    device uint8 [B * nvfp4_tiled_scales_bytes(R, C)] (output), 16-byte aligned
 *
 * Layout, with rb = row / 16, r = row % 16, nch = ceil(C / 128), nwin = ceil(C / 1024):
 *   codes : 1 KB tile per (matrix b, rb, chunk c) at ((b * R/16 + rb) * nch + c) * 1024;
 *           bytes 16 (16 g + r) .. +15 of the tile are the codes of columns
 *           128 c + 32 g .. +31 of the row (g = 0..3), zero past C.
 *   scales: 1 KB tile per (matrix b, rb, window w) at ((b * R/16 + rb) * nwin + w) * 1024;
 *           bytes 16 (16 g + r) + 2 u and + 2 u + 1 are the scales of columns
 *           128 (8 w + u) + 32 g + {0..15} and {16..31} of the row (u = 0..7), zero past C.
 * (One GPU wave then reads a 16-row x 128-column block of codes, in the lane order of the
 * matrix-core operand, as 1 KB of contiguous memory.)
 * ------------------------------------------------------------------------- */
nvfp4moe_status nvfp4_weights_tile(const uint8_t* packed, const uint8_t* scales, int64_t B, int64_t R,
                                   int64_t C, uint8_t* tiled_codes, uint8_t* tiled_scales, void* stream);
/* Bytes of one tiled [R, C] matrix: (R/16) * ceil(C/128) * 1024 codes, (R/16) * ceil(C/1024) *
 * 1024 scales; 0 if R or C violate the constraints above. */
size_t nvfp4_tiled_codes_bytes(int64_t R, int64_t C);
size_t nvfp4_tiled_scales_bytes(int64_t R, int64_t C);

/* ---------------------------------------------------------------------------
 * moe_route_permute -- router + histogram + stable permutation.
 * [P3] "The Investigation So Far" (top-8 of 256), [P1] section 1 (top-22 of 512),
 * [P3] "Discovering the sgl_kernel Alternative" (expert scatter/gather).
 *
 *   logits          device float [T, E], finite.
 *   T, E, k         1 <= T, 1 <= k <= min(E, 64), E <= 1024, T * k <= 2^24.
 *   topk_ids        device int32 [T, k]  (output) experts by descending logit, ties to
 *                   the lower id.
 *   topk_w          device float [T, k]  (output) softmax over E, renormalised over the
 *                   k kept experts (computed in float64, stored as float32).
 *   expert_offsets  device int32 [E + 1] (output) exclusive prefix sum of rows per expert.
 *   sorted_slot     device int32 [T * k] (output) row r holds slot s = t * k + j; rows of
 *                   one expert keep ascending slot order (stable counting sort).
 *   slot_to_row     device int32 [T * k] (output) inverse of sorted_slot.
 *   active_experts  device int32 [E]     (output) experts with >= 1 row, ascending, in
 *                   entries [0, n_active); the rest are set to -1.
 *   n_active        device int32 [1]     (output)
 *   ws, ws_bytes    device scratch of at least moe_route_permute_workspace_size(T, E, k)
 *                   bytes, 4-byte aligned, caller-owned (per-chunk expert counts of the
 *                   permutation; contents on return are unspecified). Too small or NULL ->
 *                   NVFP4MOE_ERR_WORKSPACE. The size query returns 0 for invalid sizes.
 * ------------------------------------------------------------------------- */
nvfp4moe_status moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k,
                                  int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                                  int32_t* sorted_slot, int32_t* slot_to_row,
                                  int32_t* active_experts, int32_t* n_active, void* ws,
                                  size_t ws_bytes, void* stream);
size_t moe_route_permute_workspace_size(int32_t T, int32_t E, int32_t k);

/* ---------------------------------------------------------------------------
 * moe_dispatch_w4a16 -- moe_route_permute plus the W4A16 up/gate GEMM's preparation of the
 * token rows, for decode-sized batches where every launch of the layer costs several
 * microseconds: up to 16 tokens (T * k <= 1024, H <= 8192) the routing workgroup and one
 * workgroup per token row run as one launch; otherwise the rows are prepared by launches of
 * their own after the routing. [P3] "Discovering the sgl_kernel Alternative" (a fused MoE's
 * expert dispatch), [P1] section 3 (launch overhead of many small kernels), [P1] section 1
 * (FP8 activations).
 *
 *   logits, T, E, k, topk_ids .. n_active   as moe_route_permute (same outputs, same bits).
 *   x          device bf16 [T, H], 16-byte aligned; H >= 32, H % 32 == 0, T * H < 2^31.
 *   fp8_act    0, or 1: the rows first take the FP8 E4M3 round trip of
 *              act_fp8_e4m3_roundtrip (per-tensor scale over all of x), as that call writes.
 *   x_prep     device, moe_prepared_act_bytes(T, H) bytes, 16-byte aligned (output): the rows
 *              as moe_grouped_gemm_nvfp4 prepares bf16 activations for W4A16 (each row scaled
 *              by a power of two into f16 range, f16 in the kernels' operand order, and the
 *              exponents); its only reader is moe_grouped_gemm_nvfp4 in mode
 *              NVFP4MOE_W4A16_PREPARED with a = x_prep, a_rows = T, K = H.
 *   ws         moe_dispatch_w4a16_workspace_size(T, E, k, H, fp8_act) bytes, 16-byte aligned,
 *              caller-owned scratch; too small -> NVFP4MOE_ERR_WORKSPACE.
 * ------------------------------------------------------------------------- */
nvfp4moe_status moe_dispatch_w4a16(const float* logits, const void* x, int32_t T, int32_t E, int32_t k,
                                   int32_t H, int32_t fp8_act, int32_t* topk_ids, float* topk_w,
                                   int32_t* expert_offsets, int32_t* sorted_slot, int32_t* slot_to_row,
                                   int32_t* active_experts, int32_t* n_active, void* x_prep, void* ws,
                                   size_t ws_bytes, void* stream);
size_t moe_dispatch_w4a16_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t fp8_act);
/* Bytes of prepared activations for rows x K (0 for invalid sizes). */
size_t moe_prepared_act_bytes(int64_t rows, int32_t K);

/* ---------------------------------------------------------------------------
 * moe_grouped_gemm_nvfp4 -- per expert e, rows expert_offsets[e] .. expert_offsets[e+1]:
 *     P = A_rows . W_e^T  (float32 accumulation of exact products) * w_g[e] (* a_g[0])
 *     EPI_NONE  : out = P                                  [rows, Nw]
 *     EPI_SWIGLU: out = silu(P[:, :Nw/2]) * P[:, Nw/2:]    [rows, Nw/2]
 * [P3] "Discovering the sgl_kernel Alternative" (operands, block scales, alpha, out
 * dtype), [P2] "The NVFP4 Pivot" and [P4] "The Decision" (W4A16 / W4A4).
 *
 *   mode        W4A16: a is bf16 [a_rows, K]; a_scales and a_g are ignored (may be NULL).
 *               W4A4 : a is NVFP4 packed uint8 [a_rows, K/2] with a_scales uint8
 *                      [a_rows, K/16] and a_g device float[1].
 *               W4A16_PREPARED: W4A16 with a = the x_prep of moe_dispatch_w4a16 (its T =
 *                      a_rows, its H = K), so the call launches no preparation of its own.
 *   a_rows      rows of a.
 *   gather_index, gather_div
 *               NULL: GEMM row r reads a row r (a_rows must equal rows).
 *               else: GEMM row r reads a row gather_index[r] / gather_div, e.g.
 *                     sorted_slot with gather_div = k to gather token rows.
 *   w_packed, w_scales
 *               device, the E expert matrices [Nw, K] in the tiled storage: written by
 *               nvfp4_quantize with NVFP4MOE_LAYOUT_TILED (B = E), or by nvfp4_weights_tile
 *               from the row-major storage (expert e at e * nvfp4_tiled_codes_bytes(Nw, K)
 *               and e * nvfp4_tiled_scales_bytes(Nw, K)); w_g float [E], the g_out of that
 *               quantization.
 *   expert_offsets, active_experts, n_active  as written by moe_route_permute (for a
 *               dense GEMM: E = 1, offsets {0, rows}, active {0}, n_active {1}).
 *   E, rows, Nw, K  1 <= E <= 1024; rows = expert_offsets[E] >= 1; Nw >= 32, Nw % 32 == 0
 *               (EPI_SWIGLU: gate rows 0..Nw/2-1, up rows Nw/2..Nw-1); K >= 32, K % 32 == 0;
 *               rows * max(K, Nw) < 2^31, a_rows * K * 2 < 2^31, Nw * K / 2 < 2^31
 *               (K rounded up to a multiple of 128 in the last two).
 *               a, w_packed and w_scales 16-byte aligned, a_scales 2-byte aligned.
 *   out         device, out_dtype (F32 or BF16), [rows, EPI_SWIGLU ? Nw/2 : Nw].
 *   out_amax    device float[1] or NULL: if given, set to max |out| over the finite values
 *               the call writes (NaN and +-Inf excluded; with a bf16 out, of the rounded
 *               values): exactly the amax nvfp4_quantize's amax_in expects for out.
 *   ws          moe_grouped_gemm_workspace_size(mode, a_rows, rows, E, Nw, K) bytes.
 * ------------------------------------------------------------------------- */
nvfp4moe_status moe_grouped_gemm_nvfp4(nvfp4moe_mode mode, nvfp4moe_epilogue epi,
                                       const void* a, const uint8_t* a_scales, const float* a_g,
                                       int64_t a_rows, const int32_t* gather_index,
                                       int32_t gather_div, const uint8_t* w_packed,
                                       const uint8_t* w_scales, const float* w_g,
                                       const int32_t* expert_offsets,
                                       const int32_t* active_experts, const int32_t* n_active,
                                       int32_t E, int32_t rows, int32_t Nw, int32_t K, void* out,
                                       nvfp4moe_dtype out_dtype, float* out_amax, void* ws,
                                       size_t ws_bytes, void* stream);
size_t moe_grouped_gemm_workspace_size(nvfp4moe_mode mode, int64_t a_rows, int32_t rows,
                                       int32_t E, int32_t Nw, int32_t K);

/* ---------------------------------------------------------------------------
 * moe_grouped_gemm_nvfp4_combine -- the down GEMM and the weighted unpermute-reduce in one
 * call: per expert e, Y_rows = A_rows . W_e^T * w_g[e] (* a_g[0]) in float32 (as
 * moe_grouped_gemm_nvfp4 with EPI_NONE and F32 out, rows = T * k, no gather), then
 *     out[t, :] = bf16( sum_{j<k} topk_w[t, j] * Y[slot_to_row[t*k + j], :] )
 * with float32 multiply-adds in ascending j (as moe_unpermute_reduce). [P3] "Discovering the
 * sgl_kernel Alternative" (a fused MoE scatters the expert results back to the tokens).
 * The reduce runs inside the GEMM: the workgroup that stores the last of a token's k rows of
 * a column tile sums them (integer completion counters; no floating-point atomics, no
 * waiting), so out is bit for bit what moe_grouped_gemm_nvfp4 + moe_unpermute_reduce give.
 * When the call splits K (grids under one workgroup per CU) the reduce runs as a second
 * kernel of the call instead, with the same result.
 *   mode, a, a_scales, a_g, w_packed, w_scales, w_g, expert_offsets, active_experts,
 *   n_active, E, Nw, K    as for moe_grouped_gemm_nvfp4 (a has T * k rows).
 *   sorted_slot, slot_to_row, topk_w   device, as written by moe_route_permute for T tokens, k.
 *   T, k        T >= 1, 1 <= k <= min(E, 64), T * k <= 2^24, T * k * Nw < 2^31.
 *   out         device bf16 [T, Nw], 16-byte aligned.
 *   ws          moe_grouped_gemm_nvfp4_combine_workspace_size(mode, T, k, E, Nw, K) bytes,
 *               16-byte aligned (the GEMM's workspace, the float32 Y and the counters).
 * ------------------------------------------------------------------------- */
nvfp4moe_status moe_grouped_gemm_nvfp4_combine(nvfp4moe_mode mode, const void* a, const uint8_t* a_scales,
                                               const float* a_g, const uint8_t* w_packed,
                                               const uint8_t* w_scales, const float* w_g,
                                               const int32_t* expert_offsets,
                                               const int32_t* active_experts, const int32_t* n_active,
                                               const int32_t* sorted_slot, const int32_t* slot_to_row,
                                               const float* topk_w, int32_t E, int32_t T, int32_t k,
                                               int32_t Nw, int32_t K, void* out, void* ws,
                                               size_t ws_bytes, void* stream);
size_t moe_grouped_gemm_nvfp4_combine_workspace_size(nvfp4moe_mode mode, int32_t T, int32_t k, int32_t E,
                                                     int32_t Nw, int32_t K);

/* ---------------------------------------------------------------------------
 * moe_unpermute_reduce -- out[t, :] = bf16( sum_{j<k} topk_w[t, j] * y[slot_to_row[t*k+j], :] )
 * accumulated in float32 in ascending j. [P3] "Discovering the sgl_kernel Alternative"
 * (results scattered back from the experts to the tokens).
 *
 *   y           device, y_dtype (F32 or BF16), [T * k, H].
 *   slot_to_row device int32 [T * k]; topk_w device float [T, k].
 *   T, k, H     T >= 1, k >= 1, H >= 8, H % 8 == 0, T * k * H < 2^31; y, out 16-byte aligned.
 *   out         device bf16 [T, H].
 * ------------------------------------------------------------------------- */
nvfp4moe_status moe_unpermute_reduce(const void* y, nvfp4moe_dtype y_dtype,
                                     const int32_t* slot_to_row, const float* topk_w, int32_t T,
                                     int32_t k, int32_t H, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * act_fp8_e4m3_roundtrip -- FP8 E4M3 activations dequantized to bf16, per-tensor scale.
 * [P1] section 1 ("FP4 weights with FP8 activations").
 *   s_a = amax(|x|) / 448 (1 if amax == 0);  out = bf16( E4M3(min(|x / s_a|, 448)) * s_a )
 *   with the sign of x (float32 steps, round-to-nearest-even).
 *   x, out   device bf16 [n], 16-byte aligned (may alias); n >= 8, n % 8 == 0.
 *   ws       act_fp8_e4m3_roundtrip_workspace_size(n) bytes.
 * ------------------------------------------------------------------------- */
nvfp4moe_status act_fp8_e4m3_roundtrip(const void* x, int64_t n, void* out, void* ws,
                                       size_t ws_bytes, void* stream);
size_t act_fp8_e4m3_roundtrip_workspace_size(int64_t n);

/* ---------------------------------------------------------------------------
 * MXFP4 variant: FP4 (E2M1, codes and packing as above) with one UE8M0 scale per 32
 * elements and no per-tensor scale ([P2] "The NVFP4 Pivot": "MXFP4 (group-32, UE8M0)").
 * UE8M0 code s is 2^(s - 127) (s = 0..254) and NaN for s = 255; a value decodes as
 * E2M1[q] * 2^(s - 127).
 *
 * mxfp4_quantize -- quantize float rows [R, C] to MXFP4, per 32-group along C (the OCP MX
 * v1.0 conversion rule): e = max(floor(log2 amax) - 2, -127), scale byte e + 127, codes
 * E2M1_RNE_saturating(x * 2^-e) with the sign of x; NaN/Inf group -> scale 0xFF, codes 0;
 * all-zero group -> scale 0, codes +-0.
 *   x        device, x_dtype (F32 or BF16), [R, C] row-major, 16-byte aligned.
 *   R, C     R >= 1, C >= 32, C % 32 == 0.
 *   packed   device uint8 [R, C/2] (output), 16-byte aligned.
 *   scales   device uint8 [R, C/32] (output).
 * ------------------------------------------------------------------------- */
nvfp4moe_status mxfp4_quantize(const void* x, nvfp4moe_dtype x_dtype, int64_t R, int64_t C, uint8_t* packed,
                               uint8_t* scales, void* stream);

/* ---------------------------------------------------------------------------
 * mxfp4_weights_tile -- reorder B MXFP4 matrices [R, C] (as written by mxfp4_quantize)
 * into the storage moe_grouped_gemm_mxfp4 reads: the codes exactly as nvfp4_weights_tile
 * tiles them (nvfp4_tiled_codes_bytes(R, C) per matrix), the scales in 1 KB tiles per
 * (matrix b, row block rb, window w of 16 chunks of 128 columns) at
 * ((b * R/16 + rb) * ceil(C/2048) + w) * 1024, where lane l = 16 g + r holds 16 bytes: at
 * byte u the scale of columns 128 (16 w + u) + 32 g .. +31 of row 16 rb + r (zero where
 * the columns are >= C). A permutation plus zero padding; no value changes.
 *   B, R, C         1 <= B <= 65535, R >= 16, R % 16 == 0, C >= 32, C % 32 == 0,
 *                   B * R * C / 2 < 2^40; packed and both outputs 16-byte aligned.
 *   tiled_scales    device uint8 [B * mxfp4_tiled_scales_bytes(R, C)] (output).
 * mxfp4_tiled_scales_bytes returns 0 for an invalid R or C.
 * ------------------------------------------------------------------------- */
size_t mxfp4_tiled_scales_bytes(int64_t R, int64_t C);
nvfp4moe_status mxfp4_weights_tile(const uint8_t* packed, const uint8_t* scales, int64_t B, int64_t R, int64_t C,
                                   uint8_t* tiled_codes, uint8_t* tiled_scales, void* stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_gemm_mxfp4 -- W4A4 grouped GEMM with MXFP4 weights and activations:
 * per expert e, rows expert_offsets[e] .. expert_offsets[e+1]:
 *     P = A_rows . W_e^T  (float32 accumulation of the exact products E2M1 * 2^s)
 *     EPI_NONE: out = P [rows, Nw];  EPI_SWIGLU: out = silu(P[:, :Nw/2]) * P[:, Nw/2:]
 * on the scaled FP4 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4), whose operands are
 * MXFP4 blocks as stored. [P2] "The NVFP4 Pivot" (MXFP4), [P3] "Discovering the sgl_kernel
 * Alternative" (block-scaled FP4 GEMM on two FP4 operands).
 *   a, a_scales  device uint8 [a_rows, K/2] and [a_rows, K/32] (mxfp4_quantize output); a
 *                16-byte aligned.
 *   gather_index, gather_div, expert_offsets, active_experts, n_active, E, rows, out,
 *   out_dtype, out_amax   as for moe_grouped_gemm_nvfp4.
 *   w_packed, w_scales    E expert matrices [Nw, K] as written by mxfp4_weights_tile,
 *                16-byte aligned.
 *   Nw, K        Nw % 256 == 0 (else NVFP4MOE_ERR_UNSUPPORTED), K >= 32, K % 32 == 0,
 *                rows * max(K, Nw), a_rows * K / 2 and Nw * K / 2 below 2^31.
 *   ws           moe_grouped_gemm_mxfp4_workspace_size(rows, E, Nw, K) bytes, 16-byte
 *                aligned: the device-built m-tile list and, when the grid is too small to
 *                fill the chip, fixed-order split-K partial sums. Returns 0 for invalid sizes.
 * ------------------------------------------------------------------------- */
nvfp4moe_status moe_grouped_gemm_mxfp4(nvfp4moe_epilogue epi, const uint8_t* a, const uint8_t* a_scales,
                                       int64_t a_rows, const int32_t* gather_index, int32_t gather_div,
                                       const uint8_t* w_packed, const uint8_t* w_scales,
                                       const int32_t* expert_offsets, const int32_t* active_experts,
                                       const int32_t* n_active, int32_t E, int32_t rows, int32_t Nw,
                                       int32_t K, void* out, nvfp4moe_dtype out_dtype, float* out_amax, void* ws,
                                       size_t ws_bytes, void* stream);
size_t moe_grouped_gemm_mxfp4_workspace_size(int32_t rows, int32_t E, int32_t Nw, int32_t K);

/* ---------------------------------------------------------------------------
 * moe_grouped_gemm_mxfp4_swiglu_q -- the SwiGLU call of moe_grouped_gemm_mxfp4 with h written
 * as MXFP4 straight from the epilogue: h = silu(P[:, :Nw/2]) * P[:, Nw/2:] in float32, then
 * per row and group of 32 columns the rule of mxfp4_quantize (so the codes and scales are
 * those mxfp4_quantize gives for the float32 h of the unquantized call, bit for bit). This is
 * the down GEMM's activation in the MXFP4 layer; MXFP4 has no per-tensor scale, so h needs no
 * pass over all of it first. [P2] "The NVFP4 Pivot" (MXFP4, group 32, UE8M0).
 *   All arguments as for moe_grouped_gemm_mxfp4 except:
 *   h_packed     device uint8 [rows, Nw/4] (output), 16-byte aligned: MXFP4 codes of h.
 *   h_scales     device uint8 [rows, Nw/64] (output), 4-byte aligned: UE8M0 scales of h.
 *   ws           moe_grouped_gemm_mxfp4_workspace_size(rows, E, Nw, K) bytes (K is never
 *                split in this call).
 * ------------------------------------------------------------------------- */
nvfp4moe_status moe_grouped_gemm_mxfp4_swiglu_q(const uint8_t* a, const uint8_t* a_scales, int64_t a_rows,
                                                const int32_t* gather_index, int32_t gather_div,
                                                const uint8_t* w_packed, const uint8_t* w_scales,
                                                const int32_t* expert_offsets, const int32_t* active_experts,
                                                const int32_t* n_active, int32_t E, int32_t rows, int32_t Nw,
                                                int32_t K, uint8_t* h_packed, uint8_t* h_scales, void* ws,
                                                size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_gemm_mxfp4_combine -- the MXFP4 down GEMM (as moe_grouped_gemm_mxfp4 with
 * EPI_NONE, F32 Y, rows = T * k, no gather) and the weighted unpermute-reduce in one call,
 * exactly as moe_grouped_gemm_nvfp4_combine: out bf16 [T, Nw] is bit for bit
 * moe_grouped_gemm_mxfp4 + moe_unpermute_reduce. [P3] "Discovering the sgl_kernel
 * Alternative". ws: moe_grouped_gemm_mxfp4_combine_workspace_size(T, k, E, Nw, K) bytes.
 * ------------------------------------------------------------------------- */
nvfp4moe_status moe_grouped_gemm_mxfp4_combine(const uint8_t* a, const uint8_t* a_scales, const uint8_t* w_packed,
                                               const uint8_t* w_scales, const int32_t* expert_offsets,
                                               const int32_t* active_experts, const int32_t* n_active,
                                               const int32_t* sorted_slot, const int32_t* slot_to_row,
                                               const float* topk_w, int32_t E, int32_t T, int32_t k,
                                               int32_t Nw, int32_t K, void* out, void* ws, size_t ws_bytes,
                                               void* stream);
size_t moe_grouped_gemm_mxfp4_combine_workspace_size(int32_t T, int32_t k, int32_t E, int32_t Nw, int32_t K);

/* ---------------------------------------------------------------------------
 * MXFP8 (block-scaled FP8): FP8 E4M3 codes, one per byte, with one UE8M0 scale per 32
 * elements and no per-tensor scale; the block-scaled FP8 dense GEMM next to the MoE layer
 * ([P1] sections 1-2: FP8 activations, FP8 scaled-matmul kernels for the dense layers).
 * Storage of a matrix [R, C]: codes uint8 [R, C] (OCP E4M3FN), scales uint8 [R, C/32].
 *
 * mxfp8_quantize -- float rows [R, C] to MXFP8 per 32-group along C (OCP MX v1.0 rule with
 * E4M3 elements): e = max(floor(log2 amax) - 8, -127), scale byte e + 127, codes
 * E4M3_RNE(min(|x| * 2^-e, 448)) with the sign of x; NaN/Inf groups scale 0xFF and codes 0,
 * all-zero groups scale 0 and codes +-0.
 *   x              device float32 or bf16 [R, C], 16-byte aligned; C % 32 == 0.
 *   codes, scales  device uint8 [R, C] (16-byte aligned) and [R, C/32] (outputs).
 *
 * mxfp8_weights_tile -- B matrices [R, C] (R % 16 == 0) into the storage
 * moe_grouped_gemm_mxfp8 reads: code tiles of 2048 bytes per (16-row block, 128 columns; lane
 * 16 g + r holds columns 16 g .. +15 and 64 + 16 g .. +15 of row r, the scaled FP8 MFMA's
 * operand order),
 * scales tiled as by mxfp4_weights_tile (mxfp4_tiled_scales_bytes(R, C) per matrix).
 *   tiled_codes    device uint8 [B * mxfp8_tiled_codes_bytes(R, C)] (output), 16-byte aligned.
 * mxfp8_tiled_codes_bytes returns 0 for an invalid R or C.
 *
 * moe_grouped_gemm_mxfp8 -- W8A8 grouped GEMM on MXFP8 operands (the scaled FP8 matrix
 * cores, v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 on both sides): arguments as for
 * moe_grouped_gemm_mxfp4 with a [a_rows, K] codes + [a_rows, K/32] scales, weights as
 * written by mxfp8_weights_tile, and ws of moe_grouped_gemm_mxfp8_workspace_size(rows, E,
 * Nw, K) bytes. A dense GEMM is the call with E = 1 and expert_offsets {0, M}.
 * ------------------------------------------------------------------------- */
nvfp4moe_status mxfp8_quantize(const void* x, nvfp4moe_dtype x_dtype, int64_t R, int64_t C, uint8_t* codes,
                               uint8_t* scales, void* stream);
size_t mxfp8_tiled_codes_bytes(int64_t R, int64_t C);
nvfp4moe_status mxfp8_weights_tile(const uint8_t* codes, const uint8_t* scales, int64_t B, int64_t R, int64_t C,
                                   uint8_t* tiled_codes, uint8_t* tiled_scales, void* stream);
nvfp4moe_status moe_grouped_gemm_mxfp8(nvfp4moe_epilogue epi, const uint8_t* a, const uint8_t* a_scales,
                                       int64_t a_rows, const int32_t* gather_index, int32_t gather_div,
                                       const uint8_t* w_codes, const uint8_t* w_scales,
                                       const int32_t* expert_offsets, const int32_t* active_experts,
                                       const int32_t* n_active, int32_t E, int32_t rows, int32_t Nw,
                                       int32_t K, void* out, nvfp4moe_dtype out_dtype, float* out_amax, void* ws,
                                       size_t ws_bytes, void* stream);
size_t moe_grouped_gemm_mxfp8_workspace_size(int32_t rows, int32_t E, int32_t Nw, int32_t K);

/* Thread-local message describing the last non-OK status ("" if none). Never NULL. */
const char* nvfp4moe_last_error(void);
/* nvfp4moe_path of the last moe_grouped_gemm_nvfp4 call on this thread. */
int nvfp4moe_last_dispatch(void);
/* ABI version of this header (major * 100 + minor). */
int nvfp4moe_abi_version(void);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* NVFP4MOE_H */
