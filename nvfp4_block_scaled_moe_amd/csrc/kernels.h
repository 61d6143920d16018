// Internal launch interface between the C ABI layer (api.hip) and the kernel files.
// Every launcher only enqueues work on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4moe {

// ---- quantize.hip
size_t quantize_ws_bytes(int64_t B, int64_t R, int64_t C);
// tiled: write codes and scales in the tiled storage of launch_weights_tile (R % 16 == 0).
hipError_t launch_quantize(const void* x, bool x_bf16, int64_t B, int64_t R, int64_t C,
                           const float* g_in, const float* amax_in, bool tiled, uint8_t* packed,
                           uint8_t* scales, float* g_out, void* ws, hipStream_t stream);
size_t fp8_roundtrip_ws_bytes(int64_t n);
hipError_t launch_fp8_roundtrip(const void* x, int64_t n, void* out, void* ws, hipStream_t stream);

// ---- route.hip
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;
// Workspace of launch_route_permute: the per-chunk expert counts of the two-launch permutation.
size_t route_permute_ws_bytes(int T, int E, int k);
// The token rows of a W4A16 dispatch: x [T, H] bf16 (after the FP8 E4M3 round trip when fp8)
// prepared for the GEMM into a16 [T, H128] f16 + rexp [T]; rows_ws: dispatch_rows_ws_bytes of
// scratch for the separate round trip (fp8 only).
struct ActPrep {
  const uint16_t* x;
  int H;
  int fp8;
  _Float16* a16;
  int* rexp;
  void* rows_ws;
};
size_t dispatch_rows_ws_bytes(int T, int H, bool fp8);
// Routing and permutation; with prep (nullable) also the token rows' preparation.
hipError_t launch_route_permute(const float* logits, int T, int E, int k, int* topk_ids,
                                float* topk_w, int* expert_offsets, int* sorted_slot,
                                int* slot_to_row, int* active_experts, int* n_active,
                                void* ws, size_t ws_bytes, hipStream_t stream, const ActPrep* prep = nullptr);

// ---- act_prep.hip
// The m-tile list of the large-M path, built by one extra workgroup of the activation prep
// launch (no launch of its own): for the active experts in list order, their m-tiles of bm
// rows; sched_e[i] = expert, sched_r[i] = first row within the expert, sched_n[0] = count (at
// most max_tiles, the length of sched_e and sched_r). max_tiles = 0: no list.
struct MtileSched {
  const int* offsets;
  const int* active;
  const int* n_active;
  int E, bm, max_tiles;
  int* sched_e;
  int* sched_r;
  int* sched_n;
};
// The m-tile list in a launch of its own.
hipError_t launch_mtile_schedule(const MtileSched& sched, hipStream_t stream);
// bf16 rows -> f16 rows scaled by 2^-p (max |x| in [2^14, 2^15)) + p
hipError_t launch_act_prep(const uint16_t* a, int64_t rows, int K, _Float16* a16, int* rexp,
                           const MtileSched& sched, hipStream_t stream);
// NVFP4 rows (codes + E4M3 scales) -> the same f16 layout, decoded exactly (E2M1 * E4M3, the
// global scale stays in the GEMM epilogue); rexp = 0.
hipError_t launch_act_prep_fp4(const uint8_t* packed, const uint8_t* scales, int64_t rows, int K,
                               _Float16* a16, int* rexp, const MtileSched& sched, hipStream_t stream);

// ---- grouped GEMM kernels
struct GemmArgs {
  int w4a4;                        // 0: W4A16 (a16 + rexp), 1: W4A4 (a_packed + a_scales + a_g)
  int a4_staged;                   // W4A4 on the large-M path: 1 = the GEMM decodes the NVFP4 rows
                                   // itself, 0 = it reads their f16 copy (a16) from the activation prep
  const _Float16* a16;             // [a_rows, K] f16, row r scaled by 2^-rexp[r]
  const int* rexp;                 // [a_rows]
  const uint8_t* a_packed;         // [a_rows, K/2]
  const uint8_t* a_scales;         // [a_rows, K/16]
  const float* a_g;                // [1]
  const int* gather_index;         // [rows] or null
  int gather_div;
  const uint8_t* w_packed;         // tiled codes, tiled_codes_bytes(Nw, K) per expert
  const uint8_t* w_scales;         // tiled scales, tiled_scales_bytes(Nw, K) per expert
  const float* w_g;                // [E]
  const int* expert_offsets;       // [E+1]
  const int* active;               // [E]
  const int* n_active;             // [1]
  int E, rows, Nw, K;
  int a_rows;                       // rows of the activation tensor (< 2^31 bytes of it)
  int swiglu;
  void* out;
  int out_bf16;
  float* out_amax;                 // null or [1], zeroed before the GEMM
  const int* sched_e;              // large-M path: m-tile -> expert   (workspace)
  const int* sched_r;              // large-M path: m-tile -> first row (workspace)
  const int* sched_n;              // large-M path: number of m-tiles  (workspace)
  float* partial;                  // large-M split-K: [ksplit, rows, Nw] fp32 partial sums (workspace)
  int ksplit;                      // large-M: K slices (1: no split)
  int unit_alpha;                  // MXFP4: no per-tensor scales (alpha = 1 in the split-K reduce)
  uint8_t* hq_packed;              // MXFP4 SwiGLU: h quantized in the epilogue, [rows, Nw/4] codes
  uint8_t* hq_scales;              //   and [rows, Nw/64] UE8M0 scales (null: out as usual)
  // Fused unpermute + weighted reduce (down GEMM, EPI_NONE, float32 out = Y, no split K):
  const int* comb_slot;            // [rows] sorted_slot: GEMM row -> slot (null: no combine)
  const int* comb_s2r;             // [T * k] slot_to_row
  const float* comb_w;             // [T * k] top-k weights
  int* comb_count;                 // [T * Nw/32] completion counters, zero before the GEMM
  uint16_t* comb_out;              // bf16 [T, Nw]
  int comb_k;
};
// Completion counters of the fused combine: one int per (token, 32 columns), zeroed.
inline size_t comb_count_ints(int T, int Nw) { return (size_t)T * (size_t)(Nw / 32); }
hipError_t launch_zero_i32(int* p, size_t n, hipStream_t stream);
hipError_t launch_gemm_stream(const GemmArgs& a, hipStream_t stream);
// K slices for the small-M path from the sizes alone (1 unless the grid is tiny).
int stream_ksplit(int rows, int E, int Nw, int K);
// Split-K epilogue shared by both GEMM paths: out (and out_amax) from the fixed-order sum of
// the ksplit partial-sum slices in a.partial.
hipError_t launch_splitk_reduce(const GemmArgs& a, hipStream_t stream);
// Tiled weight storage (weights_tile.hip): bytes per [R, C] matrix and the reordering.
size_t tiled_codes_bytes(int64_t R, int64_t C);
size_t tiled_scales_bytes(int64_t R, int64_t C);
hipError_t launch_weights_tile(const uint8_t* packed, const uint8_t* scales, int64_t B, int64_t R, int64_t C,
                               uint8_t* tiled_codes, uint8_t* tiled_scales, hipStream_t stream);
// MXFP4: the same code tiles; UE8M0 scales tiled per (16-row block, 16-chunk window).
size_t mx_tiled_scales_bytes(int64_t R, int64_t C);
hipError_t launch_mx_weights_tile(const uint8_t* packed, const uint8_t* scales, int64_t B, int64_t R, int64_t C,
                                  uint8_t* tiled_codes, uint8_t* tiled_scales, hipStream_t stream);
// MXFP8 (quantize.hip, weights_tile.hip): n elements (n % 32 == 0) -> E4M3 codes [n] + UE8M0
// scales [n/32]; code tiles of 2 KB per (16-row block, chunk), the mx scale tiles.
hipError_t launch_mx8_quantize(const void* x, bool x_bf16, int64_t n, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream);
size_t mx8_tiled_codes_bytes(int64_t R, int64_t C);
hipError_t launch_mx8_weights_tile(const uint8_t* codes, const uint8_t* scales, int64_t B, int64_t R, int64_t C,
                                   uint8_t* tiled_codes, uint8_t* tiled_scales, hipStream_t stream);
// MXFP4 quantizer (quantize.hip): n elements (n % 32 == 0) -> packed [n/2] + UE8M0 scales [n/32].
hipError_t launch_mx_quantize(const void* x, bool x_bf16, int64_t n, uint8_t* packed, uint8_t* scales,
                              hipStream_t stream);
// large-M path: rows per m-tile, the Nw it supports, and the launcher (max_mtiles is the host
// bound ceil(rows / rows_per_mtile) + min(E, rows) on the schedule length).
int large_rows_per_mtile();
bool large_supports(int Nw);
hipError_t launch_gemm_large(const GemmArgs& a, int max_mtiles, hipStream_t stream);
// K slices for the large-M path from the sizes alone (1 when the tiles fill the GPU).
int large_ksplit(int rows, int E, int Nw, int K);
// Waves per large-M workgroup (8, or 4 for small grids), from the sizes alone.
int large_waves(int rows, int E, int Nw);
// MXFP4 W4A4 GEMM on the scaled FP4 MFMA (gemm_mx.hip): m-tile rows, supported Nw, launcher
// (a.w_packed / a.w_scales: MX tiles; a.a_packed / a.a_scales: row-major MXFP4; the m-tile
// list in a.sched_*).
int mx_rows_per_mtile(int bits);   // MX element bits: 4 (MXFP4) or 8 (MXFP8)
bool mx_supports(int Nw);
hipError_t launch_gemm_mx(const GemmArgs& a, int max_mtiles, int bits, hipStream_t stream);
// K slices of the MXFP4 GEMM from the sizes alone (1 unless the grid is under one workgroup per CU).
int mx_ksplit(int max_mtiles, int Nw, int K);
hipError_t launch_zero_f32(float* p, int n, hipStream_t stream);

// ---- reduce.hip
hipError_t launch_unpermute_reduce(const void* y, bool y_bf16, const int* slot_to_row,
                                   const float* topk_w, int T, int k, int H, uint16_t* out,
                                   hipStream_t stream);

}  // namespace nvfp4moe
