// Per-row activation arithmetic shared by the activation prep launch (act_prep.hip), the FP8
// round trip (quantize.hip) and the few-token dispatch that routes and prepares in one launch
// (route.hip), so that every path produces the same bits.
#pragma once

#include "common.h"

namespace nvfp4moe {

// |v| for finite v, 0 for NaN and +-Inf (both fail the compare): the maxima below are taken
// over the finite entries.
__device__ __forceinline__ float finite_abs(float v) {
  const float a = fabsf(v);
  return (a <= 3.402823466e38f) ? a : 0.0f;
}

// ---- FP8 E4M3 activations with a per-tensor scale ("Native FP4 Is Slower Than Emulated FP4",
// section 1): s = amax / 448 over the finite entries (1 when that amax is 0); each value goes
// to the nearest E4M3 code of v / s (saturating at 448, sign kept) and back as bf16(code * s).
__device__ __forceinline__ float fp8_scale(float amax) { return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f); }

// bf16 bits of the round trip of v (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t fp8_roundtrip_bits(float v, float s) {
  if (v != v) return 0x7fc0u;
  const float r = __fdiv_rn(v, s);
  const float mag = e4m3_to_f32(e4m3_rne(fminf(fabsf(r), 448.0f)));
  const float q = (__float_as_uint(r) >> 31) ? -mag : mag;
  return f32_to_bf16(q * s);
}

// ---- bf16 rows -> f16 rows for the f16 matrix cores (W4A16). A row is scaled by 2^-p so that
// its largest finite magnitude lies in [2^14, 2^15); the scaling and the bf16 -> f16
// conversion are exact for every value within 2^31 of that maximum, and the GEMM epilogue
// multiplies by 2^p again.
__device__ __forceinline__ int f16_row_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ex;
  (void)frexpf(amax, &ex);   // amax = f * 2^ex, f in [0.5, 1)
  return ex - 15;            // amax * 2^-p in [2^14, 2^15)
}

// Eight bf16 values (packed two per word) scaled by 2^-p and converted to f16.
__device__ __forceinline__ f16x8 bf16x8_to_f16(const uint32_t (&w)[4], int p) {
  f16x8 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = (_Float16)ldexpf(bf16_to_f32(w[j] & 0xffffu), -p);
    o[2 * j + 1] = (_Float16)ldexpf(bf16_to_f32(w[j] >> 16), -p);
  }
  return o;
}

// Finite maximum of |value| over eight bf16 values.
__device__ __forceinline__ float bf16x8_finite_max(const uint32_t (&w)[4], float m) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m = fmaxf(m, finite_abs(bf16_to_f32(w[j] & 0xffffu)));
    m = fmaxf(m, finite_abs(bf16_to_f32(w[j] >> 16)));
  }
  return m;
}

// Prepared rows are padded with zeros to whole 128-wide chunks and hold the GEMM's operand
// order: inside each chunk the 8-element pieces are transposed, logical k = 32 g + 8 j + i
// stored at 32 j + 8 g + i, so that the four lane groups of a token read 64 contiguous bytes
// per load. Position (in pieces) of logical piece i:
__device__ __forceinline__ int prepared_piece(int i) {
  const int c = i >> 4, g = (i >> 2) & 3, j = i & 3;
  return 16 * c + 4 * j + g;
}

}  // namespace nvfp4moe
