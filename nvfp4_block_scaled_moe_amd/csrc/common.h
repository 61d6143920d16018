// Device helpers shared by the gfx950 kernels of libnvfp4moe.
//
// Number formats (NVFP4 = FP4 E2M1 values with one E4M3 scale per 16 elements and a
// float32 per-tensor scale; "The Benchmark That Confirmed the Ceiling: NVFP4 Cutlass on
// sm_120", section "The NVFP4 Pivot"):
//   E2M1 : s.ee.m, bias 1, values {0, .5, 1, 1.5, 2, 3, 4, 6}; element 2i of a row is the
//          low nibble of byte i.
//   E4M3 : OCP E4M3FN, bias 7, NaN = 0x7F / 0xFF, max 448 (gfx950's native FP8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace nvfp4moe {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ host: per-device set-up
// Raise a kernel's dynamic-LDS limit once per device (the attribute is per device). `done`
// is one bit per device id < 64, owned by the caller (one per kernel).
inline hipError_t ensure_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float32 -> bf16 bits, round to nearest even; NaN stays (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// bf16 bits of a (low half) and b (high half) by the hardware pack: rounded to nearest even,
// the same bits as f32_to_bf16 for every float but NaN (which stays a NaN).
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// ------------------------------------------------------------------ E4M3
// E4M3FN byte -> float32 (exact; NaN for 0x7F/0xFF) with the hardware OCP FP8 convert.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Nearest E4M3 code (0..0x7E) to r in [0, 448], ties to the even code.
// Below 2^-6 the grid is uniform with step 2^-9 (subnormals), so the code is the
// integer nearest to r * 2^9 (ties to even; code 8 is 2^-6, the first normal).
// Above, keep 3 mantissa bits of the float32 with round-half-even on the dropped
// 20 bits; a carry moves into the exponent field, which is what E4M3 needs.
__device__ __forceinline__ uint32_t e4m3_rne(float r) {
  if (r < 0.015625f) return (uint32_t)__builtin_rintf(r * 512.0f);
  uint32_t u = __float_as_uint(r);
  u += 0x7ffffu + ((u >> 20) & 1u);
  return (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
}

// ------------------------------------------------------------------ E2M1
// Magnitude code 0..7 of the E2M1 value nearest to x >= 0 (ties to the even code,
// saturating at 6). The grid {0,.5,1,1.5,2,3,4,6} has midpoints .25,.75,1.25,1.75,
// 2.5,3.5,5; a midpoint rounds down when the lower neighbour's code is even.
__device__ __forceinline__ uint32_t e2m1_rne_mag(float x) {
  return (uint32_t)(x > 0.25f) + (uint32_t)(x >= 0.75f) + (uint32_t)(x > 1.25f) +
         (uint32_t)(x >= 1.75f) + (uint32_t)(x > 2.5f) + (uint32_t)(x >= 3.5f) +
         (uint32_t)(x > 5.0f);
}
// E2M1 codes (sign in bit 3) of a (bits 0-3) and b (bits 4-7), rounded to nearest even and
// saturating at 6, by the hardware converter with scale 1: for every finite x its code is
// sign(x) << 3 | e2m1_rne_mag(|x|) (the same bits, compared over all float bit patterns).
__device__ __forceinline__ uint32_t e2m1_pk(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0);
}

// ------------------------------------------------------------------ MXFP4 groups
// Group key of one element for the MXFP4 shared exponent: |v| as float bits when finite,
// 0xFFFFFFFF for NaN/Inf (above every finite key), so the max over a group is the finite
// amax, or the marker of a group with a non-finite element.
__device__ __forceinline__ uint32_t mx_key(float v) {
  const float a = fabsf(v);
  return a <= 3.402823466e38f ? __float_as_uint(a) : 0xFFFFFFFFu;
}
// Scale byte of a group from its key (OCP MX v1.0 rule, group of 32): NaN/Inf -> 0xFF;
// amax 0 -> 0; else e = max(floor(log2 amax) - emax, -127) (frexp gives floor(log2) exactly;
// emax is the element format's largest exponent: 2 for E2M1, 8 for E4M3) and byte e + 127.
// e is returned for the element codes (0 when unused).
__device__ __forceinline__ uint32_t mx_scale(uint32_t key, int& e, int emax = 2) {
  e = 0;
  if (key == 0xFFFFFFFFu) return 0xFFu;
  if (key == 0u) return 0u;
  int ex;
  (void)frexpf(__uint_as_float(key), &ex);   // amax = f * 2^ex, f in [0.5, 1)
  e = max(ex - 1 - emax, -127);
  return (uint32_t)(e + 127);
}
// MXFP8 element code: E4M3_RNE(min(|v| * 2^-e, 448)) with the sign bit of v; 0 in a
// non-finite group, +-0 in an all-zero group.
__device__ __forceinline__ uint32_t mx8_code(float v, uint32_t key, int e) {
  if (key == 0xFFFFFFFFu) return 0u;
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  return sign | (key != 0u ? e4m3_rne(fminf(ldexpf(fabsf(v), -e), 448.0f)) : 0u);
}
// Code (sign bit | E2M1 magnitude) of v in a group with the given key and exponent:
// E2M1_RNE_saturating(|v| * 2^-e), a power-of-two scaling (exact); 0 in a non-finite group,
// +-0 in an all-zero group.
__device__ __forceinline__ uint32_t mx_code(float v, uint32_t key, int e) {
  if (key == 0xFFFFFFFFu) return 0u;
  const uint32_t sign = (__float_as_uint(v) >> 31) << 3;
  return sign | (key != 0u ? e2m1_rne_mag(ldexpf(fabsf(v), -e)) : 0u);
}
// The codes of two elements of one group, v0 in bits 0-3 and v1 in bits 4-7 (the same bits as
// mx_code: in an all-zero group the values are +-0, whose codes are their sign bits).
__device__ __forceinline__ uint32_t mx_code2(float v0, float v1, uint32_t key, int e) {
  if (key == 0xFFFFFFFFu) return 0u;
  return e2m1_pk(ldexpf(v0, -e), ldexpf(v1, -e));
}

// ------------------------------------------------------------------ NVFP4 -> f16
// Eight E2M1 codes (one dword, element 0 in the low nibble) times an f16 block scale,
// as eight f16 values. The hardware convert produces the E2M1 values exactly (scale
// 1.0); the product E2M1 * E4M3 has at most 6 significant bits and lies in
// [2^-10, 2688], so the f16 multiply is exact as well. A NaN scale gives NaN.
__device__ __forceinline__ f16x8 decode8(uint32_t w, f16x2 s2) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Two consecutive E4M3 scale bytes (low byte first) -> their values as f16 pairs
// (s0, s0) and (s1, s1). E4M3 values are exact in f16.
__device__ __forceinline__ void decode_scale_pair(uint32_t two, f16x2& s0, f16x2& s1) {
  f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)two, false);
  f16 h0 = (f16)f[0], h1 = (f16)f[1];
  s0 = (f16x2){h0, h0};
  s1 = (f16x2){h1, h1};
}

// Read of a kernel input that stays constant while the kernel runs, through the constant
// address space: a wave-uniform read then becomes a scalar load, whose wait does not hold up
// the vector-memory queue (a vector load's wait also waits for every load issued before it).
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}
// A pointer that is the same in every lane (e.g. read from LDS) moved to scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// ------------------------------------------------------------------ wave helpers
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Key of |v| for a max over the finite values: the float bits of |v| when v is finite, 0 for
// NaN and +-Inf (float bits of non-negative floats order like the values).
__device__ __forceinline__ uint32_t finite_abs_bits(float v) {
  const uint32_t b = __float_as_uint(v) & 0x7fffffffu;
  return b < 0x7f800000u ? b : 0u;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o, kWave);
    v = v > w ? v : w;
  }
  return v;
}

// Wave-wide max of a uint32 through DPP moves (no LDS round trips): quad, half-row and row
// steps leave every row's max in all its lanes, the row broadcasts fold rows 0..3 into
// lane 63, which is read back as a wave-uniform value.
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v, int ctrl_id) {
  uint32_t t;
  switch (ctrl_id) {
    case 0: t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xb1, 0xf, 0xf, false); break;   // quad_perm 1,0,3,2
    case 1: t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4e, 0xf, 0xf, false); break;   // quad_perm 2,3,0,1
    case 2: t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false); break;  // row_half_mirror
    case 3: t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false); break;  // row_mirror
    case 4: t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false); break;  // row_bcast15
    default: t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false); break; // row_bcast31
  }
  return v > t ? v : t;
}
__device__ __forceinline__ uint32_t wave_max_u32_uniform(uint32_t v) {
#pragma unroll
  for (int s = 0; s < 6; ++s) v = dpp_max_u32(v, s);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

}  // namespace nvfp4moe
