// Pieces shared by the two grouped-GEMM kernels (gemm_stream.hip, gemm_large.hip): buffer
// loads and the epilogue.
#pragma once

#include "common.h"
#include "kernels.h"

namespace nvfp4moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 128;              // k per chunk (16 bytes of FP4 per lane)
constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past every resource: loads return 0
constexpr int kRsrcFlags = 0x00020000;   // raw buffer resource word 3 for gfx9 (32-bit data)

template <int N>
struct Int {
  static constexpr int value = N;
};

// Raw buffer resource over [base, base + bytes): 32-bit offsets, loads past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcFlags);
}
__device__ __forceinline__ u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}


// Four consecutive output values at element offset o of p.out (f32, or bf16 rounded to
// nearest even); returns amax_bits merged with the finite |value|s as written. The float32 Y
// of a combine call is stored with device-scope stores (coherent across the XCDs' L2
// caches without a write-back of the L2), which the fused reduce of another workgroup reads.
__device__ __forceinline__ uint32_t store4(const GemmArgs& p, size_t o, const float (&v)[4], uint32_t amax_bits) {
  const bool amax = p.out_amax != nullptr;   // the |value| bits are only gathered when asked for
  if (p.comb_slot) {
    if (amax) {
#pragma unroll
      for (int i = 0; i < 4; ++i) amax_bits = max(amax_bits, finite_abs_bits(v[i]));
    }
    uint64_t* q = reinterpret_cast<uint64_t*>(static_cast<float*>(p.out) + o);
    const uint64_t lo = (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32);
    const uint64_t hi = (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32);
    __hip_atomic_store(q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (p.out_bf16) {
    const uint32_t b01 = bf16x2(v[0], v[1]), b23 = bf16x2(v[2], v[3]);
    if (amax) {
      amax_bits = max(amax_bits, finite_abs_bits(__uint_as_float(b01 << 16)));
      amax_bits = max(amax_bits, finite_abs_bits(__uint_as_float(b01 & 0xffff0000u)));
      amax_bits = max(amax_bits, finite_abs_bits(__uint_as_float(b23 << 16)));
      amax_bits = max(amax_bits, finite_abs_bits(__uint_as_float(b23 & 0xffff0000u)));
    }
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) = make_uint2(b01, b23);
  } else {
    if (amax) {
#pragma unroll
      for (int i = 0; i < 4; ++i) amax_bits = max(amax_bits, finite_abs_bits(v[i]));
    }
    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + o) = make_float4(v[0], v[1], v[2], v[3]);
  }
  return amax_bits;
}

// silu(gate) * up, the SwiGLU of one output element (shared by every epilogue so that
// equal inputs give equal bits): gate / (1 + e^-gate) * up with the hardware base-2
// exponential and reciprocal, e^-gate = 2^(-gate log2 e). Relative error below
// |gate| 2^-24 + 4 ulp (about 1e-6 for |gate| < 16); +-Inf and NaN gates give the values
// of the exact formula (NaN for -Inf, Inf * up for +Inf).
__device__ __forceinline__ float swiglu1(float gv, float uv) {
  const float e = __builtin_amdgcn_exp2f(-1.44269504088896341f * gv);
  return gv * __builtin_amdgcn_rcpf(1.0f + e) * uv;
}

// Epilogue of one wave's tile: RBW blocks of 16 weight rows x TBM blocks of 16 GEMM rows,
// with MFMA 16x16 output layout (lane l holds weight rows 4*(l/16)+i of each block, GEMM
// row l%16 of each token block). GEMM rows tc .. tc+16*ntb-1 of the expert (those < M) are
// written: out = acc * alpha * 2^pexp, where pexp is the activation row's power-of-two
// scale (W4A16) or 0; with SwiGLU the first RBW/2 blocks are gate rows and the others the
// matching up rows, and silu(gate) * up is written to column blkrow(b) of the F-wide output.
// Returns the running max of |written value| over the finite values written (NaN and Inf
// excluded; with a bf16 output, of the rounded values) as float bits.
// pexp[tb] is the power-of-two exponent of the lane's GEMM row in token block tb.
template <int RBW, int TBM, bool SWIGLU, typename BlkRow>
__device__ __forceinline__ uint32_t store_tile_exp(const GemmArgs& p, const f32x4 (&acc)[RBW][TBM], int tc,
                                                   int ntb, int M, int r0, float alpha, const int (&pexps)[TBM],
                                                   BlkRow blkrow, int lane, uint32_t amax_bits) {
  const int l16 = lane & 15, g = lane >> 4;
  const int Nw = p.Nw, F = Nw >> 1;
#pragma unroll
  for (int tb = 0; tb < TBM; ++tb) {
    const int t = tc + 16 * tb + l16;
    if (tb < ntb && t < M) {
      const int row = r0 + t;
      const int pexp = pexps[tb];
      if (SWIGLU) {
#pragma unroll
        for (int b = 0; b < RBW / 2; ++b) {
          float h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gv = ldexpf(acc[b][tb][i] * alpha, pexp);
            const float uv = ldexpf(acc[b + RBW / 2][tb][i] * alpha, pexp);
            h[i] = swiglu1(gv, uv);
          }
          const size_t o = (size_t)row * F + blkrow(b) + 4 * g;
          amax_bits = store4(p, o, h, amax_bits);
        }
      } else {
#pragma unroll
        for (int b = 0; b < RBW; ++b) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[i] = ldexpf(acc[b][tb][i] * alpha, pexp);
          }
          const size_t o = (size_t)row * Nw + blkrow(b) + 4 * g;
          amax_bits = store4(p, o, v, amax_bits);
        }
      }
    }
  }
  return amax_bits;
}

// Power-of-two exponent of each of the lane's GEMM rows (0 without row scales or past M).
template <int TBM>
__device__ __forceinline__ void row_exponents(const GemmArgs& p, int tc, int M, int r0, bool row_exp, int lane,
                                              int (&pexps)[TBM]) {
#pragma unroll
  for (int tb = 0; tb < TBM; ++tb) {
    const int t = tc + 16 * tb + (lane & 15);
    const int row = r0 + t;
    pexps[tb] = row_exp && t < M ? p.rexp[p.gather_index ? p.gather_index[row] / p.gather_div : row] : 0;
  }
}

template <int RBW, int TBM, bool SWIGLU, typename BlkRow>
__device__ __forceinline__ uint32_t store_tile(const GemmArgs& p, const f32x4 (&acc)[RBW][TBM], int tc,
                                               int ntb, int M, int r0, float alpha, bool row_exp,
                                               BlkRow blkrow, int lane, uint32_t amax_bits) {
  int pexps[TBM];
  row_exponents<TBM>(p, tc, M, r0, row_exp, lane, pexps);
  return store_tile_exp<RBW, TBM, SWIGLU>(p, acc, tc, ntb, M, r0, alpha, pexps, blkrow, lane, amax_bits);
}

// Fused unpermute + weighted top-k reduce at the end of a down-GEMM tile (the scatter back
// from the experts to the tokens of a fused MoE: "The 2x Gap: Diagnosing Suboptimal FP4 GEMM
// Kernels on Blackwell SM120", section "Discovering the sgl_kernel Alternative").
// The workgroup (NT threads, all of them calling) has stored float32 Y rows [row0, row0 +
// nrows) x columns [col0, col0 + ncols) (ncols % 4 == 0, nrows <= kCombMaxRows) into p.out
// with device-scope stores (store4). For each of its rows it bumps the integer counter of
// (token of the row's slot, column tile); the workgroup whose bump brings a token's counter
// to k has all k rows of that token for this column tile in memory, and it writes
//     comb_out[t, c] = bf16( sum_{j<k} w[t, j] * Y[slot_to_row[t*k + j], c] )
// with float32 fused multiply-adds in ascending j: the arithmetic of the unpermute-reduce
// kernel, so the bits do not depend on which workgroup finishes a token last.
// Ordering without cache flushes: every wave waits for its own device-scope Y stores to
// complete (vmcnt 0) before the barrier that precedes the bumps, and the finishing workgroup
// reads Y with device-scope loads, issued after the barrier that follows the bump it observed.
// (A release/acquire fence at device scope would write back and invalidate the whole L2 of the
// XCD at every tile: measured 7x slower.) No workgroup ever waits for another.
constexpr int kCombMaxRows = 128;
constexpr int kCombBatch = 8;
template <int NT>
__device__ __forceinline__ void combine_tile(const GemmArgs& p, int row0, int nrows, int col0, int ncols) {
  __shared__ int tok[kCombMaxRows];
  __shared__ int ntok;
  const int tid = threadIdx.x;
  const int k = p.comb_k, Nw = p.Nw;
  const int stride = Nw >> 5, ctile = col0 >> 5;
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's Y stores have completed
  if (tid == 0) ntok = 0;
  __syncthreads();
  for (int i = tid; i < nrows; i += NT) {
    const int t = p.comb_slot[row0 + i] / k;
    const int old = __hip_atomic_fetch_add(p.comb_count + (size_t)t * stride + ctile, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    if (old == k - 1) tok[atomicAdd(&ntok, 1)] = t;
  }
  __syncthreads();
  const int n = ntok;
  if (n == 0) return;
  const float* y = static_cast<const float*>(p.out);
  const int c4 = ncols >> 2;
  for (int i = tid; i < n * c4; i += NT) {
    const int t = tok[i / c4];
    const int c = col0 + 4 * (i - (i / c4) * c4);
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    // The rows of up to kCombBatch slots are requested before the first of them is summed
    // (their latencies overlap); the sum itself stays in ascending j.
    for (int j0 = 0; j0 < k; j0 += kCombBatch) {
      uint64_t lo[kCombBatch], hi[kCombBatch];
      float w[kCombBatch];
#pragma unroll
      for (int j = 0; j < kCombBatch; ++j) {
        const bool in = j0 + j < k;
        const size_t row = in ? (size_t)p.comb_s2r[(size_t)t * k + j0 + j] : 0;
        w[j] = in ? p.comb_w[(size_t)t * k + j0 + j] : 0.f;
        const uint64_t* q = reinterpret_cast<const uint64_t*>(y + row * Nw + c);
        lo[j] = in ? __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
        hi[j] = in ? __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
      }
#pragma unroll
      for (int j = 0; j < kCombBatch; ++j) {
        if (j0 + j < k) {
          a0 = fmaf(w[j], __uint_as_float((uint32_t)lo[j]), a0);
          a1 = fmaf(w[j], __uint_as_float((uint32_t)(lo[j] >> 32)), a1);
          a2 = fmaf(w[j], __uint_as_float((uint32_t)hi[j]), a2);
          a3 = fmaf(w[j], __uint_as_float((uint32_t)(hi[j] >> 32)), a3);
        }
      }
    }
    *reinterpret_cast<uint2*>(p.comb_out + (size_t)t * Nw + c) =
        make_uint2(bf16x2(a0, a1), bf16x2(a2, a3));
  }
}

// Wave-reduced amax of the tile (finite values only), merged into *out_amax (float bits of
// non-negative values order like the values).
__device__ __forceinline__ void merge_amax(float* out_amax, uint32_t amax_bits, int lane) {
  if (!out_amax) return;
  amax_bits = wave_max_u32(amax_bits);
  if (lane == 0 && amax_bits) atomicMax(reinterpret_cast<unsigned int*>(out_amax), amax_bits);
}

}  // namespace nvfp4moe
