// 16-bit activations for the f16 MFMA path (gfx950).
//
// W4A16 multiplies 16-bit activations by FP4 weights dequantized to 16 bits ("The 24%
// Ceiling", section "The Core Insight"). gfx950 has no packed bf16 multiply, but it has
// an exact, cheap NVFP4 -> f16 decode (one convert and one packed f16 multiply per two
// weights), so the GEMMs run on f16 MFMA. bf16 activations have float32's exponent range
// and f16 does not; each row is therefore scaled by a power of two 2^-p chosen so that
// its largest finite magnitude lies in [2^14, 2^15). Scaling by a power of two and the
// bf16 -> f16 conversion are exact for every value within 2^31 of the row maximum (f16
// keeps 11 significant bits, bf16 has 8); the GEMM epilogue multiplies by 2^p again.
// Non-finite values stay Inf/NaN.
//
// Output layout (the GEMM's operand order): rows padded with zeros to K128 = K rounded up
// to 128, and inside every 128-wide chunk the 8-element pieces are transposed: logical
// k = 32*g + 8*j + i is stored at 32*j + 8*g + i. The GEMM lane group g feeds MFMA j with
// logical k 32g+8j..+7, so the four lane groups of one token read 64 contiguous bytes per
// load instruction (one cache line instead of four).
//
// One workgroup per row (bf16 input): the row is read once into registers (K up to 32768; longer
// rows are read twice), its finite amax reduced, then converted. Traffic: 2 bytes read + 2 bytes
// written per element.
#include "act_rows.h"
#include "common.h"
#include "kernels.h"

namespace nvfp4moe {

namespace {

constexpr int kPrepThreads = 256;

// The m-tile list (MtileSched) by one workgroup of kPrepThreads threads: thread a takes the
// active-list slots 4a .. 4a+3 (kMaxExperts = 1024 slots), a workgroup scan gives each its
// first list position, and it writes its experts' m-tiles in list order.
__device__ void mtile_schedule_block(const MtileSched& s) {
  static_assert(4 * kPrepThreads >= kMaxExperts, "four active-list slots per thread");
  __shared__ int wsum[kPrepThreads / kWave];
  const int a = threadIdx.x, lane = a & 63, wave = a >> 6;
  const int na = min(s.n_active[0], s.E);
  int e[4], cnt[4], tot = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * a + q;
    e[q] = i < na ? s.active[i] : 0;
    cnt[q] = i < na ? (s.offsets[e[q] + 1] - s.offsets[e[q]] + s.bm - 1) / s.bm : 0;
    tot += cnt[q];
  }
  int incl = tot;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < kPrepThreads / kWave; ++w) {
    if (w < wave) before += wsum[w];
    total += wsum[w];
  }
  int base = before + incl - tot;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    for (int i = 0; i < cnt[q] && base + i < s.max_tiles; ++i) {
      s.sched_e[base + i] = e[q];
      s.sched_r[base + i] = i * s.bm;
    }
    base += cnt[q];
  }
  if (a == 0) s.sched_n[0] = min(total, s.max_tiles);
}

// The m-tile list alone (for GEMMs with no activation prep, such as MXFP4 W4A4).
__global__ __launch_bounds__(kPrepThreads) void mtile_schedule_kernel(const MtileSched sched) {
  mtile_schedule_block(sched);
}

// VPT = 16-byte vectors held per thread (K <= 8 * kPrepThreads * VPT): the row is read once
// into registers, its amax reduced, then converted from the registers.
// With sched.max_tiles > 0, workgroup 0 builds the m-tile list (dispatched first, its chain
// of dependent reads overlaps the conversion) and workgroup r + 1 converts row r.
template <int VPT>
__global__ __launch_bounds__(kPrepThreads) void act_prep_kernel(const uint16_t* __restrict__ a,
                                                                int K,
                                                                _Float16* __restrict__ a16,
                                                                int* __restrict__ rexp, int64_t rows,
                                                                const MtileSched sched) {
  const int64_t r = (int64_t)blockIdx.x - (sched.max_tiles > 0 ? 1 : 0);
  if (r < 0) {
    mtile_schedule_block(sched);
    return;
  }
  const int K128 = (K + 127) & ~127;
  const uint16_t* row = a + r * (int64_t)K;
  _Float16* orow = a16 + r * (int64_t)K128;
  const int nvec = K / 8;
  uint4 q[VPT];
  float m = 0.0f;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int i = threadIdx.x + v * kPrepThreads;
    q[v] = i < nvec ? *reinterpret_cast<const uint4*>(row + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t w[4] = {q[v].x, q[v].y, q[v].z, q[v].w};
    m = bf16x8_finite_max(w, m);
  }
  __shared__ float red[kPrepThreads / kWave];
  m = wave_max(m);
  if ((threadIdx.x % kWave) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  float amax = red[0];
  for (int w = 1; w < kPrepThreads / kWave; ++w) amax = fmaxf(amax, red[w]);
  const int p = f16_row_exponent(amax);
  if (threadIdx.x == 0) rexp[r] = p;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int i = threadIdx.x + v * kPrepThreads;
    if (i < K128 / 8) {
      const uint32_t w[4] = {q[v].x, q[v].y, q[v].z, q[v].w};   // zeros past K
      *reinterpret_cast<f16x8*>(orow + 8 * prepared_piece(i)) = bf16x8_to_f16(w, p);
    }
  }
}

// Rows too long for registers: pass 1 finds the amax, pass 2 re-reads the row (from L2) and
// converts.
__global__ __launch_bounds__(kPrepThreads) void act_prep_loop_kernel(const uint16_t* __restrict__ a,
                                                                     int K,
                                                                     _Float16* __restrict__ a16,
                                                                     int* __restrict__ rexp, int64_t rows,
                                                                     const MtileSched sched) {
  const int64_t r = (int64_t)blockIdx.x - (sched.max_tiles > 0 ? 1 : 0);
  if (r < 0) {
    mtile_schedule_block(sched);
    return;
  }
  const int K128 = (K + 127) & ~127;
  const uint16_t* row = a + r * (int64_t)K;
  _Float16* orow = a16 + r * (int64_t)K128;
  const int nvec = K / 8;
  float m = 0.0f;
  for (int i = threadIdx.x; i < nvec; i += kPrepThreads) {
    const uint4 q = *reinterpret_cast<const uint4*>(row + 8 * i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    m = bf16x8_finite_max(w, m);
  }
  __shared__ float red[kPrepThreads / kWave];
  m = wave_max(m);
  if ((threadIdx.x % kWave) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  float amax = red[0];
  for (int w = 1; w < kPrepThreads / kWave; ++w) amax = fmaxf(amax, red[w]);
  const int p = f16_row_exponent(amax);
  if (threadIdx.x == 0) rexp[r] = p;
  for (int i = threadIdx.x; i < K128 / 8; i += kPrepThreads) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (i < nvec) {
      const uint4 q = *reinterpret_cast<const uint4*>(row + 8 * i);
      w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
    }
    *reinterpret_cast<f16x8*>(orow + 8 * prepared_piece(i)) = bf16x8_to_f16(w, p);
  }
}

// NVFP4 activations -> f16 for the large-M path. Each thread decodes one 32-element group
// (16 bytes of codes and its two E4M3 scales) exactly, as E2M1 value times block scale (<= 6
// significant bits, magnitudes 2^-10 .. 2688, all exact in f16), into the layout above; the
// per-tensor scale is applied in the GEMM epilogue, so rexp = 0. Groups past K are zero.
__global__ __launch_bounds__(kPrepThreads) void act_prep_fp4_kernel(const uint8_t* __restrict__ packed,
                                                                    const uint8_t* __restrict__ scales,
                                                                    int64_t rows, int K,
                                                                    _Float16* __restrict__ a16,
                                                                    int* __restrict__ rexp,
                                                                    const MtileSched sched) {
  const int K128 = (K + 127) & ~127;
  const int gpr = K128 / 32;   // groups per padded row
  const int64_t blk = (int64_t)blockIdx.x - (sched.max_tiles > 0 ? 1 : 0);
  if (blk < 0) {   // workgroup 0 builds the m-tile list
    mtile_schedule_block(sched);
    return;
  }
  const int64_t i = blk * kPrepThreads + threadIdx.x;
  if (i >= rows * gpr) return;
  const int64_t r = i / gpr;
  const int q = (int)(i - r * gpr);   // group: logical k 32q .. 32q+31
  const int c = q >> 2, g = q & 3;
  _Float16* orow = a16 + r * (int64_t)K128;
  f16x8 o[4];
  if (32 * q < K) {
    const uint4 w = *reinterpret_cast<const uint4*>(packed + r * (int64_t)(K / 2) + 16 * q);
    const uint32_t sv = *reinterpret_cast<const uint16_t*>(scales + r * (int64_t)(K / 16) + 2 * q);
    f16x2 s0, s1;
    decode_scale_pair(sv, s0, s1);
    o[0] = decode8(w.x, s0);
    o[1] = decode8(w.y, s0);
    o[2] = decode8(w.z, s1);
    o[3] = decode8(w.w, s1);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (f16x8){0, 0, 0, 0, 0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) *reinterpret_cast<f16x8*>(orow + 8 * (16 * c + 4 * j + g)) = o[j];
  if (q == 0) rexp[r] = 0;
}

}  // namespace

hipError_t launch_mtile_schedule(const MtileSched& sched, hipStream_t stream) {
  mtile_schedule_kernel<<<1, kPrepThreads, 0, stream>>>(sched);
  return hipGetLastError();
}

hipError_t launch_act_prep_fp4(const uint8_t* packed, const uint8_t* scales, int64_t rows, int K,
                               _Float16* a16, int* rexp, const MtileSched& sched, hipStream_t stream) {
  const int64_t n = rows * (((K + 127) & ~127) / 32);
  const unsigned blocks = (unsigned)((n + kPrepThreads - 1) / kPrepThreads) + (sched.max_tiles > 0 ? 1u : 0u);
  act_prep_fp4_kernel<<<blocks, kPrepThreads, 0, stream>>>(packed, scales, rows, K, a16, rexp, sched);
  return hipGetLastError();
}

hipError_t launch_act_prep(const uint16_t* a, int64_t rows, int K, _Float16* a16, int* rexp,
                           const MtileSched& sched, hipStream_t stream) {
  // vectors per thread covering K128 / 8 pieces (padding pieces are written as zeros)
  const int need = ((K + 127) / 128 * 16 + kPrepThreads - 1) / kPrepThreads;
  const unsigned blocks = (unsigned)rows + (sched.max_tiles > 0 ? 1u : 0u);
  if (need <= 2) act_prep_kernel<2><<<blocks, kPrepThreads, 0, stream>>>(a, K, a16, rexp, rows, sched);
  else if (need <= 4) act_prep_kernel<4><<<blocks, kPrepThreads, 0, stream>>>(a, K, a16, rexp, rows, sched);
  else if (need <= 8) act_prep_kernel<8><<<blocks, kPrepThreads, 0, stream>>>(a, K, a16, rexp, rows, sched);
  else if (need <= 16) act_prep_kernel<16><<<blocks, kPrepThreads, 0, stream>>>(a, K, a16, rexp, rows, sched);
  else act_prep_loop_kernel<<<blocks, kPrepThreads, 0, stream>>>(a, K, a16, rexp, rows, sched);
  return hipGetLastError();
}

}  // namespace nvfp4moe
