// NVFP4 quantization and the FP8 E4M3 activation round trip (gfx950).
//
// NVFP4 ("The Benchmark That Confirmed the Ceiling: NVFP4 Cutlass on sm_120", section
// "The NVFP4 Pivot"): one E4M3 scale per 16 consecutive elements of a row, E2M1 codes,
// and a float32 per-tensor scale g. Per matrix, in float32 with round-to-nearest-even:
//   g = amax / 2688 over the finite entries (1 if that amax is 0), unless given;
//   per 16-group: any NaN/Inf -> scale 0x7F, codes 0;  amax_g == 0 -> scale 0, codes +-0;
//   else s = E4M3(min(amax_g / (6 g), 448)), S = E4M3[s] * g, q = E2M1(|w| / S) with the
//   sign bit of w.
// FP8 activations ("Native FP4 Is Slower Than Emulated FP4", section 1): x -> E4M3 with a
// per-tensor scale amax / 448, back to bf16.
//
// Memory traffic: one read of x for the amax, one read of x plus 9/16 byte per element
// written for the codes; every access is a 16-byte vector access.
#include "act_rows.h"
#include "common.h"
#include "kernels.h"

namespace nvfp4moe {

namespace {

constexpr int kAmaxThreads = 256;
constexpr int kQuantThreads = 256;

template <typename T>
struct Vec8;  // eight consecutive elements as float
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float v[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <>
struct Vec8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float v[8]) {
    uint4 a = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
};

// Partial max of |x| over the finite entries: grid (nblk, B); matrix b has n elements
// (n % 8 == 0); block j scans the 8-element vectors j, j + nblk, ... of matrix b, four
// vectors per thread and step so that four loads are in flight.
template <typename T>
__global__ __launch_bounds__(kAmaxThreads) void amax_partial_kernel(const T* __restrict__ x,
                                                                    int64_t n, int nblk,
                                                                    float* __restrict__ partial) {
  const int b = blockIdx.y;
  const T* xb = x + (size_t)b * (size_t)n;
  const int64_t nvec = n / 8;
  const int64_t stride = (int64_t)nblk * kAmaxThreads;
  float m = 0.0f;
  int64_t i = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    float v[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q) Vec8<T>::load(xb + (i + q * stride) * 8, v[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, finite_abs(v[q][j]));
  }
  for (; i < nvec; i += stride) {
    float v[8];
    Vec8<T>::load(xb + i * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, finite_abs(v[j]));
  }
  __shared__ float red[kAmaxThreads / kWave];
  m = wave_max(m);
  if ((threadIdx.x % kWave) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < kAmaxThreads / kWave; ++w) r = fmaxf(r, red[w]);
    partial[(size_t)b * nblk + blockIdx.x] = r;
  }
}

// g[b] from (in order of precedence) g_in, amax_in, or the partial maxima.
// mode 0: quantizer global scale amax/2688; mode 1: FP8 activation scale amax/448.
__global__ __launch_bounds__(kWave) void finalize_scale_kernel(const float* __restrict__ g_in,
                                                               const float* __restrict__ amax_in,
                                                               const float* __restrict__ partial,
                                                               int nblk, float denom,
                                                               float* __restrict__ g_out) {
  const int b = blockIdx.x;
  float g;
  if (g_in) {
    g = g_in[b];
  } else {
    float a;
    if (amax_in) {
      a = amax_in[b];
    } else {
      a = 0.0f;
      for (int i = threadIdx.x; i < nblk; i += kWave) a = fmaxf(a, partial[(size_t)b * nblk + i]);
      a = wave_max(a);
    }
    g = (a == 0.0f) ? 1.0f : __fdiv_rn(a, denom);
  }
  if (threadIdx.x == 0) g_out[b] = g;
}

// NVFP4 codes of 32 consecutive elements (two 16-groups) at src, under global scale gb:
// four words of packed codes (element 0 in the low nibble of word 0) and, in the return
// value, the two scale bytes (low byte first).
template <typename T>
__device__ __forceinline__ uint32_t quantize32(const T* __restrict__ src, float gb, uint32_t (&words)[4]) {
  const float six_g = 6.0f * gb;
  uint32_t sc_bytes = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float v[16];
    Vec8<T>::load(src + 16 * h, v);
    Vec8<T>::load(src + 16 * h + 8, v + 8);
    float amax = 0.0f;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a = fabsf(v[i]);
      finite = finite && (a <= 3.402823466e38f);
      amax = fmaxf(amax, finite_abs(v[i]));
    }
    uint32_t s;
    float S;
    if (!finite) {
      s = 0x7f;
      S = 0.0f;
    } else if (amax == 0.0f) {
      s = 0;
      S = 0.0f;
    } else {
      float ratio = fminf(__fdiv_rn(amax, six_g), 448.0f);
      s = e4m3_rne(ratio);
      S = e4m3_to_f32(s) * gb;
    }
    sc_bytes |= s << (8 * h);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t code = 0;
      if (finite) {
        uint32_t sign = (__float_as_uint(v[i]) >> 31) << 3;
        uint32_t mag = (S == 0.0f) ? 0u : e2m1_rne_mag(__fdiv_rn(fabsf(v[i]), S));
        code = sign | mag;
      }
      if (i < 8) w0 |= code << (4 * i);
      else w1 |= code << (4 * (i - 8));
    }
    words[2 * h] = w0;
    words[2 * h + 1] = w1;
  }
  return sc_bytes;
}

// One thread per 32 consecutive elements of a row (two 16-groups): reads 32 elements,
// writes 16 packed bytes and 2 scale bytes (row-major storage).
template <typename T>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(const T* __restrict__ x,
                                                                 int64_t n_per_mat,
                                                                 int64_t total_units,
                                                                 const float* __restrict__ g,
                                                                 uint8_t* __restrict__ packed,
                                                                 uint8_t* __restrict__ scales) {
  const int64_t u = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (u >= total_units) return;
  const int64_t e0 = u * 32;               // first element (flat over all matrices)
  const int64_t b = e0 / n_per_mat;        // matrix index
  uint32_t w[4];
  const uint32_t sc = quantize32<T>(x + e0, g[b], w);
  *reinterpret_cast<uint4*>(packed + e0 / 2) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint16_t*>(scales + e0 / 16) = (uint16_t)sc;
}

// The same quantization written straight into the tiled storage the GEMMs read (the layout
// of nvfp4_weights_tile): thread i is slot i of the scale windows' chunk grid, lane
// l = 16 g + r of row block rbm (over all matrices; R % 16 == 0), chunk c of the padded
// range ceil(C / 1024) * 8. It quantizes columns 128 c + 32 g .. +31 of row 16 rb + r and
// writes their 16 code bytes at slot 16 l of code tile (rbm, c) (for c < ceil(C / 128)) and
// their two scale bytes at 16 l + 2 (c % 8) of scale tile (rbm, c / 8); columns past C get
// zero codes and scales.
template <typename T>
__global__ __launch_bounds__(kQuantThreads) void quantize_tiled_kernel(const T* __restrict__ x, int R, int C,
                                                                       int64_t total_slots,
                                                                       const float* __restrict__ g,
                                                                       uint8_t* __restrict__ codes,
                                                                       uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (i >= total_slots) return;
  const int nch = (C + 127) / 128, nwin = (C + 1023) / 1024, ncp = 8 * nwin;
  const int lane = (int)(i & 63);
  const int64_t tile = i >> 6;
  const int c = (int)(tile % ncp);
  const int64_t rbm = tile / ncp;                      // row block over all matrices
  const int rb_per_mat = R / 16;
  const int64_t b = rbm / rb_per_mat;
  const int64_t row = (rbm % rb_per_mat) * 16 + (lane & 15);
  const int col = 128 * c + 32 * (lane >> 4);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  uint32_t sc = 0;
  if (col < C) sc = quantize32<T>(x + (b * R + row) * (int64_t)C + col, g[b], w);
  if (c < nch) *reinterpret_cast<uint4*>(codes + ((rbm * nch + c) << 10) + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint16_t*>(scales + ((rbm * nwin + c / 8) << 10) + 16 * lane + 2 * (c % 8)) = (uint16_t)sc;
}

// FP8 E4M3 round trip of 8 bf16 values per thread.
// Eight bf16 activations (vector i) through E4M3 and back under the per-tensor scale s.
__device__ __forceinline__ void fp8_roundtrip8(const uint16_t* __restrict__ x, int64_t i, float s,
                                               uint16_t* __restrict__ out) {
  float v[8];
  Vec8<uint16_t>::load(x + i * 8, v);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t bits = fp8_roundtrip_bits(v[j], s);
    if (j & 1) w[j / 2] |= bits << 16;
    else w[j / 2] = bits;
  }
  *reinterpret_cast<uint4*>(out + i * 8) = make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(kQuantThreads) void fp8_roundtrip_kernel(const uint16_t* __restrict__ x,
                                                                      int64_t nvec,
                                                                      const float* __restrict__ s_a,
                                                                      uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (i >= nvec) return;
  fp8_roundtrip8(x, i, s_a[0], out);
}

// The round trip of a small tensor in one launch instead of three: every workgroup takes the
// amax over the finite entries of the whole tensor (a max, so every workgroup gets the same
// value; the tensor is read from L2), s_a = amax / 448 (1 if amax = 0, the same division as
// the scale kernel), then converts its own slice of kSmallRtVecs vectors.
constexpr int kSmallRtThreads = 1024;
constexpr int kSmallRtVecs = 512;                       // vectors of 8 per workgroup slice
constexpr int64_t kSmallRtElems = int64_t(1) << 16;     // larger tensors: three launches (measured faster)
__global__ __launch_bounds__(kSmallRtThreads) void fp8_roundtrip_small_kernel(const uint16_t* __restrict__ x,
                                                                             int64_t nvec,
                                                                             uint16_t* __restrict__ out) {
  __shared__ float red[kSmallRtThreads / kWave];
  __shared__ float s_sh;
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < nvec; i += kSmallRtThreads) {
    float v[8];
    Vec8<uint16_t>::load(x + i * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, finite_abs(v[j]));
  }
  m = wave_max(m);
  if ((threadIdx.x % kWave) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = red[0];
    for (int w = 1; w < kSmallRtThreads / kWave; ++w) a = fmaxf(a, red[w]);
    s_sh = fp8_scale(a);
  }
  __syncthreads();
  const float s = s_sh;
  const int64_t lo = (int64_t)blockIdx.x * kSmallRtVecs, hi = min(nvec, lo + kSmallRtVecs);
  for (int64_t i = lo + threadIdx.x; i < hi; i += kSmallRtThreads) fp8_roundtrip8(x, i, s, out);
}

// MXFP4 (group 32, UE8M0 scale, no per-tensor scale; "The Benchmark That Confirmed the
// Ceiling", section "The NVFP4 Pivot", read with the OCP MX v1.0 conversion rule): one thread
// per 32 consecutive elements of a row: amax over the finite entries, shared exponent
// e = max(floor(log2 amax) - 2, -127) (frexp gives floor(log2) exactly), scale byte e + 127,
// codes E2M1_RNE_saturating(w * 2^-e) (a power-of-two scaling, exact); a group with NaN/Inf
// gets scale 0xFF and codes 0, an all-zero group scale 0 and codes +-0.
template <typename T>
__global__ __launch_bounds__(kQuantThreads) void mx_quantize_kernel(const T* __restrict__ x, int64_t total_units,
                                                                    uint8_t* __restrict__ packed,
                                                                    uint8_t* __restrict__ scales) {
  const int64_t u = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (u >= total_units) return;
  const int64_t e0 = u * 32;
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) Vec8<T>::load(x + e0 + 8 * q, v + 8 * q);
  uint32_t key = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) key = max(key, mx_key(v[i]));
  int e = 0;
  const uint32_t s = mx_scale(key, e);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; i += 2) w[i >> 3] |= mx_code2(v[i], v[i + 1], key, e) << (4 * (i & 7));
  *reinterpret_cast<uint4*>(packed + e0 / 2) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[u] = (uint8_t)s;
}

// MXFP8 (E4M3 elements, one UE8M0 scale per 32; the block-scaled FP8 of the dense layers on
// "Native FP4 Is Slower Than Emulated FP4", sections 1-2, read with the OCP MX v1.0 rule):
// one thread per 32 consecutive elements of a row: e = max(floor(log2 amax) - 8, -127), scale
// byte e + 127, codes E4M3_RNE(min(|w| * 2^-e, 448)) with the sign of w; NaN/Inf groups get
// scale 0xFF and codes 0, all-zero groups scale 0 and codes +-0.
template <typename T>
__global__ __launch_bounds__(kQuantThreads) void mx8_quantize_kernel(const T* __restrict__ x, int64_t total_units,
                                                                     uint8_t* __restrict__ codes,
                                                                     uint8_t* __restrict__ scales) {
  const int64_t u = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (u >= total_units) return;
  const int64_t e0 = u * 32;
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) Vec8<T>::load(x + e0 + 8 * q, v + 8 * q);
  uint32_t key = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) key = max(key, mx_key(v[i]));
  int e = 0;
  const uint32_t s = mx_scale(key, e, 8);
  uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i >> 2] |= mx8_code(v[i], key, e) << (8 * (i & 3));
  *reinterpret_cast<uint4*>(codes + e0) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(codes + e0 + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  scales[u] = (uint8_t)s;
}

// Workgroups per matrix for the amax pass: about 8 vectors per thread, at most 2048 (8 per
// CU), so that large activations keep enough loads in flight.
inline int amax_blocks(int64_t n) {
  int64_t nb = (n / 8 + kAmaxThreads * 8 - 1) / (kAmaxThreads * 8);
  if (nb < 1) nb = 1;
  if (nb > 2048) nb = 2048;
  return (int)nb;
}

}  // namespace

size_t quantize_ws_bytes(int64_t B, int64_t R, int64_t C) {
  return (size_t)B * (size_t)amax_blocks(R * C) * sizeof(float);
}

hipError_t launch_quantize(const void* x, bool x_bf16, int64_t B, int64_t R, int64_t C,
                           const float* g_in, const float* amax_in, bool tiled, uint8_t* packed,
                           uint8_t* scales, float* g_out, void* ws, hipStream_t stream) {
  const int64_t n = R * C;
  const int nblk = amax_blocks(n);
  float* partial = static_cast<float*>(ws);
  if (!g_in && !amax_in) {
    dim3 grid(nblk, (unsigned)B);
    if (x_bf16)
      amax_partial_kernel<uint16_t><<<grid, kAmaxThreads, 0, stream>>>(
          static_cast<const uint16_t*>(x), n, nblk, partial);
    else
      amax_partial_kernel<float><<<grid, kAmaxThreads, 0, stream>>>(static_cast<const float*>(x),
                                                                      n, nblk, partial);
  }
  finalize_scale_kernel<<<(unsigned)B, kWave, 0, stream>>>(g_in, amax_in, partial, nblk, 2688.0f,
                                                            g_out);
  if (tiled) {
    const int64_t slots = B * (R / 16) * ((C + 1023) / 1024 * 8) * kWave;
    const int64_t blocks = (slots + kQuantThreads - 1) / kQuantThreads;
    if (x_bf16)
      quantize_tiled_kernel<uint16_t><<<(unsigned)blocks, kQuantThreads, 0, stream>>>(
          static_cast<const uint16_t*>(x), (int)R, (int)C, slots, g_out, packed, scales);
    else
      quantize_tiled_kernel<float><<<(unsigned)blocks, kQuantThreads, 0, stream>>>(
          static_cast<const float*>(x), (int)R, (int)C, slots, g_out, packed, scales);
    return hipGetLastError();
  }
  const int64_t units = B * n / 32;
  const int64_t blocks = (units + kQuantThreads - 1) / kQuantThreads;
  if (x_bf16)
    quantize_kernel<uint16_t><<<(unsigned)blocks, kQuantThreads, 0, stream>>>(
        static_cast<const uint16_t*>(x), n, units, g_out, packed, scales);
  else
    quantize_kernel<float><<<(unsigned)blocks, kQuantThreads, 0, stream>>>(
        static_cast<const float*>(x), n, units, g_out, packed, scales);
  return hipGetLastError();
}

hipError_t launch_mx8_quantize(const void* x, bool x_bf16, int64_t n, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream) {
  const int64_t units = n / 32;
  const unsigned blocks = (unsigned)((units + kQuantThreads - 1) / kQuantThreads);
  if (x_bf16)
    mx8_quantize_kernel<uint16_t><<<blocks, kQuantThreads, 0, stream>>>(static_cast<const uint16_t*>(x), units,
                                                                         codes, scales);
  else
    mx8_quantize_kernel<float><<<blocks, kQuantThreads, 0, stream>>>(static_cast<const float*>(x), units, codes,
                                                                      scales);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(const void* x, bool x_bf16, int64_t n, uint8_t* packed, uint8_t* scales,
                              hipStream_t stream) {
  const int64_t units = n / 32;
  const unsigned blocks = (unsigned)((units + kQuantThreads - 1) / kQuantThreads);
  if (x_bf16)
    mx_quantize_kernel<uint16_t><<<blocks, kQuantThreads, 0, stream>>>(static_cast<const uint16_t*>(x), units,
                                                                       packed, scales);
  else
    mx_quantize_kernel<float><<<blocks, kQuantThreads, 0, stream>>>(static_cast<const float*>(x), units, packed,
                                                                    scales);
  return hipGetLastError();
}

size_t fp8_roundtrip_ws_bytes(int64_t n) {
  return ((size_t)amax_blocks(n) + 64) * sizeof(float);
}

hipError_t launch_fp8_roundtrip(const void* x, int64_t n, void* out, void* ws, hipStream_t stream) {
  if (n <= kSmallRtElems) {   // decode-sized activations: one launch
    const int64_t nvec = n / 8;
    fp8_roundtrip_small_kernel<<<(unsigned)((nvec + kSmallRtVecs - 1) / kSmallRtVecs), kSmallRtThreads, 0, stream>>>(
        static_cast<const uint16_t*>(x), nvec, static_cast<uint16_t*>(out));
    return hipGetLastError();
  }
  const int nblk = amax_blocks(n);
  float* partial = static_cast<float*>(ws);
  float* s_a = partial + nblk + 32;  // keep apart from the partials
  amax_partial_kernel<uint16_t><<<dim3(nblk, 1), kAmaxThreads, 0, stream>>>(
      static_cast<const uint16_t*>(x), n, nblk, partial);
  finalize_scale_kernel<<<1, kWave, 0, stream>>>(nullptr, nullptr, partial, nblk, 448.0f, s_a);
  const int64_t nvec = n / 8;
  fp8_roundtrip_kernel<<<(unsigned)((nvec + kQuantThreads - 1) / kQuantThreads), kQuantThreads, 0,
                         stream>>>(static_cast<const uint16_t*>(x), nvec, s_a,
                                   static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace nvfp4moe
