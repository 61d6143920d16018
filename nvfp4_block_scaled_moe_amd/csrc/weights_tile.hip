// Tiled storage of NVFP4 weight matrices: the order in which the GEMM kernels read them.
//
// The GEMMs feed each weight row to v_mfma_f32_16x16x32_f16 as the 16x32 A operand: lane
// l = 16 g + r of a wave holds row r of a 16-row block and, per 128-wide k chunk, the 32
// codes k = 32 g .. 32 g + 31 (16 bytes). In the row-major NVFP4 layout one such wave load
// touches 16 rows; in the tiled layout it is 1 KB of contiguous memory:
//
//   codes : tile (matrix b, row block rb, chunk c) of 1024 bytes at
//           ((b * R/16 + rb) * ceil(C/128) + c) * 1024; lane l's 16 bytes at 16 l hold
//           codes k = 128 c + 32 g .. +31 of row 16 rb + r (zero where k >= C).
//   scales: tile (matrix b, row block rb, window w of 8 chunks) of 1024 bytes at
//           ((b * R/16 + rb) * ceil(C/1024) + w) * 1024; lane l's 16 bytes at 16 l hold,
//           for u = 0..7, the two E4M3 scales of k = 128 (8 w + u) + 32 g + {0..15, 16..31}
//           of row 16 rb + r at bytes 2 u, 2 u + 1 (zero where k >= C).
//
// MXFP4 weights use the same code tiles; their UE8M0 scales (one per 32 k) are tiled as
//   mx scales: tile (matrix b, row block rb, window w of 16 chunks) of 1024 bytes at
//           ((b * R/16 + rb) * ceil(C/2048) + w) * 1024; lane l's 16 bytes at 16 l hold, at
//           byte u = 0..15, the scale of k = 128 (16 w + u) + 32 g .. +31 of row 16 rb + r
//           (zero where k >= C): exactly the scale operand of lane l of the scaled FP4 MFMA
//           for chunk 16 w + u.
//
// MXFP8 weights (one E4M3 code per byte) use code tiles of 2048 bytes per (matrix b, row
// block rb, chunk c) at ((b * R/16 + rb) * ceil(C/128) + c) * 2048; lane l's 32 bytes at
// 32 l hold codes k = 128 c + 16 g .. +15 and then k = 128 c + 64 + 16 g .. +15 of row
// 16 rb + r (the FP8 operand of lane l of the scaled MFMA, whose lane group g holds those two
// 16-element pieces), and the mx scale tiles above.
//
// The reordering is a pure permutation plus zero padding; codes and scales are copied bit
// for bit.
#include "common.h"
#include "kernels.h"

namespace nvfp4moe {

namespace {

constexpr int kTileThreads = 256;

__global__ __launch_bounds__(kTileThreads) void tile_codes_kernel(const uint8_t* __restrict__ packed,
                                                                  int64_t n_slots, int R, int C,
                                                                  uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kTileThreads + threadIdx.x;   // 16-byte slot
  if (i >= n_slots) return;
  const int nch = (C + 127) / 128;
  const int lane = (int)(i & 63);
  const int64_t tile = i >> 6;
  const int c = (int)(tile % nch);
  const int64_t rbm = tile / nch;                 // row block over all matrices
  const int64_t row = rbm * 16 + (lane & 15);     // row over all matrices (R % 16 == 0)
  const int k0 = 128 * c + 32 * (lane >> 4);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (k0 < C) v = *reinterpret_cast<const uint4*>(packed + row * (int64_t)(C / 2) + k0 / 2);
  *reinterpret_cast<uint4*>(out + i * 16) = v;
}

__global__ __launch_bounds__(kTileThreads) void tile_codes8_kernel(const uint8_t* __restrict__ codes,
                                                                   int64_t n_slots, int R, int C,
                                                                   uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kTileThreads + threadIdx.x;   // 16-byte slot
  if (i >= n_slots) return;
  const int nch = (C + 127) / 128;
  const int half = (int)(i & 1);
  const int lane = (int)((i >> 1) & 63);
  const int64_t tile = i >> 7;
  const int c = (int)(tile % nch);
  const int64_t rbm = tile / nch;
  const int64_t row = rbm * 16 + (lane & 15);
  const int k0 = 128 * c + 16 * (lane >> 4) + 64 * half;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (k0 < C) v = *reinterpret_cast<const uint4*>(codes + row * (int64_t)C + k0);   // C % 16 == 0
  *reinterpret_cast<uint4*>(out + i * 16) = v;
}

__global__ __launch_bounds__(kTileThreads) void tile_scales_kernel(const uint8_t* __restrict__ scales,
                                                                   int64_t n_slots, int R, int C,
                                                                   uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kTileThreads + threadIdx.x;
  if (i >= n_slots) return;
  const int nwin = (C + 1023) / 1024;
  const int lane = (int)(i & 63);
  const int64_t tile = i >> 6;
  const int w = (int)(tile % nwin);
  const int64_t rbm = tile / nwin;
  const int64_t row = rbm * 16 + (lane & 15);
  const uint8_t* src = scales + row * (int64_t)(C / 16);
  uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int k0 = 128 * (8 * w + u) + 32 * (lane >> 4);
    if (k0 < C) {
      const uint32_t two = *reinterpret_cast<const uint16_t*>(src + k0 / 16);
      d[u >> 1] |= two << (16 * (u & 1));
    }
  }
  *reinterpret_cast<uint4*>(out + i * 16) = make_uint4(d[0], d[1], d[2], d[3]);
}

__global__ __launch_bounds__(kTileThreads) void tile_mx_scales_kernel(const uint8_t* __restrict__ scales,
                                                                      int64_t n_slots, int R, int C,
                                                                      uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kTileThreads + threadIdx.x;
  if (i >= n_slots) return;
  const int nwin = (C + 2047) / 2048;
  const int lane = (int)(i & 63);
  const int64_t tile = i >> 6;
  const int w = (int)(tile % nwin);
  const int64_t rbm = tile / nwin;
  const int64_t row = rbm * 16 + (lane & 15);
  const uint8_t* src = scales + row * (int64_t)(C / 32);
  uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int k0 = 128 * (16 * w + u) + 32 * (lane >> 4);
    if (k0 < C) d[u >> 2] |= (uint32_t)src[k0 / 32] << (8 * (u & 3));
  }
  *reinterpret_cast<uint4*>(out + i * 16) = make_uint4(d[0], d[1], d[2], d[3]);
}

}  // namespace

size_t mx_tiled_scales_bytes(int64_t R, int64_t C) { return (size_t)(R / 16) * (size_t)((C + 2047) / 2048) * 1024; }

hipError_t launch_mx_weights_tile(const uint8_t* packed, const uint8_t* scales, int64_t B, int64_t R, int64_t C,
                                  uint8_t* tiled_codes, uint8_t* tiled_scales, hipStream_t stream) {
  const int64_t codes_slots = B * (int64_t)(tiled_codes_bytes(R, C) / 16);
  const int64_t scale_slots = B * (int64_t)(mx_tiled_scales_bytes(R, C) / 16);
  tile_codes_kernel<<<(unsigned)((codes_slots + kTileThreads - 1) / kTileThreads), kTileThreads, 0, stream>>>(
      packed, codes_slots, (int)R, (int)C, tiled_codes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tile_mx_scales_kernel<<<(unsigned)((scale_slots + kTileThreads - 1) / kTileThreads), kTileThreads, 0, stream>>>(
      scales, scale_slots, (int)R, (int)C, tiled_scales);
  return hipGetLastError();
}

size_t mx8_tiled_codes_bytes(int64_t R, int64_t C) { return (size_t)(R / 16) * (size_t)((C + 127) / 128) * 2048; }

hipError_t launch_mx8_weights_tile(const uint8_t* codes, const uint8_t* scales, int64_t B, int64_t R, int64_t C,
                                   uint8_t* tiled_codes, uint8_t* tiled_scales, hipStream_t stream) {
  const int64_t codes_slots = B * (int64_t)(mx8_tiled_codes_bytes(R, C) / 16);
  const int64_t scale_slots = B * (int64_t)(mx_tiled_scales_bytes(R, C) / 16);
  tile_codes8_kernel<<<(unsigned)((codes_slots + kTileThreads - 1) / kTileThreads), kTileThreads, 0, stream>>>(
      codes, codes_slots, (int)R, (int)C, tiled_codes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tile_mx_scales_kernel<<<(unsigned)((scale_slots + kTileThreads - 1) / kTileThreads), kTileThreads, 0, stream>>>(
      scales, scale_slots, (int)R, (int)C, tiled_scales);
  return hipGetLastError();
}

size_t tiled_codes_bytes(int64_t R, int64_t C) { return (size_t)(R / 16) * (size_t)((C + 127) / 128) * 1024; }
size_t tiled_scales_bytes(int64_t R, int64_t C) { return (size_t)(R / 16) * (size_t)((C + 1023) / 1024) * 1024; }

hipError_t launch_weights_tile(const uint8_t* packed, const uint8_t* scales, int64_t B, int64_t R, int64_t C,
                               uint8_t* tiled_codes, uint8_t* tiled_scales, hipStream_t stream) {
  const int64_t codes_slots = B * (int64_t)(tiled_codes_bytes(R, C) / 16);
  const int64_t scale_slots = B * (int64_t)(tiled_scales_bytes(R, C) / 16);
  tile_codes_kernel<<<(unsigned)((codes_slots + kTileThreads - 1) / kTileThreads), kTileThreads, 0, stream>>>(
      packed, codes_slots, (int)R, (int)C, tiled_codes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tile_scales_kernel<<<(unsigned)((scale_slots + kTileThreads - 1) / kTileThreads), kTileThreads, 0, stream>>>(
      scales, scale_slots, (int)R, (int)C, tiled_scales);
  return hipGetLastError();
}

}  // namespace nvfp4moe
