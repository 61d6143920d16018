// MXFP4 W4A4 grouped GEMM on the scaled FP4 matrix cores of gfx950.
//
// MXFP4 is FP4 (E2M1) data with one UE8M0 (power-of-two) scale per 32 elements ("The
// Benchmark That Confirmed the Ceiling: NVFP4 Cutlass on sm_120", section "The NVFP4 Pivot":
// "MXFP4 (group-32, UE8M0)"). That is exactly the operand format of
// v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 on both sides: lane l = 16 g + r holds 32 FP4
// values (row r, k = 32 g .. +31 of a 128-wide chunk, 16 bytes) and one UE8M0 scale byte for
// them, and the instruction multiplies E2M1 * 2^(scale - 127) exactly with FP32
// accumulation. So there is no decode at all: weight codes come from the tiled code layout
// (weights_tile.hip; the lane order is that of the operand), weight scales from the MX
// scale tiles (16 chunks per 16-byte lane load), activation codes and scales from the
// row-major quantizer output through an LDS ring.
//
//   * m-tiles of 128 rows of one expert from the device-built list (MtileSched, built by
//     mtile_schedule_kernel); the tiles of the listed m-tiles are split into 8 equal ranges,
//     one per XCD, as in the f16 large-M kernel.
//   * Workgroup = 8 waves = 256 weight rows (each wave 2 blocks of 16: for SwiGLU one gate
//     and the matching up block) x one m-tile (8 token blocks of 16; a ragged m-tile runs
//     with 1, 2, 4 or 8 blocks).
//   * Per chunk (128 k) each thread stages 16 bytes of codes and one scale byte of one token
//     (512 threads = 128 tokens x 4 k-blocks) through registers into a two-slot LDS ring;
//     token rows are padded to 80 bytes, so the 16 lanes of a fragment read hit distinct
//     banks. Weights are loaded two chunks ahead into registers.
//   * 16 MFMAs (16x16x128) per wave and chunk; epilogue as in the other GEMMs with alpha 1
//     (MXFP4 has no per-tensor scale): SwiGLU, bf16 or f32 stores, amax.
#include "gemm_common.h"

namespace nvfp4moe {

namespace {

constexpr int kMxWaves = 8;
constexpr int kMxTBM = 8;                           // token blocks of 16 (m-tile of 128 rows)
constexpr int kMxRBW = 2;                           // 16-row weight blocks per wave
constexpr int kMxWin = 16;                          // chunks per scale tile (2048 k)
constexpr int kMxTok = 80;                          // LDS bytes per token and chunk (64 + pad)
constexpr int kMxCodes = 16 * kMxTBM * kMxTok;      // 10240
constexpr int kMxSlot = kMxCodes + 16 * kMxTBM * 4; // + 4 scale bytes per token
constexpr int kMxDepth = 2;                         // weight chunks in flight

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_mx(u32x4 a, uint32_t sa, u32x4 b, uint32_t sb, f32x4 c) {
  const v8i A = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const v8i B = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, (int)(sa & 0xffu), 0,
                                                          (int)(sb & 0xffu));
}

template <bool SWIGLU>
__global__ __launch_bounds__(kMxWaves* kWave) void gemm_mx_kernel(const GemmArgs p, int ntiles_n) {
  constexpr int NT = kMxWaves * kWave;
  static_assert(NT == 16 * kMxTBM * 4, "one thread per token and 32-wide k block of a chunk");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kMxSlot];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  // Tiles (m-tile, row tile) of the listed m-tiles, 8 equal ranges, one per XCD.
  const int ntiles = ld_const(p.sched_n, 0) * ntiles_n;
  const int per_xcd = (ntiles + 7) >> 3;
  const int tile = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || tile >= ntiles) return;
  const int mt = tile / ntiles_n, nb = tile - mt * ntiles_n;
  const int e = ld_const(p.sched_e, mt), tc = ld_const(p.sched_r, mt);
  const int r0 = ld_const(p.expert_offsets, e);
  const int M = ld_const(p.expert_offsets, e + 1) - r0;
  const int K = p.K, Nw = p.Nw, F = Nw >> 1;
  const int Kh = K >> 1, Ks = K >> 5;
  const int nch = (K + kChunk - 1) / kChunk;
  const int nwin = (nch + kMxWin - 1) / kMxWin;
  const int ntb = __builtin_amdgcn_readfirstlane(min(kMxTBM, (M - tc + 15) >> 4));

  auto blkrow = [&](int b) -> int {
    if (SWIGLU) return (b == 0 ? 0 : F) + (nb * kMxWaves + wave) * 16;
    return (nb * kMxWaves + wave) * 16 * kMxRBW + 16 * b;
  };
  const uint32_t wbytes = (uint32_t)(Nw / 16) * (uint32_t)nch * 1024u;
  const uint32_t sbytes = (uint32_t)(Nw / 16) * (uint32_t)nwin * 1024u;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w_packed + (size_t)e * wbytes, wbytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.w_scales + (size_t)e * sbytes, sbytes);
  const uint32_t wlane = (uint32_t)(blkrow(0) / 16) * (uint32_t)nch * 1024u + 16u * lane;
  const uint32_t slane = (uint32_t)(blkrow(0) / 16) * (uint32_t)nwin * 1024u + 16u * lane;
  uint32_t wsoff[kMxRBW], ssoff[kMxRBW];
#pragma unroll
  for (int b = 0; b < kMxRBW; ++b) {
    wsoff[b] = __builtin_amdgcn_readfirstlane((uint32_t)((blkrow(b) - blkrow(0)) / 16) * (uint32_t)nch * 1024u);
    ssoff[b] = __builtin_amdgcn_readfirstlane((uint32_t)((blkrow(b) - blkrow(0)) / 16) * (uint32_t)nwin * 1024u);
  }

  // Staging role: token tk of the m-tile, 32-wide k block q of each chunk.
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(p.a_packed, (uint32_t)p.a_rows * (uint32_t)Kh);
  const __amdgpu_buffer_rsrc_t asr = make_rsrc(p.a_scales, (uint32_t)p.a_rows * (uint32_t)Ks);
  const int tk = tid >> 2, q = tid & 3;
  const bool tok_ok = tc + tk < M;
  const uint32_t arow = tok_ok ? (uint32_t)(p.gather_index ? p.gather_index[r0 + tc + tk] / p.gather_div
                                                           : r0 + tc + tk)
                               : 0u;
  const uint32_t csrc = tok_ok ? arow * (uint32_t)Kh + 16u * q : kOOB;
  const uint32_t ssrc = tok_ok ? arow * (uint32_t)Ks + q : kOOB;
  const uint32_t cdst = tk * kMxTok + 16 * q, sdst = kMxCodes + tk * 4 + q;

  u32x4 bst[2];
  uint32_t bsc[2];
  auto b_issue = [&](int set, int c) {   // k blocks past K read zero codes and scale 0
    const bool in = c < nch && 128 * c + 32 * q < K;
    bst[set] = ld128(ar, in ? csrc + 64u * c : kOOB, 0);
    bsc[set] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(asr, in ? ssrc + 4u * c : kOOB, 0, 0);
  };
  auto b_commit = [&](int set, int slot) {
    unsigned char* base = smem + slot * kMxSlot;
    *reinterpret_cast<u32x4*>(base + cdst) = bst[set];
    base[sdst] = (unsigned char)bsc[set];
  };
  u32x4 wring[kMxDepth][kMxRBW];
  auto w_issue = [&](int d, int c) {     // codes past K are zero in the tiles
#pragma unroll
    for (int b = 0; b < kMxRBW; ++b) wring[d][b] = ld128(wr, c < nch ? wlane + (uint32_t)c * 1024u : kOOB, wsoff[b]);
  };
  u32x4 scur[kMxRBW], snext[kMxRBW];
  auto s_issue = [&](int w) {
#pragma unroll
    for (int b = 0; b < kMxRBW; ++b) snext[b] = ld128(sr, w < nwin ? slane + (uint32_t)w * 1024u : kOOB, ssoff[b]);
  };

  f32x4 acc[kMxRBW][kMxTBM];
#pragma unroll
  for (int b = 0; b < kMxRBW; ++b)
#pragma unroll
    for (int tb = 0; tb < kMxTBM; ++tb) acc[b][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // prologue: scales of window 0, weights and activations of chunks 0 and 1
  s_issue(0);
#pragma unroll
  for (int b = 0; b < kMxRBW; ++b) scur[b] = snext[b];
  b_issue(0, 0);
  b_issue(1, 1);
  w_issue(0, 0);
  w_issue(1, 1);
  b_commit(0, 0);
  __syncthreads();

  // The main loop, compiled for NTB = 8, 4, 2 or 1 token blocks (ntb rounded up; blocks past
  // the m-tile's rows hold zeros). Chunk c: LDS slot c & 1, staging set c & 1, weight ring
  // entry c % kMxDepth. Whole scale windows; the MFMAs of chunks past K are skipped.
  auto body = [&](auto ntb_tag) {
    constexpr int NTB = decltype(ntb_tag)::value;
    for (int c0 = 0; c0 < nwin * kMxWin; c0 += kMxWin) {
      s_issue(c0 / kMxWin + 1);
#pragma unroll
      for (int u = 0; u < kMxWin; ++u) {
        const int c = c0 + u;
        const int d = u % kMxDepth;
        b_issue(u & 1, c + 2);   // set u & 1 was committed last step
        const unsigned char* base = smem + (c & 1) * kMxSlot;
        u32x4 wa[kMxRBW];
        uint32_t sa[kMxRBW];
#pragma unroll
        for (int b = 0; b < kMxRBW; ++b) {
          wa[b] = wring[d][b];
          sa[b] = scur[b][u >> 2] >> (8 * (u & 3));
        }
        w_issue(d, c + kMxDepth);   // this ring entry is free again
        if (c < nch) {
          u32x4 bb[NTB];
          uint32_t sb[NTB];
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb) {
            const int t = 16 * tb + l16;
            bb[tb] = *reinterpret_cast<const u32x4*>(base + t * kMxTok + 16 * g);
            sb[tb] = base[kMxCodes + t * 4 + g];
          }
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int b = 0; b < kMxRBW; ++b) acc[b][tb] = mfma_mx(wa[b], sa[b], bb[tb], sb[tb], acc[b][tb]);
        }
        b_commit((u + 1) & 1, (c + 1) & 1);
        if (u == kMxWin - 1) {
#pragma unroll
          for (int b = 0; b < kMxRBW; ++b) scur[b] = snext[b];
        }
        __syncthreads();
      }
    }
  };
  if (ntb > 4) body(Int<8>{});
  else if (ntb > 2) body(Int<4>{});
  else if (ntb > 1) body(Int<2>{});
  else body(Int<1>{});

  const uint32_t amax_bits = store_tile<kMxRBW, kMxTBM, SWIGLU>(p, acc, tc, ntb, M, r0, 1.0f, false, blkrow, lane, 0u);
  merge_amax(p.out_amax, amax_bits, lane);
}

}  // namespace

int mx_rows_per_mtile() { return 16 * kMxTBM; }
bool mx_supports(int Nw) { return Nw % (16 * kMxRBW * kMxWaves) == 0; }

hipError_t launch_gemm_mx(const GemmArgs& a, int max_mtiles, hipStream_t stream) {
  const int ntiles_n = a.Nw / (16 * kMxRBW * kMxWaves);
  const int total = max_mtiles * ntiles_n;   // bound on the tiles
  const unsigned grid = (unsigned)((total + 7) / 8 * 8);
  if (a.swiglu) gemm_mx_kernel<true><<<grid, kMxWaves * kWave, 0, stream>>>(a, ntiles_n);
  else gemm_mx_kernel<false><<<grid, kMxWaves * kWave, 0, stream>>>(a, ntiles_n);
  return hipGetLastError();
}

}  // namespace nvfp4moe
