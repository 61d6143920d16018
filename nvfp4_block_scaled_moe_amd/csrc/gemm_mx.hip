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
//     (512 threads = 128 tokens x 4 k-blocks) through registers into a three-slot LDS ring;
//     token rows are padded to 80 bytes, so the 16 lanes of a fragment read hit distinct
//     banks. The scale bytes of a chunk sit in LDS as [k-block][row in block][token block],
//     so one 8-byte read gives a lane the scales of all 8 token blocks and the MFMA's byte
//     select (opsel) picks each one. Weights are loaded two chunks ahead into registers.
//   * Step c issues the 16 MFMAs (16x16x128) of chunk c on fragments read in step c-1 and
//     meanwhile reads chunk c+1's fragments, commits chunk c+2 to the ring and requests chunk
//     c+3: the reads never wait behind the barrier that ends the step. Epilogue as in the
//     other GEMMs with alpha 1 (MXFP4 has no per-tensor scale): SwiGLU, bf16 or f32 stores,
//     amax.
#include <utility>

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
constexpr int kMxSlots = 3;                         // LDS ring slots
constexpr int kMxDepth = 2;                         // weight chunks in flight

typedef int v8i __attribute__((ext_vector_type(8)));

// FP4 x FP4 with one UE8M0 scale per lane for each operand; OA / OB select the scale byte
// within the 32-bit scale registers.
template <int OA, int OB>
__device__ __forceinline__ f32x4 mfma_mx(u32x4 a, uint32_t sa, u32x4 b, uint32_t sb, f32x4 c) {
  const v8i A = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const v8i B = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, OA, (int)sa, OB, (int)sb);
}

// f(Int<0>{}), ..., f(Int<N-1>{}): loop indices usable as template arguments (the byte
// selects of the MFMA are immediates).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(Int<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <bool SWIGLU>
__global__ __launch_bounds__(kMxWaves* kWave) void gemm_mx_kernel(const GemmArgs p, int ntiles_n) {
  constexpr int NT = kMxWaves * kWave;
  static_assert(NT == 16 * kMxTBM * 4, "one thread per token and 32-wide k block of a chunk");
  __shared__ __attribute__((aligned(16))) unsigned char smem[kMxSlots * kMxSlot];

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
  const uint32_t cdst = tk * kMxTok + 16 * q, sdst = kMxCodes + q * 128 + (tk & 15) * 8 + (tk >> 4);

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

  // prologue: scales of window 0, weights of chunks 0 and 1, activations of chunks 0 and 1
  // committed to slots 0 and 1, chunk 2 requested (staging set 0)
  s_issue(0);
#pragma unroll
  for (int b = 0; b < kMxRBW; ++b) scur[b] = snext[b];
  b_issue(0, 0);
  b_issue(1, 1);
#pragma unroll
  for (int d = 0; d < kMxDepth; ++d) w_issue(d, d);
  b_commit(0, 0);
  b_commit(1, 1);
  b_issue(0, 2);
  __syncthreads();

  // The main loop, compiled for NTB = 8, 4, 2 or 1 token blocks (ntb rounded up; blocks past
  // the m-tile's rows hold zeros). Chunk c lives in LDS slot c % 3 and staging set c & 1,
  // its weights in ring entry c % kMxDepth. Step c: request chunk c+3 (set (c+1) & 1, whose
  // chunk c+1 was committed in step c-1), read chunk c+1's fragments (committed in step c-1),
  // MFMAs of chunk c, commit chunk c+2 to slot (c+2) % 3 (chunk c-1, read in step c-2), barrier.
  // Whole scale windows; the MFMAs of chunks past K are skipped.
  auto body = [&](auto ntb_tag) {
    constexpr int NTB = decltype(ntb_tag)::value;
    u32x4 bcur[NTB], bnext[NTB];
    uint32_t scb[2], scbn[2];
    auto b_read = [&](u32x4 (&bb)[NTB], uint32_t (&sc)[2], int slot) {
      const unsigned char* base = smem + slot * kMxSlot;
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) bb[tb] = *reinterpret_cast<const u32x4*>(base + (16 * tb + l16) * kMxTok + 16 * g);
      const uint2 sv = *reinterpret_cast<const uint2*>(base + kMxCodes + g * 128 + l16 * 8);
      sc[0] = sv.x;
      sc[1] = sv.y;
    };
    b_read(bcur, scb, 0);
    int slot = 0;   // c % 3
    for (int c0 = 0; c0 < nwin * kMxWin; c0 += kMxWin) {
      s_issue(c0 / kMxWin + 1);
      static_for<kMxWin>([&](auto u_tag) {
        constexpr int u = decltype(u_tag)::value;
        const int c = c0 + u;
        constexpr int d = u % kMxDepth;
        const int slot1 = slot == kMxSlots - 1 ? 0 : slot + 1;
        const int slot2 = slot1 == kMxSlots - 1 ? 0 : slot1 + 1;
        b_issue((u + 1) & 1, c + 3);
        u32x4 wa[kMxRBW];
#pragma unroll
        for (int b = 0; b < kMxRBW; ++b) wa[b] = wring[d][b];
        w_issue(d, c + kMxDepth);   // this ring entry is free again
        b_read(bnext, scbn, slot1);
        if (c < nch) {
          static_for<NTB>([&](auto tb_tag) {
            constexpr int tb = decltype(tb_tag)::value;
#pragma unroll
            for (int b = 0; b < kMxRBW; ++b)
              acc[b][tb] = mfma_mx<(u & 3), (tb & 3)>(wa[b], scur[b][u >> 2], bcur[tb], scb[tb >> 2], acc[b][tb]);
          });
        }
        b_commit(u & 1, slot2);
        if (u == kMxWin - 1) {
#pragma unroll
          for (int b = 0; b < kMxRBW; ++b) scur[b] = snext[b];
        }
        __syncthreads();
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) bcur[tb] = bnext[tb];
        scb[0] = scbn[0];
        scb[1] = scbn[1];
        slot = slot1;
      });
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
