// Small-M NVFP4 grouped GEMM, weight-streaming (gfx950).
//
// The decode regime of the MoE: each expert sees a handful of token rows (~16 at 512
// concurrent requests with 8 of 256 experts; "The 2x Gap: Diagnosing Suboptimal FP4 GEMM
// Kernels on Blackwell SM120", section "The Investigation So Far"), so every weight byte is
// used by at most a few rows and the kernel is bound by HBM bandwidth on weight + scale
// bytes (9/16 byte per weight). The design streams each weight exactly once:
//
//   * Workgroup = WAVES wavefronts = one (expert, block of 16*RBW*WAVES weight rows) tile.
//     Each wave owns RBW blocks of 16 rows over the whole K range (for SwiGLU: matching
//     gate and up blocks), so its FP32 accumulators hold finished dot products and the
//     epilogue needs no cross-wave reduction.
//   * Weights, in the tiled storage of weights_tile.hip: per 128-wide K chunk each lane loads
//     16 bytes (32 FP4 codes of one row), so one wave load reads a 16-row x 128-column block
//     as 1 KB of contiguous memory. Loads go through buffer resources (32-bit offsets, block
//     offsets in SGPRs, out-of-range offsets read zero) into a register ring kDepth chunks
//     deep; a ring entry is re-filled as soon as it has been decoded.
//   * Activations (the MFMA B operand) are shared by the waves: per chunk the workgroup
//     copies the 16 or 32 token rows' 128-k slice into a two-slot LDS ring with one
//     16-byte load per thread, then every wave reads its fragments from LDS. W4A16
//     activations come from an f16 copy written in MFMA operand order; W4A4 activations
//     are FP4 and are decoded like the weights. LDS rows are XOR-swizzled per token so the
//     fragment reads are bank-conflict free.
//   * Weight scales: one 16-byte load per lane, block and 1024-k window (the tiled scale
//     storage) holds the lane's two scale bytes for each of the window's 8 chunks; the
//     current and the next window stay in registers.
//   * Decode in registers: hardware FP4 -> f16 convert and one packed f16 multiply by the
//     block scale per two weights. Both steps are exact (E2M1 * E4M3 has <= 6 significant
//     bits), so the MFMA sees exactly the dequantized weights.
//   * v_mfma_f32_16x16x32_f16 with the weights as the 16x32 A operand and 16 token rows as
//     the 32x16 B operand, FP32 accumulation in registers over all of K. Experts with more
//     than 32 rows are handled in further 32-row passes.
//   * Epilogue per wave: float32 global scales (w_g; a_g for W4A4, or the power-of-two
//     row scale of the f16 activations), SwiGLU when asked, 8- or 16-byte stores; for the
//     down GEMM of a combine call, the weighted reduce of the tokens the tile completes
//     (combine_tile in gemm_common.h).
//   * Tiles are numbered expert-major and handed out XCD-major (workgroup i runs on XCD
//     i mod 8), so the tiles of one expert, which share its activation rows, share an L2.
#include <cstdio>
#include <cstdlib>

#include "gemm_common.h"

namespace nvfp4moe {

namespace {

constexpr int kWin = 8;                  // chunks per scale tile (1024 k)
constexpr int kDepth = 2;                // weight chunks in flight per wave (2 keeps 3 waves per SIMD)
constexpr uint32_t kNoDst = 0xffffffffu;

template <int TBM, bool A4>
struct Ring {
  // per slot: (16*TBM tokens) x (256 B of f16 per token | 64 B of FP4 codes), then for
  // W4A4 the tokens' 8 scale bytes of the chunk
  static constexpr int kTokBytes = A4 ? 64 : 256;
  static constexpr int kCodes = 16 * TBM * kTokBytes;
  static constexpr int kSlot = kCodes + (A4 ? 16 * TBM * 8 : 0);
  static constexpr int kBytes = 2 * kSlot;
};

template <int RBW, int WAVES, int TBM, int WDEPTH, int BDEPTH, bool SWIGLU, bool A4>
__global__ __launch_bounds__(WAVES* kWave) void gemm_stream_kernel(const GemmArgs p, int tiles_per_expert) {
  static_assert(RBW % 2 == 0, "row blocks per wave come in pairs");
  static_assert(kWin % WDEPTH == 0 && kWin % BDEPTH == 0, "ring depths divide the scale window");
  static_assert(WDEPTH <= 2 && BDEPTH <= 2, "the next item's rows are ready from step kWin - 2 on");
  using R = Ring<TBM, A4>;
  constexpr int NT = WAVES * kWave;
  constexpr int TROWS = 16 * TBM;               // GEMM rows per item
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* ring = smem;                   // [2][R::kSlot]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int K = p.K, Nw = p.Nw, Kh = K >> 1, Ks = K >> 4;
  const int K128 = (K + 127) & ~127;
  const int F = Nw >> 1;
  const int nch = (K + kChunk - 1) / kChunk;
  const int nwin = (nch + kWin - 1) / kWin;
  const int wps = (nwin + p.ksplit - 1) / p.ksplit;   // scale windows per K slice

  // One tile (K slice, active expert, row tile) per workgroup. The tiles of the experts that
  // are actually active (known only here) are numbered slice-major, expert-major and split
  // into 8 equal ranges, one per XCD (workgroup i runs on XCD i mod 8), so every XCD gets an
  // equal share however few experts are active, and the tiles in flight on one XCD are
  // neighbours that share their experts' activation rows in its L2.
  const int per_split = ld_const(p.n_active, 0) * tiles_per_expert;
  const int ntiles = per_split * p.ksplit;
  const int per_xcd = (ntiles + 7) >> 3;
  const int tile = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || tile >= ntiles) return;

  // First row of block b of this wave in row tile nb (the lane adds l16).
  auto blkrow = [&](int nb, int b) -> int {
    if (SWIGLU) {
      constexpr int hb = RBW / 2;
      const int gate0 = (nb * WAVES + wave) * 16 * hb;
      return b < hb ? gate0 + 16 * b : F + gate0 + 16 * (b - hb);
    }
    return (nb * WAVES + wave) * 16 * RBW + 16 * b;
  };
  // Tiled weights: 1 KB per (16-row block, chunk) of codes and per (16-row block, window)
  // of scales; lane l reads the 16 bytes at 16 l of a tile. The block offsets inside a row
  // tile are the same for every tile.
  const uint32_t wbytes = (uint32_t)(Nw / 16) * (uint32_t)nch * 1024u;
  const uint32_t sbytes = (uint32_t)(Nw / 16) * (uint32_t)nwin * 1024u;
  const uint32_t vlane = 16u * lane;
  uint32_t wsoff[RBW], ssoff[RBW];
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const uint32_t blk = (uint32_t)((blkrow(0, b) - blkrow(0, 0)) / 16);
    wsoff[b] = __builtin_amdgcn_readfirstlane(blk * (uint32_t)nch * 1024u);
    ssoff[b] = __builtin_amdgcn_readfirstlane(blk * (uint32_t)nwin * 1024u);
  }
  __amdgpu_buffer_rsrc_t ar, asr;
  if (A4) {
    ar = make_rsrc(p.a_packed, (uint32_t)p.a_rows * (uint32_t)Kh);
    asr = make_rsrc(p.a_scales, (uint32_t)p.a_rows * (uint32_t)Ks);
  } else {
    ar = make_rsrc(p.a16, (uint32_t)p.a_rows * (uint32_t)K128 * 2u);
    asr = ar;
  }

  // The tile: K slice ks (whole scale windows [wlo, whi), chunks [wlo * kWin, chi)), expert e
  // with GEMM rows r0 .. r0+M-1, row tile nb. All wave-uniform.
  const int ks = tile / per_split;
  const int aidx = (tile - ks * per_split) / tiles_per_expert;
  const int nb = tile - ks * per_split - aidx * tiles_per_expert;
  const int e = ld_const(p.active, aidx);
  const int r0 = ld_const(p.expert_offsets, e);
  const int M = ld_const(p.expert_offsets, e + 1) - r0;
  const int wlo = ks * wps, whi = min(nwin, wlo + wps);
  const int clo = wlo * kWin, chi = min(nch, whi * kWin);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w_packed + (size_t)e * wbytes, wbytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.w_scales + (size_t)e * sbytes, sbytes);
  const uint32_t wb = __builtin_amdgcn_readfirstlane((uint32_t)(blkrow(nb, 0) / 16) * (uint32_t)nch * 1024u);
  const uint32_t sb = __builtin_amdgcn_readfirstlane((uint32_t)(blkrow(nb, 0) / 16) * (uint32_t)nwin * 1024u);

  // Activation staging roles: thread -> (token, 16-byte piece) of a chunk slice.
  constexpr int TPT = A4 ? 4 : 16;             // threads per token
  constexpr int TPR = NT / TPT;                // tokens per round
  constexpr int ROUNDS = (TROWS + TPR - 1) / TPR;
  const int pc = tid % TPT;                    // 16-byte piece of the token's slice
  uint32_t bdst[ROUNDS], bsdst[ROUNDS];
#pragma unroll
  for (int rr = 0; rr < ROUNDS; ++rr) {
    const int tk = rr * TPR + tid / TPT;
    bdst[rr] = tk >= TROWS ? kNoDst
               : A4        ? tk * R::kTokBytes + 16 * (pc ^ (tk & 3))
                           : tk * R::kTokBytes + 16 * (pc ^ (tk & 15));
    bsdst[rr] = (A4 && tk < TROWS && pc == 0) ? R::kCodes + tk * 8 : kNoDst;
  }
  // Source offsets of this thread's staging pieces for an item, from the activation row of
  // each of its tokens (arow < 0: no such row).
  auto stage_src = [&](const int (&arow)[ROUNDS], uint32_t (&src)[ROUNDS], uint32_t (&ssrc)[ROUNDS]) {
#pragma unroll
    for (int rr = 0; rr < ROUNDS; ++rr) {
      const bool ok = arow[rr] >= 0;
      const uint32_t a = (uint32_t)arow[rr];
      if (A4) {
        src[rr] = ok ? a * (uint32_t)Kh + 16 * pc : kOOB;
        ssrc[rr] = ok && pc == 0 ? a * (uint32_t)Ks : kOOB;
      } else {
        src[rr] = ok ? (a * (uint32_t)K128 + 8 * pc) * 2 : kOOB;
        ssrc[rr] = kOOB;
      }
    }
  };
  // Activation row of each staging token of the pass starting at GEMM row tc of the tile's
  // expert (-1 past its rows). The gather read is unconditional (row r0 when not needed) so
  // that no branch splits the wait for it.
  auto stage_rows = [&](int tc, int (&arow)[ROUNDS]) {
#pragma unroll
    for (int rr = 0; rr < ROUNDS; ++rr) {
      const int tk = rr * TPR + tid / TPT;
      const bool ok = tk < TROWS && tc + tk < M;
      const int row = r0 + (ok ? tc + tk : 0);
      const int src = p.gather_index ? p.gather_index[row] : row;
      arow[rr] = ok ? src : -1;
    }
  };
  auto source_rows = [&](int (&grow)[ROUNDS]) {
    if (p.gather_index) {
#pragma unroll
      for (int rr = 0; rr < ROUNDS; ++rr) grow[rr] = grow[rr] >= 0 ? grow[rr] / p.gather_div : -1;
    }
  };

  // Register rings: activations (BDEPTH staging sets, committed to a two-slot LDS ring),
  // weight codes (WDEPTH chunks) and weight scales (current and next window).
  u32x4 bst[BDEPTH][ROUNDS];
  uint32_t bsc[BDEPTH][ROUNDS][2];
  u32x4 wring[WDEPTH][RBW];
  u32x4 scur[RBW], snext[RBW];
  // f16 rows are zero-padded to whole chunks; FP4 rows are not, so W4A4 pieces and scale
  // pairs past K read zero (a neighbouring row's NaN scale must not leak in).
  // A round whose tokens are all past the item's rows (16 * TPR * rr >= rows, wave-uniform)
  // is neither loaded nor committed.
  auto round_used = [&](int rr, int rows) { return rr == 0 || rr * TPR < rows; };
  auto b_issue = [&](int set, const uint32_t (&src)[ROUNDS], const uint32_t (&ssrc)[ROUNDS], int rows, bool cin,
                     int c) {
    const int kc = c * kChunk;
#pragma unroll
    for (int rr = 0; rr < ROUNDS; ++rr) {
      const bool in = A4 ? cin && (kc + 32 * pc) < K : cin;
      const uint32_t step = A4 ? (uint32_t)kc / 2 : (uint32_t)kc * 2;
      if (round_used(rr, rows)) bst[set][rr] = ld128(ar, in ? src[rr] + step : kOOB, 0);
    }
    if (A4) {
#pragma unroll
      for (int rr = 0; rr < ROUNDS; ++rr) {
        if (!round_used(rr, rows)) continue;
        const uint32_t so = ssrc[rr] + (uint32_t)kc / 16;
        uint32_t v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = ld16(asr, (cin && kc + 32 * q < K) ? so : kOOB, 2 * q);
        bsc[set][rr][0] = v[0] | (v[1] << 16);
        bsc[set][rr][1] = v[2] | (v[3] << 16);
      }
    }
  };
  auto b_commit = [&](int set, int rows, int slot) {
    unsigned char* base = ring + slot * R::kSlot;
#pragma unroll
    for (int rr = 0; rr < ROUNDS; ++rr)
      if (round_used(rr, rows) && bdst[rr] != kNoDst) *reinterpret_cast<u32x4*>(base + bdst[rr]) = bst[set][rr];
    if (A4) {
#pragma unroll
      for (int rr = 0; rr < ROUNDS; ++rr)
        if (round_used(rr, rows) && bsdst[rr] != kNoDst)
          *reinterpret_cast<uint2*>(base + bsdst[rr]) = make_uint2(bsc[set][rr][0], bsc[set][rr][1]);
    }
  };
  // Scales: one 16-byte load per block and window holds the lane's two scale bytes for
  // each of the window's 8 chunks.
  auto s_issue = [&](const __amdgpu_buffer_rsrc_t& sr, uint32_t voff, uint32_t sbase) {
#pragma unroll
    for (int b = 0; b < RBW; ++b) snext[b] = ld128(sr, voff, sbase + ssoff[b]);
  };
  f32x4 acc[RBW][TBM];
  // Chunk c (u = c % kWin): decode ring entry d, refill it from offset voff, then the
  // MFMAs of token block 0 and, if the item has more than 16 rows (`two`, wave-uniform),
  // of token block 1; k-step-major inside a block, so that consecutive MFMAs update
  // different accumulators.
  auto compute = [&](bool two, int d, int c, int u, uint32_t voff) {
    static_assert(TBM == 2, "token blocks 0 and 1");
    u32x4 (&wv)[RBW] = wring[d];
    const unsigned char* base = ring + (c & 1) * R::kSlot;
    f16x8 wf[RBW][4];
#pragma unroll
    for (int b = 0; b < RBW; ++b) {
      const uint32_t sv = scur[b][u >> 1] >> (16 * (u & 1));   // scales of k past K are 0
      f16x2 s0, s1;
      decode_scale_pair(sv, s0, s1);
      wf[b][0] = decode8(wv[b][0], s0);
      wf[b][1] = decode8(wv[b][1], s0);
      wf[b][2] = decode8(wv[b][2], s1);
      wf[b][3] = decode8(wv[b][3], s1);
      wv[b] = ld128(wr, voff, wb + wsoff[b]);   // this ring entry is free again
    }
    auto block = [&](int tb) {
      const int tk = 16 * tb + l16;
      u32x4 aq;
      f16x2 as0, as1;
      if (A4) {
        aq = *reinterpret_cast<const u32x4*>(base + tk * R::kTokBytes + 16 * (g ^ (tk & 3)));
        decode_scale_pair(*reinterpret_cast<const uint16_t*>(base + R::kCodes + tk * 8 + 2 * g), as0, as1);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x8 bj = A4 ? decode8(aq[j], j < 2 ? as0 : as1)
                            : *reinterpret_cast<const f16x8*>(base + tk * R::kTokBytes + 16 * ((4 * j + g) ^ (tk & 15)));
#pragma unroll
        for (int b = 0; b < RBW; ++b)
          acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[b][j], bj, acc[b][tb], 0, 0, 0);
      }
    };
    block(0);
    if (two) block(1);
  };

  // First pass: its rows, then the scales of the first window and the first chunks.
  uint32_t bsrc[ROUNDS], bssrc[ROUNDS];
  {
    int arow[ROUNDS];
    stage_rows(0, arow);
    source_rows(arow);
    stage_src(arow, bsrc, bssrc);
    s_issue(sr, vlane + (uint32_t)wlo * 1024u, sb);
#pragma unroll
    for (int b = 0; b < RBW; ++b) scur[b] = snext[b];
#pragma unroll
    for (int d = 0; d < (WDEPTH > BDEPTH ? WDEPTH : BDEPTH); ++d) {
      if (d < BDEPTH) b_issue(d, bsrc, bssrc, M, clo + d < chi, clo + d);
      if (d < WDEPTH) {
#pragma unroll
        for (int b = 0; b < RBW; ++b)
          wring[d][b] = ld128(wr, clo + d < chi ? vlane + (uint32_t)(clo + d) * 1024u : kOOB, wb + wsoff[b]);
      }
    }
    b_commit(0, M, 0);
    __syncthreads();
  }

  // Passes over up to TROWS GEMM rows (experts with more rows take several; each re-streams
  // the tile's weights).
  uint32_t amax_bits = 0;
  const float alpha = A4 ? ld_const(p.w_g, e) * ld_const(p.a_g, 0) : ld_const(p.w_g, e);
  auto blk = [&](int b) { return blkrow(nb, b); };
  for (int tc = 0;; tc += TROWS) {
#pragma unroll
    for (int b = 0; b < RBW; ++b)
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) acc[b][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int rows = M - tc;                // rows of the expert from tc on (> 0)
    const bool two = rows > 16;             // token block 1 holds rows of this pass
    const bool has_next = rows > TROWS;     // another pass follows
    const int nrows = has_next ? rows - TROWS : 0;
    // Every window but the last: chunk c uses LDS slot c & 1, staging set c % BDEPTH and
    // weight ring entry c % WDEPTH (windows start at multiples of kWin); chunks past K read
    // zero.
    for (int c0 = clo; c0 < (whi - 1) * kWin; c0 += kWin) {
      s_issue(sr, vlane + (uint32_t)(c0 / kWin + 1) * 1024u, sb);
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int c = c0 + u;
        b_issue(u % BDEPTH, bsrc, bssrc, rows, c + BDEPTH < chi, c + BDEPTH);
        compute(two, u % WDEPTH, c, u, c + WDEPTH < chi ? vlane + (uint32_t)(c + WDEPTH) * 1024u : kOOB);
        b_commit((u + 1) % BDEPTH, rows, (c + 1) & 1);
        if (u == kWin - 1) {
#pragma unroll
          for (int b = 0; b < RBW; ++b) scur[b] = snext[b];
        }
        __syncthreads();
      }
    }

    // Last window: fetch the row scales of this pass's outputs and, if another pass follows,
    // request its rows, its first window of scales and its first chunks, so that the ring
    // does not drain between passes.
    int pexps[TBM], erow[TBM], nrow[ROUNDS];
    uint32_t nsrc[ROUNDS], nssrc[ROUNDS];
    {
      const int c0 = (whi - 1) * kWin;
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int c = c0 + u;
        if (u == 0) {
          // activation rows of the lanes' outputs (unconditional reads, row r0 past M)
#pragma unroll
          for (int tb = 0; tb < TBM; ++tb) {
            const int t = tc + 16 * tb + l16;
            const int row = r0 + (t < M ? t : 0);
            erow[tb] = !A4 && p.gather_index ? p.gather_index[row] : row;
          }
          stage_rows(tc + TROWS, nrow);
        }
        if (u == 2) {
#pragma unroll
          for (int tb = 0; tb < TBM; ++tb)
            pexps[tb] = A4 ? 0 : p.rexp[p.gather_index ? erow[tb] / p.gather_div : erow[tb]];
          s_issue(sr, has_next ? vlane + (uint32_t)wlo * 1024u : kOOB, sb);
        }
        if (u == kWin - 2) {
          source_rows(nrow);
          stage_src(nrow, nsrc, nssrc);
        }
        if (u + BDEPTH < kWin) {
          b_issue(u % BDEPTH, bsrc, bssrc, rows, c + BDEPTH < chi, c + BDEPTH);
        } else {
          const int cn = clo + u + BDEPTH - kWin;
          b_issue(u % BDEPTH, nsrc, nssrc, nrows, has_next && cn < chi, cn);
        }
        if (u + WDEPTH < kWin) {
          compute(two, u % WDEPTH, c, u, c + WDEPTH < chi ? vlane + (uint32_t)(c + WDEPTH) * 1024u : kOOB);
        } else {
          const int cn = clo + u + WDEPTH - kWin;
          compute(two, u % WDEPTH, c, u, has_next && cn < chi ? vlane + (uint32_t)cn * 1024u : kOOB);
        }
        // the set committed here holds chunk c + 1: the next pass's first chunk at u = kWin - 1
        b_commit((u + 1) % BDEPTH, u + 1 < kWin ? rows : nrows, (c + 1) & 1);
        if (u == kWin - 1) {
#pragma unroll
          for (int b = 0; b < RBW; ++b) scur[b] = snext[b];
        }
        __syncthreads();
      }
    }

    if (p.ksplit > 1) {   // raw partial sums; the split-K reduce applies the epilogue
      float* part = p.partial + (size_t)ks * p.rows * Nw;
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) {
        const int t = tc + 16 * tb + l16;
        if (t < M) {
#pragma unroll
          for (int b = 0; b < RBW; ++b)
            *reinterpret_cast<float4*>(part + (size_t)(r0 + t) * Nw + blk(b) + 4 * g) =
                make_float4(acc[b][tb][0], acc[b][tb][1], acc[b][tb][2], acc[b][tb][3]);
        }
      }
    } else {
      amax_bits = store_tile_exp<RBW, TBM, SWIGLU>(p, acc, tc, TBM, M, r0, alpha, pexps, blk, lane, amax_bits);
      if (!SWIGLU && p.comb_slot)   // the weighted reduce of the tokens this pass completes
        combine_tile<NT>(p, r0 + tc, min(TROWS, M - tc), nb * WAVES * 16 * RBW, WAVES * 16 * RBW);
    }
    if (!has_next) break;
#pragma unroll
    for (int rr = 0; rr < ROUNDS; ++rr) {
      bsrc[rr] = nsrc[rr];
      bssrc[rr] = nssrc[rr];
    }
  }

  merge_amax(p.out_amax, amax_bits, lane);
}

template <int RBW, int WAVES, bool SWIGLU, bool A4>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  constexpr int TBM = 2;
  const int rows_per_tile = 16 * RBW * WAVES;
  const int tiles_per_expert = a.Nw / rows_per_tile;
  const int max_active = a.E < a.rows ? a.E : a.rows;
  const int total = max_active * tiles_per_expert * a.ksplit;   // bound on the tiles
  const int grid = (total + 7) / 8 * 8;
  const size_t shmem = (size_t)Ring<TBM, A4>::kBytes;
  gemm_stream_kernel<RBW, WAVES, TBM, kDepth, kDepth, SWIGLU, A4>
      <<<grid, WAVES * kWave, shmem, stream>>>(a, tiles_per_expert);
  if (a.ksplit <= 1) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(a, stream);
}

// Tile shape: RBW row blocks of 16 per wave, WAVES waves. NVFP4MOE_STREAM_TILE=<rbw>x<waves>
// overrides the default for tuning; a shape must divide Nw (16 * RBW * WAVES rows), and
// the 2x1 shape (32 rows) divides every valid Nw.
template <bool SWIGLU, bool A4>
hipError_t launch_sw(const GemmArgs& a, hipStream_t stream) {
  int rbw = 2, waves = 4;
  if (const char* s = std::getenv("NVFP4MOE_STREAM_TILE")) std::sscanf(s, "%dx%d", &rbw, &waves);
  if (a.Nw % (16 * rbw * waves) != 0) {
    rbw = 2;
    waves = a.Nw % 128 == 0 ? 4 : a.Nw % 64 == 0 ? 2 : 1;
  }
  if (waves == 1) return launch_cfg<2, 1, SWIGLU, A4>(a, stream);
  if (rbw == 4 && waves == 4) return launch_cfg<4, 4, SWIGLU, A4>(a, stream);
  if (rbw == 2 && waves == 8) return launch_cfg<2, 8, SWIGLU, A4>(a, stream);
  if (rbw == 4 && waves == 2) return launch_cfg<4, 2, SWIGLU, A4>(a, stream);
  if (rbw == 2 && waves == 2) return launch_cfg<2, 2, SWIGLU, A4>(a, stream);
  return launch_cfg<2, 4, SWIGLU, A4>(a, stream);
}

}  // namespace

// Split K (in whole 1024-column windows) when the grid would leave most CUs idle (under 128
// workgroups, e.g. one expert with a few rows); the bound on the active experts is
// min(E, rows). At 256 workgroups (one token over 8 experts) the unsplit kernel already
// streams at ~4.8 TB/s and the extra reduce launch costs more than splitting gains (measured).
// NVFP4MOE_STREAM_KSPLIT=<n> overrides (tests, tuning).
int stream_ksplit(int rows, int E, int Nw, int K) {
  const int nwin = (K + kChunk * kWin - 1) / (kChunk * kWin);
  const int tiles = (E < rows ? E : rows) * (Nw / 128 > 0 ? Nw / 128 : 1);
  int s = tiles >= 128 ? 1 : (512 + tiles - 1) / tiles;
  if (const char* env = std::getenv("NVFP4MOE_STREAM_KSPLIT")) s = std::atoi(env);
  if (s < 1) s = 1;
  if (s > nwin) s = nwin;
  const int wps = (nwin + s - 1) / s;
  return (nwin + wps - 1) / wps;
}

hipError_t launch_gemm_stream(const GemmArgs& a, hipStream_t stream) {
  if (a.swiglu) return a.w4a4 ? launch_sw<true, true>(a, stream) : launch_sw<true, false>(a, stream);
  return a.w4a4 ? launch_sw<false, true>(a, stream) : launch_sw<false, false>(a, stream);
}

}  // namespace nvfp4moe
