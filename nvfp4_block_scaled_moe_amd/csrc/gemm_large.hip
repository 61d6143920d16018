// Large-M NVFP4 grouped GEMM (gfx950): the prefill regime, where experts see hundreds to
// thousands of rows and the GEMMs are bound by the matrix cores, not by weight bytes
// ("The 2x Gap: Diagnosing Suboptimal FP4 GEMM Kernels on Blackwell SM120", section "The
// Pivot: Comparing FP4 Against BF16": at M=512 and beyond FP4 pays off through compute).
//
//   * m-tiles: 128 consecutive rows of one expert. One workgroup of the activation prep
//     launch lists them on the device (expert, first row) for the active experts in order
//     (act_prep.hip, MtileSched), so the grid needs no
//     host-side knowledge of the per-expert counts: grid = (upper bound on the m-tile
//     count) x (row tiles), and workgroups past the list exit at once.
//   * Workgroup = 8 waves = 256 weight rows (each wave: 2 blocks of 16 rows over all of K;
//     for SwiGLU one gate and the matching up block) x one m-tile. A ragged m-tile runs with
//     1, 2, 4 or 8 blocks of 16 rows.
//   * Weights (MFMA A operand), in the tiled storage of weights_tile.hip: each lane loads 16
//     bytes (32 FP4 codes of its row) per 128-wide chunk, WDEPTH chunks ahead, and one
//     16-byte scale load per 8 chunks, into registers; the codes are decoded exactly to f16
//     (hardware FP4 convert, one packed f16 multiply by the block scale) one chunk ahead of
//     use, interleaved with the MFMAs.
//   * Activations (B operand): f16 rows in MFMA operand order (bf16 rows scaled per row by a
//     power of two, or NVFP4 rows decoded exactly, by the activation prep), staged per chunk
//     through a three-slot LDS ring by LDS DMA (16 bytes per thread and round, no registers).
//     Alternatively (a4_staged) the NVFP4 rows themselves (9/16 byte per element instead of 2)
//     are loaded into registers two chunks ahead and decoded exactly to f16 into the same ring
//     slots, with no f16 copy written or read: the same bits, measured 3-4% slower at prefill
//     (the decode and the LDS stores cost more than the copy), so it is not the default.
//     Three slots let every wave
//     read the first fragments of chunk c+1 before the barrier that ends chunk c, so no
//     MFMA waits for LDS after a barrier. XOR-swizzled rows keep the reads conflict free.
//   * v_mfma_f32_16x16x32_f16, k-step-major: each B fragment read from LDS feeds both
//     row blocks; FP32 accumulation over all of K in registers.
//   * Epilogue as in the small-M kernel (shared in gemm_common.h).
//   * Tile numbering m-tile-major and XCD-major: the 256-row tiles of one m-tile run on the
//     same XCD and share its activation rows in that XCD's L2.
#include <cstdio>
#include <cstdlib>

#include "gemm_common.h"

namespace nvfp4moe {

namespace {

constexpr int kTBM = 8;                    // 16-row blocks per m-tile
constexpr int kRBW = 2;                    // 16-row weight blocks per wave
constexpr int kSlots = 3;                  // LDS ring slots
constexpr int kWin = 8;                    // chunks per scale tile
constexpr int kTokBytes = 256;             // f16 activations of one row and chunk
constexpr int kSlot = 16 * kTBM * kTokBytes;

// 16 bytes per lane from buffer offset voff straight into LDS (lane l at lds + 16 l). A function
// of its own: with the address-space cast inside one of the kernel's lambdas, the host-side
// compilation dropped the kernel's launch stubs without a diagnostic.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// One tile of the large-M GEMM: K slice ks = scale windows [wlo, whi) = chunks [clo, chi), row
// tile nb, m-tile = rows tc .. of expert e (GEMM rows r0 .. r0 + M - 1, ntb blocks of 16 in
// this m-tile), its epilogue scale alpha, the wave's weight code and scale offsets and the
// thread's activation DMA sources (RNDF rounds).
template <int RNDF>
struct LargeTile {
  int ks, nb, e, tc, r0, M, ntb, wlo, whi, clo, chi;
  float alpha;
  uint32_t wlane, slane;
  uint32_t bsrc[RNDF];
};

template <int WAVES, int WDEPTH, bool SWIGLU, bool A4>
__global__ __launch_bounds__(WAVES* kWave, 2) void gemm_large_kernel(const GemmArgs p, int ntiles_n) {
  static_assert(WDEPTH >= 2 && kWin % WDEPTH == 0, "the weight ring is read one chunk ahead; steps pair up");
  constexpr int NT = WAVES * kWave;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int K = p.K, Nw = p.Nw;
  const int K128 = (K + 127) & ~127;
  const int F = Nw >> 1;
  const int nch = (K + kChunk - 1) / kChunk;
  const int nwin = (nch + kWin - 1) / kWin;
  const int wps = (nwin + p.ksplit - 1) / p.ksplit;   // scale windows per K slice
  // Tiles (K slice, m-tile, row tile) of the m-tiles actually listed (known only here) are
  // numbered slice-major and split into 8 equal ranges, one per XCD (workgroup i runs on XCD
  // i mod 8): every XCD gets an equal share however far the list falls below the grid's bound,
  // and the row tiles of one m-tile, which share its activation rows, and the m-tiles of one
  // expert, which share its weights, run on one XCD and share its L2. The workgroups of an XCD
  // walk its range with a stride of their number: with f16 activations (LDS DMA) and 8 waves,
  // a grid of one workgroup per CU stays resident and requests a tile's scales, first weights
  // and first activation chunks while the previous tile's results are being stored.
  constexpr bool PERSIST = !A4 && WAVES == 8;   // the 4-wave shape is only chosen for small grids
  const int per_split = ld_const(p.sched_n, 0) * ntiles_n;
  const int ntiles = per_split * p.ksplit;
  const int per_xcd = (ntiles + 7) >> 3;
  const int tlo = (int)(blockIdx.x & 7) * per_xcd;
  const int thi = min(ntiles, tlo + per_xcd);
  const int tstride = (int)(gridDim.x >> 3);
  int tile = tlo + (int)(blockIdx.x >> 3);
  if (tile >= thi) return;
  // What the decoding of a tile reads is kept in LDS, not in scalar registers through every
  // tile's main loop (with one tile per workgroup, the kernel arguments are read directly).
  struct Ctx {
    const int* sched_e;
    const int* sched_r;
    const int* offsets;
    const int* gather;
    const float* w_g;
    int gather_div, per_split, ntiles_n;
  };
  __shared__ Ctx ctx;
  if constexpr (PERSIST) {
    if (tid == 0) ctx = Ctx{p.sched_e, p.sched_r, p.expert_offsets, p.gather_index, p.w_g, p.gather_div, per_split, ntiles_n};
    __syncthreads();
  }

  // Tiled weights (weights_tile.hip): lane l reads 16 bytes at 16 l of a 1 KB tile per
  // (16-row block, chunk) of codes and per (16-row block, 8-chunk window) of scales. The block
  // offsets within a row tile are the same for every tile (SwiGLU: the up block F rows below
  // the gate block).
  const uint32_t wbytes = (uint32_t)(Nw / 16) * (uint32_t)nch * 1024u;
  const uint32_t sbytes = (uint32_t)(Nw / 16) * (uint32_t)nwin * 1024u;
  const __amdgpu_buffer_rsrc_t ar = A4 ? make_rsrc(p.a_packed, (uint32_t)p.a_rows * (uint32_t)(K >> 1))
                                        : make_rsrc(p.a16, (uint32_t)p.a_rows * (uint32_t)K128 * 2u);
  const __amdgpu_buffer_rsrc_t asr = make_rsrc(p.a_scales, A4 ? (uint32_t)p.a_rows * (uint32_t)(K >> 4) : 0u);
  uint32_t wsoff[kRBW], ssoff[kRBW];
#pragma unroll
  for (int b = 0; b < kRBW; ++b) {
    const uint32_t blk = SWIGLU ? (b == 0 ? 0u : (uint32_t)(F / 16)) : (uint32_t)b;
    wsoff[b] = __builtin_amdgcn_readfirstlane(blk * (uint32_t)nch * 1024u);
    ssoff[b] = __builtin_amdgcn_readfirstlane(blk * (uint32_t)nwin * 1024u);
  }
  const float a_g = p.w4a4 ? ld_const(p.a_g, 0) : 1.0f;
  // Activation staging by LDS DMA (buffer_load ... lds): lane l of a wave writes the 16 bytes
  // at block + 16 l of the slot, the wave's block holding 4 rows (4 x 256 B); TPR rows per
  // round, RNDF rounds for a whole m-tile. The source of each lane is the logical piece that
  // the row's XOR swizzle puts at that position, so the fragment reads stay conflict free;
  // rows past the expert read zeros (kOOB).
  constexpr int TPR = NT / 16;
  constexpr int RNDF = 16 * kTBM / TPR;
  static_assert(TPR == 4 * WAVES && RNDF * TPR == 16 * kTBM, "4 rows per wave and round, inside one slot");

  using Tile = LargeTile<RNDF>;
  auto tile_at = [&](int t, Tile& T) {
    const int* sched_e = PERSIST ? uniform_ptr(ctx.sched_e) : p.sched_e;
    const int* sched_r = PERSIST ? uniform_ptr(ctx.sched_r) : p.sched_r;
    const int* offsets = PERSIST ? uniform_ptr(ctx.offsets) : p.expert_offsets;
    const float* w_g = PERSIST ? uniform_ptr(ctx.w_g) : p.w_g;
    const int ps = PERSIST ? __builtin_amdgcn_readfirstlane(ctx.per_split) : per_split;
    const int ntn = PERSIST ? __builtin_amdgcn_readfirstlane(ctx.ntiles_n) : ntiles_n;
    T.ks = t / ps;
    const int mn = t - T.ks * ps;
    const int mt = mn / ntn;
    T.nb = mn - mt * ntn;
    T.e = ld_const(sched_e, mt);
    T.tc = ld_const(sched_r, mt);
    T.r0 = ld_const(offsets, T.e);
    T.M = ld_const(offsets, T.e + 1) - T.r0;
    T.ntb = __builtin_amdgcn_readfirstlane(min(kTBM, (T.M - T.tc + 15) >> 4));
    T.wlo = T.ks * wps;
    T.whi = min(nwin, T.wlo + wps);
    T.clo = T.wlo * kWin;
    T.chi = min(nch, T.whi * kWin);
    T.alpha = ld_const(w_g, T.e) * a_g;
    const uint32_t blk0 = (uint32_t)(SWIGLU ? T.nb * WAVES + wave : (T.nb * WAVES + wave) * kRBW);
    T.wlane = blk0 * (uint32_t)nch * 1024u + 16u * lane;
    T.slane = blk0 * (uint32_t)nwin * 1024u + 16u * lane;
    const int* gather = PERSIST ? ctx.gather : p.gather_index;
    const int gdiv = PERSIST ? ctx.gather_div : p.gather_div;
#pragma unroll
    for (int rr = 0; rr < RNDF; ++rr) {
      const int tk = rr * TPR + wave * 4 + (lane >> 4), pp = lane & 15, tt = T.tc + tk;
      const bool ok = tt < T.M;
      const uint32_t arow = ok ? (uint32_t)(gather ? gather[T.r0 + tt] / gdiv : T.r0 + tt) : 0u;
      T.bsrc[rr] = ok ? (arow * (uint32_t)K128 + 8 * (pp ^ (tk & 15))) * 2 : kOOB;
    }
  };
  // DMA rounds that cover an m-tile of ntb blocks of 16 rows (ntb rounded up to 1, 2, 4, 8)
  auto rounds = [&](int ntb) { return ((ntb > 4 ? 128 : ntb > 2 ? 64 : ntb == 2 ? 32 : 16) + TPR - 1) / TPR; };
  // the activations of chunk c (rows per bsrc, slice end chi) into an LDS slot, rnd rounds
  auto b_dma = [&](const uint32_t (&bsrc)[RNDF], int chi, int rnd, int c, int slot) {
    const bool in = c < chi;
    unsigned char* base = smem + slot * kSlot + wave * 4 * kTokBytes;
#pragma unroll
    for (int rr = 0; rr < RNDF; ++rr)
      if (rr < rnd) dma16(ar, base + rr * TPR * kTokBytes, in ? bsrc[rr] + (uint32_t)c * 256u : kOOB);
  };
  u32x4 wring[WDEPTH][kRBW];
  auto w_issue = [&](const Tile& T, int d, int c) {   // codes past K are zero in the tiles
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w_packed + (size_t)T.e * wbytes, wbytes);
#pragma unroll
    for (int b = 0; b < kRBW; ++b) wring[d][b] = ld128(wr, c < T.chi ? T.wlane + (uint32_t)c * 1024u : kOOB, wsoff[b]);
  };
  // One 16-byte load per block and window holds the lane's two scale bytes for each of
  // the window's 8 chunks; the current and the next window stay in registers.
  u32x4 scur[kRBW], snext[kRBW];
  auto s_issue = [&](const Tile& T, int w) {
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.w_scales + (size_t)T.e * sbytes, sbytes);
#pragma unroll
    for (int b = 0; b < kRBW; ++b) snext[b] = ld128(sr, w < T.whi ? T.slane + (uint32_t)w * 1024u : kOOB, ssoff[b]);
  };
  // The requests of a tile's prologue with f16 activations: its first scale window, the
  // activations of its first two chunks into slots 0 and 1 and the weights of its first
  // WDEPTH chunks (the NVFP4-staged variant issues its own in the main loop's prologue).
  auto prologue_issue = [&](const Tile& T) {
    s_issue(T, T.wlo);
    const int rnd = rounds(T.ntb);
    b_dma(T.bsrc, T.chi, rnd, T.clo, 0);
#pragma unroll
    for (int d = 0; d < WDEPTH; ++d) w_issue(T, d, T.clo + d);
    b_dma(T.bsrc, T.chi, rnd, T.clo + 1, 1);
  };

  f32x4 acc[kRBW][kTBM];
  Tile cur, nxt;
  tile_at(tile, cur);
  if constexpr (!A4) prologue_issue(cur);

  auto body = [&](auto ntb_tag) {
    constexpr int NTB = decltype(ntb_tag)::value;
    constexpr int RND = (16 * NTB + TPR - 1) / TPR;
    const int clo = cur.clo, chi = cur.chi;
    // W4A4: NVFP4 activation rows staged through registers instead: thread -> (row, 32-column
    // piece ap) of a chunk; its 16 code bytes and 2 scale bytes are loaded one step ahead and
    // decoded exactly to f16 (as the weights) into the slot, in the same swizzled operand order.
    constexpr int ATR = NT / 4;                                  // rows per round
    constexpr int ARND = (16 * NTB + ATR - 1) / ATR;
    const int ap = tid & 3;
    uint32_t acsrc[ARND], assrc[ARND];
    u32x4 acode[2][ARND];   // two staging sets: chunk c in set c & 1, loaded two steps ahead
    uint32_t ascl[2][ARND];
    if constexpr (A4) {
#pragma unroll
      for (int rr = 0; rr < ARND; ++rr) {
        const int tk = rr * ATR + (tid >> 2), t = cur.tc + tk;
        const bool ok = tk < 16 * NTB && t < cur.M;
        const uint32_t arow = ok ? (uint32_t)(p.gather_index ? p.gather_index[cur.r0 + t] / p.gather_div : cur.r0 + t) : 0u;
        acsrc[rr] = ok ? arow * (uint32_t)(K >> 1) + 16u * ap : kOOB;
        assrc[rr] = ok ? arow * (uint32_t)(K >> 4) + 2u * ap : kOOB;
      }
    }
    auto a_load = [&](int set, int c) {   // pieces past K (or the slice) read zero codes and scales
      const bool in = c < cur.chi && 128 * c + 32 * ap < K;
#pragma unroll
      for (int rr = 0; rr < ARND; ++rr) {
        acode[set][rr] = ld128(ar, in && acsrc[rr] != kOOB ? acsrc[rr] + 64u * c : kOOB, 0);
        ascl[set][rr] = ld16(asr, in && assrc[rr] != kOOB ? assrc[rr] + 8u * c : kOOB, 0);
      }
    };
    auto a_store = [&](int set, int slot) {
      unsigned char* base = smem + slot * kSlot;
#pragma unroll
      for (int rr = 0; rr < ARND; ++rr) {
        const int tk = rr * ATR + (tid >> 2);
        if (tk < 16 * NTB) {
          f16x2 s0, s1;
          decode_scale_pair(ascl[set][rr], s0, s1);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f16x8*>(base + tk * kTokBytes + 16 * ((4 * j + ap) ^ (tk & 15))) =
                decode8(acode[set][rr][j], j < 2 ? s0 : s1);
        }
      }
    };
    auto b_read = [&](f16x8 (&dst)[NTB], int slot, int j) {
      const unsigned char* base = smem + slot * kSlot;
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const int tk = 16 * tb + l16;
        dst[tb] = *reinterpret_cast<const f16x8*>(base + tk * kTokBytes + 16 * ((4 * j + g) ^ (tk & 15)));
      }
    };
    f16x8 wf[kRBW][4], wfn[kRBW][4];   // decoded weights of chunks c and c+1
    f16x2 sc[kRBW][2];
    auto scales = [&](int u) {   // chunk u of the current window, u = 8: first of the next
#pragma unroll
      for (int b = 0; b < kRBW; ++b) {
        const uint32_t two = u < kWin ? scur[b][u >> 1] >> (16 * (u & 1)) : snext[b][0];
        decode_scale_pair(two, sc[b][0], sc[b][1]);
      }
    };
    auto decode = [&](f16x8 (&dst)[kRBW][4], int d, int j) {
#pragma unroll
      for (int b = 0; b < kRBW; ++b) dst[b][j] = decode8(wring[d][b][j], sc[b][j >> 1]);
    };

#pragma unroll
    for (int b = 0; b < kRBW; ++b)
#pragma unroll
      for (int tb = 0; tb < kTBM; ++tb) acc[b][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // prologue: activations of the first two chunks in slots 0 and 1, weights of the first
    // WDEPTH chunks requested (f16 activations: already requested), the first chunk decoded
    if constexpr (A4) {   // clo is a multiple of kWin: chunk c uses staging set c & 1 = u & 1
      s_issue(cur, cur.wlo);
      a_load(0, clo);
      a_load(1, clo + 1);
#pragma unroll
      for (int d = 0; d < WDEPTH; ++d) w_issue(cur, d, clo + d);
      a_store(0, 0);
      a_load(0, clo + 2);
      a_store(1, 1);
      a_load(1, clo + 3);
    }
#pragma unroll
    for (int b = 0; b < kRBW; ++b) scur[b] = snext[b];
    scales(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) decode(wf, 0, j);
    __syncthreads();
    f16x8 bcur[NTB], bnext[NTB];
    b_read(bcur, 0, 0);

    // Step c: MFMAs of chunk c (LDS slot c % 3, decoded weights in wf) interleaved with the
    // LDS reads of the next k-step and the decode of chunk c+1, while the activations of chunk
    // c+2 stream into slot (c+2) % 3. The barrier that ends the step waits for every load of
    // the wave (LDS DMA is counted with the vector-memory loads), so chunk c+2 is in LDS for
    // all waves when step c+1 prefetches its first fragments.
    int slot = 0;
    for (int c0 = clo; c0 < chi; c0 += kWin) {     // one scale window per iteration
      s_issue(cur, c0 / kWin + 1);
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int c = c0 + u;
        if (c < chi) {
          const int d = u % WDEPTH, dn = (u + 1) % WDEPTH;
          const int slot1 = slot == kSlots - 1 ? 0 : slot + 1;
          const int slot2 = slot1 == kSlots - 1 ? 0 : slot1 + 1;
          if constexpr (A4) {                      // slot2 was last read in step c-1
            a_store(u & 1, slot2);                 // chunk c+2, loaded in step c-2
            a_load(u & 1, c + 4);
          } else {
            b_dma(cur.bsrc, chi, RND, c + 2, slot2);
          }
          w_issue(cur, d, c + WDEPTH);             // ring entry d (chunk c) was decoded last step
          scales(u + 1);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j < 3) b_read(bnext, slot, j + 1);
            else b_read(bnext, slot1, 0);
#pragma unroll
            for (int b = 0; b < kRBW; ++b)
#pragma unroll
              for (int tb = 0; tb < NTB; ++tb)
                acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[b][j], bcur[tb], acc[b][tb], 0, 0, 0);
            decode(wfn, dn, j);                    // chunk c+1, k-step j
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) bcur[tb] = bnext[tb];
          }
#pragma unroll
          for (int b = 0; b < kRBW; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) wf[b][j] = wfn[b][j];
          if (u == kWin - 1) {
#pragma unroll
            for (int b = 0; b < kRBW; ++b) scur[b] = snext[b];
          }
          __syncthreads();
          slot = slot1;
        }
      }
    }

  };

  // The epilogue of tile T from acc: raw partial sums (K split) or the usual stores (+ amax,
  // + the fused weighted reduce of a combine call). pexps: the row scales of W4A16, read
  // before the next tile's requests so that waiting for them does not wait for those.
  auto epilogue = [&](const Tile& T, const int (&pexps)[kTBM]) {
    const int tc = T.tc, M = T.M, r0 = T.r0, ntb = T.ntb, nb = T.nb;
    auto blkrow = [&](int b) -> int {
      if (SWIGLU) return (b == 0 ? 0 : F) + (nb * WAVES + wave) * 16;
      return (nb * WAVES + wave) * 16 * kRBW + 16 * b;
    };
    if (p.ksplit > 1) {   // raw partial sums; splitk_reduce_kernel applies the epilogue
      float* part = p.partial + (size_t)T.ks * p.rows * Nw;
#pragma unroll
      for (int tb = 0; tb < kTBM; ++tb) {
        const int t = tc + 16 * tb + l16;
        if (tb < ntb && t < M) {
#pragma unroll
          for (int b = 0; b < kRBW; ++b)
            *reinterpret_cast<float4*>(part + (size_t)(r0 + t) * Nw + blkrow(b) + 4 * g) =
                make_float4(acc[b][tb][0], acc[b][tb][1], acc[b][tb][2], acc[b][tb][3]);
        }
      }
      return;
    }
    uint32_t amax_bits = store_tile_exp<kRBW, kTBM, SWIGLU>(p, acc, tc, ntb, M, r0, T.alpha, pexps, blkrow, lane, 0u);
    merge_amax(p.out_amax, amax_bits, lane);
    if (!SWIGLU && p.comb_slot)   // the weighted reduce of the tokens this tile completes
      combine_tile<NT>(p, r0 + tc, min(16 * ntb, M - tc), nb * WAVES * 16 * kRBW, WAVES * 16 * kRBW);
  };

  for (;;) {
    const int ntb = cur.ntb;
    if (ntb > 4) body(Int<8>{});
    else if (ntb > 2) body(Int<4>{});
    else if (ntb == 2) body(Int<2>{});
    else body(Int<1>{});
    int pexps[kTBM];
    row_exponents<kTBM>(p, cur.tc, cur.M, cur.r0, p.ksplit <= 1 && !p.w4a4, lane, pexps);
    // the next tile's first requests go out before this tile's results are stored
    const int next = tile + tstride;
    const bool more = PERSIST && next < thi;
    if constexpr (PERSIST) {
      if (more) {
        tile_at(next, nxt);
        prologue_issue(nxt);
      }
    }
    epilogue(cur, pexps);
    if (!more) break;
    __syncthreads();   // every wave is past the epilogue (combine calls use LDS) before the next tile
    tile = next;
    cur = nxt;
  }
}

// Split-K epilogue: out[row, col] from the fixed-order sum over K slices of the partial sums,
// then the same arithmetic as the unsplit epilogue (store_tile). One thread per row and 4
// output columns; the row's expert comes from a binary search in expert_offsets.
template <bool SWIGLU>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmArgs p) {
  const int Nw = p.Nw, ncol = SWIGLU ? Nw / 2 : Nw, c4 = ncol / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t amax_bits = 0;
  if (i < (int64_t)p.rows * c4) {
    const int row = (int)(i / c4), col = 4 * (int)(i - (int64_t)row * c4);
    int lo = 0, hi = p.E;                       // expert_offsets[lo] <= row < expert_offsets[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.expert_offsets[mid] <= row) lo = mid;
      else hi = mid;
    }
    const float alpha = p.unit_alpha ? 1.0f : (p.w4a4 ? p.w_g[lo] * p.a_g[0] : p.w_g[lo]);
    const int pexp = p.w4a4 ? 0 : p.rexp[p.gather_index ? p.gather_index[row] / p.gather_div : row];
    const size_t slice = (size_t)p.rows * Nw;
    const float* src = p.partial + (size_t)row * Nw + col;
    float4 a = *reinterpret_cast<const float4*>(src);
    float4 u = SWIGLU ? *reinterpret_cast<const float4*>(src + ncol) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 1; s < p.ksplit; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(src + s * slice);
      a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
      if (SWIGLU) {
        const float4 w = *reinterpret_cast<const float4*>(src + s * slice + ncol);
        u.x += w.x; u.y += w.y; u.z += w.z; u.w += w.w;
      }
    }
    const float av[4] = {a.x, a.y, a.z, a.w}, uv[4] = {u.x, u.y, u.z, u.w};
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (SWIGLU) {
        const float gv = ldexpf(av[q] * alpha, pexp);
        const float up = ldexpf(uv[q] * alpha, pexp);
        o[q] = swiglu1(gv, up);
      } else {
        o[q] = ldexpf(av[q] * alpha, pexp);
      }
    }
    amax_bits = store4(p, (size_t)row * ncol + col, o, amax_bits);
  }
  merge_amax(p.out_amax, amax_bits, threadIdx.x & (kWave - 1));
}

// m-tiles of bm rows over the active experts (one workgroup, n_active <= 1024):

template <int WAVES, int WDEPTH, bool SWIGLU, bool A4>
hipError_t launch_cfg(const GemmArgs& a, int max_mtiles, hipStream_t stream) {
  const auto kern = &gemm_large_kernel<WAVES, WDEPTH, SWIGLU, A4>;
  const size_t shmem = (size_t)kSlots * kSlot;
  static std::atomic<uint64_t> attr_done{0};
  const hipError_t attr = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)shmem, attr_done);
  if (attr != hipSuccess) return attr;
  const int ntiles_n = a.Nw / (16 * kRBW * WAVES);
  const int total = max_mtiles * ntiles_n * a.ksplit;   // bound on the tiles
  // 8 waves with f16 activations: one workgroup per CU at most (the LDS ring fits one), looping
  // over the tiles; the NVFP4-staged variant and the 4-wave shape: one workgroup per tile
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    cus = 256;
  const int grid = A4 || WAVES != 8 ? (total + 7) / 8 * 8 : min((total + 7) / 8 * 8, cus / 8 * 8);
  kern<<<grid, WAVES * kWave, shmem, stream>>>(a, ntiles_n);
  if (a.ksplit <= 1) return hipGetLastError();
  const hipError_t e2 = hipGetLastError();
  if (e2 != hipSuccess) return e2;
  return launch_splitk_reduce(a, stream);
}

// Weight ring depth 2: the chunk after next is in flight while a chunk is decoded (a deeper
// ring does not fit the 256 registers a wave has at two waves per SIMD).
template <bool SWIGLU, bool A4>
hipError_t launch_sw(const GemmArgs& a, int max_mtiles, hipStream_t stream) {
  if (large_waves(a.rows, a.E, a.Nw) == 4) return launch_cfg<4, 2, SWIGLU, A4>(a, max_mtiles, stream);
  return launch_cfg<8, 2, SWIGLU, A4>(a, max_mtiles, stream);
}

// Bound on the m-tiles of a call (as sized on the host).
int mtile_bound(int rows, int E) { return (rows + 16 * kTBM - 1) / (16 * kTBM) + (E < rows ? E : rows); }

}  // namespace

hipError_t launch_splitk_reduce(const GemmArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.rows * ((a.swiglu ? a.Nw / 2 : a.Nw) / 4);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (a.swiglu) splitk_reduce_kernel<true><<<blocks, 256, 0, stream>>>(a);
  else splitk_reduce_kernel<false><<<blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

int large_rows_per_mtile() { return 16 * kTBM; }

// Waves per workgroup (row tiles of 32 x waves weight rows): 8, or 4 when the 8-wave grid
// would have under 128 tiles (a small GEMM such as M = 512, N = 2048: twice the tiles, split K
// three ways instead of six, measured 34.6 -> 31.8 us for GEMM and reduce).
// NVFP4MOE_LARGE_WAVES=4|8 overrides (tests, tuning).
int large_waves(int rows, int E, int Nw) {
  int w = mtile_bound(rows, E) * (Nw / (16 * kRBW * 8)) < 128 ? 4 : 8;
  if (const char* env = std::getenv("NVFP4MOE_LARGE_WAVES")) w = std::atoi(env) == 4 ? 4 : 8;
  return w;
}

// Split K (in whole 1024-column scale windows) when the m-tile x row-tile grid is under one
// workgroup per CU: aim at two 8-wave or one 4-wave workgroup per CU (measured best at
// M = 512). NVFP4MOE_LARGE_KSPLIT=<n> overrides (tests, tuning).
int large_ksplit(int rows, int E, int Nw, int K) {
  const int nwin = (K + kChunk * kWin - 1) / (kChunk * kWin);
  const int waves = large_waves(rows, E, Nw);
  const int tiles = mtile_bound(rows, E) * (Nw / (16 * kRBW * waves));
  const int target = waves == 8 ? 512 : 256;
  int s = tiles >= 256 ? 1 : (target + tiles - 1) / tiles;
  if (const char* env = std::getenv("NVFP4MOE_LARGE_KSPLIT")) s = std::atoi(env);
  if (s < 1) s = 1;
  if (s > nwin) s = nwin;
  const int wps = (nwin + s - 1) / s;   // windows per slice; no empty slices
  return (nwin + wps - 1) / wps;
}
bool large_supports(int Nw) { return Nw % (16 * kRBW * 8) == 0; }

hipError_t launch_gemm_large(const GemmArgs& a, int max_mtiles, hipStream_t stream) {
  if (a.w4a4 && a.a4_staged)
    return a.swiglu ? launch_sw<true, true>(a, max_mtiles, stream) : launch_sw<false, true>(a, max_mtiles, stream);
  return a.swiglu ? launch_sw<true, false>(a, max_mtiles, stream) : launch_sw<false, false>(a, max_mtiles, stream);
}

}  // namespace nvfp4moe
