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
//     one per XCD, as in the f16 large-M kernel. Within an expert the m-tiles go in groups
//     (64 m-tiles for FP4, 16 for FP8) whose tiles run row-tile-major: the workgroups an XCD
//     has in flight share one weight tile (FP4: up to 32 m-tiles on the same 256 weight rows)
//     in its L2 instead of each streaming the expert's weights again. Grids that split K
//     keep the m-tile-major order.
//   * Workgroup = 8 waves = 256 weight rows (each wave 2 blocks of 16: for SwiGLU one gate
//     and the matching up block) x one m-tile (8 token blocks of 16; a ragged m-tile runs
//     with 1, 2, 4 or 8 blocks).
//   * Per chunk (128 k) each thread stages 16 bytes of codes and one scale byte of one token
//     (512 threads = 128 tokens x 4 k-blocks) through registers into a four-slot LDS ring;
//     token rows are padded by 32 bytes (96-byte rows; FP8 160), which measured 2.5x (FP8
//     ~16x) fewer LDS bank-conflict cycles than 16 bytes of padding. The scale bytes of a
//     chunk sit in LDS as [k-block][row in block][token block], so one 8-byte read gives a
//     lane the scales of all 8 token blocks and the MFMA's byte select (opsel) picks each
//     one. Weights are loaded two chunks ahead into registers.
//   * Step c issues the 16 MFMAs (16x16x128) of chunk c on fragments read in step c-1 and
//     meanwhile reads chunk c+1's fragments and requests chunk c+5; every second step commits
//     the next two chunks to the ring and ends with the barrier, so the two waves per SIMD
//     meet once per 32 MFMAs each: the reads never wait behind a barrier, and a staging load
//     has two to three steps to arrive. Epilogue as in the other GEMMs with alpha 1 (MXFP4
//     has no per-tensor scale): SwiGLU, bf16 or f32 stores, amax.
//   * SwiGLU with quantized output: h is written as MXFP4 straight from the epilogue (no
//     per-tensor scale, so no pass over all of h is needed first). A 32-column group of h
//     spans the 16 columns of two neighbouring waves; each wave reduces its half's amax key
//     per row, the pair exchanges them through LDS, and both quantize their halves with the
//     group's exponent, by the same rule and helpers as the MXFP4 quantizer; the codes and
//     scales of the workgroup's tile are gathered in LDS and written as 64 contiguous bytes
//     per row.
//   * MXFP4 grids are persistent: at most one workgroup per CU (one fits a CU), each walking
//     its XCD's tile range with a stride. After a tile's main loop the workgroup reads the
//     next tile's coordinates and requests its scale windows, first weight chunks and first
//     activation chunks, and only then runs the epilogue, so those loads arrive while the
//     results are written. MXFP8 keeps one workgroup per tile.
//   * Small grids split K into slices of whole chunks (partial sums to the workspace, then
//     the shared fixed-order split-K reduce). A slice may start inside a scale window: the
//     16 scale bytes of the slice's next 16 chunks are a byte shift of the two windows held
//     in registers, taken once per 16 chunks.
#include <cstdlib>
#include <utility>

#include "gemm_common.h"

namespace nvfp4moe {

namespace {

constexpr int kMxWaves = 8;
constexpr int kMxRBW = 2;                           // 16-row weight blocks per wave
constexpr int kMxWin = 16;                          // chunks per scale tile (2048 k)
constexpr int kMxSlots = 4;                         // LDS ring slots
constexpr int kMxDepth = 2;                         // weight chunks in flight

typedef int v8i __attribute__((ext_vector_type(8)));

// Element formats of the MX blocks: FP4 (E2M1, MXFP4) and FP8 (E4M3, MXFP8). Per 128-wide
// chunk a lane holds 32 elements of one row (LB bytes: one MFMA operand); lane group g
// (lanes 16 g .. 16 g + 15) supplies the scale of k block g (k = 32 g .. 32 g + 31). With FP4
// a lane's 32 elements are that block; with FP8 (probed on the GPU) its bytes 0-15 are
// k = 16 g .. +15 and bytes 16-31 are k = 64 + 16 g .. +15; an m-tile has TBM
// token blocks of 16 rows (FP8: 4, so that two fragment sets fit the registers); TOK = LDS
// bytes per token and chunk (row bytes + 32 of padding, against bank conflicts); FMT = the
// MFMA operand format code.
template <int BITS>
struct MxFmt;
// piece(g, h) = offset in a token's chunk row of the h-th 16 bytes of lane group g's operand.
template <>
struct MxFmt<4> {
  static constexpr int LB = 16, TBM = 8, TOK = 96, FMT = 4;
  static constexpr bool PERSIST = true;
  static constexpr int piece(int g, int h) { return 16 * g + 16 * h; }
};
template <>
struct MxFmt<8> {
  static constexpr int LB = 32, TBM = 4, TOK = 160, FMT = 0;
  static constexpr bool PERSIST = false;
  static constexpr int piece(int g, int h) { return 16 * g + 64 * h; }
};

// One MX operand fragment: LB bytes per lane.
template <int BITS>
using MxFrag = uint32_t __attribute__((ext_vector_type(MxFmt<BITS>::LB / 4)));

// A x B with one UE8M0 scale per lane for each operand; OA / OB select the scale byte within
// the 32-bit scale registers.
template <int BITS, int OA, int OB>
__device__ __forceinline__ f32x4 mfma_mx(const MxFrag<BITS>& a, uint32_t sa, const MxFrag<BITS>& b, uint32_t sb,
                                         f32x4 c) {
  v8i A = {0, 0, 0, 0, 0, 0, 0, 0}, B = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < MxFmt<BITS>::LB / 4; ++i) {
    A[i] = (int)a[i];
    B[i] = (int)b[i];
  }
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, MxFmt<BITS>::FMT, MxFmt<BITS>::FMT, OA,
                                                          (int)sa, OB, (int)sb);
}

// Bytes sh .. sh+15 of the 32-byte concatenation lo | hi (sh = 0..15, wave-uniform).
__device__ __forceinline__ u32x4 byte_shift(const u32x4& lo, const u32x4& hi, int sh) {
  const uint32_t d[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  const uint32_t bs = (uint32_t)(sh & 3);
  u32x4 r;
  switch (sh >> 2) {   // uniform branch: register indices stay compile-time constants
    case 0:
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_alignbyte(d[j + 1], d[j], bs);
      break;
    case 1:
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_alignbyte(d[j + 2], d[j + 1], bs);
      break;
    case 2:
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_alignbyte(d[j + 3], d[j + 2], bs);
      break;
    default:
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_alignbyte(d[j + 4], d[j + 3], bs);
      break;
  }
  return r;
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

template <int BITS, bool SWIGLU, bool QH>
__global__ __launch_bounds__(kMxWaves* kWave) void gemm_mx_kernel(const GemmArgs p, int ntiles_n, int mgroup) {
  using Fmt = MxFmt<BITS>;
  using Frag = MxFrag<BITS>;
  constexpr int TBM = Fmt::TBM, LB = Fmt::LB, TOK = Fmt::TOK;
  constexpr int ROWB = 4 * LB;                        // bytes of one token row per chunk
  constexpr int PPT = ROWB / 16;                      // 16-byte staging pieces per token row
  constexpr int CODES = 16 * TBM * TOK;
  constexpr int SLOT = CODES + 16 * TBM * 4;          // + 4 scale bytes per token
  constexpr int TILE = 16 * ROWB;                     // weight code tile (16 rows, one chunk)
  static_assert(!QH || (SWIGLU && BITS == 4), "h is quantized (MXFP4) in the SwiGLU epilogue");
  constexpr int NT = kMxWaves * kWave;
  static_assert(NT == 16 * TBM * PPT, "one thread per 16-byte piece of a chunk");
  __shared__ __attribute__((aligned(16))) unsigned char smem[kMxSlots * SLOT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int K = p.K, Nw = p.Nw, F = Nw >> 1;
  const int Kb = K / (8 / BITS), Ks = K >> 5;   // row bytes of codes and of scales
  const int nch = (K + kChunk - 1) / kChunk;
  const int nwin = (nch + kMxWin - 1) / kMxWin;
  const int cps = (nch + p.ksplit - 1) / p.ksplit;   // chunks per K slice
  // Tiles (K slice, m-tile, row tile) of the listed m-tiles, slice-major, 8 equal ranges,
  // one per XCD (workgroup i runs on XCD i mod 8). The workgroups of an XCD walk its range
  // with a stride of their number, so that a grid of one workgroup per CU stays resident and
  // requests a tile's first chunks while the previous tile's results are being stored.
  // One expert (a dense GEMM) needs no m-tile list (sched_e null): m-tile i is rows 16 TBM i ..
  // of expert 0.
  const int n_mtiles = p.sched_e ? ld_const(p.sched_n, 0)
                                 : (ld_const(p.expert_offsets, 1) - ld_const(p.expert_offsets, 0) + 16 * TBM - 1) / (16 * TBM);
  const int per_split = n_mtiles * ntiles_n;
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
    int gather_div, per_split, ntiles_n, mgroup;
  };
  __shared__ Ctx ctx;
  if constexpr (Fmt::PERSIST) {
    if (tid == 0) ctx = Ctx{p.sched_e, p.sched_r, p.expert_offsets, p.gather_index, p.gather_div, per_split, ntiles_n, mgroup};
    __syncthreads();
  }

  // Weight block offsets within a row tile (the same for every tile): for SwiGLU the up
  // block sits F rows below the gate block.
  const uint32_t wbytes = (uint32_t)(Nw / 16) * (uint32_t)nch * (uint32_t)TILE;
  const uint32_t sbytes = (uint32_t)(Nw / 16) * (uint32_t)nwin * 1024u;
  uint32_t wsoff[kMxRBW], ssoff[kMxRBW];
#pragma unroll
  for (int b = 0; b < kMxRBW; ++b) {
    const uint32_t blk = SWIGLU ? (b == 0 ? 0u : (uint32_t)(F / 16)) : (uint32_t)b;
    wsoff[b] = __builtin_amdgcn_readfirstlane(blk * (uint32_t)nch * (uint32_t)TILE);
    ssoff[b] = __builtin_amdgcn_readfirstlane(blk * (uint32_t)nwin * 1024u);
  }
  // Staging role: token tk of the m-tile, 16-byte piece q of its row in each chunk (32-wide k
  // block kb; with FP8 two pieces share a k block and write the same scale byte).
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(p.a_packed, (uint32_t)p.a_rows * (uint32_t)Kb);
  const __amdgpu_buffer_rsrc_t asr = make_rsrc(p.a_scales, (uint32_t)p.a_rows * (uint32_t)Ks);
  const int tk = tid / PPT, q = tid % PPT, kb = q / (PPT / 4);
  const uint32_t cdst = tk * TOK + 16 * q, sdst = CODES + kb * (16 * TBM) + (tk & 15) * TBM + (tk >> 4);

  // One tile: K slice ks = chunks [clo, chi) (its first chunk is chunk u0 of scale window
  // w0), row tile nb, m-tile = rows tc .. of expert e (rows r0 .. r0 + M - 1 of the GEMM, ntb
  // blocks of 16 of them in this m-tile); this wave's weight code and scale offsets and this
  // thread's activation code and scale offsets.
  struct Tile {
    int ks, nb, e, tc, r0, M, ntb, clo, chi, w0, u0;
    uint32_t wlane, slane, csrc, ssrc;
  };
  auto decode = [&](int t, Tile& T) {
    const int* sched_e = Fmt::PERSIST ? uniform_ptr(ctx.sched_e) : p.sched_e;
    const int* sched_r = Fmt::PERSIST ? uniform_ptr(ctx.sched_r) : p.sched_r;
    const int* offsets = Fmt::PERSIST ? uniform_ptr(ctx.offsets) : p.expert_offsets;
    const int ps = Fmt::PERSIST ? __builtin_amdgcn_readfirstlane(ctx.per_split) : per_split;
    const int ntn = Fmt::PERSIST ? __builtin_amdgcn_readfirstlane(ctx.ntiles_n) : ntiles_n;
    const int mg = Fmt::PERSIST ? __builtin_amdgcn_readfirstlane(ctx.mgroup) : mgroup;
    T.ks = t / ps;
    const int mn = t - T.ks * ps;
    int mt = mn / ntn, nb = mn - mt * ntn;
    {
      // Tile order within the expert: m-tiles in groups of mgroup (the last one shorter), the
      // tiles of a group row-tile-major. The list holds an expert's m-tiles in a row, m-tile i
      // of the expert at row i * 16 TBM, so the group follows from the m-tile's own entry.
      const int loc = sched_e ? ld_const(sched_r, mt) / (16 * TBM) : mt;
      const int ex = sched_e ? ld_const(sched_e, mt) : 0;
      const int me = (ld_const(offsets, ex + 1) - ld_const(offsets, ex) + 16 * TBM - 1) / (16 * TBM);
      const int gi = loc / mg, gs = mt - loc + gi * mg;
      const int gn = min(min(mg, me - gi * mg), ps / ntn - gs);
      const int pos = (mt - gs) * ntn + nb;
      nb = pos / gn;
      mt = gs + (pos - nb * gn);
    }
    T.nb = nb;
    T.e = sched_e ? ld_const(sched_e, mt) : 0;
    T.tc = sched_e ? ld_const(sched_r, mt) : mt * 16 * TBM;
    T.r0 = ld_const(offsets, T.e);
    T.M = ld_const(offsets, T.e + 1) - T.r0;
    T.ntb = __builtin_amdgcn_readfirstlane(min(TBM, (T.M - T.tc + 15) >> 4));
    T.clo = T.ks * cps;
    T.chi = min(nch, T.clo + cps);
    T.w0 = T.clo / kMxWin;
    T.u0 = T.clo - T.w0 * kMxWin;
    const uint32_t blk0 = (uint32_t)(SWIGLU ? nb * kMxWaves + wave : (nb * kMxWaves + wave) * kMxRBW);
    T.wlane = blk0 * (uint32_t)nch * (uint32_t)TILE + (uint32_t)LB * lane;
    T.slane = blk0 * (uint32_t)nwin * 1024u + 16u * lane;
    const bool tok_ok = T.tc + tk < T.M;
    const int* gather = Fmt::PERSIST ? ctx.gather : p.gather_index;
    const int gdiv = Fmt::PERSIST ? ctx.gather_div : p.gather_div;
    const uint32_t arow = tok_ok ? (uint32_t)(gather ? gather[T.r0 + T.tc + tk] / gdiv : T.r0 + T.tc + tk) : 0u;
    T.csrc = tok_ok ? arow * (uint32_t)Kb + 16u * q : kOOB;
    T.ssrc = tok_ok ? arow * (uint32_t)Ks + kb : kOOB;
  };

  u32x4 bst[4];   // staging sets: chunk clo + j in set j & 3 (requested two steps before its commit)
  uint32_t bsc[4];
  auto b_issue = [&](const Tile& T, int set, int c) {   // k blocks past K (or the slice) read zero codes and scale 0
    const bool in = c < T.chi && 128 * c + 32 * kb < K;
    bst[set] = ld128(ar, in ? T.csrc + (uint32_t)ROWB * c : kOOB, 0);
    bsc[set] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(asr, in ? T.ssrc + 4u * c : kOOB, 0, 0);
  };
  auto b_commit = [&](int set, int slot) {
    unsigned char* base = smem + slot * SLOT;
    *reinterpret_cast<u32x4*>(base + cdst) = bst[set];
    base[sdst] = (unsigned char)bsc[set];
  };
  Frag wring[kMxDepth][kMxRBW];
  auto w_issue = [&](const Tile& T, int d, int c) {     // codes past K are zero in the tiles
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w_packed + (size_t)T.e * wbytes, wbytes);
#pragma unroll
    for (int b = 0; b < kMxRBW; ++b) {
      const uint32_t off = c < T.chi ? T.wlane + (uint32_t)c * (uint32_t)TILE : kOOB;
#pragma unroll
      for (int h = 0; h < LB / 16; ++h) {
        const u32x4 v = ld128(wr, off == kOOB ? kOOB : off + 16u * h, wsoff[b]);
#pragma unroll
        for (int i = 0; i < 4; ++i) wring[d][b][4 * h + i] = v[i];
      }
    }
  };
  // Scale windows: sa = window w0 + i, sb = w0 + i + 1 while chunks clo + 16 i .. + 15 run;
  // sn = w0 + i + 2 in flight.
  u32x4 sa[kMxRBW], sb[kMxRBW], sn[kMxRBW];
  auto s_issue = [&](const Tile& T, u32x4 (&dst)[kMxRBW], int w) {
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.w_scales + (size_t)T.e * sbytes, sbytes);
#pragma unroll
    for (int b = 0; b < kMxRBW; ++b) dst[b] = ld128(sr, w < nwin ? T.slane + (uint32_t)w * 1024u : kOOB, ssoff[b]);
  };
  // A tile's prologue in two halves: the requests (scale windows w0 and w0 + 1, the weights of
  // its first kMxDepth chunks, the activations of its first four chunks), issued before the
  // previous tile's epilogue; then the commit of the first three chunks to slots 0 - 2, the
  // request of the fifth (staging set 0) and a barrier.
  auto prologue_issue = [&](const Tile& T) {
    s_issue(T, sa, T.w0);
    s_issue(T, sb, T.w0 + 1);
    b_issue(T, 0, T.clo);
    b_issue(T, 1, T.clo + 1);
    b_issue(T, 2, T.clo + 2);
    b_issue(T, 3, T.clo + 3);
#pragma unroll
    for (int d = 0; d < kMxDepth; ++d) w_issue(T, d, T.clo + d);
  };
  auto prologue_commit = [&](const Tile& T) {
    b_commit(0, 0);
    b_commit(1, 1);
    b_commit(2, 2);
    b_issue(T, 0, T.clo + 4);
    __syncthreads();
  };

  f32x4 acc[kMxRBW][TBM];
  Tile cur, nxt;
  decode(tile, cur);
  prologue_issue(cur);

  // The main loop of tile cur, compiled for NTB = 8, 4, 2 or 1 token blocks (ntb rounded up;
  // blocks past the m-tile's rows hold zeros). With j = c - clo: chunk c lives in LDS slot j & 3
  // and staging set j & 3, its weights in ring entry j % kMxDepth. Step c: request chunk c+5
  // (set (j+1) & 3, whose chunk c+1 was committed in step c-1 or c-2), read chunk c+1's
  // fragments (committed by the last odd step before c), MFMAs of chunk c; then, for odd j,
  // commit chunks c+2 and c+3 (requested in steps c-3 and c-2) to slots (j+2) & 3 and
  // (j+3) & 3, whose chunks c-2 and c-1 were read in steps c-3 and c-2, before the barrier of
  // step c-2, and end with a barrier. The read of chunk 0 before the loop has a barrier of its
  // own, since step 1 rewrites slot 0. Steps come in blocks of 16, so j & 3 = u & 3 is a
  // constant.
  auto body = [&](auto ntb_tag) {
    const int clo = cur.clo, chi = cur.chi, w0 = cur.w0, u0 = cur.u0;
    constexpr int NTB = decltype(ntb_tag)::value;
    Frag bcur[NTB], bnext[NTB];
    uint32_t scb[2], scbn[2];
    auto b_read = [&](Frag (&bb)[NTB], uint32_t (&sc)[2], int slot) {
      const unsigned char* base = smem + slot * SLOT;
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
#pragma unroll
        for (int h = 0; h < LB / 16; ++h) {   // 16-byte reads: rows are 16-byte aligned
          const u32x4 v = *reinterpret_cast<const u32x4*>(base + (16 * tb + l16) * TOK + Fmt::piece(g, h));
#pragma unroll
          for (int i = 0; i < 4; ++i) bb[tb][4 * h + i] = v[i];
        }
      }
      if constexpr (TBM == 8) {
        const uint2 sv = *reinterpret_cast<const uint2*>(base + CODES + g * (16 * TBM) + l16 * TBM);
        sc[0] = sv.x;
        sc[1] = sv.y;
      } else {
        sc[0] = *reinterpret_cast<const uint32_t*>(base + CODES + g * (16 * TBM) + l16 * TBM);
        sc[1] = 0u;
      }
    };
    b_read(bcur, scb, 0);
    __syncthreads();   // slot 0 is rewritten in step 1
    for (int c0 = clo; c0 < chi; c0 += kMxWin) {
      u32x4 scs[kMxRBW];   // scale bytes of chunks c0 .. c0 + 15
#pragma unroll
      for (int b = 0; b < kMxRBW; ++b) scs[b] = byte_shift(sa[b], sb[b], u0);
      s_issue(cur, sn, (c0 - clo) / kMxWin + w0 + 2);
      // Step u of the window. The second half of a window runs only if the slice reaches it
      // (wave-uniform), so a slice of 8 mod 16 chunks runs no steps past its last chunk; the
      // MFMAs of any other chunk past the slice are skipped.
      auto step = [&](auto u_tag) {
        constexpr int u = decltype(u_tag)::value;
        const int c = c0 + u;
        constexpr int d = u % kMxDepth;
        b_issue(cur, (u + 1) & 3, c + 5);
        Frag wa[kMxRBW];
#pragma unroll
        for (int b = 0; b < kMxRBW; ++b) wa[b] = wring[d][b];
        w_issue(cur, d, c + kMxDepth);   // this ring entry is free again
        b_read(bnext, scbn, (u + 1) & 3);
        if (c < chi) {
          static_for<NTB>([&](auto tb_tag) {
            constexpr int tb = decltype(tb_tag)::value;
#pragma unroll
            for (int b = 0; b < kMxRBW; ++b)
              acc[b][tb] = mfma_mx<BITS, (u & 3), (tb & 3)>(wa[b], scs[b][u >> 2], bcur[tb], scb[tb >> 2], acc[b][tb]);
          });
        }
        if (u & 1) {
          b_commit((u + 2) & 3, (u + 2) & 3);
          b_commit((u + 3) & 3, (u + 3) & 3);
        }
        if (u == kMxWin - 1) {
#pragma unroll
          for (int b = 0; b < kMxRBW; ++b) {
            sa[b] = sb[b];
            sb[b] = sn[b];
          }
        }
        if (u & 1) __syncthreads();
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) bcur[tb] = bnext[tb];
        scb[0] = scbn[0];
        scb[1] = scbn[1];
      };
      static_for<kMxWin / 2>([&](auto u_tag) { step(u_tag); });
      if (c0 + kMxWin / 2 < chi)
        static_for<kMxWin / 2>([&](auto u_tag) { step(Int<decltype(u_tag)::value + kMxWin / 2>{}); });
    }
  };
  // The epilogue of tile T from acc: MXFP4 h (QH), raw partial sums (K split), or the usual
  // stores (+ amax, + the fused weighted reduce of a combine call).
  auto epilogue = [&](const Tile& T) {
    const int tc = T.tc, M = T.M, r0 = T.r0, ntb = T.ntb, nb = T.nb;
    auto blkrow = [&](int b) -> int {
      if (SWIGLU) return (b == 0 ? 0 : F) + (nb * kMxWaves + wave) * 16;
      return (nb * kMxWaves + wave) * 16 * kMxRBW + 16 * b;
    };
    if constexpr (QH) {   // MXFP4 h: rows of the m-tile, the wave's 16 h columns
      __syncthreads();     // every wave is past its last ring read
      uint32_t* xch = reinterpret_cast<uint32_t*>(smem);       // [kMxWaves][TBM][16] amax keys
      unsigned char* qc = smem + 4096;                          // [128 rows][64 B] codes of the tile
      unsigned char* qs = qc + 16 * TBM * 64;                // [128 rows][4] scale bytes
      const int F2 = F >> 1, F32 = F >> 5;
      float h[TBM][4];
      uint32_t key[TBM];
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) {
        key[tb] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[tb][i] = swiglu1(acc[0][tb][i], acc[1][tb][i]);
          key[tb] = max(key[tb], mx_key(h[tb][i]));
        }
        key[tb] = max(key[tb], (uint32_t)__shfl_xor((int)key[tb], 16, kWave));
        key[tb] = max(key[tb], (uint32_t)__shfl_xor((int)key[tb], 32, kWave));
        if (g == 0) xch[(wave * TBM + tb) * 16 + l16] = key[tb];
      }
      __syncthreads();
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) {
        const uint32_t gk = max(key[tb], xch[((wave ^ 1) * TBM + tb) * 16 + l16]);
        int ex = 0;
        const uint32_t sc = mx_scale(gk, ex);
        const uint32_t q = mx_code2(h[tb][0], h[tb][1], gk, ex) | (mx_code2(h[tb][2], h[tb][3], gk, ex) << 8);
        const int tr = 16 * tb + l16;   // row of the m-tile
        *reinterpret_cast<uint16_t*>(qc + tr * 64 + wave * 8 + 2 * g) = (uint16_t)q;
        if ((wave & 1) == 0 && g == 0) qs[tr * 4 + (wave >> 1)] = (unsigned char)sc;
      }
      __syncthreads();
      // 64 bytes of codes (the workgroup's 128 h columns) per row: 16 bytes per thread; the 4
      // scale bytes of a row as one word.
      const int tr = tid >> 2, piece = tid & 3;
      const int col0 = nb * kMxWaves * 16;   // first h column of the workgroup
      if (tr < 16 * ntb && tc + tr < M) {
        const size_t row = (size_t)(r0 + tc + tr);
        *reinterpret_cast<u32x4*>(p.hq_packed + row * F2 + col0 / 2 + 16 * piece) =
            *reinterpret_cast<const u32x4*>(qc + tr * 64 + 16 * piece);
        if (piece == 0)
          *reinterpret_cast<uint32_t*>(p.hq_scales + row * F32 + col0 / 32) =
              *reinterpret_cast<const uint32_t*>(qs + tr * 4);
      }
    } else if (p.ksplit > 1) {   // raw partial sums; the split-K reduce applies the epilogue
      float* part = p.partial + (size_t)T.ks * p.rows * Nw;
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) {
        const int t = tc + 16 * tb + l16;
        if (tb < ntb && t < M) {
#pragma unroll
          for (int b = 0; b < kMxRBW; ++b)
            *reinterpret_cast<float4*>(part + (size_t)(r0 + t) * Nw + blkrow(b) + 4 * g) =
                make_float4(acc[b][tb][0], acc[b][tb][1], acc[b][tb][2], acc[b][tb][3]);
        }
      }
    } else {
      const uint32_t amax_bits = store_tile<kMxRBW, TBM, SWIGLU>(p, acc, tc, ntb, M, r0, 1.0f, false, blkrow, lane, 0u);
      merge_amax(p.out_amax, amax_bits, lane);
      if (!SWIGLU && p.comb_slot)   // the weighted reduce of the tokens this tile completes
        combine_tile<NT>(p, r0 + tc, min(16 * ntb, M - tc), nb * kMxWaves * 16 * kMxRBW, kMxWaves * 16 * kMxRBW);
    }
  };

  for (;;) {
    prologue_commit(cur);
#pragma unroll
    for (int b = 0; b < kMxRBW; ++b)
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) acc[b][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int ntb = cur.ntb;
    if constexpr (TBM == 8) {
      if (ntb > 4) body(Int<8>{});
      else if (ntb > 2) body(Int<4>{});
      else if (ntb > 1) body(Int<2>{});
      else body(Int<1>{});
    } else {
      if (ntb > 2) body(Int<4>{});
      else if (ntb > 1) body(Int<2>{});
      else body(Int<1>{});
    }
    // the next tile's first requests go out before this tile's results are stored
    const int next = tile + tstride;
    const bool more = Fmt::PERSIST && next < thi;
    if (more) {
      decode(next, nxt);
      prologue_issue(nxt);
    }
    epilogue(cur);
    if (!more) break;
    __syncthreads();   // every wave is past the epilogue's LDS use before slots 0 - 2 are rewritten
    tile = next;
    cur = nxt;
  }
}

}  // namespace

int mx_rows_per_mtile(int bits) { return bits == 8 ? 16 * MxFmt<8>::TBM : 16 * MxFmt<4>::TBM; }
bool mx_supports(int Nw) { return Nw % (16 * kMxRBW * kMxWaves) == 0; }

// K slices when the m-tile x row-tile grid is under one workgroup per CU: about 256
// workgroups, at least 4 chunks per slice. NVFP4MOE_MX_KSPLIT=<n> overrides (tests, tuning).
int mx_ksplit(int max_mtiles, int Nw, int K) {
  const int nch = (K + kChunk - 1) / kChunk;
  const int tiles = max_mtiles * (Nw / (16 * kMxRBW * kMxWaves));
  int s = tiles >= 256 ? 1 : (256 + tiles - 1) / tiles;
  if (s > nch / 4) s = nch / 4;
  if (const char* env = std::getenv("NVFP4MOE_MX_KSPLIT")) s = std::atoi(env);
  if (s < 1) s = 1;
  if (s > nch) s = nch;
  const int cps = (nch + s - 1) / s;   // chunks per slice; no empty slices
  return (nch + cps - 1) / cps;
}

hipError_t launch_gemm_mx(const GemmArgs& a, int max_mtiles, int bits, hipStream_t stream) {
  const int ntiles_n = a.Nw / (16 * kMxRBW * kMxWaves);
  // m-tiles per row-tile-major group (measured best); a split-K grid is resident at once,
  // where m-tile-major order measured faster
  int mgroup = a.ksplit > 1 ? 1 : bits == 8 ? 16 : 64;
  if (const char* env = std::getenv("NVFP4MOE_MX_GROUP")) mgroup = std::atoi(env);
  if (mgroup < 1) mgroup = 1;
  // MXFP4: one workgroup per CU at most (one fits a CU), looping over the tiles; MXFP8: one
  // workgroup per tile.
  const int total = max_mtiles * ntiles_n * a.ksplit;   // bound on the tiles
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    cus = 256;
  const unsigned grid = (unsigned)(bits == 8 ? (total + 7) / 8 * 8 : min((total + 7) / 8 * 8, cus / 8 * 8));
  if (bits == 8) {
    if (a.swiglu) gemm_mx_kernel<8, true, false><<<grid, kMxWaves * kWave, 0, stream>>>(a, ntiles_n, mgroup);
    else gemm_mx_kernel<8, false, false><<<grid, kMxWaves * kWave, 0, stream>>>(a, ntiles_n, mgroup);
  } else if (a.hq_packed) {
    gemm_mx_kernel<4, true, true><<<grid, kMxWaves * kWave, 0, stream>>>(a, ntiles_n, mgroup);
  } else if (a.swiglu) {
    gemm_mx_kernel<4, true, false><<<grid, kMxWaves * kWave, 0, stream>>>(a, ntiles_n, mgroup);
  } else {
    gemm_mx_kernel<4, false, false><<<grid, kMxWaves * kWave, 0, stream>>>(a, ntiles_n, mgroup);
  }
  if (a.ksplit <= 1) return hipGetLastError();
  const hipError_t e2 = hipGetLastError();
  if (e2 != hipSuccess) return e2;
  return launch_splitk_reduce(a, stream);
}

}  // namespace nvfp4moe
