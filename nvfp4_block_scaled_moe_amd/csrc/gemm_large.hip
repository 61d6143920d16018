// Large-M NVFP4 grouped GEMM (gfx950): the prefill regime, where experts see hundreds to
// thousands of rows and the GEMMs are bound by the matrix cores, not by weight bytes
// ("The 2x Gap: Diagnosing Suboptimal FP4 GEMM Kernels on Blackwell SM120", section "The
// Pivot: Comparing FP4 Against BF16": at M=512 and beyond FP4 pays off through compute).
//
//   * m-tiles: 128 consecutive rows of one expert. mtile_schedule_kernel lists them on the
//     device (expert, first row) for the active experts in order, so the grid needs no
//     host-side knowledge of the per-expert counts: grid = (upper bound on the m-tile
//     count) x (row tiles), and workgroups past the list exit at once.
//   * Workgroup = 8 waves = 256 weight rows (each wave: 2 blocks of 16 rows over all of K;
//     for SwiGLU one gate and the matching up block) x one m-tile. A ragged m-tile runs with
//     1, 2, 4 or 8 blocks of 16 rows.
//   * Weights (MFMA A operand): each lane loads 16 bytes (32 FP4 codes) of its row per
//     128-wide chunk and the two E4M3 scale bytes that cover them, WDEPTH chunks ahead, into
//     registers; they are decoded exactly to f16 (hardware FP4 convert, one packed f16
//     multiply by the block scale) one chunk ahead of use, interleaved with the MFMAs.
//   * Activations (B operand): f16 rows in MFMA operand order (bf16 rows scaled per row by a
//     power of two, or NVFP4 rows decoded exactly), staged per chunk through a three-slot
//     LDS ring (one 16-byte load and store per thread and round). Three slots let every wave
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

template <int WAVES, int WDEPTH, bool SWIGLU>
__global__ __launch_bounds__(WAVES* kWave, 2) void gemm_large_kernel(const GemmArgs p, int ntiles_n,
                                                                     int total_tiles) {
  static_assert(WDEPTH >= 2 && kWin % WDEPTH == 0, "the weight ring is read one chunk ahead; steps pair up");
  constexpr int NT = WAVES * kWave;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int per_xcd = gridDim.x >> 3;
  const int tile = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (tile >= total_tiles) return;
  const int mt = tile / ntiles_n;            // m-tile
  const int nb = tile - mt * ntiles_n;       // row tile
  if (mt >= p.sched_n[0]) return;
  const int e = p.sched_e[mt], tc = p.sched_r[mt];
  const int r0 = p.expert_offsets[e];
  const int M = p.expert_offsets[e + 1] - r0;
  const int K = p.K, Nw = p.Nw;
  const int K128 = (K + 127) & ~127;
  const int F = Nw >> 1;
  const int nch = (K + kChunk - 1) / kChunk;
  const int nwin = (nch + kWin - 1) / kWin;
  const int ntb = __builtin_amdgcn_readfirstlane(min(kTBM, (M - tc + 15) >> 4));

  auto blkrow = [&](int b) -> int {
    if (SWIGLU) return (b == 0 ? 0 : F) + (nb * WAVES + wave) * 16;
    return (nb * WAVES + wave) * 16 * kRBW + 16 * b;
  };
  // Tiled weights (weights_tile.hip): lane l reads 16 bytes at 16 l of a 1 KB tile per
  // (16-row block, chunk) of codes and per (16-row block, 8-chunk window) of scales.
  const uint32_t wbytes = (uint32_t)(Nw / 16) * (uint32_t)nch * 1024u;
  const uint32_t sbytes = (uint32_t)(Nw / 16) * (uint32_t)nwin * 1024u;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w_packed + (size_t)e * wbytes, wbytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.w_scales + (size_t)e * sbytes, sbytes);
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(p.a16, (uint32_t)p.a_rows * (uint32_t)K128 * 2u);
  const uint32_t wlane = (uint32_t)(blkrow(0) / 16) * (uint32_t)nch * 1024u + 16u * lane;
  const uint32_t slane = (uint32_t)(blkrow(0) / 16) * (uint32_t)nwin * 1024u + 16u * lane;
  uint32_t wsoff[kRBW], ssoff[kRBW];
#pragma unroll
  for (int b = 0; b < kRBW; ++b) {
    wsoff[b] = __builtin_amdgcn_readfirstlane((uint32_t)((blkrow(b) - blkrow(0)) / 16) * (uint32_t)nch * 1024u);
    ssoff[b] = __builtin_amdgcn_readfirstlane((uint32_t)((blkrow(b) - blkrow(0)) / 16) * (uint32_t)nwin * 1024u);
  }
  const float alpha = p.w4a4 ? p.w_g[e] * p.a_g[0] : p.w_g[e];

  auto body = [&](auto ntb_tag) {
    constexpr int NTB = decltype(ntb_tag)::value;
    constexpr int TPT = 16;                          // threads per row (16 x 16 bytes)
    constexpr int TPR = NT / TPT;                    // rows per staging round
    constexpr int RND = (16 * NTB + TPR - 1) / TPR;
    uint32_t bsrc[RND], bdst[RND];
#pragma unroll
    for (int rr = 0; rr < RND; ++rr) {
      const int tk = rr * TPR + tid / TPT, pc = tid % TPT, t = tc + tk;
      const bool ok = tk < 16 * NTB && t < M;
      const uint32_t arow = ok ? (uint32_t)(p.gather_index ? p.gather_index[r0 + t] / p.gather_div : r0 + t) : 0u;
      bsrc[rr] = ok ? (arow * (uint32_t)K128 + 8 * pc) * 2 : kOOB;
      bdst[rr] = tk * kTokBytes + 16 * (pc ^ (tk & 15));   // tk < 128: inside the slot
    }
    u32x4 bst[2][RND];   // two staging sets: chunk c's loads are in flight for two steps
    auto b_issue = [&](int c, int set) {   // set: c % 2, passed as a constant
      const bool in = c < nch;
#pragma unroll
      for (int rr = 0; rr < RND; ++rr) bst[set][rr] = ld128(ar, in ? bsrc[rr] + (uint32_t)c * 256u : kOOB, 0);
    };
    // Rows past the tile's rows are loaded as zeros (kOOB) and stored like the others: every
    // store lands inside the slot, so the commit has no branch.
    static_assert(RND * TPR <= 16 * kTBM, "staging rounds stay inside one slot");
    auto b_commit = [&](int set, int slot) {
      unsigned char* base = smem + slot * kSlot;
#pragma unroll
      for (int rr = 0; rr < RND; ++rr) *reinterpret_cast<u32x4*>(base + bdst[rr]) = bst[set][rr];
    };
    auto b_read = [&](f16x8 (&dst)[NTB], int slot, int j) {
      const unsigned char* base = smem + slot * kSlot;
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const int tk = 16 * tb + l16;
        dst[tb] = *reinterpret_cast<const f16x8*>(base + tk * kTokBytes + 16 * ((4 * j + g) ^ (tk & 15)));
      }
    };
    u32x4 wring[WDEPTH][kRBW];
    auto w_issue = [&](int d, int c) {   // codes past K are zero in the tiles
#pragma unroll
      for (int b = 0; b < kRBW; ++b) wring[d][b] = ld128(wr, c < nch ? wlane + (uint32_t)c * 1024u : kOOB, wsoff[b]);
    };
    // One 16-byte load per block and window holds the lane's two scale bytes for each of
    // the window's 8 chunks; the current and the next window stay in registers.
    u32x4 scur[kRBW], snext[kRBW];
    auto s_issue = [&](int w) {
#pragma unroll
      for (int b = 0; b < kRBW; ++b) snext[b] = ld128(sr, w < nwin ? slane + (uint32_t)w * 1024u : kOOB, ssoff[b]);
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

    f32x4 acc[kRBW][kTBM];
#pragma unroll
    for (int b = 0; b < kRBW; ++b)
#pragma unroll
      for (int tb = 0; tb < kTBM; ++tb) acc[b][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // prologue: activations of chunks 0 and 1 into slots 0 and 1 (chunk 2 requested),
    // weights of chunks 0..WDEPTH-1 requested, chunk 0 decoded
    s_issue(0);
    b_issue(0, 0);
#pragma unroll
    for (int d = 0; d < WDEPTH; ++d) w_issue(d, d);
    b_commit(0, 0);
    b_issue(1, 1);
    b_commit(1, 1);
    b_issue(2, 0);
#pragma unroll
    for (int b = 0; b < kRBW; ++b) scur[b] = snext[b];
    scales(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) decode(wf, 0, j);
    __syncthreads();
    f16x8 bcur[NTB], bnext[NTB];
    b_read(bcur, 0, 0);

    // Step c: MFMAs of chunk c (LDS slot c % 3, decoded weights in wf) interleaved with the
    // LDS reads of the next k-step and the decode of chunk c+1. Activations of chunk c+2,
    // requested one step earlier, are stored to slot (c+2) % 3 before the step's barrier,
    // and those of chunk c+3 are requested. Vector-memory counters retire in order, so the
    // store waits only on requests at least one step old.
    int slot = 0;
    for (int c0 = 0; c0 < nch; c0 += kWin) {       // one scale window per iteration
      s_issue(c0 / kWin + 1);
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int c = c0 + u;
        if (c < nch) {
          const int d = u % WDEPTH, dn = (u + 1) % WDEPTH;
          const int slot1 = slot == kSlots - 1 ? 0 : slot + 1;
          const int slot2 = slot1 == kSlots - 1 ? 0 : slot1 + 1;
          b_issue(c + 3, (u + 1) & 1);             // c0 is even: chunk x uses set x % 2
          w_issue(d, c + WDEPTH);                  // ring entry d (chunk c) was decoded last step
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
          b_commit(u & 1, slot2);
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

    uint32_t amax_bits = store_tile<kRBW, kTBM, SWIGLU>(p, acc, tc, ntb, M, r0, alpha, !p.w4a4, blkrow, lane, 0u);
    merge_amax(p.out_amax, amax_bits, lane);
  };
  if (ntb > 4) body(Int<8>{});
  else if (ntb > 2) body(Int<4>{});
  else if (ntb == 2) body(Int<2>{});
  else body(Int<1>{});
}

// m-tiles of bm rows over the active experts (one workgroup, n_active <= 1024):
// sched_e[i] = expert, sched_r[i] = first row within the expert, sched_n[0] = count
// (at most max_tiles, the length of sched_e and sched_r).
__global__ __launch_bounds__(1024) void mtile_schedule_kernel(const int* __restrict__ offsets,
                                                             const int* __restrict__ active,
                                                             const int* __restrict__ n_active, int E,
                                                             int bm, int max_tiles, int* __restrict__ sched_e,
                                                             int* __restrict__ sched_r,
                                                             int* __restrict__ sched_n) {
  __shared__ int wsum[1024 / kWave];
  const int a = threadIdx.x, lane = a & 63, wave = a >> 6;
  const int na = min(n_active[0], E);
  int e = 0, cnt = 0;
  if (a < na) {
    e = active[a];
    cnt = (offsets[e + 1] - offsets[e] + bm - 1) / bm;
  }
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < 1024 / kWave; ++w) {
    if (w < wave) before += wsum[w];
    total += wsum[w];
  }
  const int base = before + incl - cnt;
  for (int i = 0; i < cnt && base + i < max_tiles; ++i) {
    sched_e[base + i] = e;
    sched_r[base + i] = i * bm;
  }
  if (a == 0) sched_n[0] = min(total, max_tiles);
}

template <int WAVES, int WDEPTH, bool SWIGLU>
hipError_t launch_cfg(const GemmArgs& a, int max_mtiles, hipStream_t stream) {
  const auto kern = &gemm_large_kernel<WAVES, WDEPTH, SWIGLU>;
  const size_t shmem = (size_t)kSlots * kSlot;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
  if (attr != hipSuccess) return attr;
  mtile_schedule_kernel<<<1, 1024, 0, stream>>>(a.expert_offsets, a.active, a.n_active, a.E, 16 * kTBM,
                                                max_mtiles, const_cast<int*>(a.sched_e),
                                                const_cast<int*>(a.sched_r), const_cast<int*>(a.sched_n));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ntiles_n = a.Nw / (16 * kRBW * WAVES);
  const int total = max_mtiles * ntiles_n;
  const int grid = (total + 7) / 8 * 8;
  kern<<<grid, WAVES * kWave, shmem, stream>>>(a, ntiles_n, total);
  return hipGetLastError();
}

// Weight ring depth 2: the chunk after next is in flight while a chunk is decoded (a deeper
// ring does not fit the 256 registers a wave has at two waves per SIMD).
template <bool SWIGLU>
hipError_t launch_sw(const GemmArgs& a, int max_mtiles, hipStream_t stream) {
  return launch_cfg<8, 2, SWIGLU>(a, max_mtiles, stream);
}

}  // namespace

int large_rows_per_mtile() { return 16 * kTBM; }
bool large_supports(int Nw) { return Nw % (16 * kRBW * 8) == 0; }

hipError_t launch_gemm_large(const GemmArgs& a, int max_mtiles, hipStream_t stream) {
  return a.swiglu ? launch_sw<true>(a, max_mtiles, stream) : launch_sw<false>(a, max_mtiles, stream);
}

}  // namespace nvfp4moe
