// Small-M NVFP4 grouped GEMM, weight-streaming (gfx950).
//
// The decode regime of the MoE: each expert sees a handful of token rows (~16 at 512
// concurrent requests with 8 of 256 experts; "The 2x Gap: Diagnosing Suboptimal FP4 GEMM
// Kernels on Blackwell SM120", section "The Investigation So Far"), so every weight byte is
// used by at most a few rows and the kernel is bound by HBM bandwidth on weight + scale
// bytes (9/16 byte per weight). The design streams each weight exactly once:
//
//   * Workgroup = WAVES wavefronts = one (expert, block of 16*RB weight rows) tile; the
//     waves split K in 128-wide chunks (wave w takes chunks w, w+WAVES, ...), so the
//     activation fragments a wave needs are needed by no other wave of the workgroup.
//   * Each lane loads 16 bytes of one weight row per chunk (32 FP4 codes); lanes
//     16g..16g+15 take 16 consecutive rows at k-offset 32g. Loads go through buffer
//     resources: 32-bit offsets, the row-block offset in an SGPR, and out-of-range offsets
//     returning zero, which handles the K tail and padded token lanes without branches.
//   * The tile's E4M3 scales are copied to LDS once with coalesced 16-byte loads; per chunk
//     a lane reads its two scale bytes from LDS. (Reading them from memory per chunk costs
//     a cache-line access per 2 bytes and starved the L1.)
//   * Activations (W4A16) come from the f16 copy written in MFMA operand order, so the four
//     lane groups of a token read one contiguous 64-byte piece per load instruction.
//   * Software pipelining: the fragments of the wave's next chunk are in flight while the
//     current chunk is decoded and multiplied (two register buffers).
//   * Decode in registers: hardware FP4 -> f16 convert and one packed f16 multiply by the
//     block scale per two weights. Both steps are exact (E2M1 * E4M3 has <= 6 significant
//     bits), so the MFMA sees exactly the dequantized weights.
//   * v_mfma_f32_16x16x32_f16 with the weights as the 16x32 A operand and up to 16 token
//     rows as the 32x16 B operand, FP32 accumulation in registers over the wave's K range.
//     Rows of an expert beyond 16*TBM are handled in further passes.
//   * The K partial sums of the waves are added in LDS in a fixed order (deterministic);
//     the epilogue applies the float32 global scales (w_g, and a_g for W4A4, or the
//     power-of-two row scale of the f16 activations), SwiGLU when asked, and stores.
//   * Tiles are numbered expert-major and handed out XCD-major (workgroup i runs on XCD
//     i mod 8), so the tiles of one expert, which share its activation rows, share an L2.
#include <cstdio>
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace nvfp4moe {

namespace {

constexpr int kChunk = 128;              // k per lane-load round (16 bytes of FP4 per lane)
constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past every resource: loads return 0
constexpr int kRsrcFlags = 0x00020000;   // raw buffer resource word 3 for gfx9 (32-bit data)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcFlags);
}
__device__ __forceinline__ u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

template <int RB, int NTB, bool A4>
struct Frag {
  u32x4 w[RB];               // 32 FP4 weights of this lane's row, per row block
  u32x4 b[NTB][A4 ? 1 : 4];  // W4A16: 4 x 8 f16 activations; W4A4: 32 FP4 codes
  uint32_t bs[NTB];          // W4A4: two E4M3 activation scales
};

template <int N>
struct Int {
  static constexpr int value = N;
};

// LDS row pitch of the staged weight scales (16-byte aligned, padded against bank conflicts).
__host__ __device__ constexpr int scale_pitch(int Ks) { return ((Ks + 15) & ~15) + 16; }

template <int RB, int WAVES, int TBM, bool SWIGLU, bool A4>
__global__ __launch_bounds__(WAVES * kWave) void gemm_stream_kernel(const GemmArgs p,
                                                                    int tiles_per_expert,
                                                                    int total_tiles) {
  static_assert(RB % 2 == 0, "row blocks come in pairs");
  static_assert(TBM == 2, "token blocks per pass");
  constexpr int NT = WAVES * kWave;
  constexpr int PER_BLK = TBM * 256;  // floats of one 16-row block for TBM token blocks
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int per_xcd = gridDim.x >> 3;
  const int tile = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (tile >= total_tiles) return;
  const int aidx = tile / tiles_per_expert;
  const int nb = tile - aidx * tiles_per_expert;
  if (aidx >= p.n_active[0]) return;
  const int e = p.active[aidx];
  const int r0 = p.expert_offsets[e];
  const int M = p.expert_offsets[e + 1] - r0;
  const int K = p.K, Nw = p.Nw, Kh = K >> 1, Ks = K >> 4;
  const int K128 = (K + 127) & ~127;
  const int F = Nw >> 1;
  const int Ksp = scale_pitch(Ks);
  unsigned char* sc = smem;                                    // [16*RB][Ksp] weight scales
  float* red = reinterpret_cast<float*>(smem + 16 * RB * Ksp);  // [WAVES][2][PER_BLK]

  // Weight rows: tile row 0, lane row of block 0, and the (uniform) row offset of block b.
  const int row0 = SWIGLU ? nb * 8 * RB : nb * 16 * RB;
  auto blkrow = [&](int b) -> int {
    if (SWIGLU) return b < RB / 2 ? 16 * b : F + 16 * (b - RB / 2);
    return 16 * b;
  };
  const unsigned char* wsc = p.w_scales + (size_t)e * Nw * Ks;
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(p.w_packed + (size_t)e * Nw * Kh, (uint32_t)Nw * (uint32_t)Kh);
  const uint32_t wlane = (uint32_t)(row0 + l16) * Kh + 16 * g;
  const float alpha = A4 ? p.w_g[e] * p.a_g[0] : p.w_g[e];
  const int nch = (K + kChunk - 1) / kChunk;
  const int n_it = (nch + WAVES - 1) / WAVES;  // chunk rounds per wave (same for all waves)
  uint32_t amax_bits = 0;

  // Activation resources sized to the real tensors, so kOOB offsets read zero.
  __amdgpu_buffer_rsrc_t ar, asr;
  if (A4) {
    ar = make_rsrc(p.a_packed, (uint32_t)p.a_rows * (uint32_t)Kh);
    asr = make_rsrc(p.a_scales, (uint32_t)p.a_rows * (uint32_t)Ks);
  } else {
    ar = make_rsrc(p.a16, (uint32_t)p.a_rows * (uint32_t)K128 * 2u);
    asr = ar;
  }

  // Stage the tile's weight scales in LDS with coalesced loads (once per tile).
  auto stage_scales = [&]() {
    if ((Ks & 15) == 0) {
      const int per_row = Ks >> 4;
      for (int u = tid; u < 16 * RB * per_row; u += NT) {
        const int lr = u / per_row, cu = u - lr * per_row;
        const int row = row0 + blkrow(lr >> 4) + (lr & 15);
        *reinterpret_cast<uint4*>(sc + lr * Ksp + 16 * cu) =
            *reinterpret_cast<const uint4*>(wsc + (size_t)row * Ks + 16 * cu);
      }
    } else {
      const int per_row = Ks >> 1;
      for (int u = tid; u < 16 * RB * per_row; u += NT) {
        const int lr = u / per_row, cu = u - lr * per_row;
        const int row = row0 + blkrow(lr >> 4) + (lr & 15);
        *reinterpret_cast<uint16_t*>(sc + lr * Ksp + 2 * cu) =
            *reinterpret_cast<const uint16_t*>(wsc + (size_t)row * Ks + 2 * cu);
      }
    }
  };

  bool staged = false;
  for (int tc = 0; tc < M; tc += 16 * TBM) {
    const int ntb = __builtin_amdgcn_readfirstlane(min(TBM, (M - tc + 15) >> 4));
    // B-operand row offsets of this lane (token column l16 of each token block).
    uint32_t boff[TBM], bsoff[TBM];
#pragma unroll
    for (int tb = 0; tb < TBM; ++tb) {
      const int t = tc + 16 * tb + l16;
      const int r = r0 + t;
      const uint32_t arow = (t < M) ? (uint32_t)(p.gather_index ? p.gather_index[r] / p.gather_div : r) : 0u;
      const bool ok = t < M;
      if (A4) {
        boff[tb] = ok ? arow * (uint32_t)Kh + 16 * g : kOOB;
        bsoff[tb] = ok ? arow * (uint32_t)Ks + 2 * g : kOOB;
      } else {
        boff[tb] = ok ? (arow * (uint32_t)K128 + 8 * g) * 2 : kOOB;
        bsoff[tb] = 0;
      }
    }

    f32x4 acc[RB][TBM];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) acc[b][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};

    auto kloop = [&](auto ntb_tag) {
      constexpr int NTB = decltype(ntb_tag)::value;
      auto load = [&](Frag<RB, NTB, A4>& f, int it) {
        const int c = wave + it * WAVES;
        const int kc = c * kChunk;
        const bool kin = c < nch && (kc + 32 * g) < K;   // this lane group's 32 k are inside K
        const uint32_t wo = kin ? wlane + (uint32_t)(kc >> 1) : kOOB;
#pragma unroll
        for (int b = 0; b < RB; ++b) f.w[b] = ld128(wr, wo, (uint32_t)blkrow(b) * Kh);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          if (A4) {
            f.b[tb][0] = ld128(ar, kin ? boff[tb] + (uint32_t)(kc >> 1) : kOOB, 0);
            f.bs[tb] = ld16(asr, kin ? bsoff[tb] + (uint32_t)(kc >> 4) : kOOB, 0);
          } else {
            // padded rows: only chunks past the end need the out-of-range offset
            const uint32_t o = c < nch ? boff[tb] + (uint32_t)kc * 2 : kOOB;
#pragma unroll
            for (int j = 0; j < 4; ++j) f.b[tb][j] = ld128(ar, o, 64 * j);
            f.bs[tb] = 0;
          }
        }
      };
      auto compute = [&](const Frag<RB, NTB, A4>& f, int it) {
        const int kc = (wave + it * WAVES) * kChunk;
        f16x8 bf[NTB][4];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          if (A4) {
            f16x2 s0, s1;
            decode_scale_pair(f.bs[tb], s0, s1);
            bf[tb][0] = decode8(f.b[tb][0][0], s0);
            bf[tb][1] = decode8(f.b[tb][0][1], s0);
            bf[tb][2] = decode8(f.b[tb][0][2], s1);
            bf[tb][3] = decode8(f.b[tb][0][3], s1);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) bf[tb][j] = __builtin_bit_cast(f16x8, f.b[tb][j]);
          }
        }
        // Scales of the lane's 32 k: two bytes in LDS (zero past the end of K, as the
        // weights read there are zero too).
        const int soff = (kc >> 4) + 2 * g;
        const bool sin = (kc + 32 * g) < K;
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const uint32_t sv = sin ? *reinterpret_cast<const uint16_t*>(sc + (16 * b + l16) * Ksp + soff) : 0u;
          f16x2 s0, s1;
          decode_scale_pair(sv, s0, s1);
          const f16x8 w0 = decode8(f.w[b][0], s0), w1 = decode8(f.w[b][1], s0);
          const f16x8 w2 = decode8(f.w[b][2], s1), w3 = decode8(f.w[b][3], s1);
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb) {
            acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w0, bf[tb][0], acc[b][tb], 0, 0, 0);
            acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w1, bf[tb][1], acc[b][tb], 0, 0, 0);
            acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w2, bf[tb][2], acc[b][tb], 0, 0, 0);
            acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w3, bf[tb][3], acc[b][tb], 0, 0, 0);
          }
        }
      };
      // Two-deep software pipeline over this wave's chunks.
      Frag<RB, NTB, A4> f0, f1;
      load(f0, 0);
      if (!staged) {        // first pass: the scale copy overlaps the first weight loads
        stage_scales();
        __syncthreads();
        staged = true;
      }
      int it = 0;
      for (; it + 1 < n_it; it += 2) {
        load(f1, it + 1);
        compute(f0, it);
        load(f0, it + 2);   // past the last round the offsets are out of range: loads return 0
        compute(f1, it + 1);
      }
      if (it < n_it) compute(f0, it);
    };
    if (ntb == 1) kloop(Int<1>{});
    else kloop(Int<2>{});

    // Cross-wave K reduction (fixed order) and epilogue, two row blocks at a time.
    // D layout of v_mfma_f32_16x16x32: lane l holds rows 4*(l/16)+i, column l%16.
#pragma unroll
    for (int q = 0; q < RB / 2; ++q) {
      const int b0 = q, b1 = q + RB / 2;
      float* my0 = red + (wave * 2 + 0) * PER_BLK + lane * 4;
      float* my1 = red + (wave * 2 + 1) * PER_BLK + lane * 4;
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) {
        *reinterpret_cast<f32x4*>(my0 + tb * 256) = acc[b0][tb];
        *reinterpret_cast<f32x4*>(my1 + tb * 256) = acc[b1][tb];
      }
      __syncthreads();
      for (int idx = tid; idx < ntb * 256; idx += NT) {
        const int tb = idx >> 8, ln = (idx >> 2) & 63, i = idx & 3;
        const int t = tc + 16 * tb + (ln & 15);
        if (t >= M) continue;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
          s0 += red[(w * 2 + 0) * PER_BLK + idx];
          s1 += red[(w * 2 + 1) * PER_BLK + idx];
        }
        const int row = r0 + t;
        int pexp = 0;
        if (!A4) {
          const int a_r = p.gather_index ? p.gather_index[row] / p.gather_div : row;
          pexp = p.rexp[a_r];
        }
        const float v0 = ldexpf(s0 * alpha, pexp);
        const float v1 = ldexpf(s1 * alpha, pexp);
        const int coff = 4 * (ln >> 4) + i;
        if (SWIGLU) {
          const float h = v0 / (1.0f + expf(-v0)) * v1;
          const size_t o = (size_t)row * F + nb * 8 * RB + 16 * q + coff;
          if (p.out_bf16) static_cast<uint16_t*>(p.out)[o] = (uint16_t)f32_to_bf16(h);
          else static_cast<float*>(p.out)[o] = h;
          amax_bits = max(amax_bits, abs_bits(h));
        } else {
          const size_t o0 = (size_t)row * Nw + nb * 16 * RB + 16 * b0 + coff;
          const size_t o1 = (size_t)row * Nw + nb * 16 * RB + 16 * b1 + coff;
          if (p.out_bf16) {
            static_cast<uint16_t*>(p.out)[o0] = (uint16_t)f32_to_bf16(v0);
            static_cast<uint16_t*>(p.out)[o1] = (uint16_t)f32_to_bf16(v1);
          } else {
            static_cast<float*>(p.out)[o0] = v0;
            static_cast<float*>(p.out)[o1] = v1;
          }
          amax_bits = max(amax_bits, max(abs_bits(v0), abs_bits(v1)));
        }
      }
      __syncthreads();
    }
  }

  if (p.out_amax) {
    amax_bits = wave_max_u32(amax_bits);
    if (lane == 0 && amax_bits) atomicMax(reinterpret_cast<unsigned int*>(p.out_amax), amax_bits);
  }
}

template <int RB, int WAVES, bool SWIGLU, bool A4>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  constexpr int TBM = 2;
  const int tiles_per_expert = a.Nw / (16 * RB);
  const int max_active = a.E < a.rows ? a.E : a.rows;
  const int total = max_active * tiles_per_expert;
  const int grid = (total + 7) / 8 * 8;
  const size_t shmem = (size_t)16 * RB * scale_pitch(a.K / 16) + (size_t)WAVES * 2 * TBM * 256 * sizeof(float);
  gemm_stream_kernel<RB, WAVES, TBM, SWIGLU, A4>
      <<<grid, WAVES * kWave, shmem, stream>>>(a, tiles_per_expert, total);
  return hipGetLastError();
}

// Tile shape (row blocks per tile, waves per workgroup). NVFP4MOE_STREAM_TILE=<rb>x<waves>
// overrides the default for tuning; a shape that does not divide Nw falls back to RB=2.
template <bool SWIGLU, bool A4>
hipError_t launch_sw(const GemmArgs& a, hipStream_t stream) {
  const int blocks16 = a.Nw / 16;  // even, since Nw % 32 == 0
  int rb = 4, waves = 4;
  if (const char* s = std::getenv("NVFP4MOE_STREAM_TILE")) std::sscanf(s, "%dx%d", &rb, &waves);
  if (blocks16 % rb != 0) rb = blocks16 % 4 == 0 ? 4 : 2;
  if (rb == 8 && waves == 4) return launch_cfg<8, 4, SWIGLU, A4>(a, stream);
  if (rb == 8 && waves == 2) return launch_cfg<8, 2, SWIGLU, A4>(a, stream);
  if (rb == 4 && waves == 8) return launch_cfg<4, 8, SWIGLU, A4>(a, stream);
  if (rb == 4 && waves == 2) return launch_cfg<4, 2, SWIGLU, A4>(a, stream);
  if (rb == 4) return launch_cfg<4, 4, SWIGLU, A4>(a, stream);
  return launch_cfg<2, 4, SWIGLU, A4>(a, stream);
}

}  // namespace

hipError_t launch_gemm_stream(const GemmArgs& a, hipStream_t stream) {
  if (a.swiglu) return a.w4a4 ? launch_sw<true, true>(a, stream) : launch_sw<true, false>(a, stream);
  return a.w4a4 ? launch_sw<false, true>(a, stream) : launch_sw<false, false>(a, stream);
}

}  // namespace nvfp4moe
