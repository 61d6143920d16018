// Small-M NVFP4 grouped GEMM, weight-streaming (gfx950).
//
// The decode regime of the MoE: each expert sees a handful of token rows (~16 at 512
// concurrent requests with 8 of 256 experts; "The 2x Gap: Diagnosing Suboptimal FP4 GEMM
// Kernels on Blackwell SM120", section "The Investigation So Far"), so every weight byte is
// used by at most a few rows and the kernel is bound by HBM bandwidth on weight + scale
// bytes (9/16 byte per weight). The design streams each weight exactly once:
//
//   * Workgroup = 8 wavefronts = one (expert, block of 16*RB weight rows) tile; the waves
//     split K in 128-wide chunks (wave w takes chunks w, w+8, ...), so the activation
//     fragments a wave needs are not needed by any other wave of the workgroup.
//   * Each lane loads 16 bytes of one weight row per chunk (32 FP4 codes) and the two E4M3
//     scales that cover them. Lanes 16g..16g+15 take 16 consecutive rows at k-offset 32g,
//     so a wave load reads 16 rows x 64 contiguous bytes.
//   * Decode in registers: hardware FP4 -> f16 convert and one packed f16 multiply by the
//     block scale per two weights. Both steps are exact (E2M1 * E4M3 has <= 6 significant
//     bits), so the MFMA sees exactly the dequantized weights.
//   * v_mfma_f32_16x16x32_f16 with the weights as the 16x32 A operand and up to 16 token
//     rows as the 32x16 B operand; the FP32 accumulators stay in registers for the whole K
//     range. Rows of an expert beyond 16*TBM are handled in further passes.
//   * The K partial sums of the 8 waves are added in LDS in a fixed order (deterministic),
//     then the epilogue applies the float32 global scales (w_g, and a_g for W4A4, or the
//     power-of-two row scale of the f16 activations), SwiGLU when asked, and stores.
//   * Tiles are numbered expert-major and handed out XCD-major (workgroup i runs on XCD
//     i mod 8), so the tiles of one expert, which share its activation rows, share an L2.
#include "common.h"
#include "kernels.h"

namespace nvfp4moe {

namespace {

constexpr int kStreamWaves = 8;
constexpr int kStreamThreads = kStreamWaves * kWave;
constexpr int kChunk = 128;  // k per lane-load round (16 bytes of FP4 per lane)

template <int RB, int TBM, bool SWIGLU, bool A4>
__global__ __launch_bounds__(kStreamThreads) void gemm_stream_kernel(const GemmArgs p,
                                                                     int tiles_per_expert,
                                                                     int total_tiles) {
  static_assert(RB % 2 == 0, "row blocks come in pairs");
  constexpr int PER_BLK = TBM * 256;  // floats of one 16-row block for TBM token blocks
  extern __shared__ float red[];      // [kStreamWaves][2][PER_BLK]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const int F = Nw >> 1;

  // Row (within the expert) of block 0 for this lane, and the row offset of block b.
  const int rowbase = SWIGLU ? nb * 8 * RB + l16 : nb * 16 * RB + l16;
  auto blkrow = [&](int b) -> int {
    if (SWIGLU) return b < RB / 2 ? 16 * b : F + 16 * (b - RB / 2);
    return 16 * b;
  };
  const uint8_t* wbase = p.w_packed + ((size_t)e * Nw + rowbase) * (size_t)Kh + 16 * g;
  const uint8_t* sbase = p.w_scales + ((size_t)e * Nw + rowbase) * (size_t)Ks + 2 * g;
  const float alpha = A4 ? p.w_g[e] * p.a_g[0] : p.w_g[e];
  const int nch = (K + kChunk - 1) / kChunk;
  uint32_t amax_bits = 0;

  for (int tc = 0; tc < M; tc += 16 * TBM) {
    const int ntb = min(TBM, (M - tc + 15) >> 4);
    // B-operand rows of this lane (token column l16 of each token block).
    size_t arow[TBM];
    bool tval[TBM];
#pragma unroll
    for (int tb = 0; tb < TBM; ++tb) {
      const int t = tc + 16 * tb + l16;
      tval[tb] = t < M;
      const int r = r0 + t;
      arow[tb] = tval[tb] ? (size_t)(p.gather_index ? p.gather_index[r] / p.gather_div : r) : 0;
    }

    f32x4 acc[RB][TBM];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) acc[b][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};

    for (int c = wave; c < nch; c += kStreamWaves) {
      const int kc = c * kChunk;
      const bool kin = (kc + 32 * g) < K;  // this lane group's 32 k lie inside K
      uint4 wv[RB];
      uint32_t sv[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        if (kin) {
          wv[b] = *reinterpret_cast<const uint4*>(wbase + (size_t)blkrow(b) * Kh + (kc >> 1));
          sv[b] = *reinterpret_cast<const uint16_t*>(sbase + (size_t)blkrow(b) * Ks + (kc >> 4));
        } else {
          wv[b] = make_uint4(0, 0, 0, 0);
          sv[b] = 0;
        }
      }
      f16x8 bf[TBM][4];
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) {
        const bool ld = tb < ntb && kin && tval[tb];
        if (A4) {
          uint4 av = make_uint4(0, 0, 0, 0);
          uint32_t as = 0;
          if (ld) {
            av = *reinterpret_cast<const uint4*>(p.a_packed + arow[tb] * (size_t)Kh + 16 * g + (kc >> 1));
            as = *reinterpret_cast<const uint16_t*>(p.a_scales + arow[tb] * (size_t)Ks + 2 * g + (kc >> 4));
          }
          f16x2 s0, s1;
          decode_scale_pair(as, s0, s1);
          bf[tb][0] = decode8(av.x, s0);
          bf[tb][1] = decode8(av.y, s0);
          bf[tb][2] = decode8(av.z, s1);
          bf[tb][3] = decode8(av.w, s1);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf[tb][j] = ld ? *reinterpret_cast<const f16x8*>(p.a16 + arow[tb] * (size_t)K + kc + 32 * g + 8 * j)
                           : (f16x8){0, 0, 0, 0, 0, 0, 0, 0};
          }
        }
      }
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        f16x2 s0, s1;
        decode_scale_pair(sv[b], s0, s1);
        const f16x8 w0 = decode8(wv[b].x, s0), w1 = decode8(wv[b].y, s0);
        const f16x8 w2 = decode8(wv[b].z, s1), w3 = decode8(wv[b].w, s1);
#pragma unroll
        for (int tb = 0; tb < TBM; ++tb) {
          if (tb < ntb) {
            acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w0, bf[tb][0], acc[b][tb], 0, 0, 0);
            acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w1, bf[tb][1], acc[b][tb], 0, 0, 0);
            acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w2, bf[tb][2], acc[b][tb], 0, 0, 0);
            acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w3, bf[tb][3], acc[b][tb], 0, 0, 0);
          }
        }
      }
    }

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
      for (int idx = tid; idx < PER_BLK; idx += kStreamThreads) {
        const int tb = idx >> 8, ln = (idx >> 2) & 63, i = idx & 3;
        const int t = tc + 16 * tb + (ln & 15);
        if (t >= M) continue;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int w = 0; w < kStreamWaves; ++w) {
          s0 += red[(w * 2 + 0) * PER_BLK + idx];
          s1 += red[(w * 2 + 1) * PER_BLK + idx];
        }
        const int row = r0 + t;
        int pexp = 0;
        if (!A4) {
          const int ar = p.gather_index ? p.gather_index[row] / p.gather_div : row;
          pexp = p.rexp[ar];
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

template <int RB, bool SWIGLU, bool A4>
hipError_t launch_rb(const GemmArgs& a, hipStream_t stream) {
  constexpr int TBM = 2;
  const int tiles_per_expert = a.Nw / (16 * RB);
  const int max_active = a.E < a.rows ? a.E : a.rows;
  const int total = max_active * tiles_per_expert;
  const int grid = (total + 7) / 8 * 8;
  const size_t shmem = (size_t)kStreamWaves * 2 * TBM * 256 * sizeof(float);
  gemm_stream_kernel<RB, TBM, SWIGLU, A4><<<grid, kStreamThreads, shmem, stream>>>(a, tiles_per_expert, total);
  return hipGetLastError();
}

template <bool SWIGLU, bool A4>
hipError_t launch_sw(const GemmArgs& a, hipStream_t stream) {
  const int blocks16 = a.Nw / 16;  // even, since Nw % 32 == 0
  if (blocks16 % 8 == 0) return launch_rb<8, SWIGLU, A4>(a, stream);
  if (blocks16 % 4 == 0) return launch_rb<4, SWIGLU, A4>(a, stream);
  return launch_rb<2, SWIGLU, A4>(a, stream);
}

}  // namespace

hipError_t launch_gemm_stream(const GemmArgs& a, hipStream_t stream) {
  if (a.swiglu) return a.w4a4 ? launch_sw<true, true>(a, stream) : launch_sw<true, false>(a, stream);
  return a.w4a4 ? launch_sw<false, true>(a, stream) : launch_sw<false, false>(a, stream);
}

}  // namespace nvfp4moe
