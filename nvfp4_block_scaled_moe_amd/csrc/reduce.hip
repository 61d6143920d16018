// Unpermute + weighted top-k reduce (gfx950).
//
// The scatter half of the MoE's expert scatter/gather ("The 2x Gap: Diagnosing Suboptimal
// FP4 GEMM Kernels on Blackwell SM120", section "Discovering the sgl_kernel Alternative"):
//   out[t, :] = bf16( sum_{j<k} w[t, j] * Y[slot_to_row[t*k + j], :] ),
// float32 fused multiply-adds in ascending j, so the result does not depend on thread
// timing. HBM-bound: k rows of Y read and one bf16 row written per token; each thread
// handles 8 consecutive columns with 16/32-byte vector accesses, and requests the rows of
// 8 slots at a time so their latencies overlap. Many tokens: one workgroup per token
// (H/8 threads rounded up to whole waves, up to 1024), so no workgroup idles on a partial
// column block; few tokens: 256-thread column blocks, spreading a token over more CUs.
#include "common.h"
#include "kernels.h"

namespace nvfp4moe {

namespace {

constexpr int kRedThreads = 256;       // column block for few tokens
constexpr int kRedMaxThreads = 1024;   // one workgroup per token from kRedRowTokens tokens on
constexpr int kRedRowTokens = 256;

constexpr int kRedBatch = 8;   // slots whose rows are requested together

// NT = 0: one workgroup per token of blockDim.x threads (up to kRedMaxThreads); else column
// blocks of NT threads.
template <bool YBF16, int NT>
__global__ __launch_bounds__(NT ? NT : kRedMaxThreads) void unpermute_reduce_kernel(const void* __restrict__ y,
                                                                       const int* __restrict__ slot_to_row,
                                                                       const float* __restrict__ topk_w,
                                                                       int k, int H,
                                                                       uint16_t* __restrict__ out) {
  int t, c;
  if (NT) {
    const int cblocks = (H / 8 + NT - 1) / NT;
    t = blockIdx.x / cblocks;
    c = ((blockIdx.x - t * cblocks) * NT + threadIdx.x) * 8;
  } else {
    t = blockIdx.x;
    c = threadIdx.x * 8;
  }
  if (c >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // Up to kRedBatch rows are requested before the first of them is summed; the sum itself
  // stays in ascending j.
  for (int j0 = 0; j0 < k; j0 += kRedBatch) {
    const int n = min(kRedBatch, k - j0);
    size_t row[kRedBatch];
    float w[kRedBatch];
#pragma unroll
    for (int j = 0; j < kRedBatch; ++j) {
      // the token is uniform over the workgroup: scalar loads
      row[j] = j < n ? (size_t)ld_const(slot_to_row, (int64_t)t * k + j0 + j) : 0;
      w[j] = j < n ? ld_const(topk_w, (int64_t)t * k + j0 + j) : 0.f;
    }
    float v[kRedBatch][8];
#pragma unroll
    for (int j = 0; j < kRedBatch; ++j) {
      if (j < n) {
        if (YBF16) {
          uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(y) + row[j] * H + c);
          uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[j][2 * i] = bf16_to_f32(u[i] & 0xffffu);
            v[j][2 * i + 1] = bf16_to_f32(u[i] >> 16);
          }
        } else {
          const float* yr = static_cast<const float*>(y) + row[j] * H + c;
          float4 a = *reinterpret_cast<const float4*>(yr);
          float4 b = *reinterpret_cast<const float4*>(yr + 4);
          v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
          v[j][4] = b.x; v[j][5] = b.y; v[j][6] = b.z; v[j][7] = b.w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kRedBatch; ++j) {
      if (j < n) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[j], v[j][i], acc[i]);
      }
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = bf16x2(acc[2 * i], acc[2 * i + 1]);
  *reinterpret_cast<uint4*>(out + (size_t)t * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_unpermute_reduce(const void* y, bool y_bf16, const int* slot_to_row,
                                   const float* topk_w, int T, int k, int H, uint16_t* out,
                                   hipStream_t stream) {
  const int per = H / 8;   // threads a token's row needs
  if (T >= kRedRowTokens && per <= kRedMaxThreads) {
    const int nt = (per + kWave - 1) / kWave * kWave;
    if (y_bf16)
      unpermute_reduce_kernel<true, 0><<<T, nt, 0, stream>>>(y, slot_to_row, topk_w, k, H, out);
    else
      unpermute_reduce_kernel<false, 0><<<T, nt, 0, stream>>>(y, slot_to_row, topk_w, k, H, out);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((per + kRedThreads - 1) / kRedThreads) * (unsigned)T;
  if (y_bf16)
    unpermute_reduce_kernel<true, kRedThreads><<<grid, kRedThreads, 0, stream>>>(y, slot_to_row, topk_w, k, H, out);
  else
    unpermute_reduce_kernel<false, kRedThreads><<<grid, kRedThreads, 0, stream>>>(y, slot_to_row, topk_w, k, H, out);
  return hipGetLastError();
}

}  // namespace nvfp4moe
