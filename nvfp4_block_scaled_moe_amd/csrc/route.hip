// Router (softmax top-k, renormalised) and the histogram/permutation pass (gfx950).
//
// Shapes from "The 2x Gap: Diagnosing Suboptimal FP4 GEMM Kernels on Blackwell SM120",
// section "The Investigation So Far" (8 of 256 experts per token) and "Native FP4 Is
// Slower Than Emulated FP4", section 1 (22 of 512). The permutation is the
// expert-scatter/gather of a fused MoE ("The 2x Gap", section "Discovering the sgl_kernel
// Alternative"): rows of one expert become contiguous so each expert runs one GEMM.
//
// Router: one wavefront per token. Each lane holds E/64 logits in registers; k rounds of
// a wave-wide arg-max (ties to the lower id) pick the experts. The arg-max is two DPP
// max-reductions (no LDS round trips): of the value as an order-preserving uint32, then,
// among the lanes holding that value, of the complemented expert id. The weights
// exp(l_j - l_max) / sum_j' exp(l_j' - l_max) over the k kept logits equal softmax over E
// followed by renormalisation; they are computed in float64 and rounded once.
//
// Permutation: one 1024-thread workgroup, deterministic by construction:
//   1. each wave counts the experts of its contiguous slice of slots (LDS integer atomics:
//      the counts do not depend on their order);
//   2. per expert: prefix over waves, then a block-wide exclusive scan over experts gives
//      expert_offsets, every wave's first row per expert, and the compacted active list;
//   3. each wave walks its slice again 64 slots at a time; a lane's rank among the lanes
//      holding the same expert comes from wavefront ballots over the bits of the expert id
//      (lanes with equal ids = AND of matching ballots) and a popcount of the lower lanes.
//      Slots therefore land in ascending order within each expert: a stable counting sort.
#include "common.h"
#include "kernels.h"

namespace nvfp4moe {

namespace {

constexpr int kRouterWaves = 4;
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

template <int PL>
__global__ __launch_bounds__(kRouterWaves* kWave) void router_kernel(const float* __restrict__ logits,
                                                                     int T, int E, int k,
                                                                     int* __restrict__ ids,
                                                                     float* __restrict__ w) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kRouterWaves + threadIdx.x / kWave;
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[PL];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + kWave * i;
    v[i] = -INFINITY;
    if (e < E) {
      const float x = row[e];
      v[i] = (x != x) ? -INFINITY : x;
      avail |= 1u << i;
    }
  }
  float selv = 0.0f;
  int seli = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + kWave * i;
      if (((avail >> i) & 1u) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
    // wave argmax: the largest value (as an order-preserving uint32, zeros made +0 so that
    // -0 == +0), then the lowest expert id among the lanes holding it
    const float cv = bv == 0.0f ? 0.0f : bv;
    const uint32_t ub = __float_as_uint(cv);
    const uint32_t key = (ub & 0x80000000u) ? ~ub : (ub | 0x80000000u);
    const uint32_t kmax = wave_max_u32_uniform(key);
    be = (int)~wave_max_u32_uniform(key == kmax ? ~(uint32_t)be : 0u);
    bv = __uint_as_float((kmax & 0x80000000u) ? (kmax & 0x7fffffffu) : ~kmax);
    if ((be % kWave) == lane) avail &= ~(1u << (be / kWave));
    if (lane == j) {
      selv = bv;
      seli = be;
    }
  }
  const double m = (double)__shfl(selv, 0, kWave);  // the first pick is the row maximum
  double ex = (lane < k) ? exp((double)selv - m) : 0.0;
  double sum = ex;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
  if (lane < k) {
    ids[(size_t)t * k + lane] = seli;
    w[(size_t)t * k + lane] = (float)(ex / sum);
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int* __restrict__ ids, int S,
                                                               int E, int nbits,
                                                               int* __restrict__ offsets,
                                                               int* __restrict__ sorted_slot,
                                                               int* __restrict__ slot_to_row,
                                                               int* __restrict__ active,
                                                               int* __restrict__ n_active) {
  extern __shared__ int sm[];
  int* cnt = sm;                          // [kPermWaves][E]
  int* wsum = sm + kPermWaves * E;        // [kPermWaves] row totals per wave
  int* wflag = wsum + kPermWaves;         // [kPermWaves] active-expert totals per wave
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

  for (int i = tid; i < kPermWaves * E; i += kPermThreads) cnt[i] = 0;
  __syncthreads();

  const int per = ((S + kPermWaves - 1) / kPermWaves + kWave - 1) / kWave * kWave;
  const int lo = min(S, wave * per), hi = min(S, lo + per);
  for (int s = lo + lane; s < hi; s += kWave) atomicAdd(&cnt[wave * E + ids[s]], 1);
  __syncthreads();

  // 2. per expert e = tid: prefix over waves, then scans over experts.
  const int e = tid;
  int tot = 0;
  if (e < E) {
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = tot;
      tot += c;
    }
  }
  const int flag = (e < E && tot > 0) ? 1 : 0;
  int incl = tot, fincl = flag;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int a = __shfl_up(incl, o, kWave);
    const int b = __shfl_up(fincl, o, kWave);
    if (lane >= o) {
      incl += a;
      fincl += b;
    }
  }
  if (lane == kWave - 1) {
    wsum[wave] = incl;
    wflag[wave] = fincl;
  }
  __syncthreads();
  int before = 0, fbefore = 0, nact = 0;
  for (int w = 0; w < kPermWaves; ++w) {
    if (w < wave) {
      before += wsum[w];
      fbefore += wflag[w];
    }
    nact += wflag[w];
  }
  const int base = before + incl - tot;     // exclusive prefix over experts
  const int fpos = fbefore + fincl - flag;  // position in the active list
  if (e < E) {
    offsets[e] = base;
    for (int w = 0; w < kPermWaves; ++w) cnt[w * E + e] += base;
    if (e >= nact) active[e] = -1;
    if (flag) active[fpos] = e;
    if (e == E - 1) {
      offsets[E] = base + tot;
      n_active[0] = nact;
    }
  }
  __syncthreads();

  // 3. stable scatter, 64 slots per step, ranks from ballots.
  for (int s0 = lo; s0 < hi; s0 += kWave) {
    const int s = s0 + lane;
    const bool valid = s < hi;
    const int ex = valid ? ids[s] : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (ex >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    const int start = valid ? cnt[wave * E + ex] : 0;
    const bool leader = valid && ((peers >> lane) == 1ull);  // highest lane of its group
    if (leader) cnt[wave * E + ex] = start + __popcll(peers);
    if (valid) {
      const int row = start + rank;
      sorted_slot[row] = s;
      slot_to_row[s] = row;
    }
  }
}


}  // namespace

hipError_t launch_route_permute(const float* logits, int T, int E, int k, int* topk_ids,
                                float* topk_w, int* expert_offsets, int* sorted_slot,
                                int* slot_to_row, int* active_experts, int* n_active,
                                hipStream_t stream) {
  const unsigned rgrid = (unsigned)((T + kRouterWaves - 1) / kRouterWaves);
  const int pl = (E + kWave - 1) / kWave;
  if (pl <= 1)
    router_kernel<1><<<rgrid, kRouterWaves * kWave, 0, stream>>>(logits, T, E, k, topk_ids, topk_w);
  else if (pl <= 2)
    router_kernel<2><<<rgrid, kRouterWaves * kWave, 0, stream>>>(logits, T, E, k, topk_ids, topk_w);
  else if (pl <= 4)
    router_kernel<4><<<rgrid, kRouterWaves * kWave, 0, stream>>>(logits, T, E, k, topk_ids, topk_w);
  else if (pl <= 8)
    router_kernel<8><<<rgrid, kRouterWaves * kWave, 0, stream>>>(logits, T, E, k, topk_ids, topk_w);
  else
    router_kernel<16><<<rgrid, kRouterWaves * kWave, 0, stream>>>(logits, T, E, k, topk_ids, topk_w);

  static std::atomic<uint64_t> perm_attr_done{0};
  const hipError_t attr = ensure_dynamic_lds(reinterpret_cast<const void*>(&permute_kernel),
                                             (kPermWaves * kMaxExperts + 2 * kPermWaves) * (int)sizeof(int),
                                             perm_attr_done);
  if (attr != hipSuccess) return attr;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const size_t shmem = (size_t)(kPermWaves * E + 2 * kPermWaves) * sizeof(int);
  permute_kernel<<<1, kPermThreads, shmem, stream>>>(topk_ids, T * k, E, nbits, expert_offsets,
                                                     sorted_slot, slot_to_row, active_experts,
                                                     n_active);
  return hipGetLastError();
}

}  // namespace nvfp4moe
