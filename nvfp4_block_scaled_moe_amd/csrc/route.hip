// Router (softmax top-k, renormalised) and the histogram/permutation pass (gfx950).
//
// Shapes from "The 2x Gap: Diagnosing Suboptimal FP4 GEMM Kernels on Blackwell SM120",
// section "The Investigation So Far" (8 of 256 experts per token) and "Native FP4 Is
// Slower Than Emulated FP4", section 1 (22 of 512). The permutation is the
// expert-scatter/gather of a fused MoE ("The 2x Gap", section "Discovering the sgl_kernel
// Alternative"): rows of one expert become contiguous so each expert runs one GEMM.
//
// Router: one wavefront per token. Each lane holds E/64 logits in registers; a bitwise search
// over order-preserving keys finds the k-th largest logit with wave ballots, and the k kept
// experts are ranked (descending logit, ties to the lower id) one per lane. The weights
// exp(l_j - l_max) / sum_j' exp(l_j' - l_max) over the k kept logits equal softmax over E
// followed by renormalisation; they are computed in float64 and rounded once. (Fewer than
// 256 tokens: a workgroup per token sorts instead.)
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
// Many slots (>= 16384): the same in two launches over chunks of slots. Few tokens (<= 16):
// routing and permutation in one workgroup and one launch (route_permute_small_kernel), with
// k rounds of wave argmax below top-16 and a threshold select from top-16 on, and up to 64
// slots a permutation that every wave derives from the slot ids alone, with no barrier.
#include <cstdlib>
#include <cstring>

#include "act_rows.h"
#include "common.h"
#include "kernels.h"

namespace nvfp4moe {

namespace {

constexpr int kRouterWaves = 4;
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kPermBatch = 16;   // 64-slot groups whose expert ids are loaded together

// Order-preserving uint32 key of a logit (NaN as -inf, -0 as +0): key order = value order.
__device__ __forceinline__ uint32_t logit_key(float x) {
  if (x != x) x = -INFINITY;
  if (x == 0.0f) x = 0.0f;
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_count(bool pred) { return __popcll(__ballot(pred)); }

// Router for one token per workgroup (max(NE/2, 64) threads, NE = E rounded up to a power of two,
// 64 <= NE <= 1024): a bitonic sort in LDS of 64-bit keys (order-preserving logit key << 32 |
// ~expert id) in descending order puts the experts by descending logit, ties to the lower id,
// first; padding entries get key 0, below every real logit. The sort has no serial per-expert
// chain, so one token costs log2(NE) * (log2(NE) + 1) / 2 short barrier-separated steps.
// Weights as in router_kernel, from the first k entries (one wave, float64).
template <int NE>
constexpr int router_sort_threads() { return NE / 2 > kWave ? NE / 2 : kWave; }

template <int NE>
__global__ __launch_bounds__(router_sort_threads<NE>()) void router_sort_kernel(const float* __restrict__ logits,
                                                                              int E, int k, int* __restrict__ ids,
                                                                              float* __restrict__ w) {
  constexpr int NT = router_sort_threads<NE>();
  __shared__ uint64_t s[NE];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const float* row = logits + (size_t)t * E;
  for (int e = tid; e < NE; e += NT) {
    const uint32_t key = e < E ? logit_key(row[e]) : 0u;
    s[e] = ((uint64_t)key << 32) | (uint32_t)~e;
  }
  __syncthreads();
#pragma unroll
  for (int size = 2; size <= NE; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (tid < NE / 2) {
        const int i = 2 * stride * (tid / stride) + (tid % stride), j = i + stride;
        const uint64_t a = s[i], b = s[j];
        const bool down = (i & size) == 0;   // this run is sorted descending
        if (down ? a < b : a > b) {
          s[i] = b;
          s[j] = a;
        }
      }
      __syncthreads();
    }
  }
  if (tid < kWave) {
    const int lane = tid;
    const int e = lane < k ? (int)~(uint32_t)s[lane] : 0;
    float x = lane < k ? row[e] : 0.0f;
    x = (x != x) ? -INFINITY : x;
    const double m = (double)__shfl(x, 0, kWave);   // the first entry holds the maximum
    const double ex = lane < k ? exp((double)x - m) : 0.0;
    double sum = ex;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
    if (lane < k) {
      ids[(size_t)t * k + lane] = e;
      w[(size_t)t * k + lane] = (float)(ex / sum);
    }
  }
}

// Top-k of one token by one wave without k serial rounds (the few-token kernel below also
// has route_token_rounds; both give the same ids, order and weights):
// the k-th largest key th is found bit by bit (the largest th with at least k keys >= th; a
// ballot per register and bit), the keys above th are kept and the lowest ids among those
// equal to th fill the rest, the k kept (key, id, logit) go to the wave's LDS scratch in id
// order, lane j takes entry j and counts the kept entries ahead of it (larger key, or equal
// key and lower id), and lane r then takes the entry of rank r, as round r would have.
// scratch: 3 x 64 words of the wave's own LDS.
template <int PL>
__device__ __forceinline__ void route_token_thresh(const float* __restrict__ row, int E, int k, int lane,
                                                   int* __restrict__ ids, float* __restrict__ w, int* lds_ids,
                                                   uint32_t* scratch) {
  uint32_t key[PL];
  float v[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + kWave * i;
    const float x = e < E ? row[e] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;
    key[i] = e < E ? logit_key(x) : 0u;   // every real key is >= logit_key(-inf) > 0
  }
  uint32_t th = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = th | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) cnt += wave_count(key[i] >= cand);
    if (cnt >= k) th = cand;
  }
  int need = k;
#pragma unroll
  for (int i = 0; i < PL; ++i) need -= wave_count(key[i] > th);
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int base = 0;   // kept entries in the registers before i (ids ascend with i, then lane)
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const uint64_t eq = __ballot(key[i] == th);
    const bool kept = key[i] > th || (((eq >> lane) & 1ull) && __popcll(eq & below) < need);
    const int c = __popcll(eq);
    need = need > c ? need - c : 0;
    const uint64_t km = __ballot(kept);
    if (kept) {
      const int pos = base + __popcll(km & below);
      scratch[pos] = key[i];
      scratch[kWave + pos] = (uint32_t)(lane + kWave * i);
      scratch[2 * kWave + pos] = __float_as_uint(v[i]);
    }
    base += __popcll(km);
  }
  uint32_t kj = 0, ej = 0, xj = 0;
  if (lane < k) {
    kj = scratch[lane];
    ej = scratch[kWave + lane];
    xj = scratch[2 * kWave + lane];
  }
  int rank = 0;
  for (int m = 0; m < k; ++m) {
    const uint32_t km = (uint32_t)__builtin_amdgcn_readlane((int)kj, m);
    const uint32_t em = (uint32_t)__builtin_amdgcn_readlane((int)ej, m);
    rank += (km > kj || (km == kj && em < ej)) ? 1 : 0;
  }
  if (lane < k) {
    scratch[rank] = ej;
    scratch[kWave + rank] = xj;
  }
  int my_e = 0;
  float my_x = 0.0f;
  if (lane < k) {
    my_e = (int)scratch[lane];
    my_x = __uint_as_float(scratch[kWave + lane]);
  }
  const double m = (double)__uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(my_x), 0));
  const double ex = lane < k ? exp((double)my_x - m) : 0.0;
  double sum = ex;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
  if (lane < k) {
    ids[lane] = my_e;
    w[lane] = (float)(ex / sum);
    if (lds_ids) lds_ids[lane] = my_e;
  }
}

// The permutation of at most 64 slots without further barriers: every wave holds the slot ids
// in its lanes (slot s in lane s) and derives its share of the outputs by counting over the
// slots: slot s goes to row offsets[id_s] + (earlier slots with its id), offsets[e] counts
// the slots with a lower id, and the active list holds the distinct ids in ascending order
// (an id's position counts the distinct ids below it). Wave 0 writes the per-slot rows, the
// active ids and their count; the threads write offsets[0 .. E] (thread e, and thread 0 also
// entry 1024 when E = 1024) and the -1 past the active ids. Same outputs, bit for bit, as
// permute_block.
__device__ __forceinline__ void permute_few(const int* ids, int S, int E, int* __restrict__ offsets,
                                            int* __restrict__ sorted_slot, int* __restrict__ slot_to_row,
                                            int* __restrict__ active, int* __restrict__ n_active) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int id = lane < S ? ids[lane] : 0x7fffffff;
  int same_before = 0, lower = 0;
  for (int t = 0; t < S; ++t) {
    const int it = __builtin_amdgcn_readlane(id, t);
    same_before += (t < lane && it == id) ? 1 : 0;
    lower += it < id ? 1 : 0;
  }
  const bool first = lane < S && same_before == 0;
  const uint64_t fm = __ballot(first);
  const int nact = __popcll(fm);
  for (int e = tid; e <= E; e += kPermThreads) {
    int cnt = 0;
    for (int t = 0; t < S; ++t) cnt += __builtin_amdgcn_readlane(id, t) < e ? 1 : 0;
    offsets[e] = cnt;
    if (e >= nact && e < E) active[e] = -1;
  }
  if (wave == 0) {
    int drank = 0;
    uint64_t m = fm;
    while (m) {
      const int t = __builtin_ctzll(m);
      m &= m - 1;
      drank += __builtin_amdgcn_readlane(id, t) < id ? 1 : 0;
    }
    if (lane < S) {
      const int row = lower + same_before;
      slot_to_row[lane] = row;
      sorted_slot[row] = lane;
      if (first) active[drank] = id;
    }
    if (lane == 0) n_active[0] = nact;
  }
}

template <int PL>
__global__ __launch_bounds__(kRouterWaves* kWave) void router_kernel(const float* __restrict__ logits,
                                                                     int T, int E, int k,
                                                                     int* __restrict__ ids,
                                                                     float* __restrict__ w) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int t = blockIdx.x * kRouterWaves + wave;
  __shared__ uint32_t scratch[kRouterWaves][3 * kWave];
  if (t >= T) return;   // t is the same for the whole wave
  route_token_thresh<PL>(logits + (size_t)t * E, E, k, lane, ids + (size_t)t * k, w + (size_t)t * k, nullptr,
                         scratch[wave]);
}

// Histogram of ids[lo, hi) into one wave's counter row (LDS atomics); the ids of kPermBatch
// 64-slot groups are requested before any is counted.
__device__ __forceinline__ void wave_histogram(const int* __restrict__ ids, int lo, int hi, int* cnt, int lane) {
  for (int s0 = lo; s0 < hi; s0 += kWave * kPermBatch) {
    int ex[kPermBatch];
#pragma unroll
    for (int b = 0; b < kPermBatch; ++b) {
      const int s = s0 + b * kWave + lane;
      ex[b] = s < hi ? ids[s] : -1;
    }
#pragma unroll
    for (int b = 0; b < kPermBatch; ++b)
      if (ex[b] >= 0) atomicAdd(&cnt[ex[b]], 1);
  }
}

// Stable scatter of slots [lo, hi) by one wave, 64 slots per step in slot order: cnt[e] holds
// the next row of expert e for this wave; a lane's rank among the lanes holding the same
// expert comes from ballots over the bits of the expert id and a popcount of the lower lanes.
__device__ __forceinline__ void wave_scatter(const int* __restrict__ ids, int lo, int hi, int* cnt, int nbits,
                                             int lane, int* __restrict__ sorted_slot,
                                             int* __restrict__ slot_to_row) {
  for (int sb = lo; sb < hi; sb += kWave * kPermBatch) {
    int exb[kPermBatch];
#pragma unroll
    for (int b = 0; b < kPermBatch; ++b) {
      const int s = sb + b * kWave + lane;
      exb[b] = s < hi ? ids[s] : 0;
    }
#pragma unroll
    for (int b = 0; b < kPermBatch; ++b) {
      const int s0 = sb + b * kWave;
      if (s0 >= hi) break;
      const int s = s0 + lane;
      const bool valid = s < hi;
      const int ex = exb[b];
      uint64_t peers = __ballot(valid);
      for (int bt = 0; bt < nbits; ++bt) {
        const bool bit = (ex >> bt) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
      }
      const int rank = __popcll(peers & ((1ull << lane) - 1ull));
      const int start = valid ? cnt[ex] : 0;
      const bool leader = valid && ((peers >> lane) == 1ull);  // highest lane of its group
      if (leader) cnt[ex] = start + __popcll(peers);
      if (valid) {
        const int row = start + rank;
        sorted_slot[row] = s;
        slot_to_row[s] = row;
      }
    }
  }
}

// The one-workgroup permutation (kPermThreads threads) over ids[0, S) (global memory or
// LDS); sm: (kPermWaves * E + 2 * kPermWaves) ints of LDS.
__device__ __forceinline__ void permute_block(const int* ids, int S, int E, int nbits, int* sm,
                                              int* __restrict__ offsets, int* __restrict__ sorted_slot,
                                              int* __restrict__ slot_to_row, int* __restrict__ active,
                                              int* __restrict__ n_active) {
  int* cnt = sm;                          // [kPermWaves][E]
  int* wsum = sm + kPermWaves * E;        // [kPermWaves] row totals per wave
  int* wflag = wsum + kPermWaves;         // [kPermWaves] active-expert totals per wave
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

  // slot slices of `per` slots (a multiple of 64) per wave; only the first nw waves hold slots
  const int per = ((S + kPermWaves - 1) / kPermWaves + kWave - 1) / kWave * kWave;
  const int nw = per > 0 ? min(kPermWaves, (S + per - 1) / per) : 0;
  const int lo = min(S, wave * per), hi = min(S, lo + per);
  for (int i = tid; i < nw * E; i += kPermThreads) cnt[i] = 0;
  __syncthreads();

  // 1. per-wave histograms
  wave_histogram(ids, lo, hi, cnt + wave * E, lane);
  __syncthreads();

  // 2. per expert e = tid: prefix over waves, then scans over experts.
  const int e = tid;
  int tot = 0;
  if (e < E) {
    for (int w = 0; w < nw; ++w) {
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
    for (int w = 0; w < nw; ++w) cnt[w * E + e] += base;
    if (e >= nact) active[e] = -1;
    if (flag) active[fpos] = e;
    if (e == E - 1) {
      offsets[E] = base + tot;
      n_active[0] = nact;
    }
  }
  __syncthreads();

  // 3. stable scatter of each wave's slice
  wave_scatter(ids, lo, hi, cnt + wave * E, nbits, lane, sorted_slot, slot_to_row);
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int* __restrict__ ids, int S, int E,
                                                               int nbits, int* __restrict__ offsets,
                                                               int* __restrict__ sorted_slot,
                                                               int* __restrict__ slot_to_row,
                                                               int* __restrict__ active,
                                                               int* __restrict__ n_active) {
  extern __shared__ int sm[];
  permute_block(ids, S, E, nbits, sm, offsets, sorted_slot, slot_to_row, active, n_active);
}

// Few tokens (T <= kPermWaves, T * k <= kSmallSlots): routing and permutation in one
// workgroup and one launch. Wave t routes token t. Below top-16 by k rounds of wave argmax
// (route_token_rounds): each round takes the largest order-preserving logit key (DPP max over
// the wave) and, among the experts holding it, the lowest id (ballots; registers ascend in id,
// lanes within a register), and removes it. From top-16 on by route_token_thresh, whose cost
// does not grow with k (many-small layer, top-22 of 512: 2.5-4.5 us less per step at 1, 4
// and 16 tokens; decode, top-8 of 256: the rounds ~1.5 us faster). Both give the same ids in
// the same order and the same weights: float64 exp(l - l_max) over the kept, summed over the
// wave with lane r holding rank r. The ids also go to LDS, from which the workgroup permutes
// as permute_kernel does.
constexpr int kSmallSlots = 1024;

template <int PL>
__device__ __forceinline__ void route_token_rounds(const float* __restrict__ row, int E, int k, int lane,
                                                   int* __restrict__ ids, float* __restrict__ w, int* lds_ids) {
  uint32_t key[PL];
  float v[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + kWave * i;
    const float x = e < E ? row[e] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;
    key[i] = e < E ? logit_key(x) : 0u;   // every real key is >= logit_key(-inf) > 0
  }
  int my_e = 0;
  float my_x = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < PL; ++i) best = max(best, key[i]);
    best = wave_max_u32_uniform(best);
    int e = -1;
    float x = 0.0f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const uint64_t m = __ballot(key[i] == best);
      if (e < 0 && m) {
        const int l = __builtin_ctzll(m);
        e = kWave * i + l;
        x = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v[i]), l));
      }
    }
    if (lane == j) {
      my_e = e;
      my_x = x;
    }
#pragma unroll
    for (int i = 0; i < PL; ++i)
      if (kWave * i + lane == e) key[i] = 0u;
  }
  const double m = (double)__uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(my_x), 0));
  const double ex = lane < k ? exp((double)my_x - m) : 0.0;
  double sum = ex;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
  if (lane < k) {
    ids[lane] = my_e;
    w[lane] = (float)(ex / sum);
    lds_ids[lane] = my_e;
  }
}

// Token row r of a few-token dispatch (workgroup r + 1 of the launch, kPermThreads threads,
// H <= 8 * kPermThreads): the bf16 row, after the FP8 E4M3 round trip when asked (per-tensor
// scale from the finite maximum over all T rows, which every such workgroup reads), is
// prepared for the W4A16 GEMM (row exponent, f16 in operand order) with the arithmetic of the
// round-trip and prep launches (act_rows.h), so the bits are theirs.
__device__ void dispatch_prepare_row(const ActPrep& ap, int T, int r, float* red) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int H = ap.H, nvec = H / 8, H128 = (H + 127) & ~127;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (tid < nvec) {
    const uint4 q = *reinterpret_cast<const uint4*>(ap.x + (size_t)r * H + 8 * tid);
    w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
  }
  auto block_max = [&](float m) {
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    float a = red[0];
    for (int i = 1; i < kPermWaves; ++i) a = fmaxf(a, red[i]);
    __syncthreads();   // red is reused
    return a;
  };
  if (ap.fp8) {
    float m = 0.0f;
    for (int i = tid; i < T * nvec; i += kPermThreads) {
      const uint4 q = *reinterpret_cast<const uint4*>(ap.x + 8 * (size_t)i);
      const uint32_t v[4] = {q.x, q.y, q.z, q.w};
      m = bf16x8_finite_max(v, m);
    }
    const float sc = fp8_scale(block_max(m));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = fp8_roundtrip_bits(bf16_to_f32(w[j] & 0xffffu), sc) | (fp8_roundtrip_bits(bf16_to_f32(w[j] >> 16), sc) << 16);
  }
  const int p = f16_row_exponent(block_max(bf16x8_finite_max(w, 0.0f)));
  if (tid == 0) ap.rexp[r] = p;
  if (tid < H128 / 8) *reinterpret_cast<f16x8*>(ap.a16 + (size_t)r * H128 + 8 * prepared_piece(tid)) = bf16x8_to_f16(w, p);
}

template <int PL>
__global__ __launch_bounds__(kPermThreads) void route_permute_small_kernel(const float* __restrict__ logits,
                                                                           int T, int E, int k, int nbits,
                                                                           int* __restrict__ ids,
                                                                           float* __restrict__ w,
                                                                           int* __restrict__ offsets,
                                                                           int* __restrict__ sorted_slot,
                                                                           int* __restrict__ slot_to_row,
                                                                           int* __restrict__ active,
                                                                           int* __restrict__ n_active,
                                                                           int thresh, int full_permute,
                                                                           const ActPrep ap) {
  extern __shared__ int sm[];
  if (blockIdx.x > 0) {   // a dispatch's token row (the whole workgroup)
    dispatch_prepare_row(ap, T, (int)blockIdx.x - 1, reinterpret_cast<float*>(sm));
    return;
  }
  int* s_ids = sm;                   // [T * k] expert ids
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (wave < T) {
    if (thresh)
      route_token_thresh<PL>(logits + (size_t)wave * E, E, k, lane, ids + (size_t)wave * k, w + (size_t)wave * k,
                             s_ids + wave * k,
                             reinterpret_cast<uint32_t*>(sm + kSmallSlots + kPermWaves * E + 2 * kPermWaves) +
                                 wave * 3 * kWave);
    else
      route_token_rounds<PL>(logits + (size_t)wave * E, E, k, lane, ids + (size_t)wave * k, w + (size_t)wave * k,
                             s_ids + wave * k);
  }
  __syncthreads();
  if (T * k <= kWave && !full_permute)
    permute_few(s_ids, T * k, E, offsets, sorted_slot, slot_to_row, active, n_active);
  else
    permute_block(s_ids, T * k, E, nbits, sm + kSmallSlots, offsets, sorted_slot, slot_to_row, active, n_active);
}

// Many slots: the permutation in two launches over chunks of slots, so that the scattered
// row writes are spread over many CUs (one workgroup issues about one scattered line per
// clock). perm_count_kernel: counts[b][e] = rows of expert e in chunk b. perm_scatter_kernel:
// workgroup b derives every expert's first row (exclusive scan over experts of the totals)
// and its own first row per expert (the counts of chunks before b), then scatters its chunk
// wave by wave exactly as the one-workgroup kernel does. Same result, bit for bit.
constexpr int kPmThreads = 256;
constexpr int kPmWaves = kPmThreads / kWave;
constexpr int kPmChunk = 2048;        // slots per workgroup, at least
constexpr int kPmMaxBlocks = 64;      // chunks grow beyond kPmChunk to keep the count reads small
constexpr int kPmMinSlots = 16384;    // fewer slots: the one-workgroup kernel

__global__ __launch_bounds__(kPmThreads) void perm_count_kernel(const int* __restrict__ ids, int S, int E,
                                                                int chunk, int* __restrict__ counts) {
  extern __shared__ int cnt[];   // [E]
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += kPmThreads) cnt[i] = 0;
  __syncthreads();
  const int lo = blockIdx.x * chunk, hi = min(S, lo + chunk);
  const int wave = tid / kWave, lane = tid % kWave;
  const int per = ((hi - lo + kPmWaves - 1) / kPmWaves + kWave - 1) / kWave * kWave;
  const int wlo = min(hi, lo + wave * per), whi = min(hi, wlo + per);
  wave_histogram(ids, wlo, whi, cnt, lane);
  __syncthreads();
  for (int i = tid; i < E; i += kPmThreads) counts[(size_t)blockIdx.x * E + i] = cnt[i];
}

// Exclusive prefix of v over the threads of the workgroup (thread order); total = sum.
__device__ __forceinline__ int block_excl_scan(int v, int* red, int& total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int a = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += a;
  }
  if (lane == kWave - 1) red[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kPmWaves; ++w) {
    const int x = red[w];
    if (w < wave) before += x;
    total += x;
  }
  __syncthreads();
  return before + incl - v;
}

__global__ __launch_bounds__(kPmThreads) void perm_scatter_kernel(const int* __restrict__ ids, int S, int E,
                                                                  int nbits, int chunk,
                                                                  const int* __restrict__ counts, int nblk,
                                                                  int* __restrict__ offsets,
                                                                  int* __restrict__ sorted_slot,
                                                                  int* __restrict__ slot_to_row,
                                                                  int* __restrict__ active,
                                                                  int* __restrict__ n_active) {
  extern __shared__ int sm[];
  int* wcnt = sm;                     // [kPmWaves][E]
  int* red = sm + kPmWaves * E;       // [kPmWaves]
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int b = blockIdx.x;
  // 1. each thread owns up to 4 consecutive experts (E <= 1024): total rows over all chunks
  //    and rows in the chunks before this one
  constexpr int EPT = kMaxExperts / kPmThreads;
  const int ept = (E + kPmThreads - 1) / kPmThreads;
  const int e0 = min(E, tid * ept);
  int tot[EPT], pre[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) tot[i] = pre[i] = 0;
#pragma unroll 4
  for (int bb = 0; bb < nblk; ++bb) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = e0 + i;
      if (i < ept && e < E) {
        const int c = counts[(size_t)bb * E + e];
        tot[i] += c;
        pre[i] += bb < b ? c : 0;
      }
    }
  }
  int tsum = 0, tact = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    if (i < ept && e0 + i < E) {
      tsum += tot[i];
      tact += tot[i] > 0 ? 1 : 0;
    }
  }
  int total = 0, nact = 0;
  int run = block_excl_scan(tsum, red, total);
  int arun = block_excl_scan(tact, red, nact);
  // 2. offsets and the active list (chunk 0 writes them); this chunk's first row per expert
  int first[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = e0 + i;
    first[i] = 0;
    if (i < ept && e < E) {
      if (b == 0) {
        offsets[e] = run;
        if (tot[i] > 0) active[arun] = e;
      }
      first[i] = run + pre[i];
      run += tot[i];
      arun += tot[i] > 0 ? 1 : 0;
    }
  }
  if (b == 0) {
    if (tid == 0) {
      offsets[E] = total;
      n_active[0] = nact;
    }
    for (int e = nact + tid; e < E; e += kPmThreads) active[e] = -1;
  }
  // 3. per-wave histograms of this chunk, then each wave's first row per expert
  for (int i = tid; i < kPmWaves * E; i += kPmThreads) wcnt[i] = 0;
  __syncthreads();
  const int lo = b * chunk, hi = min(S, lo + chunk);
  const int per = ((hi - lo + kPmWaves - 1) / kPmWaves + kWave - 1) / kWave * kWave;
  const int wlo = min(hi, lo + wave * per), whi = min(hi, wlo + per);
  wave_histogram(ids, wlo, whi, wcnt + wave * E, lane);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = e0 + i;
    if (i < ept && e < E) {
      int r = first[i];
#pragma unroll
      for (int w = 0; w < kPmWaves; ++w) {
        const int c = wcnt[w * E + e];
        wcnt[w * E + e] = r;
        r += c;
      }
    }
  }
  __syncthreads();
  // 4. stable scatter of each wave's slice
  wave_scatter(ids, wlo, whi, wcnt + wave * E, nbits, lane, sorted_slot, slot_to_row);
}

}  // namespace

namespace {
void perm_plan(int S, int& chunk, int& nblk) {
  const int need = (S + kPmMaxBlocks - 1) / kPmMaxBlocks;
  chunk = need <= kPmChunk ? kPmChunk : (need + kPmThreads - 1) / kPmThreads * kPmThreads;
  nblk = (S + chunk - 1) / chunk;
}
}  // namespace

template <int PL>
hipError_t launch_small(const float* logits, int T, int E, int k, int nbits, int* topk_ids, float* topk_w,
                        int* expert_offsets, int* sorted_slot, int* slot_to_row, int* active_experts,
                        int* n_active, const ActPrep& ap, hipStream_t stream) {
  static std::atomic<uint64_t> attr_done{0};
  constexpr int kScratch = kPermWaves * 3 * kWave;   // the routing waves' selection scratch
  const hipError_t attr = ensure_dynamic_lds(reinterpret_cast<const void*>(&route_permute_small_kernel<PL>),
                                             (kSmallSlots + kPermWaves * kMaxExperts + 2 * kPermWaves + kScratch) *
                                                 (int)sizeof(int),
                                             attr_done);
  if (attr != hipSuccess) return attr;
  const size_t shmem = (size_t)(kSmallSlots + kPermWaves * E + 2 * kPermWaves + kScratch) * sizeof(int);
  // k rounds cost ~0.24 us (256 experts) to ~0.39 us (512) each, the threshold select about
  // as much as 14 rounds; NVFP4MOE_SMALL_SELECT=rounds|thresh forces one (tests, tuning)
  const char* sel = std::getenv("NVFP4MOE_SMALL_SELECT");
  const int thresh = sel ? (!std::strcmp(sel, "thresh") ? 1 : 0) : (k >= 16 ? 1 : 0);
  // up to 64 slots the permutation needs no further barrier (permute_few);
  // NVFP4MOE_SMALL_PERMUTE=full keeps the general one (tests)
  const char* pf = std::getenv("NVFP4MOE_SMALL_PERMUTE");
  const int full_permute = pf && !std::strcmp(pf, "full") ? 1 : 0;
  const unsigned grid = 1u + (ap.x ? (unsigned)T : 0u);   // + one workgroup per token row to prepare
  route_permute_small_kernel<PL><<<grid, kPermThreads, shmem, stream>>>(logits, T, E, k, nbits, topk_ids, topk_w,
                                                                       expert_offsets, sorted_slot, slot_to_row,
                                                                       active_experts, n_active, thresh,
                                                                       full_permute, ap);
  return hipGetLastError();
}

size_t route_permute_ws_bytes(int T, int E, int k) {
  int chunk = 0, nblk = 0;
  perm_plan(T * k, chunk, nblk);
  return (size_t)nblk * (size_t)E * sizeof(int);
}

namespace {
// The routing launches; with `fused` (token rows to prepare) the one-workgroup launch also
// prepares them and *prepared is set.
hipError_t route_launches(const float* logits, int T, int E, int k, int* topk_ids, float* topk_w,
                          int* expert_offsets, int* sorted_slot, int* slot_to_row, int* active_experts,
                          int* n_active, void* ws, size_t ws_bytes, hipStream_t stream, const ActPrep& fused,
                          bool* prepared) {
  // Up to 16 tokens: routing and permutation in one workgroup and one launch. More tokens:
  // a router launch, then the permutation. Router: for fewer than 256 tokens a workgroup per
  // token sorts (no serial chain, measured 15.7 -> 9.1 us at one token of 512 experts,
  // top-22), for more a wave per token selects (more tokens per CU; 8192 tokens of 256
  // experts: 18 us against 33 us sorted). Overrides (tests, tuning):
  // NVFP4MOE_ROUTER=small|sort|wave and NVFP4MOE_PERMUTE=small|single|multi; any value but
  // "small" selects the separate launches.
  const char* force = std::getenv("NVFP4MOE_ROUTER");
  const char* pforce = std::getenv("NVFP4MOE_PERMUTE");
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int pl = (E + kWave - 1) / kWave;   // experts per lane
  const bool small = T <= kPermWaves && T * k <= kSmallSlots &&
                     (force ? !std::strcmp(force, "small") : true) && (pforce ? !std::strcmp(pforce, "small") : true);
  if (small) {
    *prepared = fused.x != nullptr;
#define NVFP4MOE_LAUNCH_SMALL(P)                                                                                  \
  return launch_small<P>(logits, T, E, k, nbits, topk_ids, topk_w, expert_offsets, sorted_slot, slot_to_row, \
                         active_experts, n_active, fused, stream)
    if (pl <= 1) NVFP4MOE_LAUNCH_SMALL(1);
    if (pl <= 2) NVFP4MOE_LAUNCH_SMALL(2);
    if (pl <= 4) NVFP4MOE_LAUNCH_SMALL(4);
    if (pl <= 8) NVFP4MOE_LAUNCH_SMALL(8);
    NVFP4MOE_LAUNCH_SMALL(16);
#undef NVFP4MOE_LAUNCH_SMALL
  }
  const bool sort_router = force ? !std::strcmp(force, "sort") : T < 256;
  if (sort_router) {
    if (E <= 64) router_sort_kernel<64><<<T, router_sort_threads<64>(), 0, stream>>>(logits, E, k, topk_ids, topk_w);
    else if (E <= 128) router_sort_kernel<128><<<T, router_sort_threads<128>(), 0, stream>>>(logits, E, k, topk_ids, topk_w);
    else if (E <= 256) router_sort_kernel<256><<<T, router_sort_threads<256>(), 0, stream>>>(logits, E, k, topk_ids, topk_w);
    else if (E <= 512) router_sort_kernel<512><<<T, router_sort_threads<512>(), 0, stream>>>(logits, E, k, topk_ids, topk_w);
    else router_sort_kernel<1024><<<T, router_sort_threads<1024>(), 0, stream>>>(logits, E, k, topk_ids, topk_w);
  } else {
    const unsigned rgrid = (unsigned)((T + kRouterWaves - 1) / kRouterWaves);
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
  }

  const int S = T * k;
  // Many slots: the two-launch permutation (scattered writes spread over the chunks'
  // workgroups); NVFP4MOE_PERMUTE=single|multi forces one (tests).
  const bool multi = pforce ? !std::strcmp(pforce, "multi") : S >= kPmMinSlots;
  if (multi) {
    int chunk = 0, nblk = 0;
    perm_plan(S, chunk, nblk);
    if (!ws || ws_bytes < route_permute_ws_bytes(T, E, k)) return hipErrorInvalidValue;
    int* counts = static_cast<int*>(ws);
    perm_count_kernel<<<nblk, kPmThreads, (size_t)E * sizeof(int), stream>>>(topk_ids, S, E, chunk, counts);
    perm_scatter_kernel<<<nblk, kPmThreads, (size_t)(kPmWaves * E + kPmWaves) * sizeof(int), stream>>>(
        topk_ids, S, E, nbits, chunk, counts, nblk, expert_offsets, sorted_slot, slot_to_row, active_experts,
        n_active);
    return hipGetLastError();
  }

  static std::atomic<uint64_t> perm_attr_done{0};
  const hipError_t attr = ensure_dynamic_lds(reinterpret_cast<const void*>(&permute_kernel),
                                             (kPermWaves * kMaxExperts + 2 * kPermWaves) * (int)sizeof(int),
                                             perm_attr_done);
  if (attr != hipSuccess) return attr;
  const size_t shmem = (size_t)(kPermWaves * E + 2 * kPermWaves) * sizeof(int);
  permute_kernel<<<1, kPermThreads, shmem, stream>>>(topk_ids, T * k, E, nbits, expert_offsets,
                                                     sorted_slot, slot_to_row, active_experts,
                                                     n_active);
  return hipGetLastError();
}
}  // namespace

size_t dispatch_rows_ws_bytes(int T, int H, bool fp8) {
  if (!fp8) return 0;
  const size_t rows = ((size_t)T * H * 2 + 255) / 256 * 256;   // the round trip's bf16 output
  return rows + fp8_roundtrip_ws_bytes((int64_t)T * H);
}

hipError_t launch_route_permute(const float* logits, int T, int E, int k, int* topk_ids,
                                float* topk_w, int* expert_offsets, int* sorted_slot,
                                int* slot_to_row, int* active_experts, int* n_active,
                                void* ws, size_t ws_bytes, hipStream_t stream, const ActPrep* prep) {
  // A dispatch's token rows are prepared by extra workgroups of the one-workgroup routing
  // launch when it runs (up to 16 tokens, rows of up to 8 * kPermThreads columns), otherwise
  // after the routing by the round-trip and prep launches.
  const ActPrep fused = prep && prep->H <= 8 * kPermThreads ? *prep : ActPrep{};
  bool prepared = false;
  hipError_t e = route_launches(logits, T, E, k, topk_ids, topk_w, expert_offsets, sorted_slot, slot_to_row,
                                active_experts, n_active, ws, ws_bytes, stream, fused, &prepared);
  if (e != hipSuccess || !prep || prepared) return e;
  const uint16_t* rows = prep->x;
  if (prep->fp8) {
    if (!prep->rows_ws) return hipErrorInvalidValue;
    uint16_t* rt = static_cast<uint16_t*>(prep->rows_ws);
    char* rt_ws = static_cast<char*>(prep->rows_ws) + ((size_t)T * prep->H * 2 + 255) / 256 * 256;
    e = launch_fp8_roundtrip(prep->x, (int64_t)T * prep->H, rt, rt_ws, stream);
    if (e != hipSuccess) return e;
    rows = rt;
  }
  return launch_act_prep(rows, T, prep->H, prep->a16, prep->rexp, MtileSched{}, stream);
}

}  // namespace nvfp4moe
