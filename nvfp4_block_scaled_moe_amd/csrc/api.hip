// C ABI of libnvfp4moe (declared in include/nvfp4moe.h): argument validation on the host,
// workspace carving, kernel-path dispatch, and status/error reporting. No call allocates
// memory or synchronizes the device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "kernels.h"
#include "nvfp4moe.h"

using namespace nvfp4moe;

namespace {

thread_local std::string g_last_error;
thread_local int g_last_dispatch = NVFP4MOE_PATH_NONE;

nvfp4moe_status fail(nvfp4moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

nvfp4moe_status ok() {
  g_last_error.clear();
  return NVFP4MOE_OK;
}

nvfp4moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(NVFP4MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
// Prepared W4A16 rows (moe_dispatch_w4a16's x_prep): f16 [rows, K128] in the GEMM's operand
// order, then the rows' exponents int32 [rows].
size_t prepared_rows_bytes(int64_t rows, int32_t K) { return round_up((size_t)rows * (((size_t)K + 127) / 128 * 128) * 2); }

__global__ void zero_f32_kernel(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// W4A4 on the large-M path: decode the NVFP4 activation rows in the GEMM's staging instead
// of reading an f16 copy (NVFP4MOE_LARGE_A4=1; measured slower, off by default).
bool large_a4_staged() {
  const char* s = std::getenv("NVFP4MOE_LARGE_A4");
  return s && s[0] == '1';
}

// Kernel path override for tests/measurement: NVFP4MOE_FORCE_PATH=stream|mfma.
int forced_path() {
  const char* s = std::getenv("NVFP4MOE_FORCE_PATH");
  if (!s) return NVFP4MOE_PATH_NONE;
  if (!std::strcmp(s, "stream")) return NVFP4MOE_PATH_STREAM;
  if (!std::strcmp(s, "mfma")) return NVFP4MOE_PATH_MFMA;
  return NVFP4MOE_PATH_NONE;
}

// Mean rows per expert from which the m-tiled MFMA path is used: below it every weight
// byte feeds too few rows for the MFMA tile to pay, and the weight-streaming path wins.
constexpr int64_t kLargeMeanRows = 64;

// Path of one grouped GEMM, decided on the host from the sizes alone (the per-expert row
// counts live on the device): NVFP4MOE_PATH_STREAM or _MFMA, or NONE if a forced path
// cannot run this shape.
int gemm_path(int32_t rows, int32_t E, int32_t Nw) {
  const int forced = forced_path();
  const bool large_ok = large_supports(Nw);
  if (forced == NVFP4MOE_PATH_MFMA) return large_ok ? NVFP4MOE_PATH_MFMA : NVFP4MOE_PATH_NONE;
  if (forced == NVFP4MOE_PATH_STREAM) return NVFP4MOE_PATH_STREAM;
  const int64_t groups = E < rows ? E : rows;
  return large_ok && (int64_t)rows >= kLargeMeanRows * groups ? NVFP4MOE_PATH_MFMA : NVFP4MOE_PATH_STREAM;
}

// Workspace layout of moe_grouped_gemm_nvfp4: f16 activations in MFMA operand order and
// their row exponents (W4A16 on both paths, W4A4 on the MFMA path unless the GEMM decodes
// the FP4 rows itself), and the m-tile schedule of the MFMA path.
struct GemmWs {
  size_t a16_bytes, rexp_bytes, sched_bytes, partial_bytes, total;
  int max_mtiles, ksplit;
};
GemmWs gemm_ws_layout(int path, nvfp4moe_mode mode, int64_t a_rows, int32_t rows, int32_t E, int32_t Nw,
                      int32_t K) {
  GemmWs w{0, 0, 0, 0, 0, 0, 1};
  // (prepared W4A16 rows come with the call, in moe_dispatch_w4a16's x_prep)
  if (mode == NVFP4MOE_W4A16 || (mode == NVFP4MOE_W4A4 && path == NVFP4MOE_PATH_MFMA && !large_a4_staged())) {
    const size_t K128 = ((size_t)K + 127) / 128 * 128;  // rows padded to whole 128-k chunks
    w.a16_bytes = round_up((size_t)a_rows * K128 * 2);
    w.rexp_bytes = round_up((size_t)a_rows * 4);
  }
  if (path == NVFP4MOE_PATH_MFMA) {
    const int bm = large_rows_per_mtile();
    // sum over experts of ceil(M_e / bm) <= ceil(rows / bm) + (number of non-empty experts)
    w.max_mtiles = (rows + bm - 1) / bm + (E < rows ? E : rows);
    w.sched_bytes = 2 * round_up((size_t)w.max_mtiles * 4) + kAlign;
    w.ksplit = large_ksplit(rows, E, Nw, K);
  } else {
    w.ksplit = stream_ksplit(rows, E, Nw, K);
  }
  if (w.ksplit > 1) w.partial_bytes = round_up((size_t)w.ksplit * rows * Nw * 4);
  w.total = w.a16_bytes + w.rexp_bytes + w.sched_bytes + w.partial_bytes;
  return w;
}

}  // namespace

hipError_t nvfp4moe::launch_zero_f32(float* p, int n, hipStream_t stream) {
  zero_f32_kernel<<<(n + 255) / 256, 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

namespace {
__global__ void zero_i32_kernel(int4* p, size_t n4) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) p[i] = make_int4(0, 0, 0, 0);
}
}  // namespace

// n ints at p (16-byte aligned, n rounded up to a multiple of 4 inside the caller's buffer).
hipError_t nvfp4moe::launch_zero_i32(int* p, size_t n, hipStream_t stream) {
  const size_t n4 = (n + 3) / 4;
  zero_i32_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, stream>>>(reinterpret_cast<int4*>(p), n4);
  return hipGetLastError();
}

namespace {
// The fused unpermute + weighted reduce of a down-GEMM call: routing of the T tokens and the
// bf16 [T, Nw] output.
struct Combine {
  const int32_t* sorted_slot;
  const int32_t* slot_to_row;
  const float* topk_w;
  int32_t T, k;
  void* out;
};

nvfp4moe_status combine_checks(const char* fn, const Combine& c, int32_t E, int32_t Nw) {
  if (!c.sorted_slot || !c.slot_to_row || !c.topk_w || !c.out)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (c.T < 1 || c.k < 1 || c.k > E || c.k > kMaxTopK || (int64_t)c.T * c.k > (1 << 24))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need T >= 1, 1 <= k <= min(E, %d), T * k <= 2^24 (T=%d k=%d)", fn,
                kMaxTopK, c.T, c.k);
  if ((int64_t)c.T * c.k * Nw >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: T * k * Nw must be < 2^31", fn);
  if (!aligned(c.out, 16)) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: out must be 16-byte aligned", fn);
  return NVFP4MOE_OK;
}

// Workspace added by the combine: the float32 Y [T*k, Nw] and the completion counters.
size_t combine_ws_bytes(int32_t T, int32_t k, int32_t Nw) {
  return round_up((size_t)T * k * Nw * 4) + round_up(comb_count_ints(T, Nw) * 4);
}

// Point g at Y and the counters in `base` (combine_ws_bytes of memory) and enqueue the
// counter reset; with split K the GEMM writes Y and the reduce kernel runs after it instead.
hipError_t combine_setup(GemmArgs& g, const Combine& c, char* base, int32_t Nw, hipStream_t s) {
  g.out = base;
  g.out_bf16 = 0;
  g.out_amax = nullptr;
  if (g.ksplit > 1) return hipSuccess;
  g.comb_slot = c.sorted_slot;
  g.comb_s2r = c.slot_to_row;
  g.comb_w = c.topk_w;
  g.comb_k = c.k;
  g.comb_out = static_cast<uint16_t*>(c.out);
  g.comb_count = reinterpret_cast<int*>(base + round_up((size_t)c.T * c.k * Nw * 4));
  return launch_zero_i32(g.comb_count, comb_count_ints(c.T, Nw), s);
}

hipError_t combine_finish(const GemmArgs& g, const Combine& c, int32_t Nw, hipStream_t s) {
  if (g.comb_slot) return hipSuccess;   // fused into the GEMM
  return launch_unpermute_reduce(g.out, false, c.slot_to_row, c.topk_w, c.T, c.k, Nw, static_cast<uint16_t*>(c.out), s);
}
}  // namespace

extern "C" {

const char* nvfp4moe_last_error(void) { return g_last_error.c_str(); }
int nvfp4moe_last_dispatch(void) { return g_last_dispatch; }
int nvfp4moe_abi_version(void) { return 302; }

// ------------------------------------------------------------------ quantize
size_t nvfp4_quantize_workspace_size(int64_t B, int64_t R, int64_t C) {
  if (B < 1 || R < 1 || C < 1) return 0;
  return round_up(quantize_ws_bytes(B, R, C));
}

}  // extern "C"

namespace {
// Argument checks shared by nvfp4_quantize and nvfp4_quantize_noalloc.
nvfp4moe_status quantize_checks(const char* fn, const void* x, nvfp4moe_dtype x_dtype, int64_t B, int64_t R,
                                int64_t C, nvfp4moe_layout layout, const uint8_t* packed, const uint8_t* scales,
                                const float* g_out) {
  if (layout != NVFP4MOE_LAYOUT_ROW_MAJOR && layout != NVFP4MOE_LAYOUT_TILED)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: bad layout %d", fn, (int)layout);
  if (!x || !packed || !scales || !g_out) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: x_dtype must be F32 or BF16", fn);
  if (B < 1 || R < 1 || C < 32 || C % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID_ARG,
                "%s: need B >= 1, R >= 1, C >= 32 and C %% 32 == 0 (B=%lld R=%lld C=%lld)", fn, (long long)B,
                (long long)R, (long long)C);
  if (B > 65535 || (double)B * (double)R * (double)C > 4.0e12)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: tensor too large", fn);
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(g_out, 4))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: x and packed must be 16-byte aligned, scales 2-byte aligned", fn);
  if (layout == NVFP4MOE_LAYOUT_TILED) {
    if (R < 16 || R % 16 != 0)
      return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: the tiled layout needs R %% 16 == 0 (R=%lld)", fn, (long long)R);
    if (B * R * (C / 2) >= (int64_t(1) << 40) || R > (int64_t(1) << 30) || C > (int64_t(1) << 30))
      return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: matrices too large for the tiled layout", fn);
    if (!aligned(scales, 16))
      return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: the tiled scales must be 16-byte aligned", fn);
  }
  return NVFP4MOE_OK;
}
}  // namespace

extern "C" {

nvfp4moe_status nvfp4_quantize(const void* x, nvfp4moe_dtype x_dtype, int64_t B, int64_t R,
                               int64_t C, const float* g_in, const float* amax_in,
                               nvfp4moe_layout layout, uint8_t* packed, uint8_t* scales, float* g_out,
                               void* ws, size_t ws_bytes, void* stream) {
  const nvfp4moe_status chk =
      quantize_checks("nvfp4_quantize", x, x_dtype, B, R, C, layout, packed, scales, g_out);
  if (chk != NVFP4MOE_OK) return chk;
  if (!g_in && !amax_in) {
    const size_t need = nvfp4_quantize_workspace_size(B, R, C);
    if (!ws || ws_bytes < need)
      return fail(NVFP4MOE_ERR_WORKSPACE, "nvfp4_quantize: workspace of %zu bytes needed, %zu given",
                  need, ws_bytes);
  }
  return hip_status(launch_quantize(x, x_dtype == NVFP4MOE_BF16, B, R, C, g_in, amax_in,
                                    layout == NVFP4MOE_LAYOUT_TILED, packed, scales, g_out, ws,
                                    static_cast<hipStream_t>(stream)),
                    "nvfp4_quantize");
}

}  // extern "C"

// ------------------------------------------------------------------ no-allocation quantize
// Scratch of nvfp4_quantize_noalloc: the amax pass's per-workgroup partial maxima
// (B * amax-workgroups floats). Each GPU the library runs on holds its own copy until the
// process ends. In host code the array's name is not a device address: the address comes
// from hipGetSymbolAddress, once per device with that device current, and only that pointer
// is passed to kernels.
constexpr size_t kNoAllocScratchBytes = 64 * 1024;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device id

// Device address of the current device's scratch (looked up on the first call on a device).
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

extern "C" {

nvfp4moe_status nvfp4_quantize_noalloc(const void* x, nvfp4moe_dtype x_dtype, int64_t B, int64_t R, int64_t C,
                                       const float* g_in, const float* amax_in, nvfp4moe_layout layout,
                                       uint8_t* packed, uint8_t* scales, float* g_out, void* stream) {
  const char* fn = "nvfp4_quantize_noalloc";
  const nvfp4moe_status chk = quantize_checks(fn, x, x_dtype, B, R, C, layout, packed, scales, g_out);
  if (chk != NVFP4MOE_OK) return chk;
  void* ws = nullptr;
  if (!g_in && !amax_in) {
    const size_t need = nvfp4_quantize_workspace_size(B, R, C);
    if (need > kNoAllocScratchBytes)
      return fail(NVFP4MOE_ERR_WORKSPACE,
                  "%s: the amax pass needs %zu bytes of scratch, more than the %zu this entry point holds "
                  "(fewer matrices per call, or nvfp4_quantize with a workspace)",
                  fn, need, kNoAllocScratchBytes);
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e, fn);
    if (stream) {
      hipDevice_t sdev = 0;
      e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
      if (e != hipSuccess) return hip_status(e, fn);
      if ((int)sdev != cur)
        return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: the stream belongs to device %d, the current device is %d", fn,
                    (int)sdev, cur);
    }
    e = noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return hip_status(launch_quantize(x, x_dtype == NVFP4MOE_BF16, B, R, C, g_in, amax_in,
                                    layout == NVFP4MOE_LAYOUT_TILED, packed, scales, g_out, ws,
                                    static_cast<hipStream_t>(stream)),
                    fn);
}

// ------------------------------------------------------------------ route + permute
size_t moe_route_permute_workspace_size(int32_t T, int32_t E, int32_t k) {
  if (T < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E || (int64_t)T * k > (1 << 24)) return 0;
  return route_permute_ws_bytes(T, E, k);
}

nvfp4moe_status moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k,
                                  int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                                  int32_t* sorted_slot, int32_t* slot_to_row,
                                  int32_t* active_experts, int32_t* n_active, void* ws,
                                  size_t ws_bytes, void* stream) {
  if (!logits || !topk_ids || !topk_w || !expert_offsets || !sorted_slot || !slot_to_row ||
      !active_experts || !n_active)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "moe_route_permute: null tensor pointer");
  if (T < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E || k > kMaxTopK)
    return fail(NVFP4MOE_ERR_INVALID_ARG,
                "moe_route_permute: need T >= 1, 1 <= k <= min(E, %d), E <= %d (T=%d E=%d k=%d)",
                kMaxTopK, kMaxExperts, T, E, k);
  if ((int64_t)T * k > (1 << 24))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "moe_route_permute: T * k must be <= 2^24");
  const size_t need = route_permute_ws_bytes(T, E, k);
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(NVFP4MOE_ERR_WORKSPACE, "moe_route_permute: workspace of %zu bytes needed, %zu given", need,
                ws_bytes);
  if (!aligned(ws, 4))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "moe_route_permute: workspace must be 4-byte aligned");
  return hip_status(launch_route_permute(logits, T, E, k, topk_ids, topk_w, expert_offsets,
                                         sorted_slot, slot_to_row, active_experts, n_active, ws, ws_bytes,
                                         static_cast<hipStream_t>(stream)),
                    "moe_route_permute");
}

// ------------------------------------------------------------------ dispatch (route + row prep)
size_t moe_prepared_act_bytes(int64_t rows, int32_t K) {
  if (rows < 1 || K < 32 || K % 32 != 0) return 0;
  return prepared_rows_bytes(rows, K) + round_up((size_t)rows * 4);
}

size_t moe_dispatch_w4a16_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t fp8_act) {
  if (T < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E || (int64_t)T * k > (1 << 24) || H < 32 || H % 32 != 0 ||
      (int64_t)T * H >= (int64_t(1) << 31))
    return 0;
  return round_up(route_permute_ws_bytes(T, E, k)) + dispatch_rows_ws_bytes(T, H, fp8_act != 0);
}

nvfp4moe_status moe_dispatch_w4a16(const float* logits, const void* x, int32_t T, int32_t E, int32_t k,
                                   int32_t H, int32_t fp8_act, int32_t* topk_ids, float* topk_w,
                                   int32_t* expert_offsets, int32_t* sorted_slot, int32_t* slot_to_row,
                                   int32_t* active_experts, int32_t* n_active, void* x_prep, void* ws,
                                   size_t ws_bytes, void* stream) {
  const char* fn = "moe_dispatch_w4a16";
  if (!logits || !x || !topk_ids || !topk_w || !expert_offsets || !sorted_slot || !slot_to_row || !active_experts ||
      !n_active || !x_prep)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (T < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E || k > kMaxTopK)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need T >= 1, 1 <= k <= min(E, %d), E <= %d (T=%d E=%d k=%d)", fn,
                kMaxTopK, kMaxExperts, T, E, k);
  if ((int64_t)T * k > (1 << 24)) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: T * k must be <= 2^24", fn);
  if (H < 32 || H % 32 != 0 || (int64_t)T * H >= (int64_t(1) << 31) ||
      (int64_t)T * ((H + 127) / 128 * 128) * 2 >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need H >= 32, H %% 32 == 0 and T * H * 2 < 2^31 (H=%d)", fn, H);
  if (fp8_act != 0 && fp8_act != 1) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: fp8_act must be 0 or 1", fn);
  if (!aligned(x, 16) || !aligned(x_prep, 16) || !aligned(ws, 16))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: x, x_prep and ws must be 16-byte aligned", fn);
  const size_t route_ws = round_up(route_permute_ws_bytes(T, E, k));
  const size_t need = route_ws + dispatch_rows_ws_bytes(T, H, fp8_act != 0);
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(NVFP4MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
  char* xp = static_cast<char*>(x_prep);
  const ActPrep prep{static_cast<const uint16_t*>(x), H, fp8_act, reinterpret_cast<_Float16*>(xp),
                     reinterpret_cast<int*>(xp + prepared_rows_bytes(T, H)),
                     fp8_act ? static_cast<char*>(ws) + route_ws : nullptr};
  return hip_status(launch_route_permute(logits, T, E, k, topk_ids, topk_w, expert_offsets, sorted_slot, slot_to_row,
                                         active_experts, n_active, ws, route_ws, static_cast<hipStream_t>(stream),
                                         &prep),
                    fn);
}

// ------------------------------------------------------------------ weight tiling
size_t nvfp4_tiled_codes_bytes(int64_t R, int64_t C) {
  if (R < 16 || R % 16 != 0 || C < 32 || C % 32 != 0) return 0;
  return tiled_codes_bytes(R, C);
}
size_t nvfp4_tiled_scales_bytes(int64_t R, int64_t C) {
  if (R < 16 || R % 16 != 0 || C < 32 || C % 32 != 0) return 0;
  return tiled_scales_bytes(R, C);
}

nvfp4moe_status nvfp4_weights_tile(const uint8_t* packed, const uint8_t* scales, int64_t B, int64_t R,
                                   int64_t C, uint8_t* tiled_codes, uint8_t* tiled_scales, void* stream) {
  const char* fn = "nvfp4_weights_tile";
  if (!packed || !scales || !tiled_codes || !tiled_scales)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (B < 1 || B > 65535 || R < 16 || R % 16 != 0 || C < 32 || C % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID_ARG,
                "%s: need 1 <= B <= 65535, R >= 16, R %% 16 == 0, C >= 32, C %% 32 == 0 (B=%lld R=%lld C=%lld)",
                fn, (long long)B, (long long)R, (long long)C);
  if (B * R * (C / 2) >= (int64_t(1) << 40) || R > (int64_t(1) << 30) || C > (int64_t(1) << 30))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: matrices too large", fn);
  if (!aligned(packed, 16) || !aligned(scales, 2) || !aligned(tiled_codes, 16) || !aligned(tiled_scales, 16))
    return fail(NVFP4MOE_ERR_INVALID_ARG,
                "%s: packed and the tiled outputs must be 16-byte aligned, scales 2-byte aligned", fn);
  return hip_status(launch_weights_tile(packed, scales, B, R, C, tiled_codes, tiled_scales,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

// ------------------------------------------------------------------ grouped GEMM
size_t moe_grouped_gemm_workspace_size(nvfp4moe_mode mode, int64_t a_rows, int32_t rows,
                                       int32_t E, int32_t Nw, int32_t K) {
  if (a_rows < 1 || rows < 1 || E < 1 || K < 1) return 0;
  return gemm_ws_layout(gemm_path(rows, E, Nw), mode, a_rows, rows, E, Nw, K).total;
}

size_t moe_grouped_gemm_nvfp4_combine_workspace_size(nvfp4moe_mode mode, int32_t T, int32_t k, int32_t E, int32_t Nw,
                                                     int32_t K) {
  if (T < 1 || k < 1 || E < 1 || K < 1 || Nw < 32 || (int64_t)T * k >= (int64_t(1) << 31)) return 0;
  const int32_t rows = T * k;
  return gemm_ws_layout(gemm_path(rows, E, Nw), mode, rows, rows, E, Nw, K).total + combine_ws_bytes(T, k, Nw);
}

}  // extern "C"

namespace {
nvfp4moe_status grouped_gemm_nvfp4_impl(const char* fn, nvfp4moe_mode mode, nvfp4moe_epilogue epi,
                                        const void* a, const uint8_t* a_scales, const float* a_g,
                                        int64_t a_rows, const int32_t* gather_index,
                                        int32_t gather_div, const uint8_t* w_packed,
                                        const uint8_t* w_scales, const float* w_g,
                                        const int32_t* expert_offsets,
                                        const int32_t* active_experts, const int32_t* n_active,
                                        int32_t E, int32_t rows, int32_t Nw, int32_t K, void* out,
                                        nvfp4moe_dtype out_dtype, float* out_amax, void* ws,
                                        size_t ws_bytes, void* stream, const Combine* comb) {
  if (mode != NVFP4MOE_W4A16 && mode != NVFP4MOE_W4A4 && mode != NVFP4MOE_W4A16_PREPARED)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: bad mode %d", fn, (int)mode);
  const bool prepared = mode == NVFP4MOE_W4A16_PREPARED;
  if (epi != NVFP4MOE_EPI_NONE && epi != NVFP4MOE_EPI_SWIGLU)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: bad epilogue %d", fn, (int)epi);
  if (out_dtype != NVFP4MOE_F32 && out_dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: out_dtype must be F32 or BF16", fn);
  if (!a || !w_packed || !w_scales || !w_g || !expert_offsets || !active_experts || !n_active || !out)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (mode == NVFP4MOE_W4A4 && (!a_scales || !a_g))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: W4A4 needs a_scales and a_g", fn);
  if (E < 1 || E > kMaxExperts)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need 1 <= E <= %d (E=%d)", fn, kMaxExperts, E);
  if (rows < 1 || a_rows < 1)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need rows >= 1 and a_rows >= 1", fn);
  if (Nw < 32 || Nw % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need Nw >= 32 and Nw %% 32 == 0 (Nw=%d)", fn, Nw);
  if (K < 32 || K % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need K >= 32 and K %% 32 == 0 (K=%d)", fn, K);
  if ((int64_t)rows * (K > Nw ? K : Nw) >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: rows * max(K, Nw) must be < 2^31", fn);
  if (a_rows * (int64_t)((K + 127) / 128 * 128) * 2 >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: a_rows * K * 2 must be < 2^31", fn);
  if ((int64_t)Nw * ((K + 127) / 128 * 64) >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: Nw * K / 2 must be < 2^31", fn);
  if (!gather_index && a_rows != rows)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: without gather_index a_rows must equal rows", fn);
  if (gather_index && gather_div < 1)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: gather_div must be >= 1", fn);
  if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(w_scales, 16) ||
      (a_scales && !aligned(a_scales, 2)) || !aligned(out, out_dtype == NVFP4MOE_F32 ? 4 : 2))
    return fail(NVFP4MOE_ERR_INVALID_ARG,
                "%s: a and the tiled weights must be 16-byte aligned, a_scales 2-byte aligned", fn);
  const int path = gemm_path(rows, E, Nw);
  if (path == NVFP4MOE_PATH_NONE)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "%s: the forced MFMA path needs Nw %% 256 == 0 (Nw=%d)", fn, Nw);
  const GemmWs lay = gemm_ws_layout(path, mode, a_rows, rows, E, Nw, K);
  const size_t need = lay.total + (comb ? combine_ws_bytes(comb->T, comb->k, Nw) : 0);
  if (need && (!ws || ws_bytes < need))
    return fail(NVFP4MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
  if (need && !aligned(ws, 16))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);

  hipStream_t s = static_cast<hipStream_t>(stream);
  GemmArgs g{};
  g.w4a4 = mode == NVFP4MOE_W4A4;
  g.gather_index = gather_index;
  g.gather_div = gather_div < 1 ? 1 : gather_div;
  g.w_packed = w_packed;
  g.w_scales = w_scales;
  g.w_g = w_g;
  g.expert_offsets = expert_offsets;
  g.active = active_experts;
  g.n_active = n_active;
  g.E = E;
  g.rows = rows;
  g.Nw = Nw;
  g.K = K;
  g.a_rows = (int)a_rows;
  g.swiglu = epi == NVFP4MOE_EPI_SWIGLU;
  g.out = out;
  g.out_bf16 = out_dtype == NVFP4MOE_BF16;
  g.out_amax = out_amax;

  hipError_t err = hipSuccess;
  char* base = static_cast<char*>(ws);
  g.ksplit = lay.ksplit;
  if (comb) err = combine_setup(g, *comb, base + lay.total, Nw, s);
  if (out_amax && err == hipSuccess) err = launch_zero_f32(out_amax, 1, s);
  if (err != hipSuccess) return hip_status(err, fn);
  if (lay.a16_bytes) {
    g.a16 = reinterpret_cast<_Float16*>(base);
    g.rexp = reinterpret_cast<int*>(base + lay.a16_bytes);
  }
  // The MFMA path's m-tile list is built by one extra workgroup of the activation prep launch.
  MtileSched sched{};
  if (path == NVFP4MOE_PATH_MFMA) {
    char* sp = base + lay.a16_bytes + lay.rexp_bytes;
    const size_t arr = round_up((size_t)lay.max_mtiles * 4);
    g.sched_e = reinterpret_cast<const int*>(sp);
    g.sched_r = reinterpret_cast<const int*>(sp + arr);
    g.sched_n = reinterpret_cast<const int*>(sp + 2 * arr);
    sched = MtileSched{expert_offsets, active_experts, n_active, E, large_rows_per_mtile(), lay.max_mtiles,
                       const_cast<int*>(g.sched_e), const_cast<int*>(g.sched_r), const_cast<int*>(g.sched_n)};
  }
  if (prepared) {   // the rows and exponents of moe_dispatch_w4a16's x_prep
    g.a16 = static_cast<const _Float16*>(a);
    g.rexp = reinterpret_cast<const int*>(static_cast<const char*>(a) + prepared_rows_bytes(a_rows, K));
    if (path == NVFP4MOE_PATH_MFMA) err = launch_mtile_schedule(sched, s);
  } else if (mode == NVFP4MOE_W4A16) {
    err = launch_act_prep(static_cast<const uint16_t*>(a), a_rows, K, const_cast<_Float16*>(g.a16),
                          const_cast<int*>(g.rexp), sched, s);
  } else {
    g.a_packed = static_cast<const uint8_t*>(a);
    g.a_scales = a_scales;
    g.a_g = a_g;
    g.a4_staged = path == NVFP4MOE_PATH_MFMA && large_a4_staged();
    if (g.a4_staged)
      err = launch_mtile_schedule(sched, s);   // the GEMM decodes the FP4 rows itself
    else if (path == NVFP4MOE_PATH_MFMA)
      err = launch_act_prep_fp4(g.a_packed, a_scales, a_rows, K, const_cast<_Float16*>(g.a16),
                                const_cast<int*>(g.rexp), sched, s);
  }
  if (err != hipSuccess) return hip_status(err, fn);
  g_last_dispatch = path;
  g.partial = lay.partial_bytes
                  ? reinterpret_cast<float*>(base + lay.a16_bytes + lay.rexp_bytes + lay.sched_bytes)
                  : nullptr;
  err = path == NVFP4MOE_PATH_MFMA ? launch_gemm_large(g, lay.max_mtiles, s) : launch_gemm_stream(g, s);
  if (err == hipSuccess && comb) err = combine_finish(g, *comb, Nw, s);
  return hip_status(err, fn);
}
}  // namespace

extern "C" {

nvfp4moe_status moe_grouped_gemm_nvfp4(nvfp4moe_mode mode, nvfp4moe_epilogue epi,
                                       const void* a, const uint8_t* a_scales, const float* a_g,
                                       int64_t a_rows, const int32_t* gather_index,
                                       int32_t gather_div, const uint8_t* w_packed,
                                       const uint8_t* w_scales, const float* w_g,
                                       const int32_t* expert_offsets,
                                       const int32_t* active_experts, const int32_t* n_active,
                                       int32_t E, int32_t rows, int32_t Nw, int32_t K, void* out,
                                       nvfp4moe_dtype out_dtype, float* out_amax, void* ws,
                                       size_t ws_bytes, void* stream) {
  return grouped_gemm_nvfp4_impl("moe_grouped_gemm_nvfp4", mode, epi, a, a_scales, a_g, a_rows, gather_index,
                                 gather_div, w_packed, w_scales, w_g, expert_offsets, active_experts, n_active, E,
                                 rows, Nw, K, out, out_dtype, out_amax, ws, ws_bytes, stream, nullptr);
}

nvfp4moe_status moe_grouped_gemm_nvfp4_combine(nvfp4moe_mode mode, const void* a, const uint8_t* a_scales,
                                               const float* a_g, const uint8_t* w_packed, const uint8_t* w_scales,
                                               const float* w_g, const int32_t* expert_offsets,
                                               const int32_t* active_experts, const int32_t* n_active,
                                               const int32_t* sorted_slot, const int32_t* slot_to_row,
                                               const float* topk_w, int32_t E, int32_t T, int32_t k, int32_t Nw,
                                               int32_t K, void* out, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_grouped_gemm_nvfp4_combine";
  const Combine c{sorted_slot, slot_to_row, topk_w, T, k, out};
  const nvfp4moe_status chk = combine_checks(fn, c, E, Nw);
  if (chk != NVFP4MOE_OK) return chk;
  return grouped_gemm_nvfp4_impl(fn, mode, NVFP4MOE_EPI_NONE, a, a_scales, a_g, (int64_t)T * k, nullptr, 1, w_packed,
                                 w_scales, w_g, expert_offsets, active_experts, n_active, E, T * k, Nw, K, out,
                                 NVFP4MOE_F32, nullptr, ws, ws_bytes, stream, &c);
}

// ------------------------------------------------------------------ MXFP4
nvfp4moe_status mxfp4_quantize(const void* x, nvfp4moe_dtype x_dtype, int64_t R, int64_t C, uint8_t* packed,
                               uint8_t* scales, void* stream) {
  const char* fn = "mxfp4_quantize";
  if (!x || !packed || !scales) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: x_dtype must be F32 or BF16", fn);
  if (R < 1 || C < 32 || C % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need R >= 1, C >= 32 and C %% 32 == 0 (R=%lld C=%lld)", fn,
                (long long)R, (long long)C);
  if ((double)R * (double)C > 4.0e12) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: tensor too large", fn);
  if (!aligned(x, 16) || !aligned(packed, 16))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: x and packed must be 16-byte aligned", fn);
  return hip_status(launch_mx_quantize(x, x_dtype == NVFP4MOE_BF16, R * C, packed, scales,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

size_t mxfp4_tiled_scales_bytes(int64_t R, int64_t C) {
  if (R < 16 || R % 16 != 0 || C < 32 || C % 32 != 0) return 0;
  return mx_tiled_scales_bytes(R, C);
}

nvfp4moe_status mxfp4_weights_tile(const uint8_t* packed, const uint8_t* scales, int64_t B, int64_t R, int64_t C,
                                   uint8_t* tiled_codes, uint8_t* tiled_scales, void* stream) {
  const char* fn = "mxfp4_weights_tile";
  if (!packed || !scales || !tiled_codes || !tiled_scales)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (B < 1 || B > 65535 || R < 16 || R % 16 != 0 || C < 32 || C % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID_ARG,
                "%s: need 1 <= B <= 65535, R >= 16, R %% 16 == 0, C >= 32, C %% 32 == 0 (B=%lld R=%lld C=%lld)",
                fn, (long long)B, (long long)R, (long long)C);
  if (B * R * (C / 2) >= (int64_t(1) << 40) || R > (int64_t(1) << 30) || C > (int64_t(1) << 30))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: matrices too large", fn);
  if (!aligned(packed, 16) || !aligned(tiled_codes, 16) || !aligned(tiled_scales, 16))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: packed and the tiled outputs must be 16-byte aligned", fn);
  return hip_status(launch_mx_weights_tile(packed, scales, B, R, C, tiled_codes, tiled_scales,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

namespace {
int mx_max_mtiles(int32_t rows, int32_t E, int bits) {
  const int bm = mx_rows_per_mtile(bits);
  return (rows + bm - 1) / bm + (E < rows ? E : rows);
}

// Workspace of the MX GEMMs: the m-tile list (sched_e, sched_r, sched_n) and, when K is
// split, the [ksplit, rows, Nw] fp32 partial sums.
size_t mx_workspace_size(int32_t rows, int32_t E, int32_t Nw, int32_t K, int bits) {
  if (rows < 1 || E < 1 || Nw < 1 || K < 32) return 0;
  const int mt = mx_max_mtiles(rows, E, bits);
  const int ks = mx_supports(Nw) ? mx_ksplit(mt, Nw, K) : 1;
  const size_t partial = ks > 1 ? round_up((size_t)ks * rows * Nw * 4) : 0;
  return 3 * round_up((size_t)mt * 4) + partial + kAlign;
}
}  // namespace

size_t moe_grouped_gemm_mxfp4_workspace_size(int32_t rows, int32_t E, int32_t Nw, int32_t K) {
  return mx_workspace_size(rows, E, Nw, K, 4);
}
size_t moe_grouped_gemm_mxfp8_workspace_size(int32_t rows, int32_t E, int32_t Nw, int32_t K) {
  return mx_workspace_size(rows, E, Nw, K, 8);
}

namespace {
// Both MXFP4 GEMM entry points: out/out_dtype/out_amax, or (SwiGLU only) h quantized to
// MXFP4 into hq_packed/hq_scales.
nvfp4moe_status mx_gemm_call(const char* fn, int bits, nvfp4moe_epilogue epi, const uint8_t* a, const uint8_t* a_scales,
                             int64_t a_rows, const int32_t* gather_index, int32_t gather_div,
                             const uint8_t* w_packed, const uint8_t* w_scales, const int32_t* expert_offsets,
                             const int32_t* active_experts, const int32_t* n_active, int32_t E, int32_t rows,
                             int32_t Nw, int32_t K, void* out, nvfp4moe_dtype out_dtype, float* out_amax,
                             uint8_t* hq_packed, uint8_t* hq_scales, void* ws, size_t ws_bytes, void* stream,
                             const Combine* comb = nullptr) {
  const bool qh = hq_packed != nullptr;
  if (epi != NVFP4MOE_EPI_NONE && epi != NVFP4MOE_EPI_SWIGLU)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: bad epilogue %d", fn, (int)epi);
  if (out_dtype != NVFP4MOE_F32 && out_dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: out_dtype must be F32 or BF16", fn);
  if (!a || !a_scales || !w_packed || !w_scales || !expert_offsets || !active_experts || !n_active ||
      (qh ? !hq_scales : !out))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (E < 1 || E > kMaxExperts)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need 1 <= E <= %d (E=%d)", fn, kMaxExperts, E);
  if (rows < 1 || a_rows < 1) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need rows >= 1 and a_rows >= 1", fn);
  if (K < 32 || K % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need K >= 32 and K %% 32 == 0 (K=%d)", fn, K);
  if (!mx_supports(Nw))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "%s: needs Nw %% 256 == 0 (Nw=%d)", fn, Nw);
  const int64_t kbytes = bits == 8 ? (int64_t)K : (int64_t)(K / 2);   // code bytes of a row
  if ((int64_t)rows * (K > Nw ? K : Nw) >= (int64_t(1) << 31) || a_rows * kbytes >= (int64_t(1) << 31) ||
      (int64_t)Nw * ((K + 127) / 128 * 128) * bits / 8 >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: rows * max(K, Nw) and the code bytes of a and w must be < 2^31", fn);
  if (!gather_index && a_rows != rows)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: without gather_index a_rows must equal rows", fn);
  if (gather_index && gather_div < 1) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: gather_div must be >= 1", fn);
  if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(w_scales, 16) ||
      (qh ? !aligned(hq_packed, 16) || !aligned(hq_scales, 4) : !aligned(out, out_dtype == NVFP4MOE_F32 ? 4 : 2)))
    return fail(NVFP4MOE_ERR_INVALID_ARG,
                "%s: a and the tiled weights must be 16-byte aligned, the output to its element", fn);
  const size_t mx_need = mx_workspace_size(rows, E, Nw, K, bits);
  const size_t need = mx_need + (comb ? combine_ws_bytes(comb->T, comb->k, Nw) : 0);
  if (!ws || ws_bytes < need)
    return fail(NVFP4MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
  if (!aligned(ws, 16)) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int max_mtiles = mx_max_mtiles(rows, E, bits);
  const size_t arr = round_up((size_t)max_mtiles * 4);
  char* base = static_cast<char*>(ws);
  GemmArgs g{};
  g.w4a4 = 1;
  g.a_packed = a;
  g.a_scales = a_scales;
  g.gather_index = gather_index;
  g.gather_div = gather_div < 1 ? 1 : gather_div;
  g.w_packed = w_packed;
  g.w_scales = w_scales;
  g.expert_offsets = expert_offsets;
  g.active = active_experts;
  g.n_active = n_active;
  g.E = E;
  g.rows = rows;
  g.Nw = Nw;
  g.K = K;
  g.a_rows = (int)a_rows;
  g.swiglu = epi == NVFP4MOE_EPI_SWIGLU;
  g.out = out;
  g.out_bf16 = out_dtype == NVFP4MOE_BF16;
  g.out_amax = out_amax;
  const bool dense = E == 1;   // one expert: the GEMM numbers its m-tiles itself, no list
  g.sched_e = dense ? nullptr : reinterpret_cast<const int*>(base);
  g.sched_r = dense ? nullptr : reinterpret_cast<const int*>(base + arr);
  g.sched_n = dense ? nullptr : reinterpret_cast<const int*>(base + 2 * arr);
  g.hq_packed = hq_packed;
  g.hq_scales = hq_scales;
  g.ksplit = qh ? 1 : mx_ksplit(max_mtiles, Nw, K);   // the quantized epilogue needs whole sums
  g.partial = g.ksplit > 1 ? reinterpret_cast<float*>(base + 3 * arr) : nullptr;
  g.unit_alpha = 1;
  if ((int64_t)g.ksplit * rows * Nw >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: split-K partial sums too large (ksplit %d)", fn, g.ksplit);
  hipError_t err = hipSuccess;
  if (comb) err = combine_setup(g, *comb, base + mx_need, Nw, s);
  if (out_amax && err == hipSuccess) err = launch_zero_f32(out_amax, 1, s);
  if (err != hipSuccess) return hip_status(err, fn);
  const MtileSched sched{expert_offsets, active_experts, n_active, E, mx_rows_per_mtile(bits), max_mtiles,
                         const_cast<int*>(g.sched_e), const_cast<int*>(g.sched_r), const_cast<int*>(g.sched_n)};
  if (!dense) err = launch_mtile_schedule(sched, s);
  if (err == hipSuccess) err = launch_gemm_mx(g, max_mtiles, bits, s);
  if (err == hipSuccess && comb) err = combine_finish(g, *comb, Nw, s);
  return hip_status(err, fn);
}
}  // namespace

nvfp4moe_status moe_grouped_gemm_mxfp4(nvfp4moe_epilogue epi, const uint8_t* a, const uint8_t* a_scales,
                                       int64_t a_rows, const int32_t* gather_index, int32_t gather_div,
                                       const uint8_t* w_packed, const uint8_t* w_scales,
                                       const int32_t* expert_offsets, const int32_t* active_experts,
                                       const int32_t* n_active, int32_t E, int32_t rows, int32_t Nw,
                                       int32_t K, void* out, nvfp4moe_dtype out_dtype, float* out_amax, void* ws,
                                       size_t ws_bytes, void* stream) {
  return mx_gemm_call("moe_grouped_gemm_mxfp4", 4, epi, a, a_scales, a_rows, gather_index, gather_div, w_packed,
                      w_scales, expert_offsets, active_experts, n_active, E, rows, Nw, K, out, out_dtype, out_amax,
                      nullptr, nullptr, ws, ws_bytes, stream);
}

size_t moe_grouped_gemm_mxfp4_combine_workspace_size(int32_t T, int32_t k, int32_t E, int32_t Nw, int32_t K) {
  if (T < 1 || k < 1 || E < 1 || K < 32 || Nw < 32 || (int64_t)T * k >= (int64_t(1) << 31)) return 0;
  return mx_workspace_size(T * k, E, Nw, K, 4) + combine_ws_bytes(T, k, Nw);
}

nvfp4moe_status moe_grouped_gemm_mxfp4_combine(const uint8_t* a, const uint8_t* a_scales, const uint8_t* w_packed,
                                               const uint8_t* w_scales, const int32_t* expert_offsets,
                                               const int32_t* active_experts, const int32_t* n_active,
                                               const int32_t* sorted_slot, const int32_t* slot_to_row,
                                               const float* topk_w, int32_t E, int32_t T, int32_t k, int32_t Nw,
                                               int32_t K, void* out, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_grouped_gemm_mxfp4_combine";
  const Combine c{sorted_slot, slot_to_row, topk_w, T, k, out};
  const nvfp4moe_status chk = combine_checks(fn, c, E, Nw);
  if (chk != NVFP4MOE_OK) return chk;
  return mx_gemm_call(fn, 4, NVFP4MOE_EPI_NONE, a, a_scales, (int64_t)T * k, nullptr, 1, w_packed, w_scales,
                      expert_offsets, active_experts, n_active, E, T * k, Nw, K, out, NVFP4MOE_F32, nullptr, nullptr,
                      nullptr, ws, ws_bytes, stream, &c);
}

nvfp4moe_status moe_grouped_gemm_mxfp4_swiglu_q(const uint8_t* a, const uint8_t* a_scales, int64_t a_rows,
                                                const int32_t* gather_index, int32_t gather_div,
                                                const uint8_t* w_packed, const uint8_t* w_scales,
                                                const int32_t* expert_offsets, const int32_t* active_experts,
                                                const int32_t* n_active, int32_t E, int32_t rows, int32_t Nw,
                                                int32_t K, uint8_t* h_packed, uint8_t* h_scales, void* ws,
                                                size_t ws_bytes, void* stream) {
  if (!h_packed) return fail(NVFP4MOE_ERR_INVALID_ARG, "moe_grouped_gemm_mxfp4_swiglu_q: null tensor pointer");
  return mx_gemm_call("moe_grouped_gemm_mxfp4_swiglu_q", 4, NVFP4MOE_EPI_SWIGLU, a, a_scales, a_rows, gather_index,
                      gather_div, w_packed, w_scales, expert_offsets, active_experts, n_active, E, rows, Nw, K,
                      nullptr, NVFP4MOE_F32, nullptr, h_packed, h_scales, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ unpermute-reduce
nvfp4moe_status moe_unpermute_reduce(const void* y, nvfp4moe_dtype y_dtype,
                                     const int32_t* slot_to_row, const float* topk_w, int32_t T,
                                     int32_t k, int32_t H, void* out, void* stream) {
  const char* fn = "moe_unpermute_reduce";
  if (!y || !slot_to_row || !topk_w || !out)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (y_dtype != NVFP4MOE_F32 && y_dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: y_dtype must be F32 or BF16", fn);
  if (T < 1 || k < 1 || H < 8 || H % 8 != 0)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need T >= 1, k >= 1, H >= 8, H %% 8 == 0", fn);
  if ((int64_t)T * k * H >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: T * k * H must be < 2^31", fn);
  if (!aligned(y, 16) || !aligned(out, 16))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: y and out must be 16-byte aligned", fn);
  return hip_status(launch_unpermute_reduce(y, y_dtype == NVFP4MOE_BF16, slot_to_row, topk_w, T, k,
                                            H, static_cast<uint16_t*>(out),
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

// ------------------------------------------------------------------ FP8 activations
size_t act_fp8_e4m3_roundtrip_workspace_size(int64_t n) {
  if (n < 1) return 0;
  return round_up(fp8_roundtrip_ws_bytes(n));
}

nvfp4moe_status act_fp8_e4m3_roundtrip(const void* x, int64_t n, void* out, void* ws,
                                       size_t ws_bytes, void* stream) {
  const char* fn = "act_fp8_e4m3_roundtrip";
  if (!x || !out) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (n < 8 || n % 8 != 0 || n > (int64_t(1) << 40))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need n >= 8 and n %% 8 == 0", fn);
  if (!aligned(x, 16) || !aligned(out, 16))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: x and out must be 16-byte aligned", fn);
  const size_t need = act_fp8_e4m3_roundtrip_workspace_size(n);
  if (!ws || ws_bytes < need)
    return fail(NVFP4MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                ws_bytes);
  return hip_status(launch_fp8_roundtrip(x, n, out, ws, static_cast<hipStream_t>(stream)), fn);
}

// ------------------------------------------------------------------ MXFP8
nvfp4moe_status mxfp8_quantize(const void* x, nvfp4moe_dtype x_dtype, int64_t R, int64_t C, uint8_t* codes,
                               uint8_t* scales, void* stream) {
  const char* fn = "mxfp8_quantize";
  if (!x || !codes || !scales) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: x_dtype must be F32 or BF16", fn);
  if (R < 1 || C < 32 || C % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: need R >= 1, C >= 32 and C %% 32 == 0 (R=%lld C=%lld)", fn,
                (long long)R, (long long)C);
  if ((double)R * (double)C > 4.0e12) return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: tensor too large", fn);
  if (!aligned(x, 16) || !aligned(codes, 16))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: x and codes must be 16-byte aligned", fn);
  return hip_status(launch_mx8_quantize(x, x_dtype == NVFP4MOE_BF16, R * C, codes, scales,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

size_t mxfp8_tiled_codes_bytes(int64_t R, int64_t C) {
  if (R < 16 || R % 16 != 0 || C < 32 || C % 32 != 0) return 0;
  return mx8_tiled_codes_bytes(R, C);
}

nvfp4moe_status mxfp8_weights_tile(const uint8_t* codes, const uint8_t* scales, int64_t B, int64_t R, int64_t C,
                                   uint8_t* tiled_codes, uint8_t* tiled_scales, void* stream) {
  const char* fn = "mxfp8_weights_tile";
  if (!codes || !scales || !tiled_codes || !tiled_scales)
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (B < 1 || B > 65535 || R < 16 || R % 16 != 0 || C < 32 || C % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID_ARG,
                "%s: need 1 <= B <= 65535, R >= 16, R %% 16 == 0, C >= 32, C %% 32 == 0 (B=%lld R=%lld C=%lld)",
                fn, (long long)B, (long long)R, (long long)C);
  if (B * R * C >= (int64_t(1) << 40) || R > (int64_t(1) << 30) || C > (int64_t(1) << 30))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: matrices too large", fn);
  if (!aligned(codes, 16) || !aligned(tiled_codes, 16) || !aligned(tiled_scales, 16))
    return fail(NVFP4MOE_ERR_INVALID_ARG, "%s: codes and the tiled outputs must be 16-byte aligned", fn);
  return hip_status(launch_mx8_weights_tile(codes, scales, B, R, C, tiled_codes, tiled_scales,
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

nvfp4moe_status moe_grouped_gemm_mxfp8(nvfp4moe_epilogue epi, const uint8_t* a, const uint8_t* a_scales,
                                       int64_t a_rows, const int32_t* gather_index, int32_t gather_div,
                                       const uint8_t* w_codes, const uint8_t* w_scales,
                                       const int32_t* expert_offsets, const int32_t* active_experts,
                                       const int32_t* n_active, int32_t E, int32_t rows, int32_t Nw,
                                       int32_t K, void* out, nvfp4moe_dtype out_dtype, float* out_amax, void* ws,
                                       size_t ws_bytes, void* stream) {
  return mx_gemm_call("moe_grouped_gemm_mxfp8", 8, epi, a, a_scales, a_rows, gather_index, gather_div, w_codes,
                      w_scales, expert_offsets, active_experts, n_active, E, rows, Nw, K, out, out_dtype, out_amax,
                      nullptr, nullptr, ws, ws_bytes, stream);
}

}  // extern "C"
