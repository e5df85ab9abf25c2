// Host side of the C ABI declared in include/wq.h: argument checks, path
// choice, the MoE combine workspace, and error reporting.
//
// The argument checks follow the pages' own: k must be a multiple of 32
// (wavo src/gpu/mod.rs `Gpu::upload_linear`; hanzo-ml src/wgpu_backend.rs
// `matvec_q4_0_gpu` / `matvec_q8_0_gpu`), buffers must hold what the sizes
// say (`moe_matvec_gpu`), and the bias flag follows the presence of a bias
// (cortiq-engine src/gpu_wgpu/nemotron_audio.rs `AudioEncoder::gemm` sets
// flag 1 exactly when a bias is given). Every check runs before any HIP call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "wq.h"
#include "wq_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(WQ_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

void clear_error() { g_err[0] = '\0'; }

constexpr int64_t kIntMax = 0x7fffffff;
// Row counts the kernels round up to whole tiles (at most 256 rows) in 32-bit ints.
constexpr int64_t kMaxRows = kIntMax - 512;
// Elements of an output: tile counts (64 x 64 and larger tiles) then fit in 28 bits, so the
// GEMM's grid of tile numbers fits in an int. 2^40 floats are 4 TiB, beyond any device.
constexpr int64_t kMaxOutputs = int64_t(1) << 40;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges; empty ranges never overlap).
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(nb) && b0 < a0 + static_cast<uintptr_t>(na);
}

int check_wtype(int wtype) {
  if (wtype != WQ_W_BF16 && wtype != WQ_W_Q8_0 && wtype != WQ_W_Q4_0 && wtype != WQ_W_F32 && wtype != WQ_W_F16 &&
      wtype != WQ_W_Q4_K)
    return fail(WQ_ERR_WTYPE, "unknown weight type %d (0 = bf16, 1 = Q8_0, 2 = Q4_0, 3 = f32, 4 = f16, 5 = Q4_K)",
                wtype);
  return WQ_OK;
}

int check_k(int64_t k, int wtype) {
  if (k <= 0 || k % 32 != 0) return fail(WQ_ERR_SHAPE, "k must be a positive multiple of 32, got %lld", (long long)k);
  if (k > kIntMax / 4) return fail(WQ_ERR_SHAPE, "k = %lld is too large", (long long)k);
  if (wtype == WQ_W_Q4_K && k % 256 != 0)
    return fail(WQ_ERR_SHAPE, "Q4_K weights need k % 256 == 0 (256-weight super-blocks), got %lld", (long long)k);
  return WQ_OK;
}

// ---- MoE combine workspace: per (device, stream), grown on demand, kept for the process ----
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// The caller holds g_ws_mu until the work that uses the buffer is queued: another thread that
// grows the same (device, stream) buffer then waits for that work before freeing it, instead of
// freeing it between this call's lookup and its launches.
int workspace(hipStream_t stream, size_t bytes, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  Workspace& w = g_ws[{dev, stream}];
  if (w.bytes < bytes) {
    if (w.ptr) {
      // The old buffer may still be read by work queued on this stream.
      e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      e = hipFree(w.ptr);
      if (e != hipSuccess) return hip_fail(e, "hipFree");
      w.ptr = nullptr;
      w.bytes = 0;
    }
    size_t want = bytes < (size_t(1) << 20) ? (size_t(1) << 20) : bytes;
    e = hipMalloc(&w.ptr, want);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc (MoE workspace)");
    w.bytes = want;
  }
  *out = w.ptr;
  return WQ_OK;
}

// ---- no-allocation scratch (wq_moe_matvec_noalloc) ----
// The per-slot products of a gated MoE call, before the combine. A file-scope device array: each
// GPU the library runs on holds its own copy from the module's load until the process ends. Host
// code never uses the name itself (in host code it is a stand-in, not a device address); it takes
// the address from hipGetSymbolAddress once per device, with that device current.
constexpr size_t kScratchFloats = size_t(8) << 20;  // 32 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

std::mutex g_scratch_mu;
float* g_scratch_ptr[64] = {};

int scratch_address(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(WQ_ERR_HIP, "device index %d outside the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (MoE scratch)");
    if (ptr == nullptr) return fail(WQ_ERR_HIP, "hipGetSymbolAddress gave a null scratch address");
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return WQ_OK;
}

// io (inside the library only): bit 0, x holds bf16 bit patterns; bit 1, y receives them. Both
// take bf16 weights on the bf16 matrix-core path (which rounds X to bf16 anyway), and a bf16 y
// takes no residual and no dual outputs. dry: run the checks only (a caller that launches several
// steps checks them all before its first launch).
int gemm_checked(const float* x, const void* w, int wtype, const float* bias, unsigned flags, float alpha,
                 float* y, int64_t n, int64_t m, int64_t k, int64_t dual, int path, void* stream, int io = 0,
                 bool dry = false) {
  clear_error();
  if (int r = check_wtype(wtype)) return r;
  constexpr unsigned kActs = WQ_GELU | WQ_SILU | WQ_RELU | WQ_TANH;
  if (flags & ~(WQ_BIAS | WQ_RESIDUAL | kActs)) return fail(WQ_ERR_FLAGS, "unknown flag bits 0x%x", flags);
  if (__builtin_popcount(flags & kActs) > 1)
    return fail(WQ_ERR_FLAGS, "at most one activation flag (GELU, SILU, RELU, TANH), got 0x%x", flags);
  if (!std::isfinite(alpha)) return fail(WQ_ERR_FLAGS, "alpha must be finite");
  if (((flags & WQ_BIAS) != 0) != (bias != nullptr))
    return fail(WQ_ERR_FLAGS, "WQ_BIAS must be set exactly when a bias pointer is given");
  if (path != WQ_PATH_AUTO && path != WQ_PATH_MATVEC && path != WQ_PATH_MFMA && path != WQ_PATH_MFMA_F32)
    return fail(WQ_ERR_SHAPE, "unknown path %d", path);
  if (n < 0 || m < 0) return fail(WQ_ERR_SHAPE, "negative size n = %lld, m = %lld", (long long)n, (long long)m);
  if (int r = check_k(k, wtype)) return r;
  if (n > kMaxRows || m > kMaxRows) return fail(WQ_ERR_SHAPE, "n or m exceeds 2^31 - 513");
  if (dual < 0 || dual > m) return fail(WQ_ERR_SHAPE, "dual must be in [0, m], got %lld", (long long)dual);
  if (m + dual > kMaxRows) return fail(WQ_ERR_SHAPE, "m + dual exceeds 2^31 - 513");
  if (n > 0 && (m + dual) > kMaxOutputs / n) return fail(WQ_ERR_SHAPE, "n * (m + dual) exceeds 2^40");
  if (wtype == WQ_W_Q4_K && (path == WQ_PATH_MFMA || path == WQ_PATH_MFMA_F32 || n > WQ_MATVEC_MAX_N))
    return fail(WQ_ERR_WTYPE, "Q4_K weights take the matvec path only (n <= %d), got n = %lld, path %d", WQ_MATVEC_MAX_N,
                (long long)n, path);
  if (path == WQ_PATH_AUTO) path = n <= WQ_MATVEC_MAX_N ? WQ_PATH_MATVEC : WQ_PATH_MFMA;
  if (path == WQ_PATH_MATVEC && n > WQ_MATVEC_MAX_N)
    return fail(WQ_ERR_SHAPE, "the matvec path takes n <= %d, got %lld", WQ_MATVEC_MAX_N, (long long)n);
  if ((path == WQ_PATH_MFMA || path == WQ_PATH_MFMA_F32) && n > 65535LL * 128)
    return fail(WQ_ERR_SHAPE, "n = %lld exceeds the GEMM grid (65535 x 128 rows)", (long long)n);
  if (io != 0 && (wtype != WQ_W_BF16 || path != WQ_PATH_MFMA || dual != 0 || ((io & 2) && (flags & WQ_RESIDUAL))))
    return fail(WQ_ERR_SHAPE, "bf16 activations take bf16 weights on the bf16 matrix-core path");
  if (n == 0 || m == 0) return WQ_OK;
  if (!x || !w || !y) return fail(WQ_ERR_NULL, "x, w and y must not be NULL");
  if (!aligned(x, 16) || !aligned(w, 16)) return fail(WQ_ERR_ALIGN, "x and w must be 16-byte aligned");
  if (!aligned(y, 4) || (bias && !aligned(bias, 4))) return fail(WQ_ERR_ALIGN, "y and bias must be 4-byte aligned");
  const int64_t wbytes = wq_weight_bytes(wtype, m, k);
  const int64_t ybytes = n * (m + dual) * ((io & 2) ? 2 : 4);
  if (overlap(y, ybytes, x, n * k * ((io & 1) ? 2 : 4)) || overlap(y, ybytes, w, wbytes) ||
      overlap(y, ybytes, bias, (m + dual) * 4))
    return fail(WQ_ERR_ALIAS, "y overlaps x, w or bias");
  if (dry) return WQ_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  const long long rowbytes = static_cast<long long>(wbytes / m);
  if (path == WQ_PATH_MATVEC) {
    wq::MatvecParams p{};
    p.x = x;
    p.w = static_cast<const uint8_t*>(w);
    p.expert_bytes = 0;
    p.bias = bias;
    p.y = y;
    p.ids = nullptr;
    p.n_slots = static_cast<int>(n);
    p.top_k = 1;
    p.n_exp = 1;
    p.m = static_cast<int>(m);
    p.k = static_cast<int>(k);
    p.rowbytes = rowbytes;
    p.flags = flags;
    p.alpha = alpha;
    p.ystride = static_cast<int>(m + dual);
    p.dual = static_cast<int>(dual);
    e = wq::launch_matvec(wtype, p, static_cast<int>(n), s);
  } else {
    wq::GemmParams p{};
    p.x = x;
    p.w = static_cast<const uint8_t*>(w);
    p.bias = bias;
    p.y = y;
    p.n = static_cast<int>(n);
    p.m = static_cast<int>(m);
    p.k = static_cast<int>(k);
    p.rowbytes = rowbytes;
    p.flags = flags;
    p.alpha = alpha;
    p.ystride = static_cast<int>(m + dual);
    p.dual = static_cast<int>(dual);
    p.x_parts = path == WQ_PATH_MFMA_F32 ? 3 : 1;
    p.x_bf16 = io & 1;
    p.y_bf16 = (io >> 1) & 1;
    e = wq::launch_gemm(wtype, p, s);
  }
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return WQ_OK;
}

}  // namespace

extern "C" {

int64_t wq_weight_bytes(int wtype, int64_t m, int64_t k) {
  if (m < 0 || k < 0 || k % 32 != 0) return -1;
  switch (wtype) {
    case WQ_W_Q4_K: return k % 256 != 0 ? -1 : 144 * m * (k / 256);
    case WQ_W_BF16: return 2 * m * k;
    case WQ_W_Q8_0: return 34 * m * (k / 32);
    case WQ_W_Q4_0: return 18 * m * (k / 32);
    case WQ_W_F32: return 4 * m * k;
    case WQ_W_F16: return 2 * m * k;
    default: return -1;
  }
}

int wq_gemm_path(int64_t n, int64_t m, int64_t k, int wtype) {
  clear_error();
  if (int r = check_wtype(wtype)) return r;
  if (n < 0 || m < 0) return fail(WQ_ERR_SHAPE, "negative size");
  if (int r = check_k(k, wtype)) return r;
  if (wtype == WQ_W_Q4_K && n > WQ_MATVEC_MAX_N)
    return fail(WQ_ERR_WTYPE, "Q4_K weights take the matvec path only (n <= %d)", WQ_MATVEC_MAX_N);
  return n <= WQ_MATVEC_MAX_N ? WQ_PATH_MATVEC : WQ_PATH_MFMA;
}

int wq_gemm(const float* x, const void* w, int wtype, const float* bias, unsigned flags, float* y, int64_t n,
            int64_t m, int64_t k, void* stream) {
  return gemm_checked(x, w, wtype, bias, flags, 1.0f, y, n, m, k, 0, WQ_PATH_AUTO, stream);
}

int wq_gemm_ex(const float* x, const void* w, int wtype, const float* bias, unsigned flags, float* y, int64_t n,
               int64_t m, int64_t k, int path, void* stream) {
  return gemm_checked(x, w, wtype, bias, flags, 1.0f, y, n, m, k, 0, path, stream);
}

int wq_linear(const float* x, const void* w, int wtype, const float* bias, unsigned flags, float alpha, float* y,
              int64_t n, int64_t m, int64_t k, int path, void* stream) {
  return gemm_checked(x, w, wtype, bias, flags, alpha, y, n, m, k, 0, path, stream);
}

int wq_linear_dual(const float* x, const void* w, int wtype, const float* bias, unsigned flags, float alpha,
                   float* y, int64_t n, int64_t m, int64_t k, int64_t dual, int path, void* stream) {
  return gemm_checked(x, w, wtype, bias, flags, alpha, y, n, m, k, dual, path, stream);
}

}  // extern "C"

namespace {

// Both MoE entry points: `noalloc` takes the per-slot products into the library's fixed scratch
// array instead of the grown workspace.
int moe_checked(const float* x, const void* w_experts, int wtype, const int32_t* expert_ids,
                const float* gate_w, float* y, int64_t n_tok, int64_t top_k, int64_t n_experts, int64_t m,
                int64_t k, void* stream, bool noalloc) {
  clear_error();
  if (int r = check_wtype(wtype)) return r;
  if (n_tok < 0 || m < 0) return fail(WQ_ERR_SHAPE, "negative size");
  if (n_experts < 1 || n_experts > 65534) return fail(WQ_ERR_SHAPE, "n_experts must be in [1, 65534]");
  if (top_k < 1 || top_k > n_experts) return fail(WQ_ERR_SHAPE, "top_k must be in [1, n_experts]");
  if (int r = check_k(k, wtype)) return r;
  if (m > kMaxRows) return fail(WQ_ERR_SHAPE, "m exceeds 2^31 - 513");
  if (n_tok * top_k > 4096) return fail(WQ_ERR_SHAPE, "n_tok * top_k must be <= 4096");
  if (n_tok * top_k * m > kMaxOutputs) return fail(WQ_ERR_SHAPE, "n_tok * top_k * m exceeds 2^40");
  if (n_tok == 0 || m == 0) return WQ_OK;
  if (!x || !w_experts || !expert_ids || !y) return fail(WQ_ERR_NULL, "x, w_experts, expert_ids and y must not be NULL");
  if (!aligned(x, 16) || !aligned(w_experts, 16))
    return fail(WQ_ERR_ALIGN, "x and w_experts must be 16-byte aligned");
  if (!aligned(y, 4) || !aligned(expert_ids, 4) || (gate_w && !aligned(gate_w, 4)))
    return fail(WQ_ERR_ALIGN, "y, expert_ids and gate_w must be 4-byte aligned");
  const int64_t n_slots = n_tok * top_k;
  const int64_t ebytes = wq_weight_bytes(wtype, m, k);
  const int64_t ybytes = (gate_w ? n_tok : n_slots) * m * 4;
  if (overlap(y, ybytes, x, n_tok * k * 4) || overlap(y, ybytes, w_experts, ebytes * n_experts) ||
      overlap(y, ybytes, expert_ids, n_slots * 4) || overlap(y, ybytes, gate_w, n_slots * 4))
    return fail(WQ_ERR_ALIAS, "y overlaps x, w_experts, expert_ids or gate_w");

  if (noalloc && gate_w && n_slots * m > static_cast<int64_t>(kScratchFloats))
    return fail(WQ_ERR_SHAPE, "n_tok * top_k * m = %lld exceeds the %lld floats of the no-allocation scratch",
                (long long)(n_slots * m), (long long)kScratchFloats);

  hipStream_t s = static_cast<hipStream_t>(stream);
  float* slots = y;
  std::unique_lock<std::mutex> ws_lock(g_ws_mu, std::defer_lock);  // held through the launches
  if (gate_w && noalloc) {
    if (int r = scratch_address(&slots)) return r;
  } else if (gate_w) {
    ws_lock.lock();
    void* ws = nullptr;
    if (int r = workspace(s, static_cast<size_t>(n_slots * m * 4), &ws)) return r;
    slots = static_cast<float*>(ws);
  }
  wq::MatvecParams p{};
  p.x = x;
  p.w = static_cast<const uint8_t*>(w_experts);
  p.expert_bytes = ebytes;
  p.bias = nullptr;
  p.y = slots;
  p.ids = expert_ids;
  p.n_slots = static_cast<int>(n_slots);
  p.top_k = static_cast<int>(top_k);
  p.n_exp = static_cast<int>(n_experts);
  p.m = static_cast<int>(m);
  p.k = static_cast<int>(k);
  p.rowbytes = ebytes / m;
  p.flags = 0;
  p.alpha = 1.0f;
  p.ystride = static_cast<int>(m);
  p.dual = 0;
  // Twice the mean count of slots per expert picks the tokens-per-pass variant: an expert
  // holding more than that is rare, and is still served exactly by a further pass over its rows.
  const int64_t per_expert = 2 * ((n_slots + n_experts - 1) / n_experts);
  hipError_t e = wq::launch_matvec(wtype, p, static_cast<int>(per_expert < n_tok ? per_expert : n_tok), s);
  if (e != hipSuccess) return hip_fail(e, "MoE matvec launch");
  if (gate_w) {
    e = wq::launch_moe_combine(slots, gate_w, y, static_cast<int>(n_tok), static_cast<int>(top_k),
                               static_cast<int>(m), s);
    if (e != hipSuccess) return hip_fail(e, "MoE combine launch");
  }
  return WQ_OK;
}

}  // namespace

extern "C" {

int wq_moe_matvec(const float* x, const void* w_experts, int wtype, const int32_t* expert_ids,
                  const float* gate_w, float* y, int64_t n_tok, int64_t top_k, int64_t n_experts, int64_t m,
                  int64_t k, void* stream) {
  return moe_checked(x, w_experts, wtype, expert_ids, gate_w, y, n_tok, top_k, n_experts, m, k, stream, false);
}

int wq_moe_matvec_noalloc(const float* x, const void* w_experts, int wtype, const int32_t* expert_ids,
                          const float* gate_w, float* y, int64_t n_tok, int64_t top_k, int64_t n_experts,
                          int64_t m, int64_t k, void* stream) {
  return moe_checked(x, w_experts, wtype, expert_ids, gate_w, y, n_tok, top_k, n_experts, m, k, stream, true);
}

int wq_dequantize(const void* w, int wtype, float* out, int64_t m, int64_t k, void* stream) {
  clear_error();
  if (int r = check_wtype(wtype)) return r;
  if (m < 0) return fail(WQ_ERR_SHAPE, "negative m");
  if (int r = check_k(k, wtype)) return r;
  if (m > kMaxRows || m * (k / 32) > kIntMax * 128LL) return fail(WQ_ERR_SHAPE, "m * k too large");
  if (m == 0) return WQ_OK;
  if (!w || !out) return fail(WQ_ERR_NULL, "w and out must not be NULL");
  if (!aligned(w, 16) || !aligned(out, 16)) return fail(WQ_ERR_ALIGN, "w and out must be 16-byte aligned");
  if (overlap(out, m * k * 4, w, wq_weight_bytes(wtype, m, k))) return fail(WQ_ERR_ALIAS, "out overlaps w");
  hipError_t e = wq::launch_dequantize(wtype, static_cast<const uint8_t*>(w), out, static_cast<int>(m),
                                       static_cast<int>(k), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  return WQ_OK;
}

int64_t wq_padded_k(int64_t k) { return k < 1 || k > kIntMax / 4 ? -1 : (k + 31) / 32 * 32; }

int wq_pad_weight(const void* w, int wtype, float* out, int64_t m, int64_t k, void* stream) {
  clear_error();
  if (wtype != WQ_W_F32 && wtype != WQ_W_F16 && wtype != WQ_W_BF16)
    return fail(WQ_ERR_WTYPE, "padding takes f32, f16 or bf16 weights (3, 4 or 0), got %d", wtype);
  if (m < 0) return fail(WQ_ERR_SHAPE, "negative m");
  const int64_t kp = wq_padded_k(k);
  if (kp < 0) return fail(WQ_ERR_SHAPE, "k must be in [1, 2^29 - 1], got %lld", (long long)k);
  if (m > kMaxRows || m * kp > kMaxOutputs) return fail(WQ_ERR_SHAPE, "m * k too large");
  if (m == 0) return WQ_OK;
  if (!w || !out) return fail(WQ_ERR_NULL, "w and out must not be NULL");
  const int64_t width = wtype == WQ_W_F32 ? 4 : 2;
  if (!aligned(w, static_cast<uintptr_t>(width)) || !aligned(out, 4))
    return fail(WQ_ERR_ALIGN, "w must be aligned to its element size and out to 4 bytes");
  if (overlap(out, m * kp * 4, w, m * k * width)) return fail(WQ_ERR_ALIAS, "out overlaps w");
  hipError_t e = wq::launch_pad_weight(wtype, static_cast<const uint8_t*>(w), out, m, static_cast<int>(k),
                                       static_cast<int>(kp), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pad weight launch");
  return WQ_OK;
}

// ---- encoder block ------------------------------------------------------------------------------

int wq_layer_norm(const float* x, const float* wb, float* y, int64_t n, int64_t d, void* stream) {
  clear_error();
  if (n < 0 || d < 1) return fail(WQ_ERR_SHAPE, "need n >= 0 and d >= 1, got n = %lld, d = %lld", (long long)n, (long long)d);
  if (n > kMaxRows || d > kIntMax / 2) return fail(WQ_ERR_SHAPE, "n or d too large");
  if (n > 0 && d > kMaxOutputs / n) return fail(WQ_ERR_SHAPE, "n * d exceeds 2^40");
  if (n == 0) return WQ_OK;
  if (!x || !wb || !y) return fail(WQ_ERR_NULL, "x, wb and y must not be NULL");
  if (!aligned(x, 4) || !aligned(wb, 4) || !aligned(y, 4)) return fail(WQ_ERR_ALIGN, "x, wb and y must be 4-byte aligned");
  const int64_t bytes = n * d * 4;
  if ((y != x && overlap(y, bytes, x, bytes)) || overlap(y, bytes, wb, 2 * d * 4))
    return fail(WQ_ERR_ALIAS, "y overlaps wb, or overlaps x without being x");
  hipError_t e = wq::launch_layer_norm(x, wb, y, static_cast<int>(n), static_cast<int>(d),
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "layer norm launch");
  return WQ_OK;
}

int wq_rope_table(float* cs, int64_t n, int64_t rot) {
  clear_error();
  if (n < 0 || rot < 2 || rot % 2 != 0) return fail(WQ_ERR_SHAPE, "need n >= 0 and an even rot >= 2");
  if (n > kMaxRows || rot > kIntMax / 2 || (n > 0 && rot > kMaxOutputs / n)) return fail(WQ_ERR_SHAPE, "n * rot too large");
  if (n == 0) return WQ_OK;
  if (!cs) return fail(WQ_ERR_NULL, "cs must not be NULL");
  const int64_t half = rot / 2;
  for (int64_t i = 0; i < half; ++i) {
    const float inv = 1.0f / std::pow(10000.0f, static_cast<float>(2 * i) / static_cast<float>(rot));
    for (int64_t t = 0; t < n; ++t) {
      const float ang = static_cast<float>(t) * inv;
      cs[t * half + i] = std::cos(ang);
      cs[n * half + t * half + i] = std::sin(ang);
    }
  }
  return WQ_OK;
}

}  // extern "C"

namespace {

int qk_checked(float* qkv, const float* qn, const float* kn, const float* cs, int64_t n, int64_t heads, int64_t hd,
               int64_t rot, void* stream) {
  if (n < 0 || heads < 1 || hd < 1 || hd > 256) return fail(WQ_ERR_SHAPE, "need n >= 0, heads >= 1 and 1 <= hd <= 256");
  if (rot < 0 || rot > hd || rot % 2 != 0) return fail(WQ_ERR_SHAPE, "rot must be even and in [0, hd], got %lld", (long long)rot);
  if (n > (int64_t(1) << 22) || heads > (int64_t(1) << 20) || n * heads * hd * 3 > kMaxOutputs)
    return fail(WQ_ERR_SHAPE, "n, heads or n * 3 * heads * hd too large");
  if ((qn == nullptr) != (kn == nullptr)) return fail(WQ_ERR_NULL, "give both qn and kn, or neither");
  if (n == 0) return WQ_OK;
  if (!qkv || (rot > 0 && !cs)) return fail(WQ_ERR_NULL, "qkv (and cs when rot > 0) must not be NULL");
  if (!aligned(qkv, 4) || (qn && !aligned(qn, 4)) || (kn && !aligned(kn, 4)) || (cs && !aligned(cs, 4)))
    return fail(WQ_ERR_ALIGN, "qkv, qn, kn and cs must be 4-byte aligned");
  const int64_t bytes = n * 3 * heads * hd * 4;
  if (overlap(qkv, bytes, qn, 2 * hd * 4) || overlap(qkv, bytes, kn, 2 * hd * 4) || overlap(qkv, bytes, cs, n * rot * 4))
    return fail(WQ_ERR_ALIAS, "qn, kn or cs overlaps qkv");
  hipError_t e = wq::launch_qk_norm_rope(qkv, qn, kn, cs, static_cast<int>(n), static_cast<int>(heads),
                                         static_cast<int>(hd), static_cast<int>(rot), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "q/k norm launch");
  return WQ_OK;
}

bool attention_sizes_ok(int64_t n, int64_t heads, int64_t hd) {
  // heads is a grid dimension of the pack kernel (at most 65535); 4096 is far beyond any model.
  return n >= 0 && n <= (int64_t(1) << 22) && heads >= 1 && heads <= 4096 && hd >= 1 && hd <= 128 &&
         n * heads * hd * 3 <= kMaxOutputs;
}

int attention_checked(const float* qkv, const int32_t* valid, float* o, void* ws, int64_t ws_bytes, int64_t n,
                      int64_t heads, int64_t hd, float scale, void* stream) {
  if (!attention_sizes_ok(n, heads, hd))
    return fail(WQ_ERR_SHAPE, "need 0 <= n <= 2^22, 1 <= heads <= 4096, 1 <= hd <= 128 (n = %lld, heads = %lld, hd = %lld)",
                (long long)n, (long long)heads, (long long)hd);
  if (!std::isfinite(scale)) return fail(WQ_ERR_FLAGS, "scale must be finite");
  if (n == 0) return WQ_OK;
  if (!qkv || !valid || !o || !ws) return fail(WQ_ERR_NULL, "qkv, valid, o and workspace must not be NULL");
  if (!aligned(qkv, 4) || !aligned(valid, 4) || !aligned(o, 4) || !aligned(ws, 256))
    return fail(WQ_ERR_ALIGN, "qkv, valid and o must be 4-byte aligned, the workspace 256-byte aligned");
  const int64_t need = static_cast<int64_t>(wq::attention_workspace_bytes(n, heads, hd));
  if (ws_bytes < need)
    return fail(WQ_ERR_SHAPE, "the workspace holds %lld bytes, %lld needed", (long long)ws_bytes, (long long)need);
  const int64_t obytes = n * heads * hd * 4;
  if (overlap(o, obytes, qkv, 3 * obytes) || overlap(o, obytes, valid, n * 4) || overlap(o, obytes, ws, need) ||
      overlap(ws, need, qkv, 3 * obytes) || overlap(ws, need, valid, n * 4))
    return fail(WQ_ERR_ALIAS, "o or the workspace overlaps qkv, valid or each other");
  hipError_t e = wq::launch_attention(qkv, valid, o, ws, static_cast<int>(n), static_cast<int>(heads),
                                      static_cast<int>(hd), scale, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return WQ_OK;
}

// Layout of wq_encoder_layer's workspace: a [n][d], qkv [n][3d], att [n][d], f [n][inter], then
// the attention workspace; each part starts on a 256-byte boundary.
struct EncoderWs {
  int64_t a, qkv, att, f, attn, total;
};

EncoderWs encoder_ws(int64_t n, int64_t d, int64_t heads, int64_t inter) {
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  EncoderWs w{};
  w.a = 0;
  w.qkv = w.a + up(n * d * 4);
  w.att = w.qkv + up(n * 3 * d * 4);
  w.f = w.att + up(n * d * 4);
  w.attn = w.f + up(n * inter * 4);
  w.total = w.attn + static_cast<int64_t>(wq::attention_workspace_bytes(n, heads, d / heads));
  return w;
}

bool encoder_sizes_ok(int64_t n, int64_t d, int64_t heads, int64_t inter) {
  return n >= 0 && n <= (int64_t(1) << 22) && d >= 32 && d % 32 == 0 && d <= kIntMax / 4 && inter >= 32 &&
         inter % 32 == 0 && inter <= kIntMax / 4 && heads >= 1 && d % heads == 0 && d / heads <= 128 &&
         n * 3 * d <= kMaxOutputs && n * inter <= kMaxOutputs;
}

}  // namespace

extern "C" {

int wq_qk_norm_rope(float* qkv, const float* qn, const float* kn, const float* cs, int64_t n, int64_t heads,
                    int64_t hd, int64_t rot, void* stream) {
  clear_error();
  return qk_checked(qkv, qn, kn, cs, n, heads, hd, rot, stream);
}

int64_t wq_attention_workspace_bytes(int64_t n, int64_t heads, int64_t hd) {
  if (!attention_sizes_ok(n, heads, hd)) return -1;
  return static_cast<int64_t>(wq::attention_workspace_bytes(n, heads, hd));
}

int wq_attention(const float* qkv, const int32_t* valid, float* o, void* workspace, int64_t workspace_bytes,
                 int64_t n, int64_t heads, int64_t hd, float scale, void* stream) {
  clear_error();
  return attention_checked(qkv, valid, o, workspace, workspace_bytes, n, heads, hd, scale, stream);
}

int64_t wq_encoder_workspace_bytes(int64_t n, int64_t d, int64_t heads, int64_t inter) {
  if (!encoder_sizes_ok(n, d, heads, inter)) return -1;
  return encoder_ws(n, d, heads, inter).total;
}

int wq_encoder_layer(const wq_encoder_layer_t* l, int wtype, float* h, const int32_t* valid, const float* cs,
                     void* workspace, int64_t workspace_bytes, int64_t n, int64_t d, int64_t heads, int64_t rot,
                     int64_t inter, int path, void* stream) {
  clear_error();
  if (!encoder_sizes_ok(n, d, heads, inter))
    return fail(WQ_ERR_SHAPE,
                "need 0 <= n <= 2^22, d and inter positive multiples of 32, d %% heads == 0 and d / heads <= 128");
  const int64_t hd = d / heads;
  if (rot < 0 || rot > hd || rot % 2 != 0) return fail(WQ_ERR_SHAPE, "rot must be even and in [0, hd]");
  if (path != WQ_PATH_AUTO && path != WQ_PATH_MFMA && path != WQ_PATH_MFMA_F32)
    return fail(WQ_ERR_SHAPE, "path must be WQ_PATH_AUTO, WQ_PATH_MFMA or WQ_PATH_MFMA_F32");
  if (int r = check_wtype(wtype)) return r;
  if (!l) return fail(WQ_ERR_NULL, "layer must not be NULL");
  if (!l->ln1 || !l->qkv_w || !l->out_w || !l->out_b || !l->ln2 || !l->fc1_w || !l->fc1_b || !l->fc2_w || !l->fc2_b)
    return fail(WQ_ERR_NULL, "every layer weight except qkv_b, qn and kn must be given");
  if ((l->qn == nullptr) != (l->kn == nullptr)) return fail(WQ_ERR_NULL, "give both qn and kn, or neither");
  if (n == 0) return WQ_OK;
  if (!h || !valid || !workspace || (rot > 0 && !cs)) return fail(WQ_ERR_NULL, "h, valid, workspace (and cs) must not be NULL");
  if (!aligned(h, 16) || !aligned(workspace, 256))
    return fail(WQ_ERR_ALIGN, "h must be 16-byte aligned and the workspace 256-byte aligned");
  if (!aligned(valid, 4) || (cs && !aligned(cs, 4)) || (l->qn && !aligned(l->qn, 4)) || (l->kn && !aligned(l->kn, 4)))
    return fail(WQ_ERR_ALIGN, "valid, cs, qn and kn must be 4-byte aligned");
  const EncoderWs w = encoder_ws(n, d, heads, inter);
  if (workspace_bytes < w.total)
    return fail(WQ_ERR_SHAPE, "the workspace holds %lld bytes, %lld needed", (long long)workspace_bytes, (long long)w.total);
  if (overlap(h, n * d * 4, workspace, w.total)) return fail(WQ_ERR_ALIAS, "h overlaps the workspace");
  uint8_t* base = static_cast<uint8_t*>(workspace);
  float* a = reinterpret_cast<float*>(base + w.a);
  float* qkv = reinterpret_cast<float*>(base + w.qkv);
  float* att = reinterpret_cast<float*>(base + w.att);
  float* f = reinterpret_cast<float*>(base + w.f);
  void* attn_ws = base + w.attn;
  const float scale = 1.0f / std::sqrt(static_cast<float>(hd));
  // With bf16 weights on the bf16 matrix cores each product rounds its input to bf16 as it reads
  // it, so the LayerNorms, the attention and the MLP's first product hand their outputs over in
  // bf16, rounded the same way: half the bytes, and the block's output is bit-identical. The
  // f32-accurate path, the matvec path (n <= 16) and the other weight types keep f32 hand-offs.
  const int gpath = path == WQ_PATH_AUTO ? (n <= WQ_MATVEC_MAX_N ? WQ_PATH_MATVEC : WQ_PATH_MFMA) : path;
  // The bf16 products address their operands with 32-bit byte offsets (checked again by their
  // launcher): every bf16 activation (n x d, n x inter) and weight under 4 GiB.
  const bool b16 = wtype == WQ_W_BF16 && gpath == WQ_PATH_MFMA && d % 64 == 0 && inter % 64 == 0 &&
                   n * std::max(d, inter) * 2 < (int64_t(1) << 32) && 3 * d * d * 2 < (int64_t(1) << 32) &&
                   inter * d * 2 < (int64_t(1) << 32);
  // Every step's checks run here, before the first launch, so a refused call leaves h as it was
  // (only a launch that fails returns with h partly updated). The steps write h and the
  // workspace; nothing they read may lie there.
  const int64_t hbytes = n * d * 4;
  auto outside = [&](const void* p, int64_t bytes) {
    return !overlap(p, bytes, h, hbytes) && !overlap(p, bytes, workspace, w.total);
  };
  const float* vecs[] = {l->ln1, l->ln2, l->qkv_b, l->qn, l->kn, l->out_b, l->fc1_b, l->fc2_b};
  const int64_t vbytes[] = {2 * d * 4, 2 * d * 4, 3 * d * 4, 2 * hd * 4, 2 * hd * 4, d * 4, inter * 4, d * 4};
  for (int i = 0; i < 8; ++i) {
    if (vecs[i] && !aligned(vecs[i], 4)) return fail(WQ_ERR_ALIGN, "the layer's vectors must be 4-byte aligned");
    if (!outside(vecs[i], vbytes[i])) return fail(WQ_ERR_ALIAS, "a layer vector overlaps h or the workspace");
  }
  const void* mats[] = {l->qkv_w, l->out_w, l->fc1_w, l->fc2_w};
  const int64_t mbytes[] = {wq_weight_bytes(wtype, 3 * d, d), wq_weight_bytes(wtype, d, d),
                            wq_weight_bytes(wtype, inter, d), wq_weight_bytes(wtype, d, inter)};
  for (int i = 0; i < 4; ++i)
    if (!outside(mats[i], mbytes[i])) return fail(WQ_ERR_ALIAS, "a layer weight overlaps h or the workspace");
  if (!outside(valid, n * 4) || (rot > 0 && !outside(cs, n * rot * 4)))
    return fail(WQ_ERR_ALIAS, "valid or cs overlaps h or the workspace");
  const int io_in = b16 ? 1 : 0;
  int r;
  if ((r = gemm_checked(a, l->qkv_w, wtype, l->qkv_b, l->qkv_b ? WQ_BIAS : 0u, 1.0f, qkv, n, 3 * d, d, 0, gpath, stream,
                        io_in, true)) ||
      (r = gemm_checked(att, l->out_w, wtype, l->out_b, WQ_BIAS | WQ_RESIDUAL, 1.0f, h, n, d, d, 0, gpath, stream, io_in,
                        true)) ||
      (r = gemm_checked(a, l->fc1_w, wtype, l->fc1_b, WQ_BIAS | WQ_GELU, 1.0f, f, n, inter, d, 0, gpath, stream,
                        b16 ? 3 : 0, true)) ||
      (r = gemm_checked(f, l->fc2_w, wtype, l->fc2_b, WQ_BIAS | WQ_RESIDUAL, 1.0f, h, n, d, inter, 0, gpath, stream,
                        io_in, true)))
    return r;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto norm = [&](const float* wb) -> int {
    if (!b16) return wq_layer_norm(h, wb, a, n, d, stream);
    clear_error();
    hipError_t e = wq::launch_layer_norm_bf16(h, wb, reinterpret_cast<uint16_t*>(a), static_cast<int>(n),
                                               static_cast<int>(d), hs);
    return e == hipSuccess ? WQ_OK : hip_fail(e, "LayerNorm launch");
  };
  if ((r = norm(l->ln1))) return r;
  if ((r = gemm_checked(a, l->qkv_w, wtype, l->qkv_b, l->qkv_b ? WQ_BIAS : 0u, 1.0f, qkv, n, 3 * d, d, 0, gpath, stream,
                        io_in)))
    return r;
  // The q/k norm + rotation runs fused with the attention's pack: k goes to the workspace in bf16
  // only (the f32 rows are not needed after), q is rewritten in place as wq_qk_norm_rope would.
  clear_error();
  hipError_t he = wq::launch_qk_attention(qkv, l->qn, l->kn, cs, valid, att, attn_ws, static_cast<int>(n),
                                          static_cast<int>(heads), static_cast<int>(hd), static_cast<int>(rot), scale,
                                          hs, b16 ? 1 : 0);
  if (he != hipSuccess) return hip_fail(he, "q/k norm + attention launch");
  if ((r = gemm_checked(att, l->out_w, wtype, l->out_b, WQ_BIAS | WQ_RESIDUAL, 1.0f, h, n, d, d, 0, gpath, stream,
                        io_in)))
    return r;
  if ((r = norm(l->ln2))) return r;
  if ((r = gemm_checked(a, l->fc1_w, wtype, l->fc1_b, WQ_BIAS | WQ_GELU, 1.0f, f, n, inter, d, 0, gpath, stream,
                        b16 ? 3 : 0)))
    return r;
  return gemm_checked(f, l->fc2_w, wtype, l->fc2_b, WQ_BIAS | WQ_RESIDUAL, 1.0f, h, n, d, inter, 0, gpath, stream,
                      io_in);
}

const char* wq_last_error(void) { return g_err; }

const char* wq_version(void) { return "wq 0.1.0 (gfx950)"; }

}  // extern "C"
