// The plain streaming read that sets the floor a weight-streaming kernel is measured against:
// read `bytes` from HBM once, do nothing with them but fold them into one word per workgroup (so
// the loads cannot be dropped), and time that. A matvec or MoE call that streams the same bytes
// can be no faster than this, so achieved / floor ("fraction of the speed of light") separates
// what the kernel loses from what the memory system gives.
//
// Built as its own library (libwq_bench.so), loaded by the bench only; it is not part of the
// layer's ABI (include/wq.h).
//
// Design for gfx950: one workgroup per CU slot, 256 threads; each thread keeps 8 16-byte loads in
// flight (non-temporal, as the matvec kernels' weight loads), over a grid-stride loop of
// consecutive 4 KB pieces per wave, so every load instruction of a wave covers 1 KB of
// contiguous bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq_lds_dma.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ buf, long long n16,
                                                               uint32_t* __restrict__ out) {
  // Pieces of kThreads * kUnroll 16-byte chunks; chunk u of a piece is read by thread u % kThreads.
  const long long piece = static_cast<long long>(kThreads) * kUnroll;
  uint32_t acc = 0;
  for (long long base = static_cast<long long>(blockIdx.x) * piece; base < n16;
       base += static_cast<long long>(gridDim.x) * piece) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long i = base + static_cast<long long>(u) * kThreads + threadIdx.x;
      v[u] = i < n16 ? __builtin_nontemporal_load(buf + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // One word per workgroup (every thread's bits folded in), so no load is dead.
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < kThreads; ++t) r ^= red[t];
    out[blockIdx.x] = r;
  }
}

// The same read with direct-to-LDS loads (global_load_lds_dwordx4, non-temporal), the way the
// matvec kernels stream their weights: each wave keeps kInFlight 1 KB loads in flight into a
// private LDS ring and never touches the data, so nothing but the memory system sets the pace.
constexpr int kWaves = 4;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(64 * kWaves) void stream_read_lds_kernel(const uint8_t* __restrict__ buf, long long n1k,
                                                                   uint32_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kWaves * kInFlight * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t my_ring = wq::lds_address(ring) + wave * kInFlight * 1024;
  const long long waves = static_cast<long long>(gridDim.x) * kWaves;
  long long c = static_cast<long long>(blockIdx.x) * kWaves + wave;  // 1 KB chunk of this wave
  int slot = 0;
  for (; c < n1k; c += waves) {
    // The slot is reused once the load issued kInFlight loads ago has landed.
    wq::wait_vmcnt<kInFlight - 1>();
    const uint8_t* base = buf + c * 1024;
    wq::load_lds16<true>(base, static_cast<uint32_t>(lane * 16), my_ring + slot * 1024);
    slot = slot + 1 == kInFlight ? 0 : slot + 1;
  }
  wq::wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = reinterpret_cast<const uint32_t*>(ring)[0];
}

// The shader clock under load: every workgroup runs `iters` dependent FMAs per lane between two
// readings of the shader-clock counter (s_memtime) and of the constant-rate wall counter
// (s_memrealtime); the bench turns each workgroup's cycle and tick counts into a clock rate.
__global__ __launch_bounds__(kThreads) void clock_probe_kernel(int iters, float seed, unsigned long long* __restrict__ out,
                                                                float* __restrict__ sink) {
  const unsigned long long c0 = clock64();
  const unsigned long long w0 = wall_clock64();
  float a = seed + static_cast<float>(threadIdx.x);
  for (int i = 0; i < iters; ++i) a = __builtin_fmaf(a, 1.0000001f, 1e-7f);
  asm volatile("" ::"v"(a));  // the chain is done before the second reading
  const unsigned long long c1 = clock64();
  const unsigned long long w1 = wall_clock64();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = w1 - w0;
  }
  if (a == -1.f) sink[threadIdx.x] = a;  // never true for these inputs; keeps the chain live
}

}  // namespace

extern "C" {

// Runs the clock probe on `blocks` workgroups: out receives 2 * blocks counts (shader-clock
// cycles, wall-counter ticks per workgroup), sink 256 floats that stay unwritten.
int wq_bench_clock_probe(int iters, uint64_t* out, float* sink, int blocks, void* stream) {
  if (iters <= 0 || blocks <= 0 || !out || !sink) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters, 1.f,
                     reinterpret_cast<unsigned long long*>(out), sink);
  return static_cast<int>(hipGetLastError());
}

// Rates of the wall counter and the device's maximum shader clock, in kHz (0 if unknown).
int wq_bench_clock_rates(int* wall_khz, int* max_khz) {
  int dev = 0;
  *wall_khz = 0;
  *max_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) *wall_khz = 0;
  if (hipDeviceGetAttribute(max_khz, hipDeviceAttributeClockRate, dev) != hipSuccess) *max_khz = 0;
  return 0;
}

// The direct-to-LDS read of `bytes` (a multiple of 1024, buf 16-byte aligned); `blocks` workgroups.
int wq_bench_stream_read_lds(const void* buf, int64_t bytes, uint32_t* out, int blocks, void* stream) {
  if (bytes <= 0 || bytes % 1024 != 0 || blocks <= 0 || !buf || !out) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(stream_read_lds_kernel, dim3(blocks), dim3(64 * kWaves), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(buf), static_cast<long long>(bytes / 1024), out);
  return static_cast<int>(hipGetLastError());
}

// Reads `bytes` (a multiple of 16, buf 16-byte aligned) once; writes `blocks` words to out, where
// `blocks` is what wq_bench_stream_read_blocks returns. Returns 0 or the hipError_t of the launch.
int wq_bench_stream_read(const void* buf, int64_t bytes, uint32_t* out, int blocks, void* stream) {
  if (bytes <= 0 || bytes % 16 != 0 || blocks <= 0 || !buf || !out) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), static_cast<long long>(bytes / 16), out);
  return static_cast<int>(hipGetLastError());
}

// Workgroups of the read: `per_cu` resident per CU (at most 8 fit: 256 threads, 1 KB of LDS).
int wq_bench_stream_read_blocks(int per_cu) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256 * per_cu;
  return cus * per_cu;
}

}  // extern "C"
