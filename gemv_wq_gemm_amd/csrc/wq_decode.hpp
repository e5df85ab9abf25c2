// Device-side decoding of the three weight storage types.
//
// bf16  : a 16-bit pattern that is the upper half of an f32 (the weight-pair
//         unpack of `ae_gemm`, cortiq-engine src/gpu_wgpu/nemotron_audio.rs).
// f32, f16: IEEE values as stored (wavo src/gpu/mod.rs `Linear` GEMM types 0
//         and 1, copied as they are by `Gpu::upload_linear`).
// Q8_0  : 34-byte block = little-endian f16 scale d, then 32 int8 q; w = d*q
//         (wavo src/gpu/mod.rs `Gpu::upload_linear`; hanzo-ml src/wgpu_backend.rs
//         `matvec_q8_0_gpu`).
// Q4_0  : 18-byte block = little-endian f16 scale d, then 16 bytes; byte j holds
//         element j (low nibble) and element j+16 (high nibble); w = d*(q-8)
//         (hanzo-ml `matvec_q4_0_gpu`; GGML nibble order).
//
// Blocks start at any even byte address (34- and 18-byte blocks break 4-byte
// alignment), so readers fetch the aligned dwords that cover a block and
// realign them with v_alignbyte. An aligned dword that holds at least one
// byte of the buffer lies in the buffer's pages, so these reads never leave
// mapped memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// Bytes [sh, sh+4) of the 8-byte value hi:lo (sh in 0..3).
__device__ __forceinline__ uint32_t realign(uint32_t hi, uint32_t lo, uint32_t sh) {
  return __builtin_amdgcn_alignbyte(hi, lo, sh);
}

// int8 quant in byte b of a dword, as f32 (exact).
__device__ __forceinline__ float q8_at(uint32_t word, int b) {
  return static_cast<float>(static_cast<int8_t>(word >> (8 * b)));
}

// Q4_0 nibble `pos` (0..7) of a dword that was XOR-ed with 0x88888888, as the
// signed value q-8 in f32 (exact). XOR with 8 maps q to the 4-bit two's
// complement pattern of q-8.
__device__ __forceinline__ float q4_at(uint32_t word_x8, int pos) {
  return static_cast<float>(static_cast<int32_t>(word_x8 << (28 - 4 * pos)) >> 28);
}

__device__ __forceinline__ float bf16_lo(uint32_t word) { return __uint_as_float(word << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t word) { return __uint_as_float(word & 0xFFFF0000u); }

// One block read from memory whose address is only 2-byte aligned.
// `NW` dwords of payload (bf16: 16, Q8_0: 8, Q4_0: 4) come back aligned in q[],
// and the f16 scale bits in *scale (quantized types).
template <int WT>
struct BlockWords;

template <>
struct BlockWords<0> {
  static constexpr int NW = 16;
};
template <>
struct BlockWords<1> {
  static constexpr int NW = 8;
};
template <>
struct BlockWords<2> {
  static constexpr int NW = 4;
};
template <>
struct BlockWords<3> {
  static constexpr int NW = 32;
};
template <>
struct BlockWords<4> {
  static constexpr int NW = 16;
};

// Reads the block that starts `off` bytes after the 4-byte aligned `base`
// (off even), through the aligned dwords that cover exactly
// [off & ~3, off + block_bytes). `base` may point to global memory or LDS;
// keeping it a typed pointer (no integer round trip) keeps its address space.
template <int WT, typename Off>
__device__ __forceinline__ void read_block(const uint32_t* base, Off off, uint32_t* q, uint32_t* scale) {
  const uint32_t sh = static_cast<uint32_t>(off) & 3u;  // 0 or 2
  const uint32_t* a = base + (off >> 2);
  if constexpr (WT == 0 || WT == 3 || WT == 4) {
    // bf16 / f16 (64 bytes) or f32 (128 bytes), no scale: NW + 1 covering dwords when sh == 2,
    // NW when sh == 0.
    constexpr int NW = BlockWords<WT>::NW;
    uint32_t d[NW + 1];
#pragma unroll
    for (int i = 0; i < NW; ++i) d[i] = a[i];
    d[NW] = sh ? a[NW] : 0u;
#pragma unroll
    for (int i = 0; i < NW; ++i) q[i] = realign(d[i + 1], d[i], sh);
    *scale = 0;
  } else {
    constexpr int NW = BlockWords<WT>::NW;
    // scale at off, payload at off + 2; NW + 1 dwords cover [off - sh, off + 2 + 4 NW).
    uint32_t d[NW + 1];
#pragma unroll
    for (int i = 0; i <= NW; ++i) d[i] = a[i];
    *scale = (sh ? (d[0] >> 16) : d[0]) & 0xFFFFu;
#pragma unroll
    for (int i = 0; i < NW; ++i) q[i] = sh ? d[i + 1] : realign(d[i + 1], d[i], 2u);
  }
}

// Element e (0..31) of a block of a plain type (bf16 0, f32 3, f16 4) read by read_block, exact.
template <int WT>
__device__ __forceinline__ float plain_at(const uint32_t* q, int e) {
  if constexpr (WT == 3) return __uint_as_float(q[e]);
  const uint32_t h = (e & 1) ? q[e >> 1] >> 16 : q[e >> 1] & 0xFFFFu;
  if constexpr (WT == 4) return f16_to_f32(h);
  return __uint_as_float(h << 16);
}

// erf by Abramowitz & Stegun 7.1.26 (Hastings' rational approximation), branch-free:
//    erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2), t = 1 / (1 + p z),
// with an absolute error below 1.5e-7 in exact arithmetic. In f32 it stays within about 5.3e-7
// of the exact erf over the whole range (checked against it), the most near 0, where 1 - poly e
// cancels. GELU needs 1 + erf only to absolute accuracy: 0.5 v (1 + erf) moves by at most 0.5 |v|
// times that error, under 1.8e-7 of |v| + |GELU(v)|, inside the f32 rounding the epilogue's bounds
// allow. (A Maclaurin series below |z| = 0.5 kept erf's relative accuracy there as well; without it
// the MLP up projection of the encoder chain, 1500 x 4096 x 1024, went from 26.3-26.9 to
// 25.4-25.9 us.)
__device__ __forceinline__ float erf_as(float z) {
  const float a = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, a, 1.0f));
  float poly = 1.061405429f;
  poly = __builtin_fmaf(poly, t, -1.453152027f);
  poly = __builtin_fmaf(poly, t, 1.421413741f);
  poly = __builtin_fmaf(poly, t, -0.284496736f);
  poly = __builtin_fmaf(poly, t, 0.254829592f);
  poly *= t;
  // exp(-a^2) = 2^(-a^2 log2 e); v_exp_f32 is exact to about 1 ulp and flushes to 0 far out.
  const float e = __builtin_amdgcn_exp2f(-a * a * 1.4426950408889634f);
  return copysignf(__builtin_fmaf(-poly, e, 1.0f), z);
}

__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erf_as(v * 0.70710678118654752f));
}

// Epilogue flag bits (include/wq.h): bias 1, erf-GELU 2 and accumulate into the old output 4 are
// those of cortiq-engine `ae_put`; SiLU 8, ReLU 16 and tanh 32 are the other activations of wavo
// src/gpu/mod.rs `Epilogue`. The host lets at most one activation through.
constexpr unsigned kEpiBias = 1u, kEpiGelu = 2u, kEpiResidual = 4u, kEpiSilu = 8u, kEpiRelu = 16u, kEpiTanh = 32u;
constexpr unsigned kEpiAct = kEpiGelu | kEpiSilu | kEpiRelu | kEpiTanh;

// The activation `flags` selects (v itself when none): erf-GELU as above, SiLU v / (1 + e^-v)
// (ROCm's expf; for v far below 0 the quotient is -0), ReLU max(v, 0), ROCm's tanhf.
__device__ __forceinline__ float activation(float v, unsigned flags) {
  if (flags & kEpiGelu) return gelu_erf(v);
  if (flags & kEpiSilu) return v / (1.0f + expf(-v));
  if (flags & kEpiRelu) return fmaxf(v, 0.0f);
  if (flags & kEpiTanh) return tanhf(v);
  return v;
}

// The whole epilogue of one output: (+ bias) -> activation -> times alpha -> (+ old output).
// Dual outputs (wavo `Linear.dual`) call it a second time for output j < dual, with bias[m + j]
// and the old value at column m + j.
// `bias` and `old` are read only when their flags are set.
__device__ __forceinline__ float epilogue(float acc, unsigned flags, float alpha, const float* bias,
                                          const float* old) {
  float v = acc;
  if (flags & kEpiBias) v += *bias;
  v = alpha * activation(v, flags);
  if (flags & kEpiResidual) v += *old;
  return v;
}

}  // namespace wq
