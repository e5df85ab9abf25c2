// Device-side decoding of the three weight storage types.
//
// bf16  : a 16-bit pattern that is the upper half of an f32 (the weight-pair
//         unpack of `ae_gemm`, cortiq-engine src/gpu_wgpu/nemotron_audio.rs).
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

// Reads the block that starts `off` bytes after the 4-byte aligned `base`
// (off even), through the aligned dwords that cover exactly
// [off & ~3, off + block_bytes). `base` may point to global memory or LDS;
// keeping it a typed pointer (no integer round trip) keeps its address space.
template <int WT, typename Off>
__device__ __forceinline__ void read_block(const uint32_t* base, Off off, uint32_t* q, uint32_t* scale) {
  const uint32_t sh = static_cast<uint32_t>(off) & 3u;  // 0 or 2
  const uint32_t* a = base + (off >> 2);
  if constexpr (WT == 0) {
    // 64 bytes: 17 covering dwords when sh == 2, 16 when sh == 0.
    uint32_t d[17];
#pragma unroll
    for (int i = 0; i < 16; ++i) d[i] = a[i];
    d[16] = sh ? a[16] : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = realign(d[i + 1], d[i], sh);
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

__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}

}  // namespace wq
