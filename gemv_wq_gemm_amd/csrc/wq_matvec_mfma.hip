// Matrix-core matvec for 2..16 tokens per pass and the MoE matvec, with f32 accuracy.
//
// Same contract as the other matvec kernels: y[t][j] = epilogue(sum_k x[t][k] w[j][k]) for the
// plain layer (cortiq-engine src/gpu_wgpu/nemotron_audio.rs `ae_gemm`/`ae_put`; wavo
// src/gpu/mod.rs `Pass::gemv`) and y[s][j] = sum_k W[ids[s]][j][k] x[s / top_k][k] for MoE slots
// (hanzo-ml src/wgpu_backend.rs `moe_matvec_gpu`), for Q8_0 and Q4_0 weights.
//
// Why matrix cores: with f32 FMAs every weight costs one instruction per token, so a few tokens
// (or a MoE expert's routed tokens) make the kernel bound by the vector ALU, not by HBM. Here each
// weight is decoded once and v_mfma_f32_16x16x32_bf16 applies it to up to 16 tokens.
//
// Exactness:
//  * Each activation is split into three bf16 parts, x = x1 + x2 + x3, with x1 = bf16(x),
//    x2 = bf16(x - x1), x3 = bf16(x - x1 - x2), all rounded to nearest even. Both differences are
//    exact in f32, and the last part holds the at most 8 bits left, so the three parts add up to x
//    exactly (outside the bottom of the exponent range).
//  * The integer quants q (Q8_0) and q - 8 (Q4_0, taken as (q - 8) / 16 and scaled by 16 d) are
//    exact in bf16, and products of two bf16 values are exact in f32.
//  * One 32-element block is one MFMA's k: three chained MFMAs (one per activation part, sharing
//    the decoded weights) sum the block's products into a fresh 16x16 f32 tile, which the block's
//    scale then multiplies and adds to the running sum in f32. So only f32 additions round: the
//    products of a block, 16 blocks per wave, and 8 waves -- well inside 1e-5 * sum |x w|.
//
// Layout of the work (gfx950, wave64):
//  * A workgroup has k/512 waves; wave w owns the k-slice [512 w, 512 w + 512), i.e. 16 blocks of
//    every row. MFMA roles: A = activations (16 token rows x 32 k), B = weights (32 k x 16 weight
//    rows), D[t][j] in lane 16 (t / 4) + j, value t % 4.
//  * Lane l = 16 o + j: weight row j of the tile and k-octet o of each block (elements 8o..8o+7);
//    as A it holds token l % 16 at the same octet. Its three activation parts for the 16 blocks of
//    its slice (192 VGPRs) are built once per group of tokens and reused for every tile.
//  * A tile is 16 consecutive weight rows, streamed by the workgroup into a ring of NSTAGE LDS
//    slots with direct-to-LDS loads (each wave a share of the rows, 1024 bytes per load, the last
//    load of a row on the lanes with bytes left), NSTAGE-1 tiles ahead; one barrier per tile
//    publishes it. Rows sit at a stride of their length + 16 bytes, so the 16 rows one operand
//    read touches spread over the LDS banks (at most two lanes of a half-wave per bank).
//  * Each wave writes its 16x16 partial sums to LDS; after the next tile's barrier the workgroup
//    adds the k-slices in wave order, applies the epilogue and stores. An epilogue that reads
//    memory (bias, residual) would make the compiler wait for every ring load in flight, so such
//    launches park the sums in LDS and finish them after the last tile.
//  * MoE: blockIdx.y is the expert; a ballot over the ids picks its slots, 16 per pass, so each
//    touched expert's rows stream once per 16 of its slots. One extra grid row writes NaN for
//    slots whose id is out of range.
#include <hip/hip_runtime.h>

#include "wq_decode.hpp"
#include "wq_internal.hpp"
#include "wq_lds_dma.hpp"

namespace wq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 16;    // weight rows per tile: the MFMA's N
constexpr int kSliceBlocks = 16;  // blocks per wave: 512 of k
constexpr int kMaxWaves = 8;      // k <= 4096
constexpr int kTokens = 16;       // slots per pass: the MFMA's M
constexpr int kParkTiles = 4;     // tiles whose sums a memory-reading epilogue parks in LDS

// bf16 bit patterns of two f32 values that bf16 holds exactly, packed low | high << 16.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// (q - 8) / 16 of the Q4_0 nibble in byte b of a word already XOR-ed with 0x88888888 (and shifted
// so the wanted nibbles are the low ones of each byte).
__device__ __forceinline__ float q4_byte(uint32_t word, int b) {
  return __builtin_amdgcn_cvt_off_f32_i4(b == 0 ? word : (word >> (8 * b)) & 0xFFu);
}

// The 8 weights of k-octet o of the block at LDS byte offset `off`, as MFMA B operand, and the
// factor that scales their products.
template <int WT>
__device__ __forceinline__ bf16x8 decode_octet(const uint8_t* lds, int off, int o, float& scale) {
  const float d = f16_to_f32(*reinterpret_cast<const uint16_t*>(lds + off));
  const int qo = off + 2 + (WT == kQ8_0 ? 8 * o : 8 * (o & 1));
  const uint32_t sh = static_cast<uint32_t>(qo) & 3u;
  const uint32_t* a = reinterpret_cast<const uint32_t*>(lds) + (qo >> 2);
  const uint32_t d0 = a[0], d1 = a[1], d2 = a[2];
  const uint32_t q0 = realign(d1, d0, sh), q1 = realign(d2, d1, sh);
  uint4 u;
  if constexpr (WT == kQ8_0) {
    u.x = bf16_pair(q8_at(q0, 0), q8_at(q0, 1));
    u.y = bf16_pair(q8_at(q0, 2), q8_at(q0, 3));
    u.z = bf16_pair(q8_at(q1, 0), q8_at(q1, 1));
    u.w = bf16_pair(q8_at(q1, 2), q8_at(q1, 3));
    scale = d;
  } else {
    // Octets 0, 1 are the low nibbles of bytes 0-7, 8-15; octets 2, 3 their high nibbles.
    const uint32_t s4 = 4u * static_cast<uint32_t>(o >> 1);
    const uint32_t x0 = (q0 ^ 0x88888888u) >> s4, x1 = (q1 ^ 0x88888888u) >> s4;
    u.x = bf16_pair(q4_byte(x0, 0), q4_byte(x0, 1));
    u.y = bf16_pair(q4_byte(x0, 2), q4_byte(x0, 3));
    u.z = bf16_pair(q4_byte(x1, 0), q4_byte(x1, 1));
    u.w = bf16_pair(q4_byte(x1, 2), q4_byte(x1, 3));
    scale = 16.f * d;
  }
  return __builtin_bit_cast(bf16x8, u);
}

// Three bf16 parts of 8 activations (see the exactness note above).
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8& p1, bf16x8& p2, bf16x8& p3) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h1 = static_cast<__bf16>(x[i]);
    const float r1 = x[i] - static_cast<float>(h1);
    const __bf16 h2 = static_cast<__bf16>(r1);
    const float r2 = r1 - static_cast<float>(h2);
    p1[i] = h1;
    p2[i] = h2;
    p3[i] = static_cast<__bf16>(r2);
  }
}

template <int WT, int NSTAGE>
__global__ __launch_bounds__(64 * kMaxWaves) void matvec_mfma_kernel(MatvecParams p, int tiles_per_wg) {
  constexpr int BB = block_bytes(WT);
  // A row sits in LDS at a stride of its byte length + 16: row strides that are multiples of
  // 128 bytes would put the 16 rows an MFMA operand reads at once into one LDS bank.
  constexpr int kMaxRowBytes = kMaxWaves * kSliceBlocks * BB;
  constexpr int kSlotBytes = kTileRows * (kMaxRowBytes + 16);
  // Loads per wave per tile, at least (rows per wave x loads per row, over the supported k).
  constexpr int kMinPerWave = WT == kQ8_0 ? 8 : 4;
  static_assert(NSTAGE >= 2 && 2 * kMinPerWave * (NSTAGE - 2) < 64, "vmcnt range");

  __shared__ __attribute__((aligned(16))) uint8_t ring[NSTAGE * kSlotBytes];
  __shared__ float part[2][kMaxWaves * kTileRows * kTokens];  // [buffer][wave][token][row]
  __shared__ float park[kParkTiles * kTileRows * kTokens];     // [tile][token][row]
  __shared__ int slot_lds[kTokens];                            // slot of each token row

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int e = blockIdx.y;
  const bool moe = p.ids != nullptr;
  const int ntiles = (p.m + kTileRows - 1) / kTileRows;
  const int t_begin = blockIdx.x * tiles_per_wg;
  const int t_end = min(ntiles, t_begin + tiles_per_wg);
  if (t_begin >= ntiles) return;  // workgroup-uniform

  if (moe && e == p.n_exp) {
    // Slots routed outside the bank: their outputs in this run of rows become NaN.
    for (int win = 0; win < p.n_slots; win += 64) {
      const int s = win + lane;
      int id = 0;
      if (s < p.n_slots) id = p.ids[s];
      uint64_t bad = __ballot(s < p.n_slots && (id < 0 || id >= p.n_exp));
      while (bad) {
        const int slot = win + __builtin_ctzll(bad);
        bad &= bad - 1;
        for (int row = t_begin * kTileRows + threadIdx.x; row < min(p.m, t_end * kTileRows); row += blockDim.x)
          p.y[static_cast<long long>(slot) * p.m + row] = __builtin_nanf("");
      }
    }
    return;
  }

  const bool parked = !moe && (p.flags & 5u) != 0;
  const uint8_t* wexp = p.w + static_cast<long long>(e) * p.expert_bytes;
  const uint32_t ring_addr = lds_address(ring);
  const int rowbytes = static_cast<int>(p.rowbytes);
  const int stride = rowbytes + 16;
  const int per_row = (rowbytes + 1023) / 1024;  // 1024-byte loads per row, the last one partial
  // This wave's rows of every tile.
  const int r0 = wave * kTileRows / nw;
  const int r1 = (wave + 1) * kTileRows / nw;

  auto issue = [&](int tile) {
    const int row0 = tile * kTileRows;
    const uint8_t* base = wexp + static_cast<long long>(row0) * p.rowbytes;
    const uint32_t dst = ring_addr + static_cast<uint32_t>((tile % NSTAGE) * kSlotBytes);
    for (int r = r0; r < r1; ++r) {
      const int rr = min(r, p.m - 1 - row0);  // rows past the end of W re-read its last row
      for (int c = 0; c < per_row; ++c) {
        const int b = c * 1024 + lane * 16;
        if (b < rowbytes)  // the last load of a row runs on the lanes that have bytes left
          load_lds16(base, static_cast<uint32_t>(rr * rowbytes + b), dst + r * stride + c * 1024);
      }
    }
  };

  const int j = lane & 15;  // weight row in the tile (B, D column); token row as A
  const int o = lane >> 4;  // k-octet of each block; D rows 4o .. 4o+3
  const int row_off = j * stride + wave * kSliceBlocks * BB;

  // Finishes tile `tile` from the wave partials in part[buf]: the sums of all waves, in wave order.
  auto finish = [&](int tile, int buf) {
    for (int i = threadIdx.x; i < kTileRows * kTokens; i += blockDim.x) {
      const int t = i >> 4;
      const int r = i & 15;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kMaxWaves; ++w)
        if (w < nw) v += part[buf][w * kTileRows * kTokens + i];
      if (parked) {
        park[(tile - t_begin) * kTileRows * kTokens + i] = v;
      } else {
        const int row = tile * kTileRows + r;
        const int slot = slot_lds[t];
        if (row < p.m && slot >= 0) {
          if (!moe && (p.flags & 2u)) v = gelu_erf(v);
          p.y[static_cast<long long>(slot) * p.m + row] = v;
        }
      }
    }
  };

  for (int win = 0; win < p.n_slots; win += 64) {
    uint64_t mask;
    if (moe) {
      const int s = win + lane;
      int id = -1;
      if (s < p.n_slots) id = p.ids[s];
      mask = __ballot(id == e);
    } else {
      const int left = p.n_slots - win;
      mask = left >= 64 ? ~0ull : ((1ull << left) - 1ull);
    }
    while (mask) {
      int slot_of[kTokens];
#pragma unroll
      for (int t = 0; t < kTokens; ++t) {
        if (mask) {
          slot_of[t] = win + __builtin_ctzll(mask);
          mask &= mask - 1;
        } else {
          slot_of[t] = -1;
        }
      }
      int my_slot = -1;
#pragma unroll
      for (int t = 0; t < kTokens; ++t)
        if (t == j) my_slot = slot_of[t];
      if (threadIdx.x < kTokens) slot_lds[threadIdx.x] = my_slot;  // read after the next barrier

      // Prologue: the first NSTAGE-1 tiles in flight, then the activation parts.
#pragma unroll
      for (int s = 0; s < NSTAGE - 1; ++s)
        if (t_begin + s < t_end) issue(t_begin + s);

      bf16x8 xa[3][kSliceBlocks];
      {
        const float* xs = my_slot >= 0 ? p.x + static_cast<long long>(my_slot / p.top_k) * p.k : nullptr;
#pragma unroll
        for (int bb = 0; bb < kSliceBlocks; ++bb) {
          float xv[8];
          if (xs) {
            const float4* xp = reinterpret_cast<const float4*>(xs + wave * 512 + bb * 32 + 8 * o);
            const float4 v0 = xp[0], v1 = xp[1];
            xv[0] = v0.x; xv[1] = v0.y; xv[2] = v0.z; xv[3] = v0.w;
            xv[4] = v1.x; xv[5] = v1.y; xv[6] = v1.z; xv[7] = v1.w;
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] = 0.f;
          }
          split3(xv, xa[0][bb], xa[1][bb], xa[2][bb]);
        }
      }

      for (int tile = t_begin; tile < t_end; ++tile) {
        wait_groups<kMinPerWave, NSTAGE - 2>(min(NSTAGE - 2, t_end - 1 - tile));
        __syncthreads();  // the tile is in; the slot of tile-1 and part[(tile-1)&1] are complete
        if (tile + NSTAGE - 1 < t_end) issue(tile + NSTAGE - 1);
        if (tile > t_begin) finish(tile - 1, (tile - 1) & 1);

        const int seg = (tile % NSTAGE) * kSlotBytes + row_off;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int bb = 0; bb < kSliceBlocks; ++bb) {
          float scale;
          const bf16x8 wb = decode_octet<WT>(ring, seg + bb * BB, o, scale);
          f32x4 blk = {0.f, 0.f, 0.f, 0.f};
          blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[0][bb], wb, blk, 0, 0, 0);
          blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[1][bb], wb, blk, 0, 0, 0);
          blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[2][bb], wb, blk, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(scale, blk[v], acc[v]);
        }
        float* pw = part[tile & 1] + wave * kTileRows * kTokens;
#pragma unroll
        for (int v = 0; v < 4; ++v) pw[(4 * o + v) * kTileRows + j] = acc[v];
      }
      __syncthreads();
      finish(t_end - 1, (t_end - 1) & 1);

      if (parked) {
        // Every ring load has landed (the last tile waited for all of them).
        __syncthreads();
        const int n = (t_end - t_begin) * kTileRows * kTokens;
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
          const int tl = i / (kTileRows * kTokens);
          const int t = (i >> 4) & (kTokens - 1);
          const int row = (t_begin + tl) * kTileRows + (i & 15);
          const int slot = slot_lds[t];
          if (row < p.m && slot >= 0) {
            float* yp = p.y + static_cast<long long>(slot) * p.m + row;
            float v = park[i];
            if (p.flags & 1u) v += p.bias[row];
            if (p.flags & 2u) v = gelu_erf(v);
            if (p.flags & 4u) v += *yp;
            *yp = v;
          }
        }
      }
      __syncthreads();  // part, park and the ring are reused by the next group of slots
    }
  }
}

int mfma_device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

template <int WT, int NSTAGE>
hipError_t launch_mfma(const MatvecParams& p, hipStream_t stream) {
  const int nw = p.k / 512;
  const int n_exp_rows = p.ids ? p.n_exp + 1 : 1;
  const int experts = p.ids ? p.n_exp : 1;
  const int ntiles = (p.m + kTileRows - 1) / kTileRows;
  auto kernel = matvec_mfma_kernel<WT, NSTAGE>;
  static int per_cu = 0;
  if (per_cu <= 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, 64 * kMaxWaves, 0) != hipSuccess || v <= 0) v = 1;
    per_cu = v;
  }
  int groups = per_cu * mfma_device_cus() / experts;
  if (groups < 1) groups = 1;
  if (groups > ntiles) groups = ntiles;
  int tpw = (ntiles + groups - 1) / groups;
  if (p.ids == nullptr && (p.flags & 5u) != 0 && tpw > kParkTiles) tpw = kParkTiles;
  dim3 grid((ntiles + tpw - 1) / tpw, n_exp_rows);
  hipLaunchKernelGGL(kernel, grid, dim3(64 * nw), 0, stream, p, tpw);
  return hipGetLastError();
}

}  // namespace

bool matvec_mfma_supports(int wtype, int k) {
  return (wtype == kQ8_0 || wtype == kQ4_0) && k % 512 == 0 && k >= 2048 && k <= 512 * kMaxWaves;
}

hipError_t launch_matvec_mfma(int wtype, const MatvecParams& p, hipStream_t stream) {
  if (!matvec_mfma_supports(wtype, p.k)) return hipErrorInvalidValue;
  if (wtype == kQ8_0) return launch_mfma<kQ8_0, 2>(p, stream);
  return launch_mfma<kQ4_0, 3>(p, stream);
}

}  // namespace wq
