// Matvec / small-n path (n <= 16) and the expert-major MoE matvec, all in f32.
//
// Contract: y[t][j] = epilogue(sum_k x[t][k] * w[j][k]) for the plain layer
// (cortiq-engine src/gpu_wgpu/nemotron_audio.rs, `ae_gemm` / `ae_put`;
// wavo src/gpu/mod.rs `Pass::gemv`, which keeps W unrounded), and
// y[s][j] = sum_k W[ids[s]][j][k] * x[s / top_k][k] for the MoE slots
// (hanzo-ml src/wgpu_backend.rs `moe_matvec_gpu`).
//
// Design for gfx950 (HBM-bound: every weight byte is read once per call):
//  * A wave owns RW consecutive weight rows. Each lane owns KB consecutive
//    32-element blocks of a k-chunk of 64*KB blocks, and holds the matching
//    activations of up to NTC tokens in VGPRs, reused for all RW rows.
//  * The bytes of a row's k-chunk are contiguous in memory; the wave copies
//    them with 16-byte loads (consecutive lanes, consecutive 16 bytes) into
//    a wave-private LDS region, then every lane reads its own blocks back.
//    This turns the 34- and 18-byte block stride into coalesced HBM traffic.
//  * Per block, each lane accumulates 32 products per token in f32, scales
//    the partial by d once, and adds it to the row total. The 64 lane totals
//    are summed by a butterfly across the wave. Worst-case rounding: a
//    32-term chain, a few block additions and a 6-level tree, all well inside
//    1e-5 * sum|x*w|.
//  * Tokens are taken NTC at a time; more tokens re-stream the rows (they
//    are then L2-resident). MoE workgroups are indexed by expert and find
//    their slots by a wave ballot over the ids, so an expert no token chose
//    costs no weight traffic.
#include <hip/hip_runtime.h>

#include "wq_decode.hpp"
#include "wq_internal.hpp"

namespace wq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Stop the compiler from moving LDS accesses across this point, and wait for
// this wave's outstanding LDS operations. LDS requests of one wave are served
// in order, so after this a lane sees what other lanes of its wave wrote.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int WT, int KB>
struct Geometry {
  static constexpr int BB = block_bytes(WT);
  static constexpr int kChunkBlocks = 64 * KB;
  static constexpr int kChunkBytes = kChunkBlocks * BB;
  // 16-byte pieces of a chunk that starts at any even offset inside a piece.
  static constexpr int kMaxPieces = (kChunkBytes + 15 + 15) / 16;
  static constexpr int kPiecesPerLane = (kMaxPieces + 63) / 64;
  // Staged row region: the pieces plus slack for the last block's covering dwords.
  static constexpr int kRowLds = kMaxPieces * 16 + 16;
};

template <int WT, int NTC, int KB, int RW>
__global__ __launch_bounds__(kThreads) void matvec_general_kernel(MatvecParams p) {
  using G = Geometry<WT, KB>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * RW * G::kRowLds];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int e = blockIdx.y;
  const int row0 = (blockIdx.x * kWaves + wave) * RW;
  if (row0 >= p.m) return;  // wave-uniform; the kernel has no workgroup barrier
  uint8_t* region = lds + wave * RW * G::kRowLds;
  const uint32_t* region32 = reinterpret_cast<const uint32_t*>(region);
  const bool moe = p.ids != nullptr;
  const int nb = p.k / 32;

  if (moe && e == p.n_exp) {
    // Slots routed outside the bank: their outputs become NaN.
    for (int win = 0; win < p.n_slots; win += 64) {
      const int s = win + lane;
      int id = 0;
      if (s < p.n_slots) id = p.ids[s];
      uint64_t bad = __ballot(s < p.n_slots && (id < 0 || id >= p.n_exp));
      while (bad) {
        const int slot = win + __builtin_ctzll(bad);
        bad &= bad - 1;
        if (lane < RW && row0 + lane < p.m)
          p.y[static_cast<long long>(slot) * p.m + row0 + lane] = __builtin_nanf("");
      }
    }
    return;
  }

  const uint8_t* wbase = p.w + static_cast<long long>(e) * p.expert_bytes;

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
      int slot[NTC];
#pragma unroll
      for (int t = 0; t < NTC; ++t) {
        if (mask) {
          slot[t] = win + __builtin_ctzll(mask);
          mask &= mask - 1;
        } else {
          slot[t] = -1;
        }
      }

      float acc[RW][NTC];
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < NTC; ++t) acc[r][t] = 0.f;

      for (int cb0 = 0; cb0 < nb; cb0 += G::kChunkBlocks) {
        const int cblocks = min(G::kChunkBlocks, nb - cb0);
        const int lb0 = lane * KB;

        // Stage this chunk of each row: issue every load before any LDS write.
        uint4 st[RW][G::kPiecesPerLane];
        int shift[RW];
        int pieces[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          const int row = row0 + r;
          const uint8_t* g = wbase + static_cast<long long>(row) * p.rowbytes +
                             static_cast<long long>(cb0) * G::BB;
          shift[r] = static_cast<int>(reinterpret_cast<uintptr_t>(g) & 15u);
          pieces[r] = row < p.m ? (shift[r] + cblocks * G::BB + 15) / 16 : 0;
          const uint4* src = reinterpret_cast<const uint4*>(g - shift[r]);
#pragma unroll
          for (int i = 0; i < G::kPiecesPerLane; ++i) {
            const int pc = lane + 64 * i;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (pc < pieces[r]) v = src[pc];
            st[r][i] = v;
          }
        }

        // Activations of this lane's blocks, for every token of the pass.
        float xr[NTC][KB * 32];
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
          const int tok = slot[t] >= 0 ? slot[t] / p.top_k : 0;
          const float4* xp = reinterpret_cast<const float4*>(
              p.x + static_cast<long long>(tok) * p.k + static_cast<long long>(cb0 + lb0) * 32);
#pragma unroll
          for (int j = 0; j < KB; ++j) {
            const bool ok = slot[t] >= 0 && lb0 + j < cblocks;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              float4 v = ok ? xp[j * 8 + i] : make_float4(0.f, 0.f, 0.f, 0.f);
              xr[t][j * 32 + 4 * i + 0] = v.x;
              xr[t][j * 32 + 4 * i + 1] = v.y;
              xr[t][j * 32 + 4 * i + 2] = v.z;
              xr[t][j * 32 + 4 * i + 3] = v.w;
            }
          }
        }

#pragma unroll
        for (int r = 0; r < RW; ++r) {
          uint4* dst = reinterpret_cast<uint4*>(region + r * G::kRowLds);
#pragma unroll
          for (int i = 0; i < G::kPiecesPerLane; ++i) {
            const int pc = lane + 64 * i;
            if (pc < pieces[r]) dst[pc] = st[r][i];
          }
        }
        wave_lds_sync();

#pragma unroll
        for (int r = 0; r < RW; ++r) {
#pragma unroll
          for (int j = 0; j < KB; ++j) {
            if (lb0 + j < cblocks) {
              uint32_t q[BlockWords<WT>::NW];
              uint32_t sbits;
              read_block<WT>(region32 + r * (G::kRowLds / 4), shift[r] + (lb0 + j) * G::BB, q, &sbits);
              float part[NTC];
#pragma unroll
              for (int t = 0; t < NTC; ++t) part[t] = 0.f;
              if constexpr (plain_type(WT)) {
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                  const float wv = plain_at<WT>(q, i);
#pragma unroll
                  for (int t = 0; t < NTC; ++t) part[t] = __builtin_fmaf(xr[t][j * 32 + i], wv, part[t]);
                }
#pragma unroll
                for (int t = 0; t < NTC; ++t) acc[r][t] += part[t];
              } else if constexpr (WT == kQ8_0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
#pragma unroll
                  for (int b = 0; b < 4; ++b) {
                    const float wv = q8_at(q[i], b);
#pragma unroll
                    for (int t = 0; t < NTC; ++t)
                      part[t] = __builtin_fmaf(xr[t][j * 32 + 4 * i + b], wv, part[t]);
                  }
                }
                const float d = f16_to_f32(sbits);
#pragma unroll
                for (int t = 0; t < NTC; ++t) acc[r][t] = __builtin_fmaf(d, part[t], acc[r][t]);
              } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const uint32_t qx = q[i] ^ 0x88888888u;
#pragma unroll
                  for (int b = 0; b < 4; ++b) {
                    const float lo = q4_at(qx, 2 * b), hi = q4_at(qx, 2 * b + 1);
#pragma unroll
                    for (int t = 0; t < NTC; ++t) {
                      part[t] = __builtin_fmaf(xr[t][j * 32 + 4 * i + b], lo, part[t]);
                      part[t] = __builtin_fmaf(xr[t][j * 32 + 16 + 4 * i + b], hi, part[t]);
                    }
                  }
                }
                const float d = f16_to_f32(sbits);
#pragma unroll
                for (int t = 0; t < NTC; ++t) acc[r][t] = __builtin_fmaf(d, part[t], acc[r][t]);
              }
            }
          }
        }
        wave_lds_sync();  // every lane has read the region before the next chunk overwrites it
      }

      // Sum over the wave, then one lane per (row, token) finishes the output.
#pragma unroll
      for (int r = 0; r < RW; ++r) {
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
          const float v = wave_sum(acc[r][t]);
          const int row = row0 + r;
          if (lane == r * NTC + t && slot[t] >= 0 && row < p.m) {
            float* yp = p.y + static_cast<long long>(slot[t]) * p.ystride + row;
            float o = v;
            if (!moe) {
              o = epilogue(o, p.flags, p.alpha, p.bias + row, yp);
              if (p.dual > 0 && row < p.dual)
                yp[p.m] = epilogue(v, p.flags, p.alpha, p.bias + p.m + row, yp + p.m);
            }
            *yp = o;
          }
        }
      }
    }
  }
}

template <int WT, int NTC, int KB, int RW>
hipError_t launch_variant(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  const int rows_per_wg = kWaves * RW;
  dim3 grid((p.m + rows_per_wg - 1) / rows_per_wg, n_exp_rows);
  hipLaunchKernelGGL((matvec_general_kernel<WT, NTC, KB, RW>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int WT, int NTC, int KB>
hipError_t launch_rw(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  // Enough waves to cover the chip (256 CUs, ~8 waves each), then the most
  // rows per wave (more reuse of the activations held in VGPRs).
  const long long waves_rw4 = (static_cast<long long>(p.m) + 3) / 4 * n_exp_rows;
  const long long waves_rw2 = (static_cast<long long>(p.m) + 1) / 2 * n_exp_rows;
  // Row chunks of 8 KiB (bf16, f16 at KB = 2; f32 at KB = 1) or 16 KiB (f32 at KB = 2): fewer
  // rows per wave keep the LDS of a workgroup modest.
  constexpr int kChunkBytes = Geometry<WT, KB>::kChunkBytes;
  if constexpr (kChunkBytes < 8192) {
    if (waves_rw4 >= 2048) return launch_variant<WT, NTC, KB, 4>(p, n_exp_rows, stream);
  }
  if constexpr (kChunkBytes < 16384) {
    if (waves_rw2 >= 2048) return launch_variant<WT, NTC, KB, 2>(p, n_exp_rows, stream);
  }
  return launch_variant<WT, NTC, KB, 1>(p, n_exp_rows, stream);
}

template <int WT>
hipError_t launch_wt(const MatvecParams& p, int max_tok, int n_exp_rows, hipStream_t stream) {
  if (max_tok <= 1) return launch_rw<WT, 1, 2>(p, n_exp_rows, stream);
  if (max_tok <= 2) return launch_rw<WT, 2, 2>(p, n_exp_rows, stream);
  return launch_rw<WT, 4, 1>(p, n_exp_rows, stream);
}

// ---- MoE gate combine ----------------------------------------------------------------------
// A grid-stride loop over the n_tok * m outputs (the grid is capped, so its size stays in range
// for any output size).
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* slots, const float* gates,
                                                          float* y, int n_tok, int top_k, int m) {
  const long long total = static_cast<long long>(n_tok) * m;
  for (long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<long long>(gridDim.x) * 256) {
    const int t = static_cast<int>(i / m);
    const int j = static_cast<int>(i - static_cast<long long>(t) * m);
    float v = 0.f;
    for (int s = 0; s < top_k; ++s) {
      const long long slot = static_cast<long long>(t) * top_k + s;
      v = __builtin_fmaf(gates[slot], slots[slot * m + j], v);
    }
    y[i] = v;
  }
}

// ---- exact dequantization (test hook) --------------------------------------------------------
template <int WT>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* w, float* out, int m, int k,
                                                         long long rowbytes) {
  const int nb = k / 32;
  const long long gb = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (gb >= static_cast<long long>(m) * nb) return;
  const long long row = gb / nb;
  const int blk = static_cast<int>(gb - row * nb);
  uint32_t q[BlockWords<WT>::NW];
  uint32_t sbits;
  read_block<WT>(reinterpret_cast<const uint32_t*>(w), row * rowbytes + static_cast<long long>(blk) * block_bytes(WT),
                 q, &sbits);
  float v[32];
  if constexpr (plain_type(WT)) {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = plain_at<WT>(q, i);
  } else if constexpr (WT == kQ8_0) {
    const float d = f16_to_f32(sbits);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int b = 0; b < 4; ++b) v[4 * i + b] = d * q8_at(q[i], b);
  } else {
    const float d = f16_to_f32(sbits);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qx = q[i] ^ 0x88888888u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        v[4 * i + b] = d * q4_at(qx, 2 * b);
        v[16 + 4 * i + b] = d * q4_at(qx, 2 * b + 1);
      }
    }
  }
  float4* o = reinterpret_cast<float4*>(out + row * k + static_cast<long long>(blk) * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// ---- padded-k weights (load-time conversion) -------------------------------------------------
// out[r][c] = the exact f32 value of w[r][c] for c < k, 0 for k <= c < kp: wavo's conv weights
// (`Gpu::upload_linear` with k % 32 != 0) as an f32 weight the layer can take. A grid-stride loop
// over the m * kp outputs, one element per thread per step: w need only be 2- or 4-byte aligned.
template <int WT>
__global__ __launch_bounds__(256) void pad_weight_kernel(const uint8_t* w, float* out, long long m, int k, int kp) {
  const long long total = m * kp;
  for (long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<long long>(gridDim.x) * 256) {
    const long long r = i / kp;
    const int c = static_cast<int>(i - r * kp);
    float v = 0.f;
    if (c < k) {
      const long long at = r * k + c;
      if constexpr (WT == kF32) v = reinterpret_cast<const float*>(w)[at];
      else if constexpr (WT == kF16) v = f16_to_f32(reinterpret_cast<const uint16_t*>(w)[at]);
      else v = __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(w)[at]) << 16);
    }
    out[i] = v;
  }
}

}  // namespace

hipError_t launch_pad_weight(int wtype, const uint8_t* w, float* out, long long m, int k, int kp,
                             hipStream_t stream) {
  const long long want = (m * kp + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < (1 << 20) ? want : (1 << 20));
  switch (wtype) {
    case kF32: hipLaunchKernelGGL(pad_weight_kernel<kF32>, dim3(grid), dim3(256), 0, stream, w, out, m, k, kp); break;
    case kF16: hipLaunchKernelGGL(pad_weight_kernel<kF16>, dim3(grid), dim3(256), 0, stream, w, out, m, k, kp); break;
    case kBF16: hipLaunchKernelGGL(pad_weight_kernel<kBF16>, dim3(grid), dim3(256), 0, stream, w, out, m, k, kp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_matvec(int wtype, const MatvecParams& p, int max_tok, hipStream_t stream) {
  // MoE: matrix cores (each workgroup walks many tiles, which repays building the activation
  // operands once), except for a single token, whose experts each take one slot: the f32 sliced
  // kernel streams those faster (1 token top-2 of 8 Q4_0 14336 x 4096: 21.3 against 30.4 us; with 2
  // or more slots per expert the matrix cores win, 4 tokens 52.8 against 56.7 us). The plain layer
  // takes the matrix cores from 9 tokens, where the f32 FMA kernels would stream the weights twice
  // (one pass for up to 16, measured 20.9 -> 16.3 us for Q8_0 4096 x 4096 at n = 16), and from 5
  // tokens on weights with at least two (Q4_K three) 16-row tiles per CU (matvec_mfma_takes_plain).
  // Dual outputs (wavo `Linear.dual`) are stored by this file's general kernel only: the sliced
  // and matrix-core kernels keep one output per row, since even a skipped second store in their
  // flush measured 12% slower on Q4_0 14336 x 4096 at n = 1.
  if (wtype == kQ4_K) return launch_matvec_q4k(p, max_tok, stream);
  const bool dual = p.dual > 0;
  if (!dual && matvec_mfma_supports(wtype, p.k) &&
      (p.ids != nullptr ? max_tok > 1 : matvec_mfma_takes_plain(wtype, p.m, max_tok)))
    return launch_matvec_mfma(wtype, p, stream);
  if (!dual && matvec_sliced_supports(p.k)) return launch_matvec_sliced(wtype, p, max_tok, stream);
  const int n_exp_rows = p.ids ? p.n_exp + 1 : 1;
  switch (wtype) {
    case kBF16: return launch_wt<kBF16>(p, max_tok, n_exp_rows, stream);
    case kQ8_0: return launch_wt<kQ8_0>(p, max_tok, n_exp_rows, stream);
    case kQ4_0: return launch_wt<kQ4_0>(p, max_tok, n_exp_rows, stream);
    case kF32: return launch_wt<kF32>(p, max_tok, n_exp_rows, stream);
    case kF16: return launch_wt<kF16>(p, max_tok, n_exp_rows, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_moe_combine(const float* slots, const float* gates, float* y, int n_tok, int top_k,
                              int m, hipStream_t stream) {
  const long long total = static_cast<long long>(n_tok) * m;
  const long long want = (total + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < (1 << 20) ? want : (1 << 20));
  hipLaunchKernelGGL(moe_combine_kernel, dim3(blocks), dim3(256), 0, stream, slots, gates, y, n_tok,
                     top_k, m);
  return hipGetLastError();
}

hipError_t launch_dequantize(int wtype, const uint8_t* w, float* out, int m, int k, hipStream_t stream) {
  if (wtype == kQ4_K) return launch_dequantize_q4k(w, out, m, k, stream);
  const long long blocks_total = static_cast<long long>(m) * (k / 32);
  const unsigned grid = static_cast<unsigned>((blocks_total + 255) / 256);
  const long long rowbytes = static_cast<long long>(k / 32) * block_bytes(wtype);
  switch (wtype) {
    case kBF16:
      hipLaunchKernelGGL(dequantize_kernel<kBF16>, dim3(grid), dim3(256), 0, stream, w, out, m, k, rowbytes);
      break;
    case kQ8_0:
      hipLaunchKernelGGL(dequantize_kernel<kQ8_0>, dim3(grid), dim3(256), 0, stream, w, out, m, k, rowbytes);
      break;
    case kQ4_0:
      hipLaunchKernelGGL(dequantize_kernel<kQ4_0>, dim3(grid), dim3(256), 0, stream, w, out, m, k, rowbytes);
      break;
    case kF32:
      hipLaunchKernelGGL(dequantize_kernel<kF32>, dim3(grid), dim3(256), 0, stream, w, out, m, k, rowbytes);
      break;
    case kF16:
      hipLaunchKernelGGL(dequantize_kernel<kF16>, dim3(grid), dim3(256), 0, stream, w, out, m, k, rowbytes);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace wq
