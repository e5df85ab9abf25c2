// Q4_K weights on the matvec / MoE path, and their exact dequantization.
//
// Q4_K is the k-quant type hanzo-ml src/wgpu_backend.rs takes in `matvec_q4k_gpu` and
// `moe_matvec_gpu`: rows of k/256 super-blocks of 144 bytes. The pages give only those sizes; the
// byte layout is GGML's published one. Bytes 0-1: f16 d; 2-3: f16 dmin; 4-15: the 6-bit scale
// sc_j and 6-bit min m_j of each 32-element sub-block j (j < 4: low 6 bits of bytes 4+j and 8+j;
// j >= 4: low and high nibble of byte 8+j, with their top 2 bits in the top bits of bytes j and
// 4+j); 16-143: 4-bit quants, sub-blocks 2c and 2c+1 in the low and high nibbles of bytes
// 16+32c .. 16+32c+31. Weight = d sc_j q - dmin m_j.
//
// Same contract as the other matvec kernels: y[t][j] = epilogue(sum_k x[t][k] w[j][k]) for the
// plain layer (with wavo's dual outputs), y[s][j] = sum_k W[ids[s]][j][k] x[s / top_k][k] for the
// MoE slots, all in f32.
//
// launch_matvec_q4k sends MoE calls with two or more slots per expert and 9 to 16 tokens (k a
// multiple of 256 in 2048..4096) to the matrix-core kernel (wq_matvec_mfma.hip), k a multiple of
// 1024 up to 8192 to the sliced kernel (wq_matvec_sliced.hip), which streams tiles of rows through
// an LDS ring (neither stores dual outputs). The general kernel here takes every other k (a
// multiple of 256) and the dual outputs:
//  * A wave owns RW consecutive rows; lane l walks the sub-blocks l, l+64, ... of the rows. Per
//    sub-block it loads the 16 header bytes and the 32 quant bytes of its super-block with 16-byte
//    loads (the 8 lanes of one super-block read neighbouring bytes, so the wave's loads of a row
//    cover a contiguous run), and the 32 activations of each token, shared by its RW rows.
//  * Per sub-block and token: s = sum x q over 32 products (q unsigned, exact in f32), then
//    acc += d sc_j s - dmin m_j sum(x). The lane totals are summed across the wave.
//  * Tokens are taken NTC at a time; more tokens re-stream the rows. MoE workgroups are indexed by
//    expert and find their slots by a ballot over the ids, as in the other kernels.
#include <hip/hip_runtime.h>

#include "wq_decode.hpp"
#include "wq_internal.hpp"

namespace wq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sub-block j's (d sc_j, dmin m_j) from the 16 header bytes of its super-block, both exact in f32.
__device__ __forceinline__ float2 q4k_factors(const uint4& h, int j) {
  const uint32_t jj = 8u * (j & 3);
  uint32_t sc, mn;
  if (j < 4) {
    sc = (h.y >> jj) & 63u;
    mn = (h.z >> jj) & 63u;
  } else {
    sc = ((h.w >> jj) & 15u) | (((h.y >> (jj + 6)) & 3u) << 4);
    mn = ((h.w >> (jj + 4)) & 15u) | (((h.z >> (jj + 6)) & 3u) << 4);
  }
  return make_float2(f16_to_f32(h.x & 0xFFFFu) * static_cast<float>(sc),
                     f16_to_f32(h.x >> 16) * static_cast<float>(mn));
}

// The 32 quants of sub-block j from its super-block's 32 quant bytes (low nibbles for even j,
// high for odd j), as floats. A byte 0000qqqq read as FP8 E4M3 is q * 2^-9 exactly (q = 0..15),
// so one conversion with scale 2^9 gives two quants.
__device__ __forceinline__ void q4k_quants(const uint4& a, const uint4& b, int j, float (&q)[32]) {
  const uint32_t dw[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const int sh = 4 * (j & 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t v = (dw[i] >> sh) & 0x0F0F0F0Fu;
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 512.f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 512.f, true);
    q[4 * i] = lo[0];
    q[4 * i + 1] = lo[1];
    q[4 * i + 2] = hi[0];
    q[4 * i + 3] = hi[1];
  }
}

template <int NTC, int RW>
__global__ __launch_bounds__(kThreads) void matvec_q4k_kernel(MatvecParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int e = blockIdx.y;
  const int row0 = (blockIdx.x * kWaves + wave) * RW;
  if (row0 >= p.m) return;  // wave-uniform; the kernel has no workgroup barrier
  const bool moe = p.ids != nullptr;
  const int nsub = p.k / 32;

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

      for (int sb = lane; sb < nsub; sb += 64) {
        const int sup = sb >> 3, j = sb & 7;
        // Every load of the step before any arithmetic: the RW rows' header and quant bytes.
        uint4 hd[RW], qa[RW], qb[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          const int row = min(row0 + r, p.m - 1);  // rows past m re-read the last; never stored
          const uint8_t* sp = wbase + static_cast<long long>(row) * p.rowbytes + static_cast<long long>(sup) * kQ4KBytes;
          hd[r] = *reinterpret_cast<const uint4*>(sp);
          qa[r] = *reinterpret_cast<const uint4*>(sp + 16 + 32 * (j >> 1));
          qb[r] = *reinterpret_cast<const uint4*>(sp + 32 + 32 * (j >> 1));
        }
        float xr[NTC][32], xs[NTC];
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
          const int tok = slot[t] >= 0 ? slot[t] / p.top_k : 0;
          const float4* xp =
              reinterpret_cast<const float4*>(p.x + static_cast<long long>(tok) * p.k + static_cast<long long>(sb) * 32);
          xs[t] = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float4 v = xp[i];
            xr[t][4 * i + 0] = v.x;
            xr[t][4 * i + 1] = v.y;
            xr[t][4 * i + 2] = v.z;
            xr[t][4 * i + 3] = v.w;
          }
#pragma unroll
          for (int i = 0; i < 32; ++i) xs[t] += xr[t][i];
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          float q[32];
          q4k_quants(qa[r], qb[r], j, q);
          const float2 f = q4k_factors(hd[r], j);
#pragma unroll
          for (int t = 0; t < NTC; ++t) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) s = __builtin_fmaf(xr[t][i], q[i], s);
            acc[r][t] += __builtin_fmaf(f.x, s, -(f.y * xs[t]));
          }
        }
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

template <int NTC, int RW>
hipError_t launch_general(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  const int rows_per_wg = kWaves * RW;
  dim3 grid((p.m + rows_per_wg - 1) / rows_per_wg, n_exp_rows);
  hipLaunchKernelGGL((matvec_q4k_kernel<NTC, RW>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int NTC>
hipError_t launch_general_rw(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  // Several rows per wave share each activation load, while there are enough waves to cover the
  // chip (256 CUs, ~8 waves each); one row per wave for small layers. Four tokens hold 128
  // activations per lane, so their waves take at most two rows (four would spill).
  constexpr int kRw = NTC >= 4 ? 2 : 4;
  const long long waves = (static_cast<long long>(p.m) + kRw - 1) / kRw * n_exp_rows;
  if (waves >= 2048) return launch_general<NTC, kRw>(p, n_exp_rows, stream);
  return launch_general<NTC, 1>(p, n_exp_rows, stream);
}

// One thread per 32-element sub-block: out = d sc_j q - dmin m_j with one rounding (both
// products are exact in f32, and the fused multiply-add rounds the exact difference once).
__global__ __launch_bounds__(256) void dequantize_q4k_kernel(const uint8_t* w, float* out, int m, int k,
                                                             long long rowbytes) {
  const int nsub = k / 32;
  const long long g = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (g >= static_cast<long long>(m) * nsub) return;
  const long long row = g / nsub;
  const int sb = static_cast<int>(g - row * nsub);
  const int j = sb & 7;
  const uint8_t* sp = w + row * rowbytes + static_cast<long long>(sb >> 3) * kQ4KBytes;
  const uint4 h = *reinterpret_cast<const uint4*>(sp);
  const uint4 a = *reinterpret_cast<const uint4*>(sp + 16 + 32 * (j >> 1));
  const uint4 b = *reinterpret_cast<const uint4*>(sp + 32 + 32 * (j >> 1));
  float q[32];
  q4k_quants(a, b, j, q);
  const float2 f = q4k_factors(h, j);
  float4* o = reinterpret_cast<float4*>(out + row * k + static_cast<long long>(sb) * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    o[i] = make_float4(__builtin_fmaf(f.x, q[4 * i], -f.y), __builtin_fmaf(f.x, q[4 * i + 1], -f.y),
                       __builtin_fmaf(f.x, q[4 * i + 2], -f.y), __builtin_fmaf(f.x, q[4 * i + 3], -f.y));
}

}  // namespace

hipError_t launch_matvec_q4k(const MatvecParams& p, int max_tok, hipStream_t stream) {
  if (p.k % kQ4KElems != 0) return hipErrorInvalidValue;
  // As for the other quantized types: the matrix cores for MoE with two or more slots per expert,
  // for 9 to 16 tokens (every weight decoded once for up to 16 slots) and for 5 to 8 on weights
  // with three or more 16-row tiles per CU (matvec_mfma_takes_plain); else the sliced f32 kernel.
  if (p.dual == 0 && matvec_mfma_supports(kQ4_K, p.k) &&
      (p.ids != nullptr ? max_tok > 1 : matvec_mfma_takes_plain(kQ4_K, p.m, max_tok)))
    return launch_matvec_mfma(kQ4_K, p, stream);
  if (p.dual == 0 && matvec_sliced_supports(p.k)) return launch_matvec_sliced(kQ4_K, p, max_tok, stream);
  const int n_exp_rows = p.ids ? p.n_exp + 1 : 1;
  if (max_tok <= 1) return launch_general_rw<1>(p, n_exp_rows, stream);
  if (max_tok <= 2) return launch_general_rw<2>(p, n_exp_rows, stream);
  return launch_general_rw<4>(p, n_exp_rows, stream);
}

hipError_t launch_dequantize_q4k(const uint8_t* w, float* out, int m, int k, hipStream_t stream) {
  if (k % kQ4KElems != 0) return hipErrorInvalidValue;
  const long long subs = static_cast<long long>(m) * (k / 32);
  const unsigned grid = static_cast<unsigned>((subs + 255) / 256);
  const long long rowbytes = static_cast<long long>(k / kQ4KElems) * kQ4KBytes;
  hipLaunchKernelGGL(dequantize_q4k_kernel, dim3(grid), dim3(256), 0, stream, w, out, m, k, rowbytes);
  return hipGetLastError();
}

}  // namespace wq
