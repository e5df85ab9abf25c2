// GEMM path (any n; chosen for n > 16): bf16 matrix cores, f32 accumulation.
//
// Contract: Y[n x m] = epilogue(X[n x k] . W[m x k]^T + bias) with the
// epilogue of `ae_put` (bias, then erf-GELU, then + old Y) -- the tiled GEMM
// of cortiq-engine src/gpu_wgpu/nemotron_audio.rs (`ae_gemm`, a 128x128
// register-tiled f32 kernel with bf16 weights) and wavo src/gpu/mod.rs
// (`Pass::gemm`, one pipeline per weight type).
//
// Design for gfx950:
//  * Workgroup tile 128 (rows of X) x 128 (rows of W), k step 64; four waves,
//    each owning a 64x64 quarter as 2x2 v_mfma_f32_32x32x16_bf16 tiles.
//  * X is read as f32 and rounded to bf16 (nearest even, v_cvt_pk_bf16_f32)
//    on its way into LDS. bf16 weights go to LDS as stored.
//  * Q8_0 / Q4_0 weights are decoded on the way into LDS to their integer
//    quants q (Q8_0) or q-8 (Q4_0), which bf16 holds exactly; the matrix cores
//    sum each 32-element block into a fresh accumulator and the f16 scale of
//    that (row, block) multiplies it in f32. The weights thus enter the
//    product exactly and only the bf16 rounding of X (2^-9 relative) and the
//    f32 sums contribute error: |y - y_ref| <= 2^-8 * sum|x*w|.
//  * The next k step's global loads are issued before the current step's
//    matrix-core work, so their latency hides behind it.
//  * LDS rows are padded to 144 bytes so the 16-byte fragment reads of 16
//    consecutive lanes fall in distinct banks.
#include <hip/hip_runtime.h>

#include "wq_decode.hpp"
#include "wq_internal.hpp"

namespace wq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;         // tile rows (X rows, output rows)
constexpr int BN = 128;         // tile cols (W rows, output cols)
constexpr int BK = 64;          // k per step: two 32-element blocks
constexpr int LDS_STRIDE = 72;  // bf16 per LDS row (64 + 8 padding)
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // Exact for the small integers fed here (at most 8 significant bits).
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

__device__ __forceinline__ uint2 round_bf16x4(float4 v) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 a, b;
  a[0] = static_cast<__bf16>(v.x);
  a[1] = static_cast<__bf16>(v.y);
  b[0] = static_cast<__bf16>(v.z);
  b[1] = static_cast<__bf16>(v.w);
  return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

template <int WT>
struct WStage;  // registers holding one k step of this thread's share of the W tile

template <>
struct WStage<kBF16> {
  uint4 v[4];
};
template <>
struct WStage<kQ8_0> {
  uint32_t q[8];
  uint32_t s;
  bool ok;
};
template <>
struct WStage<kQ4_0> {
  uint32_t q[4];
  uint32_t s;
  bool ok;
};

template <int WT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 sA[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) __bf16 sB[BN * LDS_STRIDE];
  __shared__ float sS[BN * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;  // 64-row half of the tile (X rows)
  const int wn = wave & 1;   // 64-col half of the tile (W rows)
  const int n0 = blockIdx.y * BM;
  const int m0 = blockIdx.x * BN;
  const int nk = (p.k + BK - 1) / BK;

  // ---- per-thread load assignments ----
  // X: 8 float4 per thread; row = tid/16 + 16 i, float4 column tid%16.
  const int xc4 = tid & 15;
  const int xr0 = tid >> 4;
  // W bf16: 4 x 16 bytes per thread; row = tid/8 + 32 i, 16-byte chunk tid%8.
  const int wc16 = tid & 7;
  const int wr0 = tid >> 3;
  // W quantized: one (row, block) per thread.
  const int qrow = tid >> 1;
  const int qblk = tid & 1;

  float4 xs[8];
  WStage<WT> ws;

  auto load_stage = [&](int s) {
    const int k0 = s * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = n0 + xr0 + 16 * i;
      const int kk = k0 + 4 * xc4;
      if (r < p.n && kk < p.k)
        xs[i] = *reinterpret_cast<const float4*>(p.x + static_cast<long long>(r) * p.k + kk);
      else
        xs[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if constexpr (WT == kBF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + wr0 + 32 * i;
        const int kk = k0 + 8 * wc16;
        if (r < p.m && kk < p.k)
          ws.v[i] = *reinterpret_cast<const uint4*>(p.w + static_cast<long long>(r) * p.rowbytes + 2LL * kk);
        else
          ws.v[i] = make_uint4(0, 0, 0, 0);
      }
    } else {
      const int r = m0 + qrow;
      const int blk = s * 2 + qblk;
      ws.ok = r < p.m && blk * 32 < p.k;
      if (ws.ok) {
        read_block<WT>(reinterpret_cast<const uint32_t*>(p.w),
                       static_cast<long long>(r) * p.rowbytes + static_cast<long long>(blk) * block_bytes(WT),
                       ws.q, &ws.s);
      }
    }
  };

  auto store_stage = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = xr0 + 16 * i;
      *reinterpret_cast<uint2*>(&sA[r * LDS_STRIDE + 4 * xc4]) = round_bf16x4(xs[i]);
    }
    if constexpr (WT == kBF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wr0 + 32 * i;
        *reinterpret_cast<uint4*>(&sB[r * LDS_STRIDE + 8 * wc16]) = ws.v[i];
      }
    } else {
      uint32_t o[16];
      if (ws.ok) {
        if constexpr (WT == kQ8_0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            o[2 * i] = pack_bf16x2(q8_at(ws.q[i], 0), q8_at(ws.q[i], 1));
            o[2 * i + 1] = pack_bf16x2(q8_at(ws.q[i], 2), q8_at(ws.q[i], 3));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t qx = ws.q[i] ^ 0x88888888u;
            // elements 4i..4i+3 (low nibbles) and 16+4i..16+4i+3 (high nibbles)
            o[2 * i] = pack_bf16x2(q4_at(qx, 0), q4_at(qx, 2));
            o[2 * i + 1] = pack_bf16x2(q4_at(qx, 4), q4_at(qx, 6));
            o[8 + 2 * i] = pack_bf16x2(q4_at(qx, 1), q4_at(qx, 3));
            o[8 + 2 * i + 1] = pack_bf16x2(q4_at(qx, 5), q4_at(qx, 7));
          }
        }
        sS[qrow * 2 + qblk] = f16_to_f32(ws.s);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = 0u;
        sS[qrow * 2 + qblk] = 0.f;
      }
      uint4* dst = reinterpret_cast<uint4*>(&sB[qrow * LDS_STRIDE + 32 * qblk]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Fragment addressing: lane l supplies row (l % 32) and k-elements 8*(l/32)..+8.
  const int frow = lane & 31;
  const int fk = 8 * (lane >> 5);

  load_stage(0);
  for (int s = 0; s < nk; ++s) {
    __syncthreads();  // the previous step's fragment reads are done
    store_stage();
    __syncthreads();
    if (s + 1 < nk) load_stage(s + 1);

    if constexpr (WT == kBF16) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          a[i] = *reinterpret_cast<const bf16x8*>(&sA[(wm * 64 + i * 32 + frow) * LDS_STRIDE + ks * 16 + fk]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[j] = *reinterpret_cast<const bf16x8*>(&sB[(wn * 64 + j * 32 + frow) * LDS_STRIDE + ks * 16 + fk]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        f32x16 part[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) part[i][j][v] = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ks = blk * 2 + h;
          bf16x8 a[2], b[2];
#pragma unroll
          for (int i = 0; i < 2; ++i)
            a[i] = *reinterpret_cast<const bf16x8*>(&sA[(wm * 64 + i * 32 + frow) * LDS_STRIDE + ks * 16 + fk]);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            b[j] = *reinterpret_cast<const bf16x8*>(&sB[(wn * 64 + j * 32 + frow) * LDS_STRIDE + ks * 16 + fk]);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], part[i][j], 0, 0, 0);
        }
        // Output column of this lane in tile j is W row wn*64 + j*32 + lane%32.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float d = sS[(wn * 64 + j * 32 + frow) * 2 + blk];
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(d, part[i][j][v], acc[i][j][v]);
        }
      }
    }
  }

  // ---- epilogue: lane holds column lane%32 and rows 8*(v/4) + 4*(lane/32) + v%4 of each tile ----
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = m0 + wn * 64 + j * 32 + frow;
    if (col >= p.m) continue;
    const float b = (p.flags & 1u) ? p.bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = n0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < p.n) {
          float o = acc[i][j][v];
          if (p.flags & 1u) o += b;
          if (p.flags & 2u) o = gelu_erf(o);
          float* yp = p.y + static_cast<long long>(row) * p.m + col;
          if (p.flags & 4u) o += *yp;
          *yp = o;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(int wtype, const GemmParams& p, hipStream_t stream) {
  dim3 grid((p.m + BN - 1) / BN, (p.n + BM - 1) / BM);
  switch (wtype) {
    case kBF16: hipLaunchKernelGGL(gemm_kernel<kBF16>, grid, dim3(kThreads), 0, stream, p); break;
    case kQ8_0: hipLaunchKernelGGL(gemm_kernel<kQ8_0>, grid, dim3(kThreads), 0, stream, p); break;
    case kQ4_0: hipLaunchKernelGGL(gemm_kernel<kQ4_0>, grid, dim3(kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace wq
