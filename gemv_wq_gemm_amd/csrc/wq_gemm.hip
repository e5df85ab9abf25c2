// GEMM path (any n; chosen for n > 16): bf16 matrix cores, f32 accumulation.
//
// Contract: Y[n x m] = epilogue(X[n x k] . W[m x k]^T + bias) with the
// epilogue of `ae_put` (bias, then erf-GELU, then + old Y) -- the tiled GEMM
// of cortiq-engine src/gpu_wgpu/nemotron_audio.rs (`ae_gemm`, a 128x128
// register-tiled f32 kernel with bf16 weights) and wavo src/gpu/mod.rs
// (`Pass::gemm`, one pipeline per weight type).
//
// Two kernels: `gemm_bf16_kernel` for bf16 weights (a deeper direct-to-LDS pipeline, described
// where it is defined) and `gemm_kernel` for Q8_0 / Q4_0 weights, described here.
//
// Design for gfx950 (quantized weights):
//  * Workgroup tile BM (rows of X) x BN (rows of W), k step 64; WM x WN waves,
//    each owning a (BM/WM) x (BN/WN) piece as v_mfma_f32_32x32x16_bf16 tiles.
//    The wide tile along W keeps the per-FLOP traffic from L2 low: X arrives as
//    f32 (4 bytes per element), W as 2 bytes or less.
//  * X is rounded to bf16 (nearest even, v_cvt_pk_bf16_f32) on its way into
//    LDS; bf16 weights go to LDS as stored. Q8_0 / Q4_0 weights are decoded on
//    the way to their integer quants q (Q8_0) or q-8 (Q4_0), exact in bf16; the
//    matrix cores sum each 32-element block into a fresh accumulator and the f16
//    scale of that (row, block) multiplies it in f32. The weights thus enter
//    exactly; only the bf16 rounding of X (at most 2^-8 relative) and the f32 sums
//    contribute error: |y - y_ref| <= 2^-8 * sum|x*w|.
//  * Two LDS buffers: while the matrix cores work on one k step, the next step
//    is loaded from global memory into registers and then written to the other
//    buffer; one workgroup barrier per k step. LDS rows are padded to 144 bytes
//    so 16-byte fragment reads of consecutive lanes spread over the banks.
//  * Tiles are numbered so that consecutive tiles share W rows, and the tile
//    numbers are dealt to the 8 XCDs in contiguous ranges (workgroup i runs on
//    XCD i % 8), so an XCD's L2 holds the panels its tiles reuse.
//  * With X in three parts (the f32-accurate path) x = p1 + p2 + p3 exactly, each part bf16:
//    the parts sit in three LDS buffers and each fragment takes three MFMAs into the same
//    accumulator, so the products are exact and only the f32 sums round.
//  * Split-K: when the output has too few tiles to fill the chip and the
//    epilogue is linear in the product (no activation, accumulate into Y), gridDim.z
//    workgroups share a tile's k range and add their partial sums into Y with
//    f32 atomics; the first one adds the bias.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <type_traits>

#include "wq_decode.hpp"
#include "wq_internal.hpp"
#include "wq_lds_dma.hpp"

namespace wq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;          // k per step: two 32-element blocks
constexpr int LDS_STRIDE = 72;  // bf16 per LDS row (64 + 8 padding)

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

// Splits four f32 values into three bf16 parts (pairs packed as round_bf16x4 packs them):
// p1 = bf16(v), p2 = bf16(v - p1), p3 = bf16(v - p1 - p2), each rounded to nearest even. Both
// differences are exact in f32, and what is left for p3 has at most 8 significant bits, so
// p1 + p2 + p3 == v exactly (for |v| where bf16 holds the parts as normal numbers).
__device__ __forceinline__ float bf16_lo_f32(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi_f32(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

__device__ __forceinline__ void split3_bf16x4(float4 v, uint2& p1, uint2& p2, uint2& p3) {
  p1 = round_bf16x4(v);
  const float4 r1 = make_float4(v.x - bf16_lo_f32(p1.x), v.y - bf16_hi_f32(p1.x), v.z - bf16_lo_f32(p1.y),
                                v.w - bf16_hi_f32(p1.y));
  p2 = round_bf16x4(r1);
  const float4 r2 = make_float4(r1.x - bf16_lo_f32(p2.x), r1.y - bf16_hi_f32(p2.x), r1.z - bf16_lo_f32(p2.y),
                                r1.w - bf16_hi_f32(p2.y));
  p3 = round_bf16x4(r2);
}

// Decoded block -> 16 dwords of bf16 pairs in element order.
template <int WT>
__device__ __forceinline__ void quants_to_bf16(const uint32_t* q, uint32_t* o) {
  if constexpr (WT == kQ8_0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[2 * i] = pack_bf16x2(q8_at(q[i], 0), q8_at(q[i], 1));
      o[2 * i + 1] = pack_bf16x2(q8_at(q[i], 2), q8_at(q[i], 3));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qx = q[i] ^ 0x88888888u;
      // elements 4i..4i+3 (low nibbles) and 16+4i..16+4i+3 (high nibbles)
      o[2 * i] = pack_bf16x2(q4_at(qx, 0), q4_at(qx, 2));
      o[2 * i + 1] = pack_bf16x2(q4_at(qx, 4), q4_at(qx, 6));
      o[8 + 2 * i] = pack_bf16x2(q4_at(qx, 1), q4_at(qx, 3));
      o[8 + 2 * i + 1] = pack_bf16x2(q4_at(qx, 5), q4_at(qx, 7));
    }
  }
}

template <int WT, int BM, int BN, int WM, int WN>
struct GemmCfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int TM = BM / WM;  // wave tile rows (X rows)
  static constexpr int TN = BN / WN;  // wave tile cols (W rows)
  static constexpr int FM = TM / 32;  // 32x32 fragments per wave
  static constexpr int FN = TN / 32;
  // X: BM rows x 16 float4 per step
  static constexpr int kXLoads = BM * 16 / kThreads;
  // W bf16: BN rows x 8 16-byte chunks per step
  static constexpr int kWLoads = BN * 8 / kThreads;
  // W quantized: BN rows x 2 blocks per step
  static constexpr int kQLoads = (BN * 2 + kThreads - 1) / kThreads;
  static_assert(BM * 16 % kThreads == 0 && BN * 8 % kThreads == 0, "tile/threads mismatch");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 fragments");
};

// One step's quantized blocks as loaded: the NW + 1 aligned dwords that cover each block and
// where in the first one it starts (byte 0 or 2). Scale and quants are pulled out only when the
// step is written to LDS, so nothing waits on these loads until then: the step's MFMAs and
// scaling run while they are in flight.
template <int WT, int NQ>
struct QStage {
  uint32_t d[NQ][BlockWords<WT>::NW + 1];
  uint32_t sh[NQ];
  bool ok[NQ];
};

template <int WT, int BM, int BN, int WM, int WN, bool SPLIT>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmParams p, int tiles_m, int tiles_n) {
  using C = GemmCfg<WT, BM, BN, WM, WN>;
  constexpr bool kQuant = !plain_type(WT);  // Q8_0 / Q4_0: integer quants and a per-block scale
  __shared__ __attribute__((aligned(16))) __bf16 sA[2][BM * LDS_STRIDE];
  // SPLIT: the second and third bf16 parts of X beside the first ones in sA.
  __shared__ __attribute__((aligned(16))) __bf16 sAm[2][SPLIT ? BM * LDS_STRIDE : 8];
  __shared__ __attribute__((aligned(16))) __bf16 sAl[2][SPLIT ? BM * LDS_STRIDE : 8];
  // W as WP exact bf16 parts (f16 weights 2, f32 weights 3, else 1), each double-buffered.
  constexpr int WP = weight_parts(WT);
  __shared__ __attribute__((aligned(16))) __bf16 sB[WP][2][BN * LDS_STRIDE];
  __shared__ float sS[2][kQuant ? BN * 2 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // ---- tile of this workgroup: contiguous ranges of tile numbers per XCD ----
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + 7) / 8;
  const int bid = blockIdx.x;
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  if (t >= tiles) return;  // workgroup-uniform
  const int tile_n = t / tiles_m;  // W-row tile (varies slowest: neighbours share W)
  const int tile_m = t - tile_n * tiles_m;
  const int n0 = tile_m * BM;  // first X row
  const int m0 = tile_n * BN;  // first W row

  // ---- k range of this split ----
  const int nk_total = (p.k + BK - 1) / BK;
  const int per_split = (nk_total + gridDim.z - 1) / gridDim.z;
  const int s_begin = blockIdx.z * per_split;
  const int s_end = min(nk_total, s_begin + per_split);
  const bool split = gridDim.z > 1;

  // ---- per-thread load assignments ----
  const int xc4 = tid & 15;   // float4 column of X
  const int xr0 = tid >> 4;   // first X row; rows xr0 + i * (threads / 16)
  const int wc16 = tid & 7;   // 16-byte chunk of a bf16 W row
  const int wr0 = tid >> 3;   // first W row; rows wr0 + i * (threads / 8)

  float4 xs[C::kXLoads];
  // Plain weights: 8 elements per chunk, 16 bytes (bf16, f16) or 32 bytes (f32).
  constexpr int kChunkU4 = WT == kF32 ? 2 : 1;
  uint4 wsb[kQuant ? 1 : C::kWLoads][kChunkU4];
  QStage<plain_type(WT) ? kQ8_0 : WT, C::kQLoads> wsq;

  auto load_stage = [&](int s) {
    const int k0 = s * BK;
#pragma unroll
    for (int i = 0; i < C::kXLoads; ++i) {
      const int r = n0 + xr0 + i * (C::kThreads / 16);
      const int kk = k0 + 4 * xc4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < p.n && kk < p.k) v = *reinterpret_cast<const float4*>(p.x + static_cast<long long>(r) * p.k + kk);
      xs[i] = v;
    }
    if constexpr (!kQuant) {
#pragma unroll
      for (int i = 0; i < C::kWLoads; ++i) {
        const int r = m0 + wr0 + i * (C::kThreads / 8);
        const int kk = k0 + 8 * wc16;
        const uint4* src = reinterpret_cast<const uint4*>(p.w + static_cast<long long>(r) * p.rowbytes +
                                                          (WT == kF32 ? 4LL : 2LL) * kk);
#pragma unroll
        for (int u = 0; u < kChunkU4; ++u) {
          uint4 v = make_uint4(0u, 0u, 0u, 0u);
          if (r < p.m && kk < p.k) v = src[u];
          wsb[i][u] = v;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::kQLoads; ++i) {
        const int e = tid + i * C::kThreads;  // (row, block) pair of the step
        const int rr = e >> 1;
        const int blk = s * 2 + (e & 1);
        const bool ok = e < BN * 2 && m0 + rr < p.m && blk * 32 < p.k;
        wsq.ok[i] = ok;
        if (ok) {
          const long long off =
              static_cast<long long>(m0 + rr) * p.rowbytes + static_cast<long long>(blk) * block_bytes(WT);
          const uint32_t* a = reinterpret_cast<const uint32_t*>(p.w) + (off >> 2);
#pragma unroll
          for (int j = 0; j <= BlockWords<WT>::NW; ++j) wsq.d[i][j] = a[j];
          wsq.sh[i] = static_cast<uint32_t>(off) & 3u;
        }
      }
    }
  };

  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kXLoads; ++i) {
      const int r = xr0 + i * (C::kThreads / 16);
      if constexpr (SPLIT) {
        uint2 p1, p2, p3;
        split3_bf16x4(xs[i], p1, p2, p3);
        *reinterpret_cast<uint2*>(&sA[buf][r * LDS_STRIDE + 4 * xc4]) = p1;
        *reinterpret_cast<uint2*>(&sAm[buf][r * LDS_STRIDE + 4 * xc4]) = p2;
        *reinterpret_cast<uint2*>(&sAl[buf][r * LDS_STRIDE + 4 * xc4]) = p3;
      } else {
        *reinterpret_cast<uint2*>(&sA[buf][r * LDS_STRIDE + 4 * xc4]) = round_bf16x4(xs[i]);
      }
    }
    if constexpr (!kQuant) {
#pragma unroll
      for (int i = 0; i < C::kWLoads; ++i) {
        const int r = wr0 + i * (C::kThreads / 8);
        const int at = r * LDS_STRIDE + 8 * wc16;
        if constexpr (WT == kBF16) {
          *reinterpret_cast<uint4*>(&sB[0][buf][at]) = wsb[i][0];
        } else {
          // f16 / f32 -> WP bf16 parts that add up to the weight exactly.
          float4 f[2];
          if constexpr (WT == kF16) {
            const uint4 h = wsb[i][0];
            f[0] = make_float4(f16_to_f32(h.x & 0xFFFFu), f16_to_f32(h.x >> 16), f16_to_f32(h.y & 0xFFFFu),
                               f16_to_f32(h.y >> 16));
            f[1] = make_float4(f16_to_f32(h.z & 0xFFFFu), f16_to_f32(h.z >> 16), f16_to_f32(h.w & 0xFFFFu),
                               f16_to_f32(h.w >> 16));
          } else {
            f[0] = __builtin_bit_cast(float4, wsb[i][0]);
            f[1] = __builtin_bit_cast(float4, wsb[i][1]);
          }
          uint2 pa[2][3];
#pragma unroll
          for (int h = 0; h < 2; ++h) split3_bf16x4(f[h], pa[h][0], pa[h][1], pa[h][2]);
#pragma unroll
          for (int wp = 0; wp < WP; ++wp)
            *reinterpret_cast<uint4*>(&sB[wp][buf][at]) = make_uint4(pa[0][wp].x, pa[0][wp].y, pa[1][wp].x, pa[1][wp].y);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::kQLoads; ++i) {
        const int e = tid + i * C::kThreads;
        if (e < BN * 2) {
          const int rr = e >> 1;
          const int half = e & 1;
          uint32_t o[16];
          if (wsq.ok[i]) {
            // The f16 scale, then the quants from 2 bytes further on (as read_block does).
            constexpr int NW = BlockWords<WT>::NW;
            const uint32_t sh = wsq.sh[i];
            uint32_t q[NW];
#pragma unroll
            for (int j = 0; j < NW; ++j) q[j] = sh ? wsq.d[i][j + 1] : realign(wsq.d[i][j + 1], wsq.d[i][j], 2u);
            quants_to_bf16<WT>(q, o);
            sS[buf][rr * 2 + half] = f16_to_f32((sh ? (wsq.d[i][0] >> 16) : wsq.d[i][0]) & 0xFFFFu);
          } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) o[j] = 0u;
            sS[buf][rr * 2 + half] = 0.f;
          }
          uint4* dst = reinterpret_cast<uint4*>(&sB[0][buf][rr * LDS_STRIDE + 32 * half]);
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[j] = make_uint4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
        }
      }
    }
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Fragment addressing: lane l supplies row (l % 32) and k-elements 8*(l/32)..+8.
  const int frow = lane & 31;
  const int fk = 8 * (lane >> 5);

  // One 16-wide k slice: every part of X (1, or 3 with SPLIT) times every part of W (WP).
  auto mfma_step = [&](int buf, int ks, f32x16 (&c)[C::FM][C::FN]) {
    bf16x8 a[C::FM], b[WP][C::FN];
#pragma unroll
    for (int wp = 0; wp < WP; ++wp)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        b[wp][j] =
            *reinterpret_cast<const bf16x8*>(&sB[wp][buf][(wn * C::TN + j * 32 + frow) * LDS_STRIDE + ks * 16 + fk]);
#pragma unroll
    for (int part = 0; part < (SPLIT ? 3 : 1); ++part) {
      const __bf16* src = part == 0 ? sA[buf] : part == 1 ? sAm[buf] : sAl[buf];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&src[(wm * C::TM + i * 32 + frow) * LDS_STRIDE + ks * 16 + fk]);
#pragma unroll
      for (int wp = 0; wp < WP; ++wp)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[wp][j], c[i][j], 0, 0, 0);
    }
  };

  if (s_begin < s_end) {
    load_stage(s_begin);
    store_stage(0);
    __syncthreads();
    for (int s = s_begin; s < s_end; ++s) {
      const int buf = (s - s_begin) & 1;
      if (s + 1 < s_end) load_stage(s + 1);
      if constexpr (!kQuant) {
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) mfma_step(buf, ks, acc);
      } else {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          f32x16 part[C::FM][C::FN];
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
              for (int v = 0; v < 16; ++v) part[i][j][v] = 0.f;
          mfma_step(buf, 2 * blk, part);
          mfma_step(buf, 2 * blk + 1, part);
          // Output column of this lane in fragment j is W row wn*TN + j*32 + lane%32.
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            const float d = sS[buf][(wn * C::TN + j * 32 + frow) * 2 + blk];
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(d, part[i][j][v], acc[i][j][v]);
          }
        }
      }
      if (s + 1 < s_end) store_stage(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds column lane%32 and rows 8*(v/4) + 4*(lane/32) + v%4 of each fragment ----
  const bool first = blockIdx.z == 0;
  // Tiles inside Y, without the k split or dual outputs: Y through a buffer resource at the
  // tile's corner, old values loaded back to back and the stores issued without waits between
  // them (a guarded per-output access compiles to a branch that waits for every earlier store),
  // with the activation chosen at compile time.
  if (!split && p.dual == 0 && n0 + BM <= p.n && m0 + BN <= p.m &&
      (static_cast<long long>(BM) * p.ystride + BN) * 4 < (1LL << 31)) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(p.y + static_cast<long long>(n0) * p.ystride + m0, 0,
                                                        0x7FFFFFFF, 0x00020000);
    const int rs = p.ystride * 4;  // bytes per row of Y
    float bv[C::FN];
#pragma unroll
    for (int j = 0; j < C::FN; ++j) bv[j] = (p.flags & kEpiBias) ? p.bias[m0 + wn * C::TN + j * 32 + frow] : 0.f;
    // Inlined by force: a call would take the accumulators' address and move them to scratch.
    auto run = [&](auto act, auto res) __attribute__((always_inline)) {
      float old[C::FM][C::FN][16];
      if constexpr (decltype(res)::value) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            const int vo = (wm * C::TM + i * 32 + 4 * (lane >> 5)) * rs + (wn * C::TN + j * 32 + frow) * 4;
#pragma unroll
            for (int v = 0; v < 16; ++v)
              old[i][j][v] = __builtin_bit_cast(
                  float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, vo, (8 * (v >> 2) + (v & 3)) * rs, 0));
          }
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int vo = (wm * C::TM + i * 32 + 4 * (lane >> 5)) * rs + (wn * C::TN + j * 32 + frow) * 4;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float o = acc[i][j][v] + bv[j];
            if constexpr (decltype(act)::value != 0) o = activation(o, decltype(act)::value);
            o *= p.alpha;
            if constexpr (decltype(res)::value) o += old[i][j][v];
            // The b32 buffer builtins move 32-bit integers: the float's bits go through unchanged.
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, o), rsrc, vo,
                                                  (8 * (v >> 2) + (v & 3)) * rs, 0);
          }
        }
    };
    auto with_residual = [&](auto act) __attribute__((always_inline)) {
      if (p.flags & kEpiResidual) run(act, std::true_type{});
      else run(act, std::false_type{});
    };
    switch (p.flags & kEpiAct) {
      case kEpiGelu: with_residual(std::integral_constant<unsigned, kEpiGelu>{}); break;
      case kEpiSilu: with_residual(std::integral_constant<unsigned, kEpiSilu>{}); break;
      case kEpiRelu: with_residual(std::integral_constant<unsigned, kEpiRelu>{}); break;
      case kEpiTanh: with_residual(std::integral_constant<unsigned, kEpiTanh>{}); break;
      default: with_residual(std::integral_constant<unsigned, 0u>{}); break;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const int col = m0 + wn * C::TN + j * 32 + frow;
    if (col >= p.m) continue;
    const float b = (p.flags & kEpiBias) && first ? p.bias[col] : 0.f;
    const float b2 = (p.flags & kEpiBias) && first && col < p.dual ? p.bias[p.m + col] : 0.f;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = n0 + wm * C::TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < p.n) {
          float* yp = p.y + static_cast<long long>(row) * p.ystride + col;
          float o = acc[i][j][v] + b;
          if (split) {
            unsafeAtomicAdd(yp, p.alpha * o);  // Y already holds the old values (residual, no activation)
            if (p.dual > 0 && col < p.dual) unsafeAtomicAdd(yp + p.m, p.alpha * (acc[i][j][v] + b2));
          } else {
            if (p.dual > 0 && col < p.dual) {
              float o2 = p.alpha * activation(acc[i][j][v] + b2, p.flags);
              if (p.flags & kEpiResidual) o2 += yp[p.m];
              yp[p.m] = o2;
            }
            o = p.alpha * activation(o, p.flags);
            if (p.flags & kEpiResidual) o += *yp;
            *yp = o;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// bf16 weights: a deeper pipeline (k step BK, NSTAGE LDS slots, NSTAGE-1 steps in flight).
//  * Both operands stream from global memory straight into LDS with global_load_lds_dwordx4, so
//    the loads in flight hold no registers; X stays f32 in LDS and is rounded to bf16 (nearest
//    even) as its fragments are read -- or, on the f32-accurate path, split there into three
//    exact bf16 parts that take three MFMAs into the same accumulator.
//  * The loads are waited for with explicit vmcnt counts (wq_lds_dma.hpp).
//  * The k step is 64: a step then takes whole 128-byte lines of every W row (and two of every X
//    row). With a step of 32, each W row gives 64 bytes per step, and such half-line pieces
//    stream into LDS at about 60% of the rate of whole lines (measured on MI355X).
//  * LDS rows are XOR-swizzled by row so that the 16 lanes served per LDS cycle read 16 distinct
//    groups of four banks (64 banks): chunk c of 16 bytes in row r sits at c ^ s(r), where s(r)
//    is r divided by the rows that fill the 64 banks, modulo the chunks per row: for k step 64,
//    X rows (64 f32 = 16 chunks) use r & 15 and W rows (64 bf16 = 8 chunks) (r >> 1) & 7.
//  * A direct-to-LDS load writes lane l's 16 bytes at (LDS base + 16 l); each lane fetches the
//    global chunk that belongs at its LDS position. Rows past the end of X or W are clamped to the
//    last row (their products land only in outputs that are never stored).

// Swizzles for a k step of BK elements: rows of 4 BK bytes (X, f32) or 2 BK bytes (W, bf16).
template <int BK>
__device__ __forceinline__ int x_swizzle(int r) {
  return (r >> (BK == 32 ? 1 : 0)) & (BK / 4 - 1);
}
template <int BK>
__device__ __forceinline__ int w_swizzle(int r) {
  return (r >> (BK == 32 ? 2 : 1)) & (BK / 8 - 1);
}

// XB: X arrives as bf16 bit patterns (a producer already rounded it), staged like W. YB: outputs
// are stored as bf16 bit patterns, rounded to nearest even (no residual, no dual outputs): the
// encoder block hands activations from one product to the next that way, since the next product
// rounds them to bf16 anyway. XR: f32 X arrives by register loads and is rounded to bf16 (nearest
// even, as at fragment reads) once per element as it is written to LDS, in XB's layout; W keeps
// its direct-to-LDS loads. Half the LDS bytes and reads of X, no rounding in every reading wave,
// the same products and sums as the f32 staging (2-slot ring only).
template <int BM, int BN, int WM, int WN, int NSTAGE, int BK, bool SPLIT, bool XB = false, bool YB = false,
          bool XR = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(GemmParams p, int tiles_m, int tiles_n, int band) {
  static_assert(BK == 32 || BK == 64, "k step");
  static_assert(!(SPLIT && (XB || YB)), "the f32-accurate path takes f32 X and Y");
  static_assert(!XR || (!XB && !SPLIT && NSTAGE == 2 && BK == 64), "X rounded once: f32 X, 2-slot ring");
  constexpr int kXC = BK / 4, kWC = BK / 8;  // 16-byte chunks per X row and per W row
  constexpr int kWaves = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr bool kXb16 = XB || XR;                  // X sits in LDS as bf16
  constexpr int kABytes = BM * BK * (kXb16 ? 2 : 4);  // f32 (bf16 when XB or XR)
  constexpr int kBBytes = BN * BK * 2;  // bf16
  constexpr int kStageBytes = kABytes + kBBytes;
  // XR: X arrives by register loads (kXI 16-byte f32 chunks per thread per step), rounded once.
  constexpr int kXI = XR ? BM * BK * 4 / 16 / (64 * kWaves) : 0;
  static_assert(!XR || (BM * BK * 4 / 16) % (64 * kWaves) == 0, "X chunks must split evenly");
  constexpr int kAInst = XR ? 0 : kABytes / 1024 / kWaves;  // direct-to-LDS loads per wave per step
  constexpr int kBInst = kBBytes / 1024 / kWaves;
  constexpr int kInst = kAInst + kBInst;
  constexpr int P = NSTAGE - 1;  // steps in flight
  static_assert((XR || kABytes % (1024 * kWaves) == 0) && kBBytes % (1024 * kWaves) == 0, "step must split evenly");
  static_assert(kInst * (P - 1) < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) uint8_t ring[NSTAGE * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps addresses in SGPRs
  const int wm = wave / WN;
  const int wn = wave % WN;

  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + 7) / 8;
  const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= tiles) return;  // workgroup-uniform
  // Tiles are numbered in bands of `band` X-tile rows, down each band's rows first: an XCD's
  // contiguous range of tile numbers is then a band x (range / band) block, which reads fewer
  // distinct X and W panels than whole columns of tiles would.
  const int band_tiles = band * tiles_n;
  const int b = t / band_tiles;
  const int r = t - b * band_tiles;
  const int rows = min(band, tiles_m - b * band);
  const int tile_m = b * band + r % rows;
  const int tile_n = r / rows;
  const int n0 = tile_m * BM;
  const int m0 = tile_n * BN;
  const int nk = p.k / BK;

  // Per-lane source offsets (bytes) of this wave's direct-to-LDS loads, for k step 0.
  uint32_t aoff[kAInst > 0 ? kAInst : 1], boff[kBInst];
#pragma unroll
  for (int i = 0; i < kAInst; ++i) {
    const int L = (wave * kAInst + i) * 64 + lane;  // 16-byte chunk index in a step's X region
    if constexpr (XB) {  // rows of 2 BK bytes, swizzled as W's
      const int r = L / kWC, pos = L % kWC;
      const int c = pos ^ w_swizzle<BK>(r);
      aoff[i] = static_cast<uint32_t>(min(n0 + r, p.n - 1)) * static_cast<uint32_t>(p.k) * 2u + c * 16u;
    } else {
      const int r = L / kXC, pos = L % kXC;
      const int c = pos ^ x_swizzle<BK>(r);
      aoff[i] = static_cast<uint32_t>(min(n0 + r, p.n - 1)) * static_cast<uint32_t>(p.k) * 4u + c * 16u;
    }
  }
#pragma unroll
  for (int i = 0; i < kBInst; ++i) {
    const int L = (wave * kBInst + i) * 64 + lane;
    const int r = L / kWC, pos = L % kWC;
    const int c = pos ^ w_swizzle<BK>(r);
    boff[i] = static_cast<uint32_t>(min(m0 + r, p.m - 1)) * static_cast<uint32_t>(p.rowbytes) + c * 16u;
  }
  const uint32_t ring_lds = lds_address(ring);
  // XR: chunk L = i * threads + tid of a step's BM x BK f32 block (row L / kXC, four values at
  // column 4 (L % kXC)); its bf16 goes to the XB layout (rows of 2 BK bytes, swizzled as W's).
  uint32_t xoff[kXI > 0 ? kXI : 1];
  int xdst[kXI > 0 ? kXI : 1];
#pragma unroll
  for (int i = 0; i < kXI; ++i) {
    const int L = i * 64 * kWaves + tid;
    const int r = L / kXC, c4 = L % kXC;
    xoff[i] = static_cast<uint32_t>(min(n0 + r, p.n - 1)) * static_cast<uint32_t>(p.k) * 4u + c4 * 16u;
    xdst[i] = r * BK * 2 + (((c4 >> 1) ^ w_swizzle<BK>(r)) << 4) + (c4 & 1) * 8;
  }

  auto issue = [&](int s) {
    const uint32_t lst = ring_lds + (s % NSTAGE) * kStageBytes;
#pragma unroll
    for (int i = 0; i < kAInst; ++i) load_lds16(p.x, aoff[i] + s * (BK * (XB ? 2u : 4u)), lst + (wave * kAInst + i) * 1024);
#pragma unroll
    for (int i = 0; i < kBInst; ++i)
      load_lds16(p.w, boff[i] + s * (BK * 2u), lst + kABytes + (wave * kBInst + i) * 1024);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int frow = lane & 31;
  const int khalf = lane >> 5;  // which 8 of the 16 k of an MFMA step

  // The epilogue's bias is fetched now, long before it is needed.
  float bias_v[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = min(m0 + wn * TN + j * 32 + frow, p.m - 1);
    bias_v[j] = (p.flags & kEpiBias) ? p.bias[col] : 0.f;
  }

  // The k step s from ring slot s % NSTAGE.
  auto compute = [&](int s) {
    const uint8_t* st = ring + (s % NSTAGE) * kStageBytes;
    const float* sa = reinterpret_cast<const float*>(st);
    const __bf16* sb = reinterpret_cast<const __bf16*>(st + kABytes);
    float4 ra[2][FM][2];
    bf16x8 fa[2][FM];
    bf16x8 fb[2][FN];
    const __bf16* sab = reinterpret_cast<const __bf16*>(st);
    auto read_frags = [&](int ks, int slot) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * TM + i * 32 + frow;
        if constexpr (kXb16) {
          const int c = 2 * ks + khalf;
          fa[slot][i] = *reinterpret_cast<const bf16x8*>(sab + r * BK + ((c ^ w_swizzle<BK>(r)) << 3));
        } else {
          const int c0 = 4 * ks + 2 * khalf;  // two f32 chunks: k = 16 ks + 8 khalf .. +8
          const int sw = x_swizzle<BK>(r);
          ra[slot][i][0] = *reinterpret_cast<const float4*>(sa + r * BK + ((c0 ^ sw) << 2));
          ra[slot][i][1] = *reinterpret_cast<const float4*>(sa + r * BK + (((c0 + 1) ^ sw) << 2));
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * TN + j * 32 + frow;
        const int c = 2 * ks + khalf;
        fb[slot][j] = *reinterpret_cast<const bf16x8*>(sb + r * BK + ((c ^ w_swizzle<BK>(r)) << 3));
      }
    };
    // Fragments of two 16-wide k slices are in registers at a time: slice ks + 2 is read into
    // the slot of slice ks once its MFMAs are issued.
    read_frags(0, 0);
    read_frags(1, 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int slot = ks & 1;
      bf16x8 a[FM], am[FM], al[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (SPLIT) {
          uint2 l1, l2, l3, h1, h2, h3;
          split3_bf16x4(ra[slot][i][0], l1, l2, l3);
          split3_bf16x4(ra[slot][i][1], h1, h2, h3);
          a[i] = __builtin_bit_cast(bf16x8, make_uint4(l1.x, l1.y, h1.x, h1.y));
          am[i] = __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
          al[i] = __builtin_bit_cast(bf16x8, make_uint4(l3.x, l3.y, h3.x, h3.y));
        } else if constexpr (kXb16) {
          a[i] = fa[slot][i];
        } else {
          const uint2 l2 = round_bf16x4(ra[slot][i][0]), h2 = round_bf16x4(ra[slot][i][1]);
          a[i] = __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], fb[slot][j], acc[i][j], 0, 0, 0);
      if constexpr (SPLIT) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[i], fb[slot][j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], fb[slot][j], acc[i][j], 0, 0, 0);
          }
      }
      if (ks + 2 < BK / 16) read_frags(ks + 2, slot);
    }
  };

  if constexpr (XR) {
    // X by register loads, rounded to bf16 once per element as it is written to LDS; W by
    // direct-to-LDS loads. Iteration s: wait for this wave's W of step s (only the X loads of step
    // s + 1, issued after it, stay outstanding), barrier, write X of step s + 1 (its loads are then
    // the only ones in flight, so the compiler's wait for them is exact) and issue W of step s + 1
    // into the slot step s - 1 used, load X of step s + 2 into registers, compute step s.
    float4 xr[kXI > 0 ? kXI : 1];
    auto xload = [&](int s) {
#pragma unroll
      for (int i = 0; i < kXI; ++i)
        xr[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const uint8_t*>(p.x) + xoff[i] + s * (BK * 4u));
    };
    auto xstore = [&](int s) {
      uint8_t* dst = ring + (s % NSTAGE) * kStageBytes;
#pragma unroll
      for (int i = 0; i < kXI; ++i) *reinterpret_cast<uint2*>(dst + xdst[i]) = round_bf16x4(xr[i]);
    };
    issue(0);
    xload(0);
    xstore(0);
    if (nk > 1) xload(1);
    for (int s = 0; s < nk; ++s) {
      if (s + 1 < nk) wait_vmcnt<kXI>();
      else wait_vmcnt<0>();
      __syncthreads();  // X and W of step s are in LDS; the slot of step s - 1 is free
      if (s + 1 < nk) {
        xstore(s + 1);
        issue(s + 1);
      }
      if (s + 2 < nk) xload(s + 2);
      compute(s);
    }
  } else {
    // Prologue: steps 0..P-1 in flight.
#pragma unroll
    for (int s = 0; s < P; ++s)
      if (s < nk) issue(s);

    for (int s = 0; s < nk; ++s) {
      // Wait for this wave's loads of step s: those of the later steps issued so far stay outstanding.
      wait_groups<kInst, P - 1>(min(P - 1, nk - 1 - s));
      __syncthreads();  // every wave's step-s data is in LDS; the slot of step s-1 is free
      if (s + P < nk) issue(s + P);
      compute(s);
    }
  }

  // The epilogue, with the flag tests taken once per workgroup and the bounds tests only on
  // tiles that reach past the edge of Y.
  const bool full = n0 + BM <= p.n && m0 + BN <= p.m;
  // Tiles inside Y: no per-output branch. A guarded load or store per output compiles to a branch
  // whose entry waits for every outstanding memory operation (the previous outputs' stores
  // included), which serialises the tile's stores. Here Y is addressed through a buffer resource
  // at the tile's corner: one 32-bit offset per fragment and lane, plus a scalar row offset per
  // output, so the old values load back to back and the stores issue without waits between
  // them. Taken when the tile's byte offsets fit in 31 bits.
  constexpr int kYBytes = YB ? 2 : 4;
  const bool fast = full && p.dual == 0 &&
                    (static_cast<long long>(BM) * p.ystride + BN) * kYBytes < (1LL << 31);
  auto store_full = [&](auto act, auto res) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<uint8_t*>(p.y) + (static_cast<long long>(n0) * p.ystride + m0) * kYBytes, 0, 0x7FFFFFFF,
        0x00020000);
    const int rs = p.ystride * kYBytes;  // bytes per row of Y
    float old[FM][FN][16];
    if constexpr (decltype(res)::value) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int vo = (wm * TM + i * 32 + 4 * (lane >> 5)) * rs + (wn * TN + j * 32 + frow) * 4;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            old[i][j][v] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, vo, (8 * (v >> 2) + (v & 3)) * rs, 0));
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int vo = (wm * TM + i * 32 + 4 * (lane >> 5)) * rs + (wn * TN + j * 32 + frow) * kYBytes;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float o = acc[i][j][v] + bias_v[j];
          if constexpr (decltype(act)::value != 0) o = activation(o, decltype(act)::value);
          o *= p.alpha;
          if constexpr (decltype(res)::value) o += old[i][j][v];
          // The buffer builtins move integers: the value's bits go through unchanged.
          if constexpr (YB)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, static_cast<__bf16>(o)), rsrc, vo,
                                                  (8 * (v >> 2) + (v & 3)) * rs, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, o), rsrc, vo, (8 * (v >> 2) + (v & 3)) * rs, 0);
        }
      }
  };
  auto store = [&](auto act, auto res) {
    if (fast) {
      store_full(act, res);
      return;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = m0 + wn * TN + j * 32 + frow;
      if (!full && col >= p.m) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = n0 + wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (full || row < p.n) {
            float o = acc[i][j][v] + bias_v[j];
            if constexpr (decltype(act)::value != 0) o = activation(o, decltype(act)::value);
            o *= p.alpha;
            if constexpr (YB) {
              reinterpret_cast<__bf16*>(p.y)[static_cast<long long>(row) * p.ystride + col] = static_cast<__bf16>(o);
            } else {
              float* yp = p.y + static_cast<long long>(row) * p.ystride + col;
              if constexpr (decltype(res)::value) o += *yp;
              *yp = o;
            }
          }
        }
      }
    }
    // wavo's dual outputs: columns below `dual` are stored again at m + col, with bias[m + col].
    // A second pass, taken only by waves that own such columns, keeps the store above unchanged.
    if (!YB && p.dual > m0 + wn * TN) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = m0 + wn * TN + j * 32 + frow;
        if (col >= p.dual) continue;
        const float b2 = (p.flags & kEpiBias) ? p.bias[p.m + col] : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = n0 + wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row < p.n) {
              float* yq = p.y + static_cast<long long>(row) * p.ystride + p.m + col;
              float o = acc[i][j][v] + b2;
              if constexpr (decltype(act)::value != 0) o = activation(o, decltype(act)::value);
              o *= p.alpha;
              if constexpr (decltype(res)::value) o += *yq;
              *yq = o;
            }
          }
        }
      }
    }
  };
  auto with_residual = [&](auto act) {
    if (!YB && (p.flags & kEpiResidual)) store(act, std::true_type{});
    else store(act, std::false_type{});
  };
  switch (p.flags & kEpiAct) {
    case kEpiGelu: with_residual(std::integral_constant<unsigned, kEpiGelu>{}); break;
    case kEpiSilu: with_residual(std::integral_constant<unsigned, kEpiSilu>{}); break;
    case kEpiRelu: with_residual(std::integral_constant<unsigned, kEpiRelu>{}); break;
    case kEpiTanh: with_residual(std::integral_constant<unsigned, kEpiTanh>{}); break;
    default: with_residual(std::integral_constant<unsigned, 0u>{}); break;
  }
}

int device_cus() {
  static std::atomic<int> cus[64];  // filled on first use; concurrent callers store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

constexpr int kLdsBytes = 160 * 1024;

// LDS of gemm_kernel: X (x_parts buffers) and W (weight_parts buffers), each double-buffered, plus
// the block scales of quantized weights.
constexpr int gemm_lds_bytes(int wt, int bm, int bn, int x_parts) {
  return 2 * bm * LDS_STRIDE * 2 * x_parts + 2 * bn * LDS_STRIDE * 2 * weight_parts(wt) +
         (plain_type(wt) ? 8 : 2 * bn * 2 * 4);
}

template <int WT, int BM, int BN, int WM, int WN>
hipError_t launch_tile(const GemmParams& p, hipStream_t stream) {
  // X in three parts needs three A buffers in LDS (and f16 / f32 weights two or three B buffers):
  // only the tiles whose buffers fit in LDS are built. The launcher never picks another.
  constexpr bool kFits1 = gemm_lds_bytes(WT, BM, BN, 1) <= kLdsBytes;
  constexpr bool kFits3 = gemm_lds_bytes(WT, BM, BN, 3) <= kLdsBytes;
  void (*kernel)(GemmParams, int, int) = nullptr;
  if (p.x_parts == 3) {
    if constexpr (kFits3) kernel = gemm_kernel<WT, BM, BN, WM, WN, true>;
  } else {
    if constexpr (kFits1) kernel = gemm_kernel<WT, BM, BN, WM, WN, false>;
  }
  if (kernel == nullptr) return hipErrorInvalidValue;
  const int tiles_m = (p.n + BM - 1) / BM;
  const int tiles_n = (p.m + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  int splits = 1;
  // Split the k range when the tiles alone leave most CUs idle and the
  // epilogue allows adding partial sums into Y (accumulate, no activation).
  const int nk = (p.k + BK - 1) / BK;
  if ((p.flags & kEpiResidual) && !(p.flags & kEpiAct)) {
    const int cus = device_cus();
    while (tiles * splits * 2 <= cus * 3 / 2 && nk / (splits * 2) >= 4) splits *= 2;
  }
  const int per_xcd = (tiles + 7) / 8;
  dim3 grid(per_xcd * 8, 1, splits);
  hipLaunchKernelGGL(kernel, grid, dim3(64 * WM * WN), 0, stream, p, tiles_m, tiles_n);
  return hipGetLastError();
}

// Band height for the tile order: the divisor of an XCD's tile count closest to its square
// root (no taller than the tile grid), so each XCD works on a near-square block of tiles.
int tile_band(int tiles_m, int per_xcd) {
  int best = 1;
  for (int d = 1; d <= per_xcd && d <= tiles_m; ++d)
    if (per_xcd % d == 0 && std::abs(d * d - per_xcd) < std::abs(best * best - per_xcd)) best = d;
  return best;
}

template <int BM, int BN, int WM, int WN, int NSTAGE, int BK>
hipError_t launch_bf16(const GemmParams& p, hipStream_t stream) {
  const int tiles_m = (p.n + BM - 1) / BM;
  const int tiles_n = (p.m + BN - 1) / BN;
  const int per_xcd = (tiles_m * tiles_n + 7) / 8;
  auto kernel = p.x_parts == 3 ? gemm_bf16_kernel<BM, BN, WM, WN, NSTAGE, BK, true>
                               : gemm_bf16_kernel<BM, BN, WM, WN, NSTAGE, BK, false>;

  hipLaunchKernelGGL(kernel, dim3(per_xcd * 8), dim3(64 * WM * WN), 0, stream, p, tiles_m, tiles_n,
                     tile_band(tiles_m, per_xcd));
  return hipGetLastError();
}

// The same tiles with X rounded once as it is staged (XR, 2-slot ring) on the plain path; the
// f32-accurate path keeps the direct-to-LDS kernel.
template <int BM, int BN, int WM, int WN>
hipError_t launch_bf16_xr(const GemmParams& p, hipStream_t stream) {
  if (p.x_parts == 3) return launch_bf16<BM, BN, WM, WN, 2, 64>(p, stream);
  const int tiles_m = (p.n + BM - 1) / BM;
  const int tiles_n = (p.m + BN - 1) / BN;
  const int per_xcd = (tiles_m * tiles_n + 7) / 8;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, 2, 64, false, false, false, true>), dim3(per_xcd * 8),
                     dim3(64 * WM * WN), 0, stream, p, tiles_m, tiles_n, tile_band(tiles_m, per_xcd));
  return hipGetLastError();
}

// bf16 X and / or bf16 Y (x_bf16, y_bf16; bf16 weights, k a multiple of 64, operands under 4 GiB):
// the products inside the encoder block. Tiles from the measurements at n = 1500 with X in bf16
// (QKV 18.3-19.0 us, output projection 10.0, MLP up 22.9, MLP down 28.6 us, against 20.8 / 12.6 /
// 31.8 / 36.8 us with f32 X): 64 x 128 tiles of 8 waves when there are more than one per CU, else
// 64 x 64 tiles of 4 waves with a 3-slot ring.
hipError_t launch_bf16_io(const GemmParams& p, hipStream_t stream) {
  if (p.k % 64 != 0 || p.x_parts != 1 || (p.y_bf16 && (p.dual != 0 || (p.flags & kEpiResidual))) ||
      static_cast<long long>(p.n) * p.k * (p.x_bf16 ? 2 : 4) >= (1LL << 32) ||
      static_cast<long long>(p.m) * p.rowbytes >= (1LL << 32))
    return hipErrorInvalidValue;
  const long long small_tiles = static_cast<long long>((p.n + 63) / 64) * ((p.m + 127) / 128);
  const bool wide = small_tiles > device_cus();
  void (*kernel)(GemmParams, int, int, int) = nullptr;
  int bm = 64, bn = wide ? 128 : 64, threads = wide ? 512 : 256;
  if (p.x_bf16 && p.y_bf16)
    kernel = wide ? gemm_bf16_kernel<64, 128, 2, 4, 2, 64, false, true, true> : gemm_bf16_kernel<64, 64, 2, 2, 3, 64, false, true, true>;
  else if (p.x_bf16)
    kernel = wide ? gemm_bf16_kernel<64, 128, 2, 4, 2, 64, false, true, false> : gemm_bf16_kernel<64, 64, 2, 2, 3, 64, false, true, false>;
  else
    kernel = wide ? gemm_bf16_kernel<64, 128, 2, 4, 2, 64, false, false, true> : gemm_bf16_kernel<64, 64, 2, 2, 3, 64, false, false, true>;
  const int tiles_m = (p.n + bm - 1) / bm;
  const int tiles_n = (p.m + bn - 1) / bn;
  const int per_xcd = (tiles_m * tiles_n + 7) / 8;
  hipLaunchKernelGGL(kernel, dim3(per_xcd * 8), dim3(threads), 0, stream, p, tiles_m, tiles_n, tile_band(tiles_m, per_xcd));
  return hipGetLastError();
}

// Test hook: with WQ_GEMM_WIDE_OFFSETS=1 in the environment (read once per process), every bf16
// GEMM takes the route that X or W of 4 GiB or more take, so that route can be checked at
// shapes a test can afford.
bool force_wide_offsets() {
  static const bool on = [] {
    const char* v = std::getenv("WQ_GEMM_WIDE_OFFSETS");
    return v != nullptr && v[0] == '1' && v[1] == '\0';
  }();
  return on;
}

template <int WT>
hipError_t launch_wt(const GemmParams& p, hipStream_t stream) {
  // The pipelined bf16 kernel addresses operands with 32-bit byte offsets; larger operands take
  // gemm_kernel, whose offsets are 64-bit.
  const bool small_enough = static_cast<long long>(p.n) * p.k * 4 < (1LL << 32) &&
                            static_cast<long long>(p.m) * p.rowbytes < (1LL << 32) && !force_wide_offsets();
  if constexpr (WT == kBF16) {
    if (!small_enough) return launch_tile<WT, 128, 128, 2, 2>(p, stream);
    const long long wide_tiles = static_cast<long long>((p.n + 127) / 128) * ((p.m + 255) / 256);
    const long long mid_tiles = static_cast<long long>((p.n + 127) / 128) * ((p.m + 127) / 128);
    if (p.k % 64 == 0) {
      // A k step of 64 (k a multiple of 64). Measured on MI355X over n x m x k from
      // 256 x 2048 x 2048 to 8192 x 8192 x 4096:
      //  * a 128 x 256 tile for every CU: those tiles (fewest operand re-reads);
      //  * more 64 x 128 tiles than CUs: tiles two workgroups per CU (2-slot rings), so one
      //    tile's epilogue and stores overlap the other's k loop. A round is two tiles per CU:
      //    64 x 128 tiles when they fit one round or 64 x 192 tiles do not either, else 64 x 192
      //    tiles of 4 waves (one round instead of a thin second one: 1500 x 3072 x 1024
      //    26.5 -> 19.1 us). With more than two 64 x 128 tiles per CU, X is rounded once as it
      //    is staged (XR): 48 KB of LDS per workgroup instead of 64 KB, so three fit on a CU
      //    (1500 x 4096 x 1024 + GELU 30.5 -> 27.0 us, 1500 x 4096 x 4096 91.5 -> 82.9 us); with
      //    up to two per CU the f32 staging was as fast or faster (2048^3 31.4 both,
      //    1500 x 2048 x 1024 15.6 against 17.4 us);
      //  * fewer: 64 x 64 tiles of 4 waves when the tiles are very few or k is short (more
      //    tiles in flight), else 64 x 128 tiles with a 4-slot ring.
      const int cus = device_cus();
      const long long small_tiles = static_cast<long long>((p.n + 63) / 64) * ((p.m + 127) / 128);
      const long long tall_tiles = static_cast<long long>((p.n + 63) / 64) * ((p.m + 191) / 192);
      if (wide_tiles >= cus) return launch_bf16<128, 256, 2, 4, 2, 64>(p, stream);
      if (small_tiles > 2LL * cus && tall_tiles <= 2LL * cus) return launch_bf16<64, 192, 2, 2, 2, 64>(p, stream);
      if (small_tiles > 2LL * cus) return launch_bf16_xr<64, 128, 2, 4>(p, stream);
      if (small_tiles > cus) return launch_bf16<64, 128, 2, 4, 2, 64>(p, stream);
      if (small_tiles <= cus / 2 || p.k <= 1024) {
        // At most four k steps: a 2-slot ring (64 x 256 x 256 + bias + GELU 5.4 -> 5.0 us). At
        // k = 1024 it is slower than 3 slots (the 24-layer chain 2.68 -> 2.72 ms).
        if (p.k <= 256) return launch_bf16<64, 64, 2, 2, 2, 64>(p, stream);
        return launch_bf16<64, 64, 2, 2, 3, 64>(p, stream);
      }
      return launch_bf16<64, 128, 2, 4, 4, 64>(p, stream);
    }
    // k an odd multiple of 32 (k step 32): measured at n = 1500, 128 x 256 tiles win once they
    // give at least half the CUs a tile; below that, 128 x 128 tiles (more of them) do.
    if (wide_tiles >= device_cus() / 2) return launch_bf16<128, 256, 2, 4, 4, 32>(p, stream);
    if (mid_tiles >= device_cus() / 2) return launch_bf16<128, 128, 2, 4, 4, 32>(p, stream);
    return launch_bf16<64, 128, 2, 4, 8, 32>(p, stream);
  }
  // 8 waves per workgroup (two per SIMD, which hides the register-staged loads): 128 x 256 tiles
  // once there are two per CU, 64 x 128 tiles below (measured on MI355X from 256 x 2048 x 2048 to
  // 4096^3; at n = 1500 about 1.7x faster than 4-wave 128 x 256 / 128 x 128 tiles).
  // (X in three parts takes 64 x 128 tiles: the parts of a 128-row tile do not fit in LDS beside W.)
  if constexpr (WT == kF32 || WT == kF16) {
    // f16 / f32 weights enter as two / three bf16 parts: 64 x 128 tiles, or 64 x 64 tiles of 4
    // waves where f32 weights meet X in three parts (their six buffers fit no larger tile).
    if (WT == kF32 && p.x_parts == 3) return launch_tile<WT, 64, 64, 2, 2>(p, stream);
    return launch_tile<WT, 64, 128, 2, 4>(p, stream);
  } else {
    const long long wide_tiles = static_cast<long long>((p.n + 127) / 128) * ((p.m + 255) / 256);
    if (wide_tiles >= 2LL * device_cus() && p.x_parts == 1) return launch_tile<WT, 128, 256, 2, 4>(p, stream);
    return launch_tile<WT, 64, 128, 2, 4>(p, stream);
  }
}

}  // namespace

hipError_t launch_gemm(int wtype, const GemmParams& p, hipStream_t stream) {
  if (p.x_bf16 || p.y_bf16) return wtype == kBF16 ? launch_bf16_io(p, stream) : hipErrorInvalidValue;
  switch (wtype) {
    case kBF16: return launch_wt<kBF16>(p, stream);
    case kQ8_0: return launch_wt<kQ8_0>(p, stream);
    case kQ4_0: return launch_wt<kQ4_0>(p, stream);
    case kF32: return launch_wt<kF32>(p, stream);
    case kF16: return launch_wt<kF16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wq
