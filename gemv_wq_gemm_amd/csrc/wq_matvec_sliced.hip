// Matvec / MoE path for k a multiple of 1024 (up to 8192): the main small-n kernel.
//
// Same contract as the general matvec kernel: y[t][j] = epilogue(sum_k x[t][k] w[j][k])
// (cortiq-engine src/gpu_wgpu/nemotron_audio.rs `ae_gemm`/`ae_put`; wavo
// src/gpu/mod.rs `Pass::gemv`), and per-slot MoE outputs
// y[s][j] = sum_k W[ids[s]][j][k] x[s / top_k][k] (hanzo-ml src/wgpu_backend.rs
// `moe_matvec_gpu`), all in f32.
//
// Layout of the work (gfx950, wave64):
//  * A workgroup has k/1024 waves; wave w owns the k-slice [1024 w, 1024 w + 1024)
//    of every row, and lane l owns 16 elements of it: half h = l & 1 of block
//    32 w + l/2. Its activations for up to NTC tokens sit in 16*NTC VGPRs and
//    are loaded once per workgroup, then reused for every row it visits.
//  * The workgroup walks a run of row tiles (R rows each). For a tile, each wave
//    copies its slice of the R rows (R contiguous segments of 32 blocks) into
//    its LDS region with 16-byte loads spread evenly over the 64 lanes; the next
//    tile's loads are in flight while the current tile is computed.
//  * A lane's 16 products per row and token are summed in f32 and scaled once by
//    the block's f16 scale. The 64 lane partials of the R rows are then summed
//    by a register transpose (v_permlane32_swap, v_permlane16_swap, DPP): each
//    step halves the values a lane holds, so R rows cost about R adds per lane
//    instead of 6 R. The k-slices of the waves are added in wave order through
//    LDS, and one lane per (row, token) applies the epilogue and stores.
//  * Rounding: a 16-term chain, one scale, a 6-level tree and at most 8 slice
//    additions per output -- far inside 1e-5 * sum |x w|.
#include <hip/hip_runtime.h>

#include "wq_decode.hpp"
#include "wq_internal.hpp"

namespace wq {
namespace {

template <int WT>
struct Slice {
  static constexpr int BB = block_bytes(WT);
  static constexpr int kSegBytes = 32 * BB;          // one wave's 1024-element slice of a row
  static constexpr int kSegPieces = kSegBytes / 16;  // 68 (Q8_0), 36 (Q4_0), 128 (bf16)
};

__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sums v[0..R) over the 64 lanes of the wave. On return, lane l holds in v[0]
// the total of row (l >> (6 - log2 R)); each row's total is in 64/R lanes.
template <int R>
__device__ __forceinline__ void transpose_sum(float (&v)[R], int lane) {
  // xor 32: v_permlane32_swap(a, b) leaves a's lower half and b's lower half in
  // the first result, the upper halves in the second; their sum holds row a
  // in lanes 0-31 and row b in lanes 32-63.
  if constexpr (R >= 2) {
#pragma unroll
    for (int i = 0; i < R / 2; ++i) {
      auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + R / 2]), false, false);
      v[i] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
  }
  // xor 16: the same per pair of 16-lane groups.
  if constexpr (R >= 4) {
#pragma unroll
    for (int i = 0; i < R / 4; ++i) {
      auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + R / 4]), false, false);
      v[i] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
  }
  // xor 8 (rotate by 8 inside 16 lanes): lanes with bit 3 clear keep the lower
  // half of their values and send the upper half, the others the reverse.
  if constexpr (R >= 8) {
    const bool hi = lane & 8;
#pragma unroll
    for (int i = 0; i < R / 8; ++i) {
      const float keep = hi ? v[i + R / 8] : v[i];
      const float send = hi ? v[i] : v[i + R / 8];
      v[i] = keep + dpp<0x128>(send);
    }
  } else {
    v[0] += dpp<0x128>(v[0]);
  }
  // xor 4 (mirror inside 8 lanes pairs lanes whose bit 2 differs).
  if constexpr (R >= 16) {
    const bool hi = lane & 4;
    const float keep = hi ? v[1] : v[0];
    const float send = hi ? v[0] : v[1];
    v[0] = keep + dpp<0x141>(send);
  } else {
    v[0] += dpp<0x141>(v[0]);
  }
  v[0] += dpp<0x4E>(v[0]);  // xor 2 inside quads
  v[0] += dpp<0xB1>(v[0]);  // xor 1 inside quads
}

template <int WT, int NTC, int R, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void matvec_sliced_kernel(MatvecParams p, int tiles_per_wg) {
  using S = Slice<WT>;
  constexpr int kTilePieces = R * S::kSegPieces;
  constexpr int NL = (kTilePieces + 63) / 64;  // 16-byte loads per lane per tile
  constexpr int kLanesPerRow = 64 / R;

  // +16: the covering dwords of a wave's last block may reach 4 bytes past its region.
  __shared__ __attribute__((aligned(16))) uint8_t seg_lds[MAXW * R * S::kSegBytes + 16];
  __shared__ float cw[2][MAXW * R * NTC];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int e = blockIdx.y;
  const bool moe = p.ids != nullptr;
  const int ntiles = (p.m + R - 1) / R;
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
        for (int row = t_begin * R + threadIdx.x; row < min(p.m, t_end * R); row += blockDim.x)
          p.y[static_cast<long long>(slot) * p.m + row] = __builtin_nanf("");
      }
    }
    return;
  }

  uint8_t* seg = seg_lds + wave * (R * S::kSegBytes);
  const uint8_t* wexp = p.w + static_cast<long long>(e) * p.expert_bytes;

  // Loop-invariant part of this lane's load addresses: piece q = lane + 64 i of
  // the tile is 16 bytes of row q / P at slice offset 16 (q % P).
  int off[NL];
  int prow[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int q = lane + 64 * i;
    const int r = q / S::kSegPieces;
    prow[i] = q < kTilePieces ? r : R;  // R marks a lane with no piece here
    off[i] = r * static_cast<int>(p.rowbytes) + wave * S::kSegBytes + (q - r * S::kSegPieces) * 16;
  }

  // This lane's share of a row: half h of block bl of the wave's slice.
  const int bl = lane >> 1;
  const int h = lane & 1;
  const int kofs = wave * 1024 + lane * 16;  // first of its 16 elements

  auto issue = [&](int tile, uint4 (&st)[NL]) {
    const int row0 = tile * R;
    const uint8_t* base = wexp + static_cast<long long>(row0) * p.rowbytes;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (prow[i] < R && row0 + prow[i] < p.m) v = *reinterpret_cast<const uint4*>(base + off[i]);
      st[i] = v;
    }
  };

  int parity = 0;
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

      uint4 st[NL];
      issue(t_begin, st);

      float xr[NTC][16];
#pragma unroll
      for (int t = 0; t < NTC; ++t) {
        if (slot[t] >= 0) {
          const float4* xp = reinterpret_cast<const float4*>(
              p.x + static_cast<long long>(slot[t] / p.top_k) * p.k + kofs);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 v = xp[i];
            xr[t][4 * i] = v.x;
            xr[t][4 * i + 1] = v.y;
            xr[t][4 * i + 2] = v.z;
            xr[t][4 * i + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) xr[t][j] = 0.f;
        }
      }

      for (int tile = t_begin; tile < t_end; ++tile) {
        // Stage this tile's slice into LDS, then start the next tile's loads.
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < NL; ++i)
          if (prow[i] < R) reinterpret_cast<uint4*>(seg)[lane + 64 * i] = st[i];
        wave_lds_sync();
        if (tile + 1 < t_end) issue(tile + 1, st);

        float acc[NTC][R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint8_t* blk = seg + r * S::kSegBytes + bl * S::BB;
          float wv[16];
          float d = 1.f;
          if constexpr (WT == kBF16) {
            const uint4 a = *reinterpret_cast<const uint4*>(blk + 32 * h);
            const uint4 b = *reinterpret_cast<const uint4*>(blk + 32 * h + 16);
            const uint32_t q[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              wv[2 * i] = bf16_lo(q[i]);
              wv[2 * i + 1] = bf16_hi(q[i]);
            }
          } else {
            d = f16_to_f32(*reinterpret_cast<const uint16_t*>(blk));
            // The 16 bytes this lane needs: Q8_0 quants 16h..16h+15; Q4_0 all 16.
            const int qo = static_cast<int>(blk - seg_lds) + 2 + (WT == kQ8_0 ? 16 * h : 0);
            const uint32_t sh = static_cast<uint32_t>(qo) & 3u;
            const uint32_t* a = reinterpret_cast<const uint32_t*>(seg_lds) + (qo >> 2);
            uint32_t dw[5];
#pragma unroll
            for (int i = 0; i < 5; ++i) dw[i] = a[i];
            uint32_t q[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = realign(dw[i + 1], dw[i], sh);
            if constexpr (WT == kQ8_0) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int b = 0; b < 4; ++b) wv[4 * i + b] = q8_at(q[i], b);
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t qx = (q[i] ^ 0x88888888u) >> (4 * h);
#pragma unroll
                for (int b = 0; b < 4; ++b) wv[4 * i + b] = q4_at(qx, 2 * b);
              }
            }
          }
#pragma unroll
          for (int t = 0; t < NTC; ++t) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) s = __builtin_fmaf(xr[t][j], wv[j], s);
            acc[t][r] = d * s;
          }
        }

#pragma unroll
        for (int t = 0; t < NTC; ++t) transpose_sum<R>(acc[t], lane);

        float* cwb = cw[parity];
        if ((lane & (kLanesPerRow - 1)) == 0) {
          const int rho = lane / kLanesPerRow;
#pragma unroll
          for (int t = 0; t < NTC; ++t) cwb[(wave * R + rho) * NTC + t] = acc[t][0];
        }
        __syncthreads();
        if (threadIdx.x < R * NTC) {
          const int rho = threadIdx.x / NTC;
          const int t = threadIdx.x - rho * NTC;
          const int row = tile * R + rho;
          int st_slot = -1;
#pragma unroll
          for (int u = 0; u < NTC; ++u)
            if (u == t) st_slot = slot[u];
          if (row < p.m && st_slot >= 0) {
            float v = 0.f;
            for (int w = 0; w < nw; ++w) v += cwb[(w * R + rho) * NTC + t];
            float* yp = p.y + static_cast<long long>(st_slot) * p.m + row;
            if (!moe) {
              if (p.flags & 1u) v += p.bias[row];
              if (p.flags & 2u) v = gelu_erf(v);
              if (p.flags & 4u) v += *yp;
            }
            *yp = v;
          }
        }
        parity ^= 1;
      }
    }
  }
}

int device_cus() {
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

// Workgroups of `kernel` that fit on one CU at once; `cache` is the caller's
// per-variant slot (filled on first use).
int groups_per_cu(void (*kernel)(MatvecParams, int), int threads, int* cache) {
  if (*cache <= 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, threads, 0) != hipSuccess || v <= 0) v = 1;
    *cache = v;
  }
  return *cache;
}

template <int WT, int NTC, int R>
hipError_t launch_r(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  const int nw = p.k / 1024;
  const int ntiles = (p.m + R - 1) / R;
  auto kernel = nw <= 4 ? matvec_sliced_kernel<WT, NTC, R, 4> : matvec_sliced_kernel<WT, NTC, R, 8>;
  // As many workgroups as are resident at once (no thin second round), split
  // over the experts; each walks a run of tiles with the next tile in flight.
  const int experts = n_exp_rows > 1 ? n_exp_rows - 1 : 1;
  static int per_cu[9];  // per variant and wave count
  int groups = groups_per_cu(kernel, 64 * nw, &per_cu[nw]) * device_cus() / experts;
  if (groups < 1) groups = 1;
  if (groups > ntiles) groups = ntiles;
  const int tpw = (ntiles + groups - 1) / groups;
  dim3 grid((ntiles + tpw - 1) / tpw, n_exp_rows);
  hipLaunchKernelGGL(kernel, grid, dim3(64 * nw), 0, stream, p, tpw);
  return hipGetLastError();
}

// Rows per tile: the largest that compiles without spills for this weight type
// and token count (more rows per tile = fewer, wider reductions).
template <int WT, int NTC>
constexpr int rows_big() {
  if constexpr (WT == kBF16) return NTC >= 4 ? 4 : 8;
  if constexpr (WT == kQ8_0) return NTC >= 2 ? 8 : 16;
  return NTC >= 4 ? 8 : 16;
}

template <int WT, int NTC>
hipError_t launch_ntc(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  constexpr int RBIG = rows_big<WT, NTC>();
  constexpr int RSMALL = RBIG > 4 ? RBIG / 2 : 4;
  const long long tiles_big = (static_cast<long long>(p.m) + RBIG - 1) / RBIG * (n_exp_rows > 1 ? n_exp_rows - 1 : 1);
  if (tiles_big >= 512) return launch_r<WT, NTC, RBIG>(p, n_exp_rows, stream);
  return launch_r<WT, NTC, RSMALL>(p, n_exp_rows, stream);
}

template <int WT>
hipError_t launch_wt(const MatvecParams& p, int max_tok, int n_exp_rows, hipStream_t stream) {
  if (max_tok <= 1) return launch_ntc<WT, 1>(p, n_exp_rows, stream);
  if (max_tok <= 2) return launch_ntc<WT, 2>(p, n_exp_rows, stream);
  return launch_ntc<WT, 4>(p, n_exp_rows, stream);
}

}  // namespace

bool matvec_sliced_supports(int k) { return k % 1024 == 0 && k >= 1024 && k <= 8192; }

hipError_t launch_matvec_sliced(int wtype, const MatvecParams& p, int max_tok, hipStream_t stream) {
  const int n_exp_rows = p.ids ? p.n_exp + 1 : 1;
  switch (wtype) {
    case kBF16: return launch_wt<kBF16>(p, max_tok, n_exp_rows, stream);
    case kQ8_0: return launch_wt<kQ8_0>(p, max_tok, n_exp_rows, stream);
    case kQ4_0: return launch_wt<kQ4_0>(p, max_tok, n_exp_rows, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wq
