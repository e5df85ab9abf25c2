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
//    of every row, and each lane owns 16 elements of it, in 2 lanes per 32-element
//    block. Its activations for up to NTC tokens sit in 16*NTC VGPRs, loaded once
//    per workgroup and reused for every row it visits.
//  * The workgroup walks a run of row tiles (R consecutive rows each, i.e. one
//    contiguous run of bytes). The waves stream each tile straight into a shared
//    ring of NSTAGE LDS slots with direct-to-LDS loads, each wave a contiguous
//    share of the tile's 1024-byte loads, NSTAGE-1 tiles ahead of the one being
//    computed; one barrier per tile publishes it to all waves. The loads hold no
//    registers while in flight.
//  * Element ownership per 32-element block (half h = lane & 1):
//      bf16, Q8_0: elements 16h .. 16h+15;
//      Q4_0:       bytes 8h .. 8h+7 of the quants, i.e. elements 8h .. 8h+7 (low
//                  nibbles) and 16+8h .. 16+8h+7 (high nibbles). A byte select
//                  (SDWA) feeds each nibble to v_cvt_off_f32_i4, which yields
//                  (q-8)/16 exactly once the nibble is XOR-ed with 8; the block
//                  scale is taken as 16 d to compensate.
//  * A lane's 16 products per row and token are summed in f32 and scaled once by
//    the block scale. The 64 lane partials of the R rows are then summed by a
//    register transpose (v_permlane32_swap, v_permlane16_swap, DPP): each step
//    halves the values a lane holds, so R rows cost about R adds per lane instead
//    of 6 R.
//  * A wave leaves its per-row partial sums in LDS. Every kFlushRows rows the
//    workgroup adds the k-slices of each row in wave order, applies the epilogue
//    and stores. An epilogue that reads memory (bias, residual) would make
//    the compiler wait for every ring load in flight, so such launches give each
//    workgroup at most one flush of rows.
//  * Rounding: a 16-term chain, one scale, a 6-level tree and at most 8 slice
//    additions per output -- far inside 1e-5 * sum |x w|.
#include <hip/hip_runtime.h>

#include "wq_decode.hpp"
#include "wq_internal.hpp"
#include "wq_lds_dma.hpp"

namespace wq {
namespace {

template <int WT>
struct Slice {
  static constexpr int BB = block_bytes(WT);
  static constexpr int kSegBytes = 32 * BB;          // one wave's 1024-element slice of a row
  static constexpr int kSegPieces = kSegBytes / 16;  // 68 (Q8_0), 36 (Q4_0), 128 (bf16)
};

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
  // xor 16: the same per pair of 16-lane groups (with one row left, both operands are that
  // row, and the sum is its total over each 32-lane half).
  if constexpr (R >= 4) {
#pragma unroll
    for (int i = 0; i < R / 4; ++i) {
      auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + R / 4]), false, false);
      v[i] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
  } else {
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false);
    v[0] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
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

// Rows whose per-wave partial sums a workgroup holds in LDS before it adds them up.
constexpr int kFlushRows = 128;

// Decodes this lane's 16 weights of one block held in LDS at byte `boff` from `lds`
// (element order as described above) and returns the factor that scales their sum.
template <int WT>
__device__ __forceinline__ float decode_lane(const uint8_t* lds, int boff, int h, float (&wv)[16]) {
  if constexpr (WT == kBF16) {
    const uint4 a = *reinterpret_cast<const uint4*>(lds + boff + 32 * h);
    const uint4 b = *reinterpret_cast<const uint4*>(lds + boff + 32 * h + 16);
    const uint32_t q[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      wv[2 * i] = bf16_lo(q[i]);
      wv[2 * i + 1] = bf16_hi(q[i]);
    }
    return 1.f;
  } else if constexpr (WT == kQ8_0) {
    const float d = f16_to_f32(*reinterpret_cast<const uint16_t*>(lds + boff));
    const int qo = boff + 2 + 16 * h;  // quants 16h .. 16h+15
    const uint32_t sh = static_cast<uint32_t>(qo) & 3u;
    const uint32_t* a = reinterpret_cast<const uint32_t*>(lds) + (qo >> 2);
    uint32_t dw[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) dw[i] = a[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t q = realign(dw[i + 1], dw[i], sh);
#pragma unroll
      for (int b = 0; b < 4; ++b) wv[4 * i + b] = q8_at(q, b);
    }
    return d;
  } else {
    const float d = f16_to_f32(*reinterpret_cast<const uint16_t*>(lds + boff));
    const int qo = boff + 2 + 8 * h;  // quant bytes 8h .. 8h+7
    const uint32_t sh = static_cast<uint32_t>(qo) & 3u;
    const uint32_t* a = reinterpret_cast<const uint32_t*>(lds) + (qo >> 2);
    uint32_t dw[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) dw[i] = a[i];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t lo = realign(dw[i + 1], dw[i], sh) ^ 0x88888888u;
      const uint32_t hi = __builtin_amdgcn_alignbit(lo, lo, 4);  // high nibbles into the low ones
      wv[4 * i] = __builtin_amdgcn_cvt_off_f32_i4(lo);
      wv[8 + 4 * i] = __builtin_amdgcn_cvt_off_f32_i4(hi);
#pragma unroll
      for (int b = 1; b < 4; ++b) {
        wv[4 * i + b] = __builtin_amdgcn_cvt_off_f32_i4((lo >> (8 * b)) & 0xFFu);
        wv[8 + 4 * i + b] = __builtin_amdgcn_cvt_off_f32_i4((hi >> (8 * b)) & 0xFFu);
      }
    }
    return 16.f * d;
  }
}

// First element, within the lane's 1024-element k-slice, of each run of 8 activations the
// lane multiplies (two runs per block; see the ownership above).
template <int WT>
__device__ __forceinline__ int x_run(int lane, int run) {
  const int bl = lane >> 1, h = lane & 1;
  if constexpr (WT == kQ4_0) return bl * 32 + 8 * h + 16 * run;
  return bl * 32 + 16 * h + 8 * run;
}

template <int WT, int NTC, int R, int NSTAGE, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void matvec_sliced_kernel(MatvecParams p, int tiles_per_wg) {
  using S = Slice<WT>;
  // A tile is R consecutive rows: R * rowbytes contiguous bytes, moved by 1024-byte loads.
  constexpr int kMaxLoads = (R * MAXW * S::kSegBytes + 1023) / 1024;
  // +16: the covering dwords of the tile's last block may reach 4 bytes past it.
  constexpr int kSlotBytes = kMaxLoads * 1024 + 16;
  // Every wave issues at least this many of a tile's loads (at most one more).
  constexpr int kMinPerWave = R * S::BB / 32;
  constexpr int kLanesPerRow = 64 / R;
  constexpr int kFlushTiles = kFlushRows / R;
  static_assert(NSTAGE >= 2 && (kMinPerWave + 1) * (NSTAGE - 2) < 64, "vmcnt range");
  static_assert(kMinPerWave >= 1, "tile too small");
  static_assert(R >= 2 && R <= 16 && (R & (R - 1)) == 0, "rows per tile: a power of two in 2..16");

  __shared__ __attribute__((aligned(16))) uint8_t ring_lds[NSTAGE * kSlotBytes];
  __shared__ float part[kFlushRows * NTC * MAXW];  // [row][token][wave]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  const uint8_t* wexp = p.w + static_cast<long long>(e) * p.expert_bytes;
  const uint32_t ring_addr = lds_address(ring_lds);
  const int rowbytes = static_cast<int>(p.rowbytes);
  const int tile_bytes = R * rowbytes;
  const int n_loads = (tile_bytes + 1023) / 1024;
  // This wave's share of a tile's loads: [ld0, ld1), contiguous bytes of the tile.
  const int ld0 = wave * n_loads / nw;
  const int ld1 = (wave + 1) * n_loads / nw;

  auto issue = [&](int tile) {
    const int row0 = tile * R;
    const uint8_t* base = wexp + static_cast<long long>(row0) * p.rowbytes;
    // Bytes past the end of W (last tile) re-read W's last 16 bytes; never stored.
    const int last = min(tile_bytes, (p.m - row0) * rowbytes) - 16;
    const uint32_t dst = ring_addr + static_cast<uint32_t>((tile % NSTAGE) * kSlotBytes);
    for (int i = ld0; i < ld1; ++i)
      load_lds16(base, static_cast<uint32_t>(min(i * 1024 + lane * 16, last)), dst + i * 1024);
  };

  const int h = lane & 1;
  const int blk_off = wave * S::kSegBytes + (lane >> 1) * S::BB;  // this lane's block in a row

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

      float xr[NTC][16];
#pragma unroll
      for (int t = 0; t < NTC; ++t) {
        if (slot[t] >= 0) {
          const float* xs = p.x + static_cast<long long>(slot[t] / p.top_k) * p.k + wave * 1024;
#pragma unroll
          for (int run = 0; run < 2; ++run) {
            const float4* xp = reinterpret_cast<const float4*>(xs + x_run<WT>(lane, run));
            const float4 v0 = xp[0], v1 = xp[1];
            xr[t][8 * run + 0] = v0.x;
            xr[t][8 * run + 1] = v0.y;
            xr[t][8 * run + 2] = v0.z;
            xr[t][8 * run + 3] = v0.w;
            xr[t][8 * run + 4] = v1.x;
            xr[t][8 * run + 5] = v1.y;
            xr[t][8 * run + 6] = v1.z;
            xr[t][8 * run + 7] = v1.w;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) xr[t][j] = 0.f;
        }
      }

      // Prologue: the first NSTAGE-1 tiles in flight.
#pragma unroll
      for (int s = 0; s < NSTAGE - 1; ++s)
        if (t_begin + s < t_end) issue(t_begin + s);

      for (int f0 = t_begin; f0 < t_end; f0 += kFlushTiles) {
        const int f1 = min(t_end, f0 + kFlushTiles);
        for (int tile = f0; tile < f1; ++tile) {
          // This wave's loads of `tile` have landed once at most those of the later tiles in
          // flight are pending (counted with the smaller per-wave share: may over-wait).
          wait_groups<kMinPerWave, NSTAGE - 2>(min(NSTAGE - 2, t_end - 1 - tile));
          __syncthreads();  // every wave's share of the tile is in; the slot of tile-1 is free
          if (tile + NSTAGE - 1 < t_end) issue(tile + NSTAGE - 1);

          const int seg = (tile % NSTAGE) * kSlotBytes + blk_off;
          float acc[NTC][R];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float wv[16];
            const float d = decode_lane<WT>(ring_lds, seg + r * rowbytes, h, wv);
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
          if ((lane & (kLanesPerRow - 1)) == 0) {
            const int rr = (tile - f0) * R + lane / kLanesPerRow;
#pragma unroll
            for (int t = 0; t < NTC; ++t) part[(rr * NTC + t) * MAXW + wave] = acc[t][0];
          }
        }

        // The k-slices of the waves, added in wave order; then the epilogue and the store.
        __syncthreads();
        const int n_out = (f1 - f0) * R * NTC;
        for (int i = threadIdx.x; i < n_out; i += blockDim.x) {
          const int rr = i / NTC;
          const int t = i - rr * NTC;
          const int row = f0 * R + rr;
          int st_slot = -1;
#pragma unroll
          for (int u = 0; u < NTC; ++u)
            if (u == t) st_slot = slot[u];
          if (row < p.m && st_slot >= 0) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < MAXW; ++w)
              if (w < nw) v += part[i * MAXW + w];
            float* yp = p.y + static_cast<long long>(st_slot) * p.m + row;
            if (!moe) {
              if (p.flags & 1u) v += p.bias[row];
              if (p.flags & 2u) v = gelu_erf(v);
              if (p.flags & 4u) v += *yp;
            }
            *yp = v;
          }
        }
        __syncthreads();  // part is refilled by the next flush
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

template <int WT, int NTC, int R, int NSTAGE, int MAXW>
hipError_t launch_r(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  const int nw = p.k / 1024;
  const int ntiles = (p.m + R - 1) / R;
  auto kernel = matvec_sliced_kernel<WT, NTC, R, NSTAGE, MAXW>;
  // As many workgroups as are resident at once (no thin second round), split over the
  // experts; each walks a run of tiles with NSTAGE-1 of them in flight.
  const int experts = n_exp_rows > 1 ? n_exp_rows - 1 : 1;
  static int per_cu[9];  // per variant and wave count
  int groups = groups_per_cu(kernel, 64 * nw, &per_cu[nw]) * device_cus() / experts;
  if (groups < 1) groups = 1;
  if (groups > ntiles) groups = ntiles;
  int tpw = (ntiles + groups - 1) / groups;
  // An epilogue that reads memory (bias, residual) makes the compiler wait for every load in
  // flight, so such launches give each workgroup no more rows than one flush holds.
  if (p.ids == nullptr && (p.flags & 5u) != 0 && tpw * R > kFlushRows) tpw = kFlushRows / R;
  dim3 grid((ntiles + tpw - 1) / tpw, n_exp_rows);
  hipLaunchKernelGGL(kernel, grid, dim3(64 * nw), 0, stream, p, tpw);
  return hipGetLastError();
}

// Rows per tile and ring depth for each weight type, token count and wave count, from sweeps on
// MI355X (Q8_0 4096x4096 at n = 1 and 4, Q4_0 14336x4096 at n = 1, bf16 4096x4096 at n = 1, and
// the 16-token top-2-of-8 Q4_0 MoE): one tile in flight per workgroup with several workgroups per
// CU beat deeper rings, and taller tiles pay off once several tokens share each decoded weight.
// Eight-wave variants (k above 4096) halve the tile to stay inside the LDS.
template <int WT, int NTC, int MAXW>
struct SlicedShape {
  static constexpr int R0 = WT == kBF16 ? (NTC >= 8 ? 2 : 4) : (NTC >= 4 ? 8 : 4);
  static constexpr int R = MAXW > 4 && R0 > 2 ? R0 / 2 : R0;
  static constexpr int NSTAGE = 2;
};

template <int WT, int NTC, int R4, int R8, int NSTAGE>
hipError_t launch_shape(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  if (p.k <= 4096) return launch_r<WT, NTC, R4, NSTAGE, 4>(p, n_exp_rows, stream);
  return launch_r<WT, NTC, R8, NSTAGE, 8>(p, n_exp_rows, stream);
}

template <int WT, int NTC>
hipError_t launch_ntc(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  using C4 = SlicedShape<WT, NTC, 4>;
  using C8 = SlicedShape<WT, NTC, 8>;
  static_assert(C4::NSTAGE == C8::NSTAGE, "one ring depth per token count");
  return launch_shape<WT, NTC, C4::R, C8::R, C4::NSTAGE>(p, n_exp_rows, stream);
}

template <int WT>
hipError_t launch_wt(const MatvecParams& p, int max_tok, int n_exp_rows, hipStream_t stream) {
  if (max_tok <= 1) return launch_ntc<WT, 1>(p, n_exp_rows, stream);
  if (max_tok <= 2) return launch_ntc<WT, 2>(p, n_exp_rows, stream);
  if (max_tok <= 4) return launch_ntc<WT, 4>(p, n_exp_rows, stream);
  return launch_ntc<WT, 8>(p, n_exp_rows, stream);
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
