// Matvec / MoE path for k a multiple of 1024 (up to 8192): the main small-n kernel.
//
// Same contract as the general matvec kernel: y[t][j] = epilogue(sum_k x[t][k] w[j][k])
// (cortiq-engine src/gpu_wgpu/nemotron_audio.rs `ae_gemm`/`ae_put`; wavo
// src/gpu/mod.rs `Pass::gemv`), and per-slot MoE outputs
// y[s][j] = sum_k W[ids[s]][j][k] x[s / top_k][k] (hanzo-ml src/wgpu_backend.rs
// `moe_matvec_gpu`), all in f32.
//
// Layout of the work (gfx950, wave64):
//  * A workgroup has k/SLICE waves (SLICE = 1024 or 512 elements of k); wave w owns
//    the k-slice [SLICE w, SLICE w + SLICE) of every row, and each lane owns
//    E = SLICE/64 elements of it (16 or 8), in 32/E lanes per 32-element block.
//    Its activations for up to NTC tokens sit in E*NTC VGPRs, loaded once per
//    workgroup and reused for every row it visits. Narrower slices spread a
//    tile's arithmetic over more waves, so fewer workgroups per CU (each of which
//    loads the whole activation rows) keep the same bytes in flight.
//  * The workgroup walks a run of row tiles (R consecutive rows each, i.e. one
//    contiguous run of bytes). The waves stream each tile straight into a shared
//    ring of NSTAGE LDS slots with direct-to-LDS loads, each wave a contiguous
//    share of the tile's 1024-byte loads, NSTAGE-1 tiles ahead of the one being
//    computed; one barrier per tile publishes it to all waves. The loads hold no
//    registers while in flight.
//  * Element ownership per 32-element block (q = lane's index among the block's
//    32/E lanes):
//      bf16, Q8_0: elements E q .. E q + E-1;
//      Q4_0:       quant bytes (E/2) q .. (E/2) q + E/2-1, i.e. those elements
//                  (low nibbles) and the same 16 further on (high nibbles). A
//                  byte select (SDWA) feeds each nibble to v_cvt_off_f32_i4,
//                  which yields (q-8)/16 exactly once the nibble is XOR-ed with
//                  8; the block scale is taken as 16 d to compensate.
//  * A lane's E products per row and token are summed in f32 and scaled once by
//    the block scale. The 64 lane partials of the R rows are then summed by a
//    register transpose (v_permlane32_swap, v_permlane16_swap, DPP): each step
//    halves the values a lane holds, so R rows cost about R adds per lane instead
//    of 6 R.
//  * A wave leaves its per-row partial sums in LDS. Every flush_rows rows the
//    workgroup adds the k-slices of each row in wave order, applies the epilogue
//    and stores. An epilogue that reads memory (bias, residual) would make
//    the compiler wait for every ring load in flight, so such launches give each
//    workgroup at most one flush of rows.
//  * Q4_K (k a multiple of 256): the unit is the 144-byte super-block of 256 weights, so 256/E
//    lanes share one. A lane's E elements E q .. E q + E-1 lie in one 32-element sub-block j, whose
//    quants are one nibble (low for even j, high for odd j) of E consecutive bytes. The lane sums
//    x q over them (q unsigned, exact in f32) and finishes with d sc_j * that - dmin m_j * sum(x),
//    the sum of its activations being formed once per token group.
//  * MoE: the grid is dealt over the experts the ids touch (wq_moe_sched.hpp; for banks of more
//    than 256 experts blockIdx.y is the expert), and a ballot over the ids finds the expert's slots.
//  * Rounding: an E-term chain, one scale, a 6-level tree and at most 16 slice
//    additions per output -- far inside 1e-5 * sum |x w|. For Q4_K the lane's closing
//    d sc_j s - dmin m_j sum(x) rounds relative to d sc_j sum|x q| + dmin m_j sum|x|, which exceeds
//    sum |x w| by the cancellation inside a sub-block whose weights straddle zero.
#include <hip/hip_runtime.h>

#include <atomic>

#include "wq_decode.hpp"
#include "wq_internal.hpp"
#include "wq_lds_dma.hpp"
#include "wq_moe_sched.hpp"
#include "wq_tile_math.hpp"

namespace wq {
namespace {

template <int WT, int SLICE>
struct Slice {
  static_assert(SLICE == 1024 || SLICE == 512, "k elements per wave: 1024 or 512");
  static constexpr int kBlockElems = WT == kQ4_K ? kQ4KElems : 32;  // Q4_K: the super-block
  static constexpr int BB = WT == kQ4_K ? kQ4KBytes : block_bytes(WT);
  static constexpr int E = SLICE / 64;                         // elements per lane and row
  static constexpr int kLanesPerBlock = kBlockElems / E;       // 2 or 4 (Q4_K: 16 or 32)
  static constexpr int kSegBytes = SLICE / kBlockElems * BB;   // one wave's slice of a row
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

// Rows whose per-wave partial sums a workgroup holds in LDS before it adds them up: 128, or
// fewer where NTC * MAXW partials per row would take more than 16 KB.
constexpr int flush_rows(int ntc, int maxw) { return 4096 / (ntc * maxw) < 128 ? 4096 / (ntc * maxw) : 128; }

// Decodes this lane's E weights of one block held in LDS at byte `boff` from `lds`
// (element order as described above) and returns the factor that scales their sum.
template <int WT, int E>
__device__ __forceinline__ float decode_lane(const uint8_t* lds, int boff, int q, float (&wv)[E]) {
  if constexpr (WT == kBF16 || WT == kF16) {
    const uint32_t* a = reinterpret_cast<const uint32_t*>(lds + boff + 2 * E * q);
    uint32_t w[E / 2];
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(a)[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      if constexpr (WT == kBF16) {
        wv[2 * i] = bf16_lo(w[i]);
        wv[2 * i + 1] = bf16_hi(w[i]);
      } else {
        wv[2 * i] = f16_to_f32(w[i] & 0xFFFFu);
        wv[2 * i + 1] = f16_to_f32(w[i] >> 16);
      }
    }
    return 1.f;
  } else if constexpr (WT == kF32) {
    const float4* a = reinterpret_cast<const float4*>(lds + boff + 4 * E * q);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 v = a[i];
      wv[4 * i] = v.x;
      wv[4 * i + 1] = v.y;
      wv[4 * i + 2] = v.z;
      wv[4 * i + 3] = v.w;
    }
    return 1.f;
  } else if constexpr (WT == kQ8_0) {
    const float d = f16_to_f32(*reinterpret_cast<const uint16_t*>(lds + boff));
    const int qo = boff + 2 + E * q;  // quants E q .. E q + E-1
    const uint32_t sh = static_cast<uint32_t>(qo) & 3u;
    const uint32_t* a = reinterpret_cast<const uint32_t*>(lds) + (qo >> 2);
    uint32_t dw[E / 4 + 1];
#pragma unroll
    for (int i = 0; i < E / 4 + 1; ++i) dw[i] = a[i];
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const uint32_t v = realign(dw[i + 1], dw[i], sh);
#pragma unroll
      for (int b = 0; b < 4; ++b) wv[4 * i + b] = q8_at(v, b);
    }
    return d;
  } else {
    const float d = f16_to_f32(*reinterpret_cast<const uint16_t*>(lds + boff));
    const int qo = boff + 2 + (E / 2) * q;  // quant bytes (E/2) q .. (E/2) q + E/2-1
    const uint32_t sh = static_cast<uint32_t>(qo) & 3u;
    const uint32_t* a = reinterpret_cast<const uint32_t*>(lds) + (qo >> 2);
    uint32_t dw[E / 8 + 1];
#pragma unroll
    for (int i = 0; i < E / 8 + 1; ++i) dw[i] = a[i];
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      const uint32_t lo = realign(dw[i + 1], dw[i], sh) ^ 0x88888888u;
      const uint32_t hi = __builtin_amdgcn_alignbit(lo, lo, 4);  // high nibbles into the low ones
      wv[4 * i] = __builtin_amdgcn_cvt_off_f32_i4(lo);
      wv[E / 2 + 4 * i] = __builtin_amdgcn_cvt_off_f32_i4(hi);
#pragma unroll
      for (int b = 1; b < 4; ++b) {
        wv[4 * i + b] = __builtin_amdgcn_cvt_off_f32_i4((lo >> (8 * b)) & 0xFFu);
        wv[E / 2 + 4 * i + b] = __builtin_amdgcn_cvt_off_f32_i4((hi >> (8 * b)) & 0xFFu);
      }
    }
    return 16.f * d;
  }
}

// Where a lane's Q4_K quants and sub-block fields sit in its super-block (lane-constant).
struct Q4KLane {
  int qs_off;  // byte offset of its E quant bytes from the super-block start
  int nib;     // 0: low nibbles (even sub-block), 4: high nibbles (odd sub-block)
  int lo_off;  // bit offset of the field's low 6 bits (j < 4) or top 2 bits (j >= 4) in bytes 4-7 / 8-11
  int lo_w;    // 6 or 2
  int hi_shl;  // 0 or 4: where those bits go
  int nb_off;  // bit offset of the field's low nibble in bytes 12-15 (j >= 4)
  int nb_w;    // 0 (j < 4) or 4
};

// Super-block layout (GGML k-quant, the type hanzo-ml src/wgpu_backend.rs `matvec_q4k_gpu` takes):
// bytes 0-1 f16 d, 2-3 f16 dmin, 4-15 the 6-bit scales sc_j and mins m_j of the eight sub-blocks
// (j < 4: low 6 bits of bytes 4+j and 8+j; j >= 4: low / high nibble of byte 8+j, top 2 bits
// from the top of bytes j and 4+j), 16-143 the quants (sub-blocks 2c, 2c+1 in the low / high
// nibbles of bytes 16+32c ..).
template <int E>
__device__ __forceinline__ Q4KLane q4k_lane(int q) {
  const int j = E * q / 32;      // the lane's sub-block
  const int o = E * q % 32;      // its first element within the sub-block
  const int jj = j & 3, hi = j >> 2;
  return Q4KLane{16 + 32 * (j >> 1) + o, 4 * (j & 1), 8 * jj + 6 * hi, hi ? 2 : 6, 4 * hi, 8 * jj, 4 * hi};
}

// The lane's E quants of the super-block at byte `boff` of `lds`, as floats in wv; returns
// (d sc_j, dmin m_j), both exact in f32.
template <int E>
__device__ __forceinline__ float2 decode_q4k(const uint8_t* lds, int boff, const Q4KLane& c, float (&wv)[E]) {
  const uint4 h = *reinterpret_cast<const uint4*>(lds + boff);  // d | dmin, scale bytes 0-3, 4-7, 8-11
  const uint32_t sc = (__builtin_amdgcn_ubfe(h.y, c.lo_off, c.lo_w) << c.hi_shl) |
                      __builtin_amdgcn_ubfe(h.w, c.nb_off, c.nb_w);
  const uint32_t mn = (__builtin_amdgcn_ubfe(h.z, c.lo_off, c.lo_w) << c.hi_shl) |
                      __builtin_amdgcn_ubfe(h.w, c.nb_off + 4, c.nb_w);
  uint32_t dw[E / 4];
  if constexpr (E == 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(lds + boff + c.qs_off);
    dw[0] = v.x;
    dw[1] = v.y;
    dw[2] = v.z;
    dw[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(lds + boff + c.qs_off);
    dw[0] = v.x;
    dw[1] = v.y;
  }
  // A byte 0000qqqq read as FP8 E4M3 is q * 2^-9 exactly (q = 0..15), so one conversion with
  // scale 2^9 gives two quants as f32.
#pragma unroll
  for (int i = 0; i < E / 4; ++i) {
    const uint32_t v = (dw[i] >> c.nib) & 0x0F0F0F0Fu;
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 512.f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 512.f, true);
    wv[4 * i] = lo[0];
    wv[4 * i + 1] = lo[1];
    wv[4 * i + 2] = hi[0];
    wv[4 * i + 3] = hi[1];
  }
  return make_float2(f16_to_f32(h.x & 0xFFFFu) * static_cast<float>(sc),
                     f16_to_f32(h.x >> 16) * static_cast<float>(mn));
}

// First element, within the lane's k-slice, of the j-th run of 4 activations the lane
// multiplies (E/4 runs, in the order of decode_lane's weights).
template <int WT, int E>
__device__ __forceinline__ int x_run(int lane, int j) {
  constexpr int kElems = WT == kQ4_K ? kQ4KElems : 32;
  const int bl = lane / (kElems / E), q = lane % (kElems / E);
  if constexpr (WT == kQ4_0) return bl * 32 + (E / 2) * q + (j < E / 8 ? 4 * j : 16 + 4 * (j - E / 8));
  return bl * kElems + E * q + 4 * j;
}

template <int WT, int NTC, int R, int NSTAGE, int MAXW, int SLICE>
__global__ __launch_bounds__(64 * MAXW) void matvec_sliced_kernel(MatvecParams p, int tiles_per_wg) {
  using S = Slice<WT, SLICE>;
  constexpr int E = S::E;
  constexpr int kFlushRows = flush_rows(NTC, MAXW);
  // A tile is R consecutive rows: R * rowbytes contiguous bytes, moved by 1024-byte loads.
  constexpr int kMaxLoads = (R * MAXW * S::kSegBytes + 1023) / 1024;
  // +16: the covering dwords of the tile's last block may reach 4 bytes past it.
  constexpr int kSlotBytes = kMaxLoads * 1024 + 16;
  // Every wave issues at least this many of a tile's loads (at most one more).
  constexpr int kMinPerWave = R * S::kSegBytes / 1024;
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
  __shared__ uint32_t touched_lds[kMoeCompactMax / 32];
  int e = blockIdx.y;
  const bool moe = p.ids != nullptr;
  const int ntiles = (p.m + R - 1) / R;
  int t_begin = blockIdx.x * tiles_per_wg;
  int t_end = min(ntiles, t_begin + tiles_per_wg);
  if (moe && p.moe_compact) {
    const MoeAssign a = moe_assign(p, ntiles, tiles_per_wg, touched_lds);
    e = a.e;
    t_begin = a.t_begin;
    t_end = a.t_end;
    if (e < 0) return;  // workgroup-uniform: no expert is touched
  }
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
    const int last = tile_last_load(tile_bytes, p.m, row0, p.rowbytes);
    const uint32_t dst = ring_addr + static_cast<uint32_t>((tile % NSTAGE) * kSlotBytes);
    for (int i = ld0; i < ld1; ++i)
      load_lds16<true>(base, static_cast<uint32_t>(min(i * 1024 + lane * 16, last)), dst + i * 1024);
  };

  const int q = lane % S::kLanesPerBlock;
  const int blk_off = wave * S::kSegBytes + (lane / S::kLanesPerBlock) * S::BB;  // this lane's block in a row
  const Q4KLane qk = q4k_lane<E>(q);  // used by Q4_K only

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

      float xr[NTC][E];
#pragma unroll
      for (int t = 0; t < NTC; ++t) {
        if (slot[t] >= 0) {
          const float* xs = p.x + static_cast<long long>(slot[t] / p.top_k) * p.k + wave * SLICE;
#pragma unroll
          for (int j = 0; j < E / 4; ++j) {
            const float4 v = *reinterpret_cast<const float4*>(xs + x_run<WT, E>(lane, j));
            xr[t][4 * j + 0] = v.x;
            xr[t][4 * j + 1] = v.y;
            xr[t][4 * j + 2] = v.z;
            xr[t][4 * j + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int j = 0; j < E; ++j) xr[t][j] = 0.f;
        }
      }
      float xsum[NTC];  // Q4_K: the sum of the lane's activations, the factor of its sub-block min
#pragma unroll
      for (int t = 0; t < NTC; ++t) {
        xsum[t] = 0.f;
        if constexpr (WT == kQ4_K) {
#pragma unroll
          for (int j = 0; j < E; ++j) xsum[t] += xr[t][j];
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
            float wv[E];
            if constexpr (WT == kQ4_K) {
              const float2 f = decode_q4k<E>(ring_lds, seg + r * rowbytes, qk, wv);
#pragma unroll
              for (int t = 0; t < NTC; ++t) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < E; ++j) s = __builtin_fmaf(xr[t][j], wv[j], s);
                acc[t][r] = __builtin_fmaf(f.x, s, -(f.y * xsum[t]));
              }
            } else {
              const float d = decode_lane<WT, E>(ring_lds, seg + r * rowbytes, q, wv);
#pragma unroll
              for (int t = 0; t < NTC; ++t) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < E; ++j) s = __builtin_fmaf(xr[t][j], wv[j], s);
                acc[t][r] = d * s;
              }
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
            if (!moe) v = epilogue(v, p.flags, p.alpha, p.bias + row, yp);
            *yp = v;
          }
        }
        __syncthreads();  // part is refilled by the next flush
      }
    }
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

// Workgroups of `kernel` that fit on one CU at once; `cache` is the caller's
// per-variant slot (filled on first use).
int groups_per_cu(void (*kernel)(MatvecParams, int), int threads, std::atomic<int>* cache) {
  int v = cache->load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, threads, 0) != hipSuccess || v <= 0) v = 1;
    cache->store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int WT, int NTC, int R, int NSTAGE, int MAXW, int SLICE>
hipError_t launch_r(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  constexpr int kFlushRows = flush_rows(NTC, MAXW);
  const int nw = p.k / SLICE;
  const int ntiles = (p.m + R - 1) / R;
  auto kernel = matvec_sliced_kernel<WT, NTC, R, NSTAGE, MAXW, SLICE>;
  // As many workgroups as are resident at once (no thin second round); each walks a run of tiles
  // with NSTAGE-1 of them in flight. MoE: dealt over the touched experts on the device
  // (wq_moe_sched.hpp), or split evenly over all experts where the bitmap cannot hold them.
  static std::atomic<int> per_cu[17];  // per variant and wave count
  const int resident = groups_per_cu(kernel, 64 * nw, &per_cu[nw]) * device_cus();
  if (p.ids != nullptr && p.n_exp <= kMoeCompactMax && resident >= p.n_exp) {
    MatvecParams q = p;
    q.moe_compact = 1;
    const int tpw = (ntiles + resident - 1) / resident;
    hipLaunchKernelGGL(kernel, dim3(resident, 2), dim3(64 * nw), 0, stream, q, tpw);
    return hipGetLastError();
  }
  const int experts = n_exp_rows > 1 ? n_exp_rows - 1 : 1;
  int groups = resident / experts;
  if (groups < 1) groups = 1;
  if (groups > ntiles) groups = ntiles;
  int tpw = (ntiles + groups - 1) / groups;
  // An epilogue that reads memory (bias, residual) makes the compiler wait for every load in
  // flight, so such launches give each workgroup no more rows than one flush holds.
  if (p.ids == nullptr && (p.flags & (kEpiBias | kEpiResidual)) != 0 && tpw * R > kFlushRows) tpw = kFlushRows / R;
  dim3 grid((ntiles + tpw - 1) / tpw, n_exp_rows);
  hipLaunchKernelGGL(kernel, grid, dim3(64 * nw), 0, stream, p, tpw);
  return hipGetLastError();
}

// Launch shape: rows per tile, ring depth and k elements per wave.
struct Shape {
  int r, nstage, slice;
};

// Shapes per weight type, token count (1, 2, 4, 8) and k class (up to 4096, up to 8192), from
// sweeps on MI355X of Q8_0 and bf16 4096 x k and Q4_0 14336 x 4096 / 4096 x 8192 at each token
// count (the token pair at k = 8192 takes its neighbours' shape). Every workgroup loads the whole
// activation rows, so the winners keep several workgroups per CU with one or two tiles in flight
// each; 512-element slices win where a tile's arithmetic is heavy for its bytes (bf16, many
// tokens), 1024-element slices where decoding dominates (Q4_0, one token).
constexpr Shape sliced_shape(int wt, int ntc, bool k8) {
  if (wt == kQ8_0) {
    if (!k8) return ntc == 1 ? Shape{4, 2, 1024} : ntc == 2 ? Shape{8, 2, 512} : ntc == 4 ? Shape{8, 2, 1024}
                                                                                             : Shape{4, 3, 512};
    return ntc == 8 ? Shape{4, 2, 512} : Shape{4, 2, 1024};
  }
  if (wt == kQ4_0 || wt == kQ4_K) {
    if (!k8) return ntc == 4 ? Shape{4, 3, 1024} : Shape{4, 2, 1024};
    return ntc == 1 ? Shape{8, 2, 1024} : Shape{4, 2, 1024};
  }
  if (wt == kF32) return k8 ? Shape{2, 2, 1024} : Shape{2, 2, 512};  // rows twice bf16's
  return k8 ? Shape{2, 2, 1024} : Shape{4, 2, 512};                  // bf16, f16
}

template <int WT, int NTC, bool K8>
hipError_t launch_shaped(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  constexpr Shape c = sliced_shape(WT, NTC, K8);
  constexpr int kMaxW = (K8 ? 8192 : 4096) / c.slice;
  return launch_r<WT, NTC, c.r, c.nstage, kMaxW, c.slice>(p, n_exp_rows, stream);
}

template <int WT, int NTC>
hipError_t launch_ntc(const MatvecParams& p, int n_exp_rows, hipStream_t stream) {
  if (p.k <= 4096) return launch_shaped<WT, NTC, false>(p, n_exp_rows, stream);
  return launch_shaped<WT, NTC, true>(p, n_exp_rows, stream);
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
    case kF32: return launch_wt<kF32>(p, max_tok, n_exp_rows, stream);
    case kF16: return launch_wt<kF16>(p, max_tok, n_exp_rows, stream);
    case kQ4_K: return launch_wt<kQ4_K>(p, max_tok, n_exp_rows, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wq
