// The MoE matvec on matrix cores, with f32 accuracy (Q8_0, Q4_0 and Q4_K weights); also the plain
// layer at 9 to 16 tokens.
//
// Contract: per routed slot s and output row j, y[s][j] = sum_k W[ids[s]][j][k] x[s / top_k][k]
// (hanzo-ml src/wgpu_backend.rs `moe_matvec_gpu`), the same as the f32 matvec kernels. Without
// ids (the plain layer) every slot takes the one weight and the store applies the epilogue
// (bias, activation, alpha, + old Y).
//
// Why matrix cores: with f32 FMAs every weight costs one instruction per routed slot, so an
// expert's several slots make the kernel bound by the vector ALU, not by HBM. Here each weight
// is decoded once and v_mfma_f32_16x16x32_bf16 applies it to up to 16 slots.
//
// Exactness:
//  * Each activation is split into three bf16 parts, x = x1 + x2 + x3, with x1 = bf16(x),
//    x2 = bf16(x - x1), x3 = bf16(x - x1 - x2), all rounded to nearest even. Both differences are
//    exact in f32, and the last part holds the at most 8 bits left, so the three parts add up to x
//    exactly (outside the bottom of the exponent range).
//  * The integer quants q (Q8_0) and q - 8 (Q4_0, taken as (q - 8) / 16 against activations
//    times 16) are exact in bf16, and products of two bf16 values are exact in f32.
//  * Q4_K (hanzo-ml `matvec_q4k_gpu`; GGML's k-quant super-block of 256 weights in 144 bytes): the
//    unsigned quants q (0..15) enter as they are, and each 32-element sub-block j adds
//    d sc_j * (its MFMA sum of x q) - dmin m_j * (the sum of its activations), the activation sums
//    being formed once per group of slots. A wave's slice is one or two whole super-blocks.
//  * One 32-element block is one MFMA's k: three chained MFMAs (one per activation part, sharing
//    the decoded weights) sum the block's products into a fresh 16x16 f32 tile, which the block's
//    scale then multiplies and adds to the running sum in f32. So only f32 additions round: the
//    products of a block, SB blocks per wave, and k/(32 SB) waves -- well inside 1e-5 * sum |x w|.
//
// Layout of the work (gfx950, wave64):
//  * A workgroup has k/(32 SB) waves; wave w owns SB blocks of every row, the k-slice
//    [32 SB w, 32 SB (w + 1)). Both types take SB = 8 (up to 16 waves): the activation parts of a
//    256-element slice need half the registers of a 512-element one, so four waves fit on each
//    SIMD instead of two and hide each other's LDS and barrier waits (9-10% faster for both
//    types, on the MoE workload and on the plain layer at 12 and 16 tokens). Q8_0 tiles are
//    twice as large, so its 16 waves keep a single buffer of partial sums (PB = 1). MFMA roles: A = activations (16 slots x 32 k), B = weights (32 k x 16 weight
//    rows), D[t][j] in lane 16 (t / 4) + j, value t % 4.
//  * Lane l = 16 o + j: weight row j of the tile and k-octet o of each block (Q8_0: elements
//    8o..8o+7; Q4_0: 4o..4o+3 and 16+4o..16+4o+3, see decode_octet); as A it holds slot j at the
//    same octet. Its three activation parts for the SB blocks of its
//    slice (12 SB VGPRs) are built once per group of slots and reused for every tile.
//  * A tile is 16 consecutive weight rows, streamed by the workgroup into a ring of NSTAGE LDS
//    slots with direct-to-LDS loads (each wave a share of the rows, 1024 bytes per load, the last
//    load of a row on the lanes with bytes left), NSTAGE-1 tiles ahead; one barrier per tile
//    publishes it. Rows sit at a stride of their length + 16 bytes: row strides that are
//    multiples of 128 bytes would put the 16 rows one operand read touches into one LDS bank.
//    From a 4-byte aligned per-lane base, every block's LDS offsets are compile-time constants.
//  * Each wave writes its 16x16 partial sums to LDS; after the next tile's barrier the workgroup
//    adds the k-slices in wave order and stores.
//  * MoE: the grid is dealt over the experts the ids touch (wq_moe_sched.hpp; for banks of more
//    than 256 experts blockIdx.y is the expert); a ballot over the ids picks the expert's slots,
//    16 per pass, so each touched expert's rows stream once per 16 of its slots. A second grid row
//    writes NaN for slots whose id is out of range.
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "wq_decode.hpp"
#include "wq_internal.hpp"
#include "wq_lds_dma.hpp"
#include "wq_moe_sched.hpp"

namespace wq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 16;     // weight rows per tile: the MFMA's N
constexpr int kMaxK = 4096;
constexpr int kSlots = 16;        // routed slots per pass: the MFMA's M
constexpr int kSchedBlocks = 2;   // blocks the scheduler may interleave

// bf16 bit patterns of two f32 values that bf16 holds exactly, packed low | high << 16.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// (q - 8) / 16 of the Q4_0 nibble in byte b of a word already XOR-ed with 0x88888888 (and shifted
// so the wanted nibbles are the low ones of each byte).
__device__ __forceinline__ float q4_byte(uint32_t word, int b) {
  return __builtin_amdgcn_cvt_off_f32_i4(b == 0 ? word : (word >> (8 * b)) & 0xFFu);
}

// The 8 weights of k-octet o of block BLK of this lane's row slice, as MFMA B operand, and the
// factor that scales their products. `q_base` (4-byte aligned) is the LDS byte offset of the
// slice's first block plus the lane's quant offset (8 o for Q8_0, 4 o for Q4_0); `s_base` is the
// slice's first block. Every other offset is a compile-time constant.
//  * Q8_0: octet o is elements 8o .. 8o+7 (quant bytes 8o .. 8o+7).
//  * Q4_0: octet o is elements 4o .. 4o+3 and 16+4o .. 16+4o+3: the low and high nibbles of quant
//    bytes 4o .. 4o+3, one dword. The MFMA sums over k in any order, so the activations (A) take
//    the same order; this layout needs one quant dword, XOR and shift per block instead of two.
template <int WT, int BLK>
__device__ __forceinline__ bf16x8 decode_octet(const uint8_t* lds, int q_base, int s_base, float& scale) {
  constexpr int BB = block_bytes(WT);
  constexpr int kQ = BLK * BB + 2;  // first quant byte of the block, from an aligned base
  constexpr int kSh = kQ & 3;       // 0 or 2
  const float d = f16_to_f32(*reinterpret_cast<const uint16_t*>(lds + s_base + BLK * BB));
  const uint32_t* a = reinterpret_cast<const uint32_t*>(lds + q_base) + (kQ >> 2);
  uint4 u;
  if constexpr (WT == kQ4_0) {
    const uint32_t q = kSh == 0 ? a[0] : realign(a[1], a[0], kSh);
    const uint32_t lo = q ^ 0x88888888u;  // nibbles of elements 4o .. 4o+3 in the low halves
    // And of 16+4o .. 16+4o+3, by a rotate the compiler keeps (a plain shift would be folded into
    // each byte extract, which then loses its byte select).
    const uint32_t hi = __builtin_amdgcn_alignbit(lo, lo, 4);
    u.x = bf16_pair(q4_byte(lo, 0), q4_byte(lo, 1));
    u.y = bf16_pair(q4_byte(lo, 2), q4_byte(lo, 3));
    u.z = bf16_pair(q4_byte(hi, 0), q4_byte(hi, 1));
    u.w = bf16_pair(q4_byte(hi, 2), q4_byte(hi, 3));
    scale = d;  // (q - 8) / 16 here; the activations enter times 16 (exact)
    return __builtin_bit_cast(bf16x8, u);
  }
  uint32_t q0, q1;
  if constexpr (kSh == 0) {
    q0 = a[0];
    q1 = a[1];
  } else {
    const uint32_t d0 = a[0], d1 = a[1], d2 = a[2];
    q0 = realign(d1, d0, kSh);
    q1 = realign(d2, d1, kSh);
  }
  u.x = bf16_pair(q8_at(q0, 0), q8_at(q0, 1));
  u.y = bf16_pair(q8_at(q0, 2), q8_at(q0, 3));
  u.z = bf16_pair(q8_at(q1, 0), q8_at(q1, 1));
  u.w = bf16_pair(q8_at(q1, 2), q8_at(q1, 3));
  scale = d;
  return __builtin_bit_cast(bf16x8, u);
}

// The three bf16 parts of 8 activations (see the exactness note above).
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8& p1, bf16x8& p2, bf16x8& p3) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h1 = static_cast<__bf16>(x[i]);
    const float r1 = x[i] - static_cast<float>(h1);
    const __bf16 h2 = static_cast<__bf16>(r1);
    p1[i] = h1;
    p2[i] = h2;
    p3[i] = static_cast<__bf16>(r1 - static_cast<float>(h2));
  }
}

// The 8 quants of k-octet o of Q4_K sub-block j, as MFMA B operand (q exact in bf16): nibble
// SH / 4 (low for even j, high for odd j) of bytes 8o .. 8o+7 of the 32 bytes that sub-blocks j and
// j^1 share, given as the two dwords d0, d1.
// A byte 0000qqqq read as an FP8 E4M3 pattern is q * 2^-9 for every q in 0..15 (exponent field 0
// or 1, three mantissa bits: subnormal q/8 * 2^-6 below 8, (1 + (q-8)/8) * 2^-6 from 8), so one
// v_cvt_scalef32_pk_bf16_fp8 with scale 2^9 turns two masked nibbles into two exact bf16 quants
// (per-byte float conversions and packing took 3.5 times the instructions: 110 -> 97 us on the
// MoE of 16 tokens top-2 of 8 experts of 14336 x 4096). Decoding each row's eight sub-block factors
// once and sharing them over the row's four lanes through LDS measured slower (126 us): the extra
// registers spill.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int SH>
__device__ __forceinline__ bf16x8 q4k_octet(uint32_t d0, uint32_t d1) {
  const uint32_t l0 = (d0 >> SH) & 0x0F0F0F0Fu, l1 = (d1 >> SH) & 0x0F0F0F0Fu;
  uint4 u;
  u.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(l0, 512.f, false));
  u.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(l0, 512.f, true));
  u.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(l1, 512.f, false));
  u.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(l1, 512.f, true));
  return __builtin_bit_cast(bf16x8, u);
}

// (d sc_j, dmin m_j) of sub-block j of a Q4_K super-block from its 16 header bytes: bytes 0-1 f16 d,
// 2-3 f16 dmin, then the 6-bit fields (j < 4: low 6 bits of scale bytes j and j+4; j >= 4: low and
// high nibble of scale byte j+4 with the top 2 bits of scale bytes j-4 and j). Both exact in f32.
template <int J>
__device__ __forceinline__ float2 q4k_factor(const uint4& h, float d, float dmin) {
  constexpr uint32_t sh = 8u * (J & 3);
  uint32_t sc, mn;
  if constexpr (J < 4) {
    sc = (h.y >> sh) & 63u;
    mn = (h.z >> sh) & 63u;
  } else {
    sc = ((h.w >> sh) & 15u) | (((h.y >> (sh + 6)) & 3u) << 4);
    mn = ((h.w >> (sh + 4)) & 15u) | (((h.z >> (sh + 6)) & 3u) << 4);
  }
  return make_float2(d * static_cast<float>(sc), dmin * static_cast<float>(mn));
}

// Calls f(integral_constant<int, I>) for I = 0 .. N-1, in order.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// PB: buffers of wave partial sums (2: a tile's partials are written while the previous tile's
// are still being added up; 1: one buffer and one more barrier per tile, for LDS).
template <int WT, int NSTAGE, int SB, int PB>
__global__ __launch_bounds__(64 * (kMaxK / (32 * SB))) void matvec_mfma_kernel(MatvecParams p, int tiles_per_wg) {
  constexpr int kSliceBlocks = SB;  // blocks per wave
  constexpr int kMaxWaves = kMaxK / (32 * SB);
  constexpr int BB = block_bytes(WT);
  constexpr int kMaxRowBytes = kMaxWaves * kSliceBlocks * BB;
  constexpr int kSlotBytes = kTileRows * (kMaxRowBytes + 16);
  constexpr int kPartWave = kSlots * kTileRows;  // one wave's partials: [slot][weight row]
  // A wave issues at most 2 rows x 5 loads per tile (k <= 4096, at least 8 waves); vmcnt holds up
  // to 63.
  constexpr int kMaxPending = 20 * (NSTAGE - 2);
  static_assert(NSTAGE >= 2 && kMaxPending < 64, "vmcnt range");

  __shared__ __attribute__((aligned(16))) uint8_t ring[NSTAGE * kSlotBytes];
  __shared__ float part[PB][kMaxWaves * kPartWave];
  __shared__ int slot_lds[kSlots];
  // Q4_K: the sum of each slot's activations over each 32-element sub-block, [sub-block][slot].
  __shared__ __attribute__((aligned(16))) float xsum_lds[WT == kQ4_K ? kMaxK / 32 * kSlots : 4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  __shared__ uint32_t touched_lds[kMoeCompactMax / 32];
  int e = blockIdx.y;
  const int ntiles = (p.m + kTileRows - 1) / kTileRows;
  const bool moe = p.ids != nullptr;
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
        for (int row = t_begin * kTileRows + threadIdx.x; row < min(p.m, t_end * kTileRows); row += blockDim.x)
          p.y[static_cast<long long>(slot) * p.m + row] = __builtin_nanf("");
      }
    }
    return;
  }

  const uint8_t* wexp = p.w + static_cast<long long>(e) * p.expert_bytes;
  const uint32_t ring_addr = lds_address(ring);
  const int rowbytes = static_cast<int>(p.rowbytes);
  const int stride = rowbytes + 16;
  const int per_row = (rowbytes + 1023) / 1024;  // 1024-byte loads per row, the last one partial
  // This wave's rows of every tile.
  const int r0 = wave * kTileRows / nw;
  const int r1 = (wave + 1) * kTileRows / nw;
  const int per_tile = (r1 - r0) * per_row;  // this wave's loads per tile (wave-uniform)

  auto issue = [&](int tile) {
    const int row0 = tile * kTileRows;
    const uint8_t* base = wexp + static_cast<long long>(row0) * p.rowbytes;
    const uint32_t dst = ring_addr + static_cast<uint32_t>((tile % NSTAGE) * kSlotBytes);
    for (int r = r0; r < r1; ++r) {
      const int rr = min(r, p.m - 1 - row0);  // rows past the end of W re-read its last row
      for (int c = 0; c < per_row; ++c) {
        const int b = c * 1024 + lane * 16;
        if (b < rowbytes)  // the last load of a row runs on the lanes that have bytes left
          load_lds16<true>(base, static_cast<uint32_t>(rr * rowbytes + b), dst + r * stride + c * 1024);
      }
    }
  };

  const int j = lane & 15;  // weight row in the tile (B, D column); slot as A
  const int o = lane >> 4;  // k-octet of each block; D rows 4o .. 4o+3
  const int s_off = j * stride + wave * kSliceBlocks * BB;         // the lane's row slice
  const int q_off = s_off + (WT == kQ8_0 ? 8 * o : WT == kQ4_K ? 16 + 8 * o : 4 * o);  // and its quant bytes

  // Finishes tile `tile` from the wave partials in part[buf]: the k-slices of all waves, added in
  // wave order.
  auto finish = [&](int tile, int buf) {
    for (int i = threadIdx.x; i < kSlots * kTileRows; i += blockDim.x) {
      const int t = i >> 4;  // slot within the pass
      const int r = i & 15;  // weight row within the tile
      const int row = tile * kTileRows + r;
      const int slot = slot_lds[t];
      if (row < p.m && slot >= 0) {
        float v = 0.f;
        // Not unrolled: this runs inside the tile loop, where registers are scarce (issuing the
        // partials' reads four at a time measured no faster on the MoE workloads).
#pragma unroll 1
        for (int w = 0; w < nw; ++w) v += part[buf][w * kPartWave + i];
        float* yp = p.y + static_cast<long long>(slot) * p.m + row;
        if (!moe) v = epilogue(v, p.flags, p.alpha, p.bias + row, yp);
        *yp = v;
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
      // This pass's slots, in order: A row (and D row) t is slot_of[t].
      int slot_of[kSlots];
#pragma unroll
      for (int t = 0; t < kSlots; ++t) {
        if (mask) {
          slot_of[t] = win + __builtin_ctzll(mask);
          mask &= mask - 1;
        } else {
          slot_of[t] = -1;
        }
      }
      int my_slot = -1;
#pragma unroll
      for (int t = 0; t < kSlots; ++t)
        if (t == j) my_slot = slot_of[t];
      if (threadIdx.x < kSlots) slot_lds[threadIdx.x] = my_slot;  // read after the next barrier
      if constexpr (WT == kQ4_K) {
        // Sub-block sums of the pass's activations, each a 32-term sum in element order; read
        // after the next barrier.
        __syncthreads();  // slot_lds is complete
        const int nsub = p.k / 32;
        for (int i = threadIdx.x; i < nsub * kSlots; i += blockDim.x) {
          const int sb = i / kSlots, t = i - sb * kSlots;
          const int st = slot_lds[t];
          float sum = 0.f;
          if (st >= 0) {
            const float4* xp = reinterpret_cast<const float4*>(p.x + static_cast<long long>(st / p.top_k) * p.k + 32 * sb);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              const float4 v = xp[c];
              sum += v.x;
              sum += v.y;
              sum += v.z;
              sum += v.w;
            }
          }
          xsum_lds[i] = sum;
        }
      }

      // Prologue: the first NSTAGE-1 tiles in flight, then the activation operands.
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
            // The k order of decode_octet: Q8_0 and Q4_K elements 8o .. 8o+7, Q4_0 4o .. 4o+3 and
            // 16+4o .. 16+4o+3.
            constexpr bool kOctet = WT == kQ8_0 || WT == kQ4_K;
            const float* xb = xs + wave * (32 * kSliceBlocks) + bb * 32;
            const float4 v0 = *reinterpret_cast<const float4*>(xb + (kOctet ? 8 * o : 4 * o));
            const float4 v1 = *reinterpret_cast<const float4*>(xb + (kOctet ? 8 * o + 4 : 16 + 4 * o));
            xv[0] = v0.x; xv[1] = v0.y; xv[2] = v0.z; xv[3] = v0.w;
            xv[4] = v1.x; xv[5] = v1.y; xv[6] = v1.z; xv[7] = v1.w;
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] = 0.f;
          }
          if constexpr (WT == kQ4_0) {
            // Q4_0 weights enter as (q - 8) / 16: the activations take the 16, a power of two, so
            // the parts stay exact and each block's scale is d itself.
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] *= 16.f;
          }
          split3(xv, xa[0][bb], xa[1][bb], xa[2][bb]);
          // Load and split a few blocks at a time: hoisting every load first runs out of registers.
          if (bb % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }

      for (int tile = t_begin; tile < t_end; ++tile) {
        // This wave's loads of `tile` have landed once only those of the later tiles in flight
        // are pending (the exact count: a smaller one would also wait for part of the next tile).
        wait_at_most<kMaxPending>(per_tile * min(NSTAGE - 2, t_end - 1 - tile));
        __syncthreads();  // the tile is in; the slot of tile-1 and the partials of tile-1 are complete
        // Stores count in vmcnt too: issued before the next tile's loads, they are never among the
        // most recent operations a wait leaves in flight, so they cannot stretch it.
        if (tile > t_begin) finish(tile - 1, (tile - 1) % PB);
        if (tile + NSTAGE - 1 < t_end) issue(tile + NSTAGE - 1);

        const int slot_base = (tile % NSTAGE) * kSlotBytes;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (WT == kQ4_K) {
          static_assert(kSliceBlocks % 8 == 0, "a Q4_K slice is whole super-blocks");
          const float* xsw = xsum_lds + wave * kSliceBlocks * kSlots + 4 * o;
          static_for<0, kSliceBlocks / 8>([&](auto ss) {
            constexpr int SS = decltype(ss)::value;  // super-block of the slice
            const uint4 h = *reinterpret_cast<const uint4*>(ring + slot_base + s_off + SS * kQ4KBytes);
            const float d = f16_to_f32(h.x & 0xFFFFu), dmin = f16_to_f32(h.x >> 16);
            static_for<0, 8>([&](auto jj) {
              constexpr int J = decltype(jj)::value;  // sub-block of the super-block
              constexpr int B = 8 * SS + J;           // block of the slice
              const uint2 qd =
                  *reinterpret_cast<const uint2*>(ring + slot_base + q_off + SS * kQ4KBytes + 32 * (J >> 1));
              const bf16x8 wb = q4k_octet<4 * (J & 1)>(qd.x, qd.y);
              const float2 f = q4k_factor<J>(h, d, dmin);
              const float4 xsum = *reinterpret_cast<const float4*>(xsw + B * kSlots);
              f32x4 blk = {0.f, 0.f, 0.f, 0.f};
              blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[0][B], wb, blk, 0, 0, 0);
              blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[1][B], wb, blk, 0, 0, 0);
              blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[2][B], wb, blk, 0, 0, 0);
              acc[0] = __builtin_fmaf(f.x, blk[0], __builtin_fmaf(-f.y, xsum.x, acc[0]));
              acc[1] = __builtin_fmaf(f.x, blk[1], __builtin_fmaf(-f.y, xsum.y, acc[1]));
              acc[2] = __builtin_fmaf(f.x, blk[2], __builtin_fmaf(-f.y, xsum.z, acc[2]));
              acc[3] = __builtin_fmaf(f.x, blk[3], __builtin_fmaf(-f.y, xsum.w, acc[3]));
              if constexpr (J % kSchedBlocks == kSchedBlocks - 1) __builtin_amdgcn_sched_barrier(0);
            });
          });
        } else {
        static_for<0, kSliceBlocks>([&](auto bb) {
          constexpr int B = decltype(bb)::value;
          float scale;
          const bf16x8 wb = decode_octet<WT, B>(ring, slot_base + q_off, slot_base + s_off, scale);
          f32x4 blk = {0.f, 0.f, 0.f, 0.f};
          blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[0][B], wb, blk, 0, 0, 0);
          blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[1][B], wb, blk, 0, 0, 0);
          blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[2][B], wb, blk, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(scale, blk[v], acc[v]);
          // Keep the scheduler within a few blocks: hoisting many decodes runs out of registers.
          if constexpr (B % kSchedBlocks == kSchedBlocks - 1) __builtin_amdgcn_sched_barrier(0);
        });
        }
        // One buffer: every thread has finished adding up the previous tile's partials.
        if constexpr (PB == 1) __syncthreads();
        float* pw = part[tile % PB] + wave * kPartWave;
#pragma unroll
        for (int v = 0; v < 4; ++v) pw[(4 * o + v) * kTileRows + j] = acc[v];
      }
      __syncthreads();
      finish(t_end - 1, (t_end - 1) % PB);
      __syncthreads();  // part, slot_lds and the ring are reused by the next group of slots
    }
  }
}

int mfma_device_cus() {
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

template <int WT, int NSTAGE, int SB, int PB>
hipError_t launch_mfma(const MatvecParams& p, hipStream_t stream) {
  constexpr int kMaxWaves = kMaxK / (32 * SB);
  const int nw = p.k / (32 * SB);
  const int ntiles = (p.m + kTileRows - 1) / kTileRows;
  auto kernel = matvec_mfma_kernel<WT, NSTAGE, SB, PB>;
  static std::atomic<int> per_cu_cache{0};  // filled on first use, as device_cus
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * kMaxWaves, 0) != hipSuccess || per_cu <= 0)
      per_cu = 1;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  // As many workgroups as are resident at once. MoE: dealt over the touched experts on the device
  // (wq_moe_sched.hpp), or split evenly over all experts where the bitmap cannot hold them.
  const int resident = per_cu * mfma_device_cus();
  if (p.ids != nullptr && p.n_exp <= kMoeCompactMax && resident >= p.n_exp) {
    MatvecParams q = p;
    q.moe_compact = 1;
    const int tpw = (ntiles + resident - 1) / resident;
    hipLaunchKernelGGL(kernel, dim3(resident, 2), dim3(64 * nw), 0, stream, q, tpw);
    return hipGetLastError();
  }
  int groups = resident / p.n_exp;
  if (groups < 1) groups = 1;
  if (groups > ntiles) groups = ntiles;
  const int tpw = (ntiles + groups - 1) / groups;
  dim3 grid((ntiles + tpw - 1) / tpw, p.ids ? p.n_exp + 1 : 1);
  hipLaunchKernelGGL(kernel, grid, dim3(64 * nw), 0, stream, p, tpw);
  return hipGetLastError();
}

}  // namespace

bool matvec_mfma_supports(int wtype, int k) {
  if (wtype == kQ4_K) return k % kQ4KElems == 0 && k >= 2048 && k <= kMaxK;
  return (wtype == kQ8_0 || wtype == kQ4_0) && k % 512 == 0 && k >= 2048 && k <= kMaxK;
}

// From 5 to 8 tokens the f32 FMA kernel runs its 8-token variant, which spends more per weight
// than the matrix cores once every CU has two or more 16-row tiles to walk (the activation parts
// are then built once for several tiles). Measured on MI355X, plain calls at n = 5 and 8,
// matrix cores against the FMA kernel: Q4_0 14336 x 4096 18.8 / 19.7 against 25.8 / 27.8 us,
// Q4_0 8192 x 4096 14.7 / 15.7 against 16.9 / 18.0, Q8_0 8192 x 4096 14.4 / 15.2 against
// 19.2 / 19.7, Q8_0 8192 x 2048 10.1 / 10.5 against 12.3 / 12.5, Q4_0 14336 x 2048 13.4 / 14.1
// against 17.1 / 18.4. With one tile per CU (4096 rows), or up to 4 tokens on the larger weights,
// the FMA kernels were as fast or faster (Q4_0 14336 x 4096 at n = 4: 18.6 against 18.9 us).
// Q4_K's decode costs the matrix-core kernel more (a scale, a min and an activation sum per
// sub-block), so it needs three tiles per CU: 14336 x 4096 at n = 5 / 8 21.6 / 23.8 against
// 25.9 / 26.6 us, but 8192 x 4096 17.0 / 19.2 against 16.9 / 17.7 us.
bool matvec_mfma_takes_plain(int wtype, int m, int n) {
  if (n > 8) return true;
  const int per_cu = wtype == kQ4_K ? 3 : 2;
  return n >= 5 && (m + kTileRows - 1) / kTileRows >= per_cu * mfma_device_cus();
}

hipError_t launch_matvec_mfma(int wtype, const MatvecParams& p, hipStream_t stream) {
  if (!matvec_mfma_supports(wtype, p.k) || (p.ids == nullptr && p.n_exp != 1)) return hipErrorInvalidValue;
  // Both run a 2-slot ring (one tile in flight behind the one in use). For Q4_0 a third slot
  // measured 3-4% slower on the MoE workload (16 tokens, top-2 of 8 experts of 14336 x 4096).
  if (wtype == kQ8_0) return launch_mfma<kQ8_0, 2, 8, 1>(p, stream);
  if (wtype == kQ4_K) {
    // Q4_K holds a sub-block sum and scale per block beside the activation parts: with 256-element
    // slices (16 waves, 128 VGPRs) it spills 56 bytes per lane; 512-element slices (8 waves, no
    // spill) measured 4% faster on 16 tokens top-2 of 8 experts of 14336 x 4096 (92-93 against
    // 96-97 us). k an odd multiple of 256 keeps the 256-element slices.
    if (p.k % 512 == 0) return launch_mfma<kQ4_K, 2, 16, 2>(p, stream);
    return launch_mfma<kQ4_K, 2, 8, 2>(p, stream);
  }
  return launch_mfma<kQ4_0, 2, 8, 2>(p, stream);
}

}  // namespace wq
