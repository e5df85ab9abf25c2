// The encoder block around the linear layer: row LayerNorm, per-head q/k LayerNorm with the
// rotary embedding, and masked bidirectional attention -- the `ae_ln`, `ae_qk` and `ae_attn`
// kernels of cortiq-engine src/gpu_wgpu/nemotron_audio.rs (`AE_WGSL`) and the order
// `AudioEncoder::run` runs them in.
//
// Design for gfx950:
//  * LayerNorm: one wave per row. The row is held in registers as float4s (d <= 4096, d a multiple
//    of 4, 16-byte aligned rows); the mean and then the summed squared deviations come from
//    butterfly sums across the wave (two passes over registers, as the page's two passes over
//    memory). Other rows take a scalar kernel that reads the row three times. HBM-bound: 8·d bytes
//    per row.
//  * q/k norm + rotation: one wave per (frame, head), its q and k vectors side by side, in place. The normalised
//    vector goes through wave-private LDS so each lane can read its rotation partner (dim i pairs
//    with dim i + rot/2). HBM-bound: 16·hd bytes per vector.
//  * Attention, in two kernels:
//     - pack: K and V of every head to bf16 (round to nearest even), K as [head][frame][dim] and V
//       transposed as [head][dim][frame], frames padded to a multiple of 64; and the key mask as an
//       additive bias (0 for a valid key, -inf for a masked or padding one). These layouts let the
//       attention kernel stream 64-key tiles into LDS with direct-to-LDS loads.
//     - attention: flash-style, f32 online softmax, bf16 matrix cores (v_mfma_f32_32x32x16_bf16)
//       for both products. A workgroup of 8 waves takes 64 queries of one
//       head: four key quarters of two waves, 32 queries per wave. Each wave computes S^T = K.Q^T
//       (keys in rows, queries in columns), so a lane's scores all belong to one query: the row maximum and the sum need
//       only in-lane work plus two cross-lane steps, and the probabilities are already the B
//       operand of O^T = V^T.P^T. Work items are numbered head-major and dealt to the 8 XCDs in
//       contiguous ranges, so each XCD's L2 holds the K and V of few heads.
#include <hip/hip_runtime.h>

#include <cmath>

#include "wq_internal.hpp"
#include "wq_lds_dma.hpp"

namespace wq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLnEps = 1e-5f;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// v[lane] combined with v[lane ^ 32] and v[lane ^ 16] (v_permlane32_swap / v_permlane16_swap with
// both operands v leave the two halves in the two results).
template <typename Op>
__device__ __forceinline__ float xor32_xor16(float v, Op op) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over the wave, in every lane: xor 32 and 16 (lane swaps), then inside each 16-lane row a
// rotation by 8, a mirror inside 8 lanes and the two quad exchanges, which together add the 8
// partial sums a row's lanes hold after the rotation.
__device__ __forceinline__ float wave_sum(float v) {
  v = xor32_xor16(v, [](float a, float b) { return a + b; });
  v += dpp<0x128>(v);  // row_ror:8
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x4E>(v);   // quad_perm xor 2
  return v + dpp<0xB1>(v);  // quad_perm xor 1
}

__device__ __forceinline__ uint16_t bf16_bits_rne(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// ---------------------------------------------------------------------------------------------
// LayerNorm
// ---------------------------------------------------------------------------------------------

// Four outputs rounded to bf16 (nearest even, as the products round their f32 inputs), packed.
__device__ __forceinline__ uint2 bf16x4_bits(float a, float b, float c, float d) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 lo, hi;
  lo[0] = static_cast<__bf16>(a);
  lo[1] = static_cast<__bf16>(b);
  hi[0] = static_cast<__bf16>(c);
  hi[1] = static_cast<__bf16>(d);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// NV float4s per lane: d <= 256·NV, d % 4 == 0, x / y rows and wb 16-byte aligned. OB: y receives
// bf16 bit patterns (8-byte aligned rows) for a product that rounds its input to bf16 anyway.
template <int NV, bool OB = false>
__global__ __launch_bounds__(256) void layer_norm_vec_kernel(const float* x, const float* __restrict__ wb, void* y,
                                                              int n, int d) {
  const int lane = threadIdx.x & 63;
  const long long row = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n) return;  // wave-uniform; no barrier follows
  const int nv = d >> 2;
  const float4* xr = reinterpret_cast<const float4*>(x + row * d);
  // Loads are unconditional (lanes past the row re-read its last float4, zeroed after), so they
  // issue back to back instead of one guarded load at a time.
  float4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = xr[min(lane + 64 * i, nv - 1)];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (lane + 64 * i >= nv) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float fd = static_cast<float>(d);
  const float mean = wave_sum(s) / fd;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (lane + 64 * i < nv) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, e = v[i].w - mean;
      q += (a * a + b * b) + (c * c + e * e);
    }
  }
  const float inv = rsqrtf(wave_sum(q) / fd + kLnEps);
  const float4* w4 = reinterpret_cast<const float4*>(wb);
  float4* yr = reinterpret_cast<float4*>(static_cast<float*>(y) + row * d);
  uint2* yb = reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + row * d);
  float4 wv[NV], bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = min(lane + 64 * i, nv - 1);
    wv[i] = w4[c];
    bv[i] = w4[nv + c];
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < nv) {
      const float4 w = wv[i], b = bv[i];
      const float4 o = make_float4((v[i].x - mean) * inv * w.x + b.x, (v[i].y - mean) * inv * w.y + b.y,
                                   (v[i].z - mean) * inv * w.z + b.z, (v[i].w - mean) * inv * w.w + b.w);
      if constexpr (OB) yb[c] = bf16x4_bits(o.x, o.y, o.z, o.w);
      else yr[c] = o;
    }
  }
}

// Any d and alignment: three passes over the row in memory, one wave per row. In place is safe:
// a lane writes y[i] only after every lane of the wave has read the row for the second time.
// OB: y receives bf16 bit patterns.
template <bool OB = false>
__global__ __launch_bounds__(256) void layer_norm_scalar_kernel(const float* x, const float* __restrict__ wb,
                                                                 void* y, int n, int d) {
  const int lane = threadIdx.x & 63;
  const long long row = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const float* xr = x + row * d;
  float s = 0.f;
  for (int i = lane; i < d; i += 64) s += xr[i];
  const float fd = static_cast<float>(d);
  const float mean = wave_sum(s) / fd;
  float q = 0.f;
  for (int i = lane; i < d; i += 64) {
    const float c = xr[i] - mean;
    q += c * c;
  }
  const float inv = rsqrtf(wave_sum(q) / fd + kLnEps);
  for (int i = lane; i < d; i += 64) {
    const float o = (xr[i] - mean) * inv * wb[i] + wb[d + i];
    if constexpr (OB) static_cast<__bf16*>(y)[row * d + i] = static_cast<__bf16>(o);
    else static_cast<float*>(y)[row * d + i] = o;
  }
}

// ---------------------------------------------------------------------------------------------
// q/k LayerNorm + rotation
// ---------------------------------------------------------------------------------------------

// Orders one wave's LDS writes before its later reads by other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One q or k vector of hd values held E per lane (element lane + 64e): its LayerNorm when nw is
// given (mean, then the summed squared deviations, then (v - mean) * inv * w + b), then the
// rotation of its first rot dims by frame t's row of the table (cos_t, sin_t). vbuf is 64·E floats
// of this wave's LDS, through which a lane reads its rotation partner.
template <int E>
__device__ __forceinline__ void qk_vector(float (&v)[E], const float* __restrict__ nw, const float* cos_t,
                                          const float* sin_t, int hd, int rot, float* vbuf, int lane) {
  // Every load below is unconditional, from an index clamped into range (the value then unused),
  // so the loads issue back to back.
  const int half = rot >> 1;
  float c_[E], s_[E], w_[E], b_[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane + 64 * e;
    if (half > 0) {
      const int t = i < half ? i : (i < rot ? i - half : 0);
      c_[e] = cos_t[t];
      s_[e] = sin_t[t];
    }
    if (nw != nullptr) {
      const int ic = min(i, hd - 1);
      w_[e] = nw[ic];
      b_[e] = nw[hd + ic];
    }
  }
  if (nw != nullptr) {  // wave-uniform
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s += v[e];
    const float fhd = static_cast<float>(hd);
    const float mean = wave_sum(s) / fhd;
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float c = lane + 64 * e < hd ? v[e] - mean : 0.f;
      q += c * c;
    }
    const float inv = rsqrtf(wave_sum(q) / fhd + kLnEps);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lane + 64 * e;
      if (i < hd) v[e] = (v[e] - mean) * inv * w_[e] + b_[e];
    }
  }
  if (rot == 0) return;
  wave_lds_sync();  // the previous vector's partner reads are done
#pragma unroll
  for (int e = 0; e < E; ++e) vbuf[lane + 64 * e] = v[e];
  wave_lds_sync();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane + 64 * e;
    const float partner = vbuf[i < half ? i + half : (i < rot ? i - half : i)];
    if (i < half) {
      v[e] = v[e] * c_[e] - partner * s_[e];
    } else if (i < rot) {
      v[e] = v[e] * c_[e] + partner * s_[e];
    }
  }
}

// E elements per lane (hd <= 64·E); one wave per (frame, head), q and k side by side, in place.
template <int E>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(float* qkv, const float* __restrict__ qn,
                                                            const float* __restrict__ kn,
                                                            const float* __restrict__ cs, int n, int heads, int hd,
                                                            int rot) {
  __shared__ float vbuf[4][2][64 * E];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const long long vec = static_cast<long long>(blockIdx.x) * 4 + wave;
  if (vec >= static_cast<long long>(n) * heads) return;  // wave-uniform; only wave-level synchronisation follows
  const long long t = vec / heads;
  const int h = static_cast<int>(vec - t * heads);
  const long long d = static_cast<long long>(heads) * hd;
  float* qb = qkv + t * 3 * d + static_cast<long long>(h) * hd;
  float* kb = qb + d;
  const int half = rot >> 1;

  float vq[E], vk[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = min(lane + 64 * e, hd - 1);  // unconditional loads (zeroed past hd below)
    vq[e] = qb[c];
    vk[e] = kb[c];
  }
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (lane + 64 * e >= hd) vq[e] = vk[e] = 0.f;
  const float* cos_t = cs + t * half;
  const float* sin_t = cs + static_cast<long long>(n) * half + t * half;
  qk_vector<E>(vq, qn, cos_t, sin_t, hd, rot, vbuf[wave][0], lane);
  qk_vector<E>(vk, kn, cos_t, sin_t, hd, rot, vbuf[wave][1], lane);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane + 64 * e;
    if (i < hd) {
      qb[i] = vq[e];
      kb[i] = vk[e];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Attention: pack
// ---------------------------------------------------------------------------------------------

constexpr int kKeyTile = 64;    // keys per tile
constexpr int kQueryTile = 64;  // queries per workgroup (16 per wave)

// Grid (npad / 64, heads). K: kb[h][t][0..HDP) bf16; V: vt[h][0..HDP)[t] bf16; dims past hd and
// frames past n are zero. Head 0's workgroups also write the key bias. vec4: hd % 4 == 0 and qkv
// 16-byte aligned, so every row's head starts on a 16-byte boundary.
template <int HDP>
__global__ __launch_bounds__(256) void attn_pack_kernel(const float* __restrict__ qkv, const int32_t* __restrict__ valid,
                                                         uint16_t* __restrict__ kb, uint16_t* __restrict__ vt,
                                                         float* __restrict__ kbias, int n, int npad, int heads, int hd,
                                                         bool vec4) {
  __shared__ __attribute__((aligned(16))) uint16_t vs[kKeyTile][HDP + 4];  // V tile, frame-major, for the transposed write
  const int t0 = blockIdx.x * kKeyTile;
  const int h = blockIdx.y;
  const long long d = static_cast<long long>(heads) * hd;
  const float* kbase = qkv + d + static_cast<long long>(h) * hd;
  const float* vbase = qkv + 2 * d + static_cast<long long>(h) * hd;
  uint16_t* kout = kb + (static_cast<long long>(h) * npad + t0) * HDP;
  if (vec4) {
    // Four dims per thread: 16-byte loads of K and V, 8-byte stores of K.
    for (int i = threadIdx.x; i < kKeyTile * HDP / 4; i += 256) {
      const int r = i / (HDP / 4), c = (i % (HDP / 4)) * 4;
      const int t = t0 + r;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (t < n && c < hd) {
        const long long off = static_cast<long long>(t) * 3 * d + c;
        kv = *reinterpret_cast<const float4*>(kbase + off);
        vv = *reinterpret_cast<const float4*>(vbase + off);
      }
      *reinterpret_cast<uint2*>(kout + r * HDP + c) =
          make_uint2(bf16_bits_rne(kv.x) | (uint32_t(bf16_bits_rne(kv.y)) << 16),
                     bf16_bits_rne(kv.z) | (uint32_t(bf16_bits_rne(kv.w)) << 16));
      *reinterpret_cast<uint2*>(&vs[r][c]) =
          make_uint2(bf16_bits_rne(vv.x) | (uint32_t(bf16_bits_rne(vv.y)) << 16),
                     bf16_bits_rne(vv.z) | (uint32_t(bf16_bits_rne(vv.w)) << 16));
    }
  } else {
    for (int i = threadIdx.x; i < kKeyTile * HDP; i += 256) {
      const int r = i / HDP, c = i % HDP;
      const int t = t0 + r;
      const bool in = t < n && c < hd;
      const long long off = static_cast<long long>(t) * 3 * d + c;
      kout[i] = in ? bf16_bits_rne(kbase[off]) : uint16_t(0);
      vs[r][c] = in ? bf16_bits_rne(vbase[off]) : uint16_t(0);
    }
  }
  if (h == 0 && threadIdx.x < kKeyTile) {
    const int t = t0 + threadIdx.x;
    kbias[t] = t < n && valid[t] != 0 ? 0.f : -INFINITY;
  }
  __syncthreads();
  // vt[h][c][t0 .. t0+63]: 8 keys (16 bytes) per store.
  uint16_t* vout = vt + static_cast<long long>(h) * HDP * npad + t0;
  for (int i = threadIdx.x; i < HDP * (kKeyTile / 8); i += 256) {
    const int c = i / (kKeyTile / 8), g = i % (kKeyTile / 8);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = static_cast<uint32_t>(vs[8 * g + 2 * j][c]) | (static_cast<uint32_t>(vs[8 * g + 2 * j + 1][c]) << 16);
    *reinterpret_cast<uint4*>(vout + static_cast<long long>(c) * npad + 8 * g) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// The q/k norm + rotation and the pack in one pass, for a block's attention: grid (npad / 8,
// heads), one frame per wave and four waves per workgroup, q and k of the frame side by side: q
// normed and rotated and written back in place (f32, as qk_norm_rope_kernel writes it), k normed,
// rotated and rounded to bf16 into kb, v rounded to bf16 and transposed into vt through LDS, as
// attn_pack_kernel lays them out; head 0's workgroups write the key bias. k is not written back to
// qkv. (HDP, E): (32, 1), (64, 1), (128, 2).
constexpr int kQkFrames = 8;  // frames per workgroup
template <int HDP, int E>
__global__ __launch_bounds__(256) void qk_pack_kernel(float* qkv, const float* __restrict__ qn,
                                                       const float* __restrict__ kn, const float* __restrict__ cs,
                                                       const int32_t* __restrict__ valid, uint16_t* __restrict__ kb,
                                                       uint16_t* __restrict__ vt, float* __restrict__ kbias, int n,
                                                       int npad, int heads, int hd, int rot) {
  static_assert(64 * E >= HDP, "a wave's lanes cover the padded head");
  __shared__ float vbuf[4][2][64 * E];
  __shared__ __attribute__((aligned(16))) uint16_t vs[kQkFrames][HDP + 8];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kQkFrames;
  const int h = blockIdx.y;
  const long long d = static_cast<long long>(heads) * hd;
  const int half = rot >> 1;
  for (int r = wave; r < kQkFrames; r += 4) {
    const int t = t0 + r;
    uint16_t* krow = kb + (static_cast<long long>(h) * npad + t) * HDP;
    if (t < n) {  // wave-uniform
      float* qrow = qkv + static_cast<long long>(t) * 3 * d + static_cast<long long>(h) * hd;
      const float* cos_t = cs + static_cast<long long>(t) * half;
      const float* sin_t = cs + static_cast<long long>(n) * half + static_cast<long long>(t) * half;
      float vq[E], vk[E], vv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int c = min(lane + 64 * e, hd - 1);  // unconditional loads (zeroed past hd below)
        vq[e] = qrow[c];
        vk[e] = qrow[d + c];
        vv[e] = qrow[2 * d + c];
      }
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (lane + 64 * e >= hd) vq[e] = vk[e] = vv[e] = 0.f;
      qk_vector<E>(vq, qn, cos_t, sin_t, hd, rot, vbuf[wave][0], lane);
      qk_vector<E>(vk, kn, cos_t, sin_t, hd, rot, vbuf[wave][1], lane);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int c = lane + 64 * e;
        if (c < hd) qrow[c] = vq[e];
        if (c < HDP) {
          krow[c] = c < hd ? bf16_bits_rne(vk[e]) : uint16_t(0);
          vs[r][c] = c < hd ? bf16_bits_rne(vv[e]) : uint16_t(0);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int c = lane + 64 * e;
        if (c < HDP) {
          krow[c] = 0;
          vs[r][c] = 0;
        }
      }
    }
  }
  if (h == 0 && threadIdx.x < kQkFrames) {
    const int t = t0 + threadIdx.x;
    kbias[t] = t < n && valid[t] != 0 ? 0.f : -INFINITY;
  }
  __syncthreads();
  // vt[h][c][t0 .. t0+7]: 8 frames (16 bytes) per store.
  uint16_t* vout = vt + static_cast<long long>(h) * HDP * npad + t0;
  for (int i = threadIdx.x; i < HDP * (kQkFrames / 8); i += 256) {
    const int c = i / (kQkFrames / 8), g = i % (kQkFrames / 8);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = static_cast<uint32_t>(vs[8 * g + 2 * j][c]) | (static_cast<uint32_t>(vs[8 * g + 2 * j + 1][c]) << 16);
    *reinterpret_cast<uint4*>(vout + static_cast<long long>(c) * npad + 8 * g) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---------------------------------------------------------------------------------------------
// Attention
// ---------------------------------------------------------------------------------------------

struct AttnParams {
  const float* qkv;
  const uint16_t* kb;
  const uint16_t* vt;
  const float* kbias;
  float* o;
  int n, npad, heads, hd;
  int qtiles;      // query tiles per head
  int items;       // heads * qtiles
  int per_xcd;     // ceil(items / 8)
  float scale_l2;  // scale * log2(e): scores enter exp2
  int v4;          // hd % 8 == 0 and qkv, o 16-byte aligned: 16-byte loads of q, stores of o
  int o_bf16;      // o receives bf16 bit patterns (for a product that rounds its input to bf16)
};

// LDS tile layout (one buffer of a 32-key tile):
//   K  [32 keys][HDP] bf16, 16-byte chunks XOR-swizzled by (key & (CPR-1)), CPR = HDP/8 chunks a row;
//   Vt [HDP dims][32 keys] bf16 (64-byte rows), chunks swizzled by ((dim >> 2) & 3);
//   bias [32] f32.
constexpr int kAttnKeys = 32;  // keys per tile
constexpr float kLazy = 8.f;   // headroom of the running maximum, in log2 units
template <int HDP>
struct AttnLds {
  static constexpr int kCpr = HDP / 8;  // 16-byte chunks per K row
  static constexpr int kKBytes = kAttnKeys * HDP * 2;
  static constexpr int kVBytes = HDP * kAttnKeys * 2;
  static constexpr int kBiasBytes = kAttnKeys * 4;
  static constexpr int kBufBytes = kKBytes + kVBytes + kBiasBytes;
  static constexpr int kKLoads = kKBytes / 1024;  // 1 KB wave loads per tile
  static constexpr int kVLoads = kVBytes / 1024;
  static_assert(HDP == 32 || HDP == 64 || HDP == 128, "head dims padded to 32, 64 or 128");
};

// Workgroup: 8 waves, 64 queries of one head. The waves form four key quarters of two; quarter k
// walks the 32-key tiles t with t % 4 == k through its own double-buffered LDS tiles, and each of
// its two waves takes 32 queries. Both products run on v_mfma_f32_32x32x16_bf16 (on gfx950 twice
// the rate per FLOP of the 16x16x32 form): a wave computes S^T = K.Q^T for 32 keys x its 32 queries,
// so lane l holds 16 scores of query l % 32 (lanes l and l ^ 32 share a query), and those weights,
// rounded to bf16, are the B operand of O^T = V^T.P^T with the k order of V^T read to match (and of
// a third product against a row of ones, which keeps their running sum). At the end quarters 1-3
// hand their running maxima, sums and outputs to quarter 0 through LDS, which merges them in
// quarter order (rescaled to the common maximum) and stores.
template <int HDP>
__global__ __launch_bounds__(512) void attention_kernel(AttnParams p) {
  using L = AttnLds<HDP>;
  constexpr int kSteps = HDP / 16;   // k-steps of the score product
  constexpr int kDTiles = HDP / 32;  // 32-dim output tiles
  constexpr int kMergeFloats = 16 * kDTiles + 2;  // per lane: outputs, maximum, sum
  static_assert(3 * 2 * 64 * kMergeFloats * 4 <= 8 * L::kBufBytes, "merge area inside the tile buffers");
  __shared__ __attribute__((aligned(16))) uint8_t lds[8 * L::kBufBytes];  // [quarter][buffer]

  // Work item: head-major, dealt to XCDs in contiguous ranges (workgroup i runs on XCD i % 8).
  const int item = (blockIdx.x & 7) * p.per_xcd + (blockIdx.x >> 3);
  if (item >= p.items) return;  // workgroup-uniform, before any barrier
  const int h = item / p.qtiles;
  const int q0 = (item % p.qtiles) * kQueryTile;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qt = wave >> 1;   // key quarter
  const int qw = wave & 1;    // which 32 of the 64 queries
  const int j = lane & 31;    // query column of every fragment this lane holds
  const int hh = lane >> 5;   // k-octet (operands) / row quad (results)
  const long long d = static_cast<long long>(p.heads) * p.hd;

  // Q fragments (B operand of S^T): query q0 + 32·qw + j, dims 16s + 8hh .. +7, rounded to bf16.
  // Rows past n read row n-1 and dims past hd are zeroed, so with p.v4 the loads are unconditional
  // 16-byte loads that issue back to back.
  bf16x8 qf[kSteps];
  {
    const int q = q0 + 32 * qw + j;
    const bool qin = q < p.n;
    const float* qr = p.qkv + static_cast<long long>(qin ? q : p.n - 1) * 3 * d + static_cast<long long>(h) * p.hd;
    if (p.v4) {
      float4 lo[kSteps], hi[kSteps];
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int c = min(16 * s + 8 * hh, p.hd - 8);  // hd % 8 == 0 with v4: in the row
        lo[s] = *reinterpret_cast<const float4*>(qr + c);
        hi[s] = *reinterpret_cast<const float4*>(qr + c + 4);
      }
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const bool in = qin && 16 * s + 8 * hh < p.hd;
        const float v[8] = {lo[s].x, lo[s].y, lo[s].z, lo[s].w, hi[s].x, hi[s].y, hi[s].z, hi[s].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[s][e] = static_cast<__bf16>(in ? v[e] : 0.f);
      }
    } else {
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = 16 * s + 8 * hh + e;
          qf[s][e] = static_cast<__bf16>(qin && c < p.hd ? qr[c] : 0.f);
        }
      }
    }
  }

  const uint32_t lds_base = lds_address(lds);
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.kb + static_cast<long long>(h) * p.npad * HDP);
  const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.vt + static_cast<long long>(h) * HDP * p.npad);
  const uint8_t* bg = reinterpret_cast<const uint8_t*>(p.kbias);
  const int ntiles = p.npad / kAttnKeys;

  // Issues this wave's share of tile `kt`'s loads into its quarter's buffer `buf`: K and V loads
  // dealt to the quarter's two waves in turn; its first wave also loads the 128-byte bias.
  auto issue = [&](int kt, int buf) {
    const uint32_t dst = lds_base + (2 * qt + buf) * L::kBufBytes;
    constexpr int kRowsPerLoad = 512 / HDP;  // K rows per 1 KB
    for (int c = qw; c < L::kKLoads; c += 2) {
      const int r = c * kRowsPerLoad + lane / L::kCpr;
      const int cc = lane % L::kCpr;
      const uint32_t src =
          static_cast<uint32_t>((kt * kAttnKeys + r) * HDP * 2 + ((cc ^ (r & (L::kCpr - 1))) * 16));
      load_lds16(kg, src, dst + c * 1024);
    }
    for (int c = qw; c < L::kVLoads; c += 2) {
      const int r = c * 16 + lane / 4;  // dim
      const int cc = lane % 4;
      const uint32_t src = static_cast<uint32_t>(static_cast<long long>(r) * p.npad * 2 + kt * kAttnKeys * 2 +
                                                 ((cc ^ ((r >> 2) & 3)) * 16));
      load_lds16(vg, src, dst + L::kKBytes + c * 1024);
    }
    if (qw == 0 && lane < 8)
      load_lds16(bg, static_cast<uint32_t>(kt * kAttnKeys * 4 + lane * 16), dst + L::kKBytes + L::kVBytes);
  };

  f32x16 acc[kDTiles];
#pragma unroll
  for (int i = 0; i < kDTiles; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  float m_run = -INFINITY;  // running maximum of this lane's query (log2 domain)
  // The running sum of the weights, on the matrix cores beside the PV product: `ones` is an A
  // operand whose row 0 is all ones and rows 1-31 zero, so row 0 of lsum = ones . P^T holds each
  // query's sum of the bf16 weights (exact products, f32 sums). Lanes 0-31 hold it in lsum[0];
  // lanes 32-63 hold a zero row there. Two MFMAs per tile take the place of 32 VALU operations
  // per lane (a widening and an add per weight): pack + attention at 1500 x 8 x 128 went from
  // 35.5 to 34.1 us.
  f32x16 lsum;
#pragma unroll
  for (int v = 0; v < 16; ++v) lsum[v] = 0.f;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(j == 0 ? 1.f : 0.f);

  const int iters = (ntiles + 3) / 4;
  if (qt < ntiles) issue(qt, 0);
  wait_vmcnt<0>();
  __syncthreads();
  for (int it = 0; it < iters; ++it) {
    const int kt = 4 * it + qt;
    const int buf = it & 1;
    if (kt + 4 < ntiles) issue(kt + 4, buf ^ 1);
    if (kt < ntiles) {  // wave-uniform (the last quarters may have one tile fewer)
      const uint8_t* kl = lds + (2 * qt + buf) * L::kBufBytes;
      const uint8_t* vl = kl + L::kKBytes;
      const float* bl = reinterpret_cast<const float*>(vl + L::kVBytes);

      // S^T: rows keys 8(v/4) + 4hh + v%4, column query j.
      f32x16 sc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int chunk = (2 * s + hh) ^ (j & (L::kCpr - 1));
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + j * HDP * 2 + chunk * 16);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sc, 0, 0, 0);
      }
      // Scale, mask, the tile's maximum per query (this lane and lane ^ 32).
      float mt = -INFINITY;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 b = *reinterpret_cast<const float4*>(bl + 8 * g4 + 4 * hh);
        sc[4 * g4 + 0] = sc[4 * g4 + 0] * p.scale_l2 + b.x;
        sc[4 * g4 + 1] = sc[4 * g4 + 1] * p.scale_l2 + b.y;
        sc[4 * g4 + 2] = sc[4 * g4 + 2] * p.scale_l2 + b.z;
        sc[4 * g4 + 3] = sc[4 * g4 + 3] * p.scale_l2 + b.w;
        mt = fmaxf(mt, fmaxf(fmaxf(sc[4 * g4], sc[4 * g4 + 1]), fmaxf(sc[4 * g4 + 2], sc[4 * g4 + 3])));
      }
      {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      // The running maximum moves only when the tile's exceeds it by more than kLazy (log2 units):
      // weights then stay below 2^kLazy, and numerator and denominator share whichever maximum is
      // used, so the result is the same up to rounding while most tiles skip the rescale.
      const float m_new = mt > m_run + kLazy ? mt : m_run;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no valid key yet: every weight is 0
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      // Weights, rounded to bf16 as the PV product takes them; lsum adds the rounded values.
      bf16x8 pb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) pb[v >> 3][v & 7] = static_cast<__bf16>(__builtin_amdgcn_exp2f(sc[v] - m_use));
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < kDTiles; ++i) acc[i] *= alpha;
        lsum[0] *= alpha;
      }
      lsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb[0], lsum, 0, 0, 0);
      lsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb[1], lsum, 0, 0, 0);
      // O^T += V^T . P^T: k slot 8hh + e of product mf is key 16mf + 4hh + e (e < 4) or
      // 16mf + 8 + 4hh + (e - 4), the keys this lane's weights belong to.
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt) {
        const int r = 32 * dt + j;  // A row: dim
        const uint8_t* vrow = vl + r * (kAttnKeys * 2);
        const int sw = (r >> 2) & 3;
#pragma unroll
        for (int mf = 0; mf < 2; ++mf) {
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (((2 * mf) ^ sw) * 16) + hh * 8);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (((2 * mf + 1) ^ sw) * 16) + hh * 8);
          const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[mf], acc[dt], 0, 0, 0);
        }
      }
    }
    wait_vmcnt<0>();
    __syncthreads();  // the next tiles are in; every wave is done with this iteration's buffers
  }
  float l_part = lsum[0];  // this lane's share of the sum of weights (lanes 32-63: 0)

  // Merge: quarters 1-3 write their state to LDS (the tile buffers are free after the last
  // barrier), laid out [quarter - 1][query half][field][lane]; quarter 0 folds them in in order.
  auto slot = [&](int quarter) {
    return reinterpret_cast<float*>(lds) + ((quarter - 1) * 2 + qw) * (kMergeFloats * 64);
  };
  if (qt > 0) {
    float* f = slot(qt);
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) f[(16 * dt + v) * 64 + lane] = acc[dt][v];
    f[(16 * kDTiles) * 64 + lane] = m_run;
    f[(16 * kDTiles + 1) * 64 + lane] = l_part;
  }
  __syncthreads();
  if (qt > 0) return;
#pragma unroll 1
  for (int other = 1; other < 4; ++other) {
    const float* f = slot(other);
    const float m1 = f[(16 * kDTiles) * 64 + lane];
    const float m = fmaxf(m_run, m1);
    const float m_use = m == -INFINITY ? 0.f : m;
    const float a0 = __builtin_amdgcn_exp2f(m_run - m_use), a1 = __builtin_amdgcn_exp2f(m1 - m_use);
    m_run = m;
    l_part = l_part * a0 + f[(16 * kDTiles + 1) * 64 + lane] * a1;
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[dt][v] = acc[dt][v] * a0 + f[(16 * dt + v) * 64 + lane] * a1;
  }

  // Normalise and store: lane holds dims 32dt + 8(v/4) + 4hh + v%4 of query q0 + 32·qw + j.
  float l;
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
    l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float inv = 1.f / l;  // no valid key: 1/0, and 0 · inf = NaN, as the page's arithmetic gives
  const int q = q0 + 32 * qw + j;
  if (q < p.n) {
    const long long obase = static_cast<long long>(q) * d + static_cast<long long>(h) * p.hd;
    float* orow = p.o + obase;
    __bf16* orow_b = reinterpret_cast<__bf16*>(p.o) + obase;
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = 32 * dt + 8 * g4 + 4 * hh;
        const f32x16& v = acc[dt];
        if (p.o_bf16) {
          if (p.v4) {
            if (c < p.hd)
              *reinterpret_cast<uint2*>(orow_b + c) =
                  bf16x4_bits(v[4 * g4] * inv, v[4 * g4 + 1] * inv, v[4 * g4 + 2] * inv, v[4 * g4 + 3] * inv);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (c + r < p.hd) orow_b[c + r] = static_cast<__bf16>(v[4 * g4 + r] * inv);
          }
        } else if (p.v4) {
          if (c < p.hd)
            *reinterpret_cast<float4*>(orow + c) =
                make_float4(v[4 * g4] * inv, v[4 * g4 + 1] * inv, v[4 * g4 + 2] * inv, v[4 * g4 + 3] * inv);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (c + r < p.hd) orow[c + r] = v[4 * g4 + r] * inv;
        }
      }
    }
  }
}

int head_pad(int hd) { return hd <= 32 ? 32 : hd <= 64 ? 64 : 128; }

}  // namespace

template <bool OB>
hipError_t launch_layer_norm_t(const float* x, const float* wb, void* y, int n, int d, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const dim3 grid((n + 3) / 4), block(256);
  const bool vec = d % 4 == 0 && d <= 4096 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(y) & (OB ? 7 : 15)) == 0 && (reinterpret_cast<uintptr_t>(wb) & 15) == 0;
  if (!vec) {
    hipLaunchKernelGGL(layer_norm_scalar_kernel<OB>, grid, block, 0, stream, x, wb, y, n, d);
  } else if (d <= 256) {
    hipLaunchKernelGGL((layer_norm_vec_kernel<1, OB>), grid, block, 0, stream, x, wb, y, n, d);
  } else if (d <= 512) {
    hipLaunchKernelGGL((layer_norm_vec_kernel<2, OB>), grid, block, 0, stream, x, wb, y, n, d);
  } else if (d <= 1024) {
    hipLaunchKernelGGL((layer_norm_vec_kernel<4, OB>), grid, block, 0, stream, x, wb, y, n, d);
  } else if (d <= 2048) {
    hipLaunchKernelGGL((layer_norm_vec_kernel<8, OB>), grid, block, 0, stream, x, wb, y, n, d);
  } else {
    hipLaunchKernelGGL((layer_norm_vec_kernel<16, OB>), grid, block, 0, stream, x, wb, y, n, d);
  }
  return hipGetLastError();
}

hipError_t launch_layer_norm(const float* x, const float* wb, float* y, int n, int d, hipStream_t stream) {
  return launch_layer_norm_t<false>(x, wb, y, n, d, stream);
}

hipError_t launch_layer_norm_bf16(const float* x, const float* wb, uint16_t* y, int n, int d, hipStream_t stream) {
  return launch_layer_norm_t<true>(x, wb, y, n, d, stream);
}

hipError_t launch_qk_norm_rope(float* qkv, const float* qn, const float* kn, const float* cs, int n, int heads,
                               int hd, int rot, hipStream_t stream) {
  const long long vecs = static_cast<long long>(n) * heads;  // (frame, head) pairs
  if (vecs == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((vecs + 3) / 4)), block(256);
  if (hd <= 64)
    hipLaunchKernelGGL(qk_norm_rope_kernel<1>, grid, block, 0, stream, qkv, qn, kn, cs, n, heads, hd, rot);
  else if (hd <= 128)
    hipLaunchKernelGGL(qk_norm_rope_kernel<2>, grid, block, 0, stream, qkv, qn, kn, cs, n, heads, hd, rot);
  else
    hipLaunchKernelGGL(qk_norm_rope_kernel<4>, grid, block, 0, stream, qkv, qn, kn, cs, n, heads, hd, rot);
  return hipGetLastError();
}

long long attention_workspace_bytes(long long n, long long heads, long long hd) {
  const long long npad = (n + kKeyTile - 1) / kKeyTile * kKeyTile;
  const long long hdp = head_pad(static_cast<int>(hd));
  // kb and vt (bf16), then the key bias (f32); each part starts on a 256-byte boundary.
  const long long kv = (heads * npad * hdp * 2 + 255) / 256 * 256;
  return 2 * kv + (npad * 4 + 255) / 256 * 256;
}

// The attention workspace for these sizes: kb and vt (bf16), then the key bias, each part on a
// 256-byte boundary.
struct AttnWs {
  uint16_t* kb;
  uint16_t* vt;
  float* kbias;
  int npad;
};

template <int HDP>
AttnWs attn_ws(void* ws, int n, int heads) {
  const int npad = (n + kKeyTile - 1) / kKeyTile * kKeyTile;
  const long long kv = (static_cast<long long>(heads) * npad * HDP * 2 + 255) / 256 * 256;
  uint8_t* w = static_cast<uint8_t*>(ws);
  return {reinterpret_cast<uint16_t*>(w), reinterpret_cast<uint16_t*>(w + kv), reinterpret_cast<float*>(w + 2 * kv),
          npad};
}

template <int HDP>
hipError_t run_attention(const float* qkv, const AttnWs& w, float* o, int n, int heads, int hd, float scale,
                         hipStream_t stream, int o_bf16 = 0) {
  AttnParams p{};
  p.qkv = qkv;
  p.kb = w.kb;
  p.vt = w.vt;
  p.kbias = w.kbias;
  p.o = o;
  p.n = n;
  p.npad = w.npad;
  p.heads = heads;
  p.hd = hd;
  p.qtiles = (n + kQueryTile - 1) / kQueryTile;
  p.items = heads * p.qtiles;
  p.per_xcd = (p.items + 7) / 8;
  p.scale_l2 = scale * 1.4426950408889634f;
  p.v4 = hd % 8 == 0 && (reinterpret_cast<uintptr_t>(qkv) & 15) == 0 && (reinterpret_cast<uintptr_t>(o) & 15) == 0;
  p.o_bf16 = o_bf16;
  hipLaunchKernelGGL(attention_kernel<HDP>, dim3(p.per_xcd * 8), dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <int HDP>
hipError_t launch_attention_hdp(const float* qkv, const int32_t* valid, float* o, void* ws, int n, int heads, int hd,
                                float scale, hipStream_t stream) {
  const AttnWs w = attn_ws<HDP>(ws, n, heads);
  const bool vec4 = hd % 4 == 0 && (reinterpret_cast<uintptr_t>(qkv) & 15) == 0;
  hipLaunchKernelGGL(attn_pack_kernel<HDP>, dim3(w.npad / kKeyTile, heads), dim3(256), 0, stream, qkv, valid, w.kb,
                     w.vt, w.kbias, n, w.npad, heads, hd, vec4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return run_attention<HDP>(qkv, w, o, n, heads, hd, scale, stream);
}

template <int HDP, int E>
hipError_t launch_qk_attention_hdp(float* qkv, const float* qn, const float* kn, const float* cs, const int32_t* valid,
                                   float* o, void* ws, int n, int heads, int hd, int rot, float scale,
                                   hipStream_t stream, int o_bf16) {
  const AttnWs w = attn_ws<HDP>(ws, n, heads);
  hipLaunchKernelGGL((qk_pack_kernel<HDP, E>), dim3(w.npad / kQkFrames, heads), dim3(256), 0, stream, qkv, qn, kn, cs,
                     valid, w.kb, w.vt, w.kbias, n, w.npad, heads, hd, rot);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return run_attention<HDP>(qkv, w, o, n, heads, hd, scale, stream, o_bf16);
}

hipError_t launch_attention(const float* qkv, const int32_t* valid, float* o, void* ws, int n, int heads, int hd,
                            float scale, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  switch (head_pad(hd)) {
    case 32: return launch_attention_hdp<32>(qkv, valid, o, ws, n, heads, hd, scale, stream);
    case 64: return launch_attention_hdp<64>(qkv, valid, o, ws, n, heads, hd, scale, stream);
    default: return launch_attention_hdp<128>(qkv, valid, o, ws, n, heads, hd, scale, stream);
  }
}

hipError_t launch_qk_attention(float* qkv, const float* qn, const float* kn, const float* cs, const int32_t* valid,
                               void* o, void* ws, int n, int heads, int hd, int rot, float scale,
                               hipStream_t stream, int o_bf16) {
  if (n == 0) return hipSuccess;
  float* of = static_cast<float*>(o);
  switch (head_pad(hd)) {
    case 32: return launch_qk_attention_hdp<32, 1>(qkv, qn, kn, cs, valid, of, ws, n, heads, hd, rot, scale, stream, o_bf16);
    case 64: return launch_qk_attention_hdp<64, 1>(qkv, qn, kn, cs, valid, of, ws, n, heads, hd, rot, scale, stream, o_bf16);
    default:
      return launch_qk_attention_hdp<128, 2>(qkv, qn, kn, cs, valid, of, ws, n, heads, hd, rot, scale, stream, o_bf16);
  }
}

}  // namespace wq
