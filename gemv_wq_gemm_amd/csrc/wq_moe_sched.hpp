// Which expert's rows a MoE workgroup streams, for the weight-streaming MoE kernels.
//
// hanzo-ml's `moe_matvec_gpu` runs the router gather and the per-expert products in one dispatch
// (src/wgpu_backend.rs). Here the launch is expert-major: each touched expert's rows are streamed
// once for all of its slots. A grid split evenly over all n_exp experts would leave the CUs of the
// untouched ones idle (one token routed to 2 of 8 experts streams with a quarter of the chip), so
// the routing is compacted on the device:
//  * blockIdx.y == 0: G workgroups are dealt over the T experts the ids touch, in expert order,
//    each touched expert getting G / T (or one more) of them and its rows split evenly among those.
//    Every workgroup builds the same bitmap of touched experts from the ids (LDS atomics), so no
//    pass over the ids precedes the launch.
//  * blockIdx.y == 1: G workgroups write NaN into the outputs of slots whose id is out of range.
// Needs n_exp <= kMoeCompactMax and G >= n_exp (every touched expert then gets a workgroup).
#pragma once

#include <hip/hip_runtime.h>

#include "wq_internal.hpp"

namespace wq {

constexpr int kMoeCompactMax = 256;  // experts the bitmap holds (8 words of LDS)

struct MoeAssign {
  int e;                // expert whose rows this workgroup streams (n_exp: the NaN writer; -1: none)
  int t_begin, t_end;   // its tiles of that expert's rows
};

// Called by every thread of the workgroup (two barriers). `bitmap` is 8 words of LDS.
// `tiles_per_wg` is the NaN writers' share of the rows: ceil(ntiles / gridDim.x).
__device__ inline MoeAssign moe_assign(const MatvecParams& p, int ntiles, int tiles_per_wg, uint32_t* bitmap) {
  MoeAssign a;
  if (blockIdx.y == 1) {
    a.e = p.n_exp;
    a.t_begin = blockIdx.x * tiles_per_wg;
    a.t_end = min(ntiles, a.t_begin + tiles_per_wg);
    return a;
  }
  if (threadIdx.x < kMoeCompactMax / 32) bitmap[threadIdx.x] = 0u;
  __syncthreads();
  for (int s = threadIdx.x; s < p.n_slots; s += blockDim.x) {
    const int id = p.ids[s];
    if (id >= 0 && id < p.n_exp) atomicOr(&bitmap[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  uint32_t words[kMoeCompactMax / 32];
  int touched = 0;
#pragma unroll
  for (int i = 0; i < kMoeCompactMax / 32; ++i) {
    words[i] = bitmap[i];
    touched += __popc(words[i]);
  }
  a.e = -1;
  a.t_begin = a.t_end = 0;
  if (touched == 0) return a;
  // Workgroups [f0, f1) go to the r-th touched expert: r = floor(b T / G), f_r = ceil(r G / T).
  const long long G = gridDim.x, T = touched, b = blockIdx.x;
  const int r = static_cast<int>(b * T / G);
  const int f0 = static_cast<int>((r * G + T - 1) / T);
  const int f1 = static_cast<int>(((r + 1) * G + T - 1) / T);
  const int tpw = (ntiles + (f1 - f0) - 1) / (f1 - f0);
  a.t_begin = (static_cast<int>(b) - f0) * tpw;
  a.t_end = min(ntiles, a.t_begin + tpw);
  // The r-th set bit of the bitmap.
  int left = r;
#pragma unroll
  for (int i = 0; i < kMoeCompactMax / 32; ++i) {
    const int c = __popc(words[i]);
    if (a.e < 0 && left < c) {
      uint32_t x = words[i];
      for (int q = 0; q < left; ++q) x &= x - 1u;
      a.e = i * 32 + __ffs(x) - 1;
    }
    left -= c;
  }
  return a;
}

}  // namespace wq
