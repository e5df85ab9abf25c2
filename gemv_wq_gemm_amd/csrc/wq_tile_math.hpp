// Byte-offset arithmetic of the weight-streaming kernels, kept in one header so that the host
// unit test (tests/host/tile_offsets_test.cpp) exercises exactly what the kernels compute.
//
// A weight of m rows of `rowbytes` bytes can pass 2 GiB (a bf16 152064 x 8192 output layer is
// 2.49 GB), so products of a row count and a row length are taken in 64 bits; only offsets that
// stay inside one tile (a few rows) are narrowed to 32 bits, which the direct-to-LDS loads take.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

// Largest start offset, relative to the first byte of the tile whose first row is `row0`, of a
// 16-byte load that stays inside W: min(tile_bytes, bytes of W from row0 on) - 16. The tile's
// loads past that point re-read W's last 16 bytes (their products land in rows that are never
// stored). tile_bytes (R rows) fits in an int; the bytes left in W need not.
__host__ __device__ inline int tile_last_load(int tile_bytes, int m, int row0, long long rowbytes) {
  const long long left = static_cast<long long>(m - row0) * rowbytes;
  return static_cast<int>((left < tile_bytes ? left : static_cast<long long>(tile_bytes)) - 16);
}

}  // namespace wq
