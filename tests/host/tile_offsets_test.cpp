// Host driver for the kernels' tile-offset arithmetic (gemv_wq_gemm_amd/csrc/wq_tile_math.hpp):
// reads "tile_bytes m row0 rowbytes" per line on stdin and prints tile_last_load for each, so the
// test can compare it with exact integer arithmetic. Runs on the CPU; no HIP call is made.
#include <cstdio>

#include "wq_tile_math.hpp"

int main() {
  long long tile_bytes, m, row0, rowbytes;
  while (std::scanf("%lld %lld %lld %lld", &tile_bytes, &m, &row0, &rowbytes) == 4)
    std::printf("%d\n", wq::tile_last_load(static_cast<int>(tile_bytes), static_cast<int>(m),
                                           static_cast<int>(row0), rowbytes));
  return 0;
}
