// 16-bit GEMM instantiations of the direct-load kernel template for ragged shapes and 128x128 blocks, A stored
// [M,K] and B stored [N,K].
#include "gemm_direct_launch.h"

namespace tg {

hipError_t launch_direct16_kk(const GemmArgs& g, int64_t grid, int dtype, bool bounds, int bs,
                              hipStream_t s) {
  return launch_direct16_layout<false, false>(g, grid, dtype, bounds, bs, s);
}

}  // namespace tg
