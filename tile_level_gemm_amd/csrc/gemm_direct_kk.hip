// 16-bit GEMM instantiations of the direct-load kernel template for ragged shapes, A stored
// [M,K] and B stored [N,K].
#include "gemm_direct_launch.h"

namespace tg {

hipError_t launch_direct16_kk(const GemmArgs& g, int64_t grid, int dtype, bool bounds,
                              hipStream_t s) {
  return launch_direct16_layout<false, false>(g, grid, dtype, bounds, s);
}

}  // namespace tg
