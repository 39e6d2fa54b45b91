// fp8 GEMM instantiations of the direct-load kernel template for A stored [K,M] and B stored [K,N].
#include "gemm_fp8_launch.h"

namespace tg {

hipError_t launch_fp8_mm(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                         hipStream_t s) {
  return launch_fp8_layout<true, true>(g, grid, af, bf, bounds, bs, s);
}

}  // namespace tg
