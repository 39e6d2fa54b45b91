// Block-scaled fp8 GEMM ([SYNC-GEMM] 七: block-scaled operands, SFA / SFB) instantiations of the
// direct-load kernel template for A stored [M,K] and B stored [N,K].
#include "gemm_fp8_launch.h"

namespace tg {

hipError_t launch_mx_kk(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                        hipStream_t s) {
  return launch_fp8_layout<false, false, true>(g, grid, af, bf, bounds, bs, s);
}

}  // namespace tg
