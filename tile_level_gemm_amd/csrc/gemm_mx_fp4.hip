// Block-scaled e2m1 GEMM ([SYNC-GEMM] 七: fp4 operands with SFA / SFB block scales) on the
// direct-load kernel template: A stored [M][K/2] and B stored [N][K/2] as packed rows, K a
// multiple of 256 (one 128-byte stage row).
#include "direct_gemm.h"

namespace tg {

hipError_t launch_fp4_direct(const GemmArgs& g, int64_t grid, bool bounds, int bs, hipStream_t s) {
  auto go = [&](auto BOUNDS, auto KS) {
    constexpr bool b = decltype(BOUNDS)::value;
    constexpr int ks = decltype(KS)::value;
    if (bs == 128) {
      hipLaunchKernelGGL((gemm_direct128<false, false, kP4, 2, 4, b, ks>), dim3((unsigned)grid),
                         dim3(512), 0, s, g);
      return hipGetLastError();
    }
    if (bs != 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_direct<false, false, kP4, 2, 4, b, ks>), dim3((unsigned)grid),
                       dim3(512), 0, s, g);
    return hipGetLastError();
  };
  auto ks = [&](auto BOUNDS) {
    if (g.K % 256 != 0 || g.K <= 0) return hipErrorInvalidValue;
    const int kt = g.K / 256;
    if (kt == 1) return go(BOUNDS, std::integral_constant<int, kSingle>{});
    if (kt & 1) return go(BOUNDS, std::integral_constant<int, kOdd>{});
    return go(BOUNDS, std::integral_constant<int, kEven>{});
  };
  return bounds ? ks(std::true_type{}) : ks(std::false_type{});
}

}  // namespace tg
