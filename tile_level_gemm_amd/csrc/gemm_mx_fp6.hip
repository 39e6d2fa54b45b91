// Block-scaled 6-bit GEMM ([SYNC-GEMM] 七: block-scaled operands with SFA / SFB; e2m3 and e3m2,
// the 6-bit members of the format family the matrix unit takes with fp4) on the direct-load
// kernel template: A stored [M][3K/4] and B stored [N][3K/4] as packed rows, K a multiple of
// 128 (one 96-byte stage row).
#include "direct_gemm.h"

namespace tg {

hipError_t launch_fp6_direct(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                             hipStream_t s) {
  auto go = [&](auto AF, auto BF, auto BOUNDS, auto KS) {
    constexpr int dt = p6_code(decltype(AF)::value, decltype(BF)::value);
    constexpr bool b = decltype(BOUNDS)::value;
    constexpr int ks = decltype(KS)::value;
    if (bs == 128) {
      hipLaunchKernelGGL((gemm_direct128<false, false, dt, 2, 4, b, ks>), dim3((unsigned)grid),
                         dim3(512), 0, s, g);
      return hipGetLastError();
    }
    if (bs != 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_direct<false, false, dt, 2, 4, b, ks>), dim3((unsigned)grid),
                       dim3(512), 0, s, g);
    return hipGetLastError();
  };
  using E23 = std::integral_constant<int, 2>;
  using E32 = std::integral_constant<int, 3>;
  auto ks = [&](auto AF, auto BF, auto BOUNDS) {
    if (g.K % 128 != 0 || g.K <= 0) return hipErrorInvalidValue;
    const int kt = g.K / 128;
    if (kt == 1) return go(AF, BF, BOUNDS, std::integral_constant<int, kSingle>{});
    if (kt & 1) return go(AF, BF, BOUNDS, std::integral_constant<int, kOdd>{});
    return go(AF, BF, BOUNDS, std::integral_constant<int, kEven>{});
  };
  auto fmt = [&](auto BOUNDS) {
    if (af == 2 && bf == 2) return ks(E23{}, E23{}, BOUNDS);
    if (af == 2 && bf == 3) return ks(E23{}, E32{}, BOUNDS);
    if (af == 3 && bf == 2) return ks(E32{}, E23{}, BOUNDS);
    if (af == 3 && bf == 3) return ks(E32{}, E32{}, BOUNDS);
    return hipErrorInvalidValue;
  };
  return bounds ? fmt(std::true_type{}) : fmt(std::false_type{});
}

}  // namespace tg
