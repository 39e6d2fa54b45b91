// Host launch of the fp8 and block-scaled fp8 instantiations of the direct-load GEMM template,
// one operand orientation per translation unit (gemm_fp8*.hip, gemm_mx*.hip) so that they
// compile in parallel.  Internal header.
#pragma once

#include "direct_gemm.h"

namespace tg {

// A_MN: A stored [K][M]; B_MN: B stored [K][N].  af / bf: the MFMA format codes (0 = e4m3,
// 1 = e5m2).  The stage-count shape (K / 128 even, odd, or one) is fixed at compile time.
// SCALED: block-scaled fp8 (g.SA, g.SB hold the E8M0 scales).  bs: block size, 256 or 128 (8
// waves in a 2 x 4 grid either way).
template <bool A_MN, bool B_MN, bool SCALED = false>
hipError_t launch_fp8_layout(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                             hipStream_t s) {
  auto go = [&](auto AF, auto BF, auto BOUNDS, auto KS) {
    constexpr int dt = SCALED ? mx_code(decltype(AF)::value, decltype(BF)::value)
                              : fp8_code(decltype(AF)::value, decltype(BF)::value);
    constexpr bool b = decltype(BOUNDS)::value;
    constexpr int ks = decltype(KS)::value;
    if (bs == 128) {
      hipLaunchKernelGGL((gemm_direct128<A_MN, B_MN, dt, 2, 4, b, ks>), dim3((unsigned)grid),
                         dim3(512), 0, s, g);
      return hipGetLastError();
    }
    if (bs != 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_direct<A_MN, B_MN, dt, 2, 4, b, ks>), dim3((unsigned)grid), dim3(512), 0,
                       s, g);
    return hipGetLastError();
  };
  using Z = std::integral_constant<int, 0>;
  using O = std::integral_constant<int, 1>;
  auto ks = [&](auto AF, auto BF, auto BOUNDS) {
    const int kt = g.K / Elem<kF8>::kBK;
    if (kt == 1) return go(AF, BF, BOUNDS, std::integral_constant<int, kSingle>{});
    if (kt & 1) return go(AF, BF, BOUNDS, std::integral_constant<int, kOdd>{});
    return go(AF, BF, BOUNDS, std::integral_constant<int, kEven>{});
  };
  auto fmt = [&](auto BOUNDS) {
    if (af == 0 && bf == 0) return ks(Z{}, Z{}, BOUNDS);
    if (af == 0) return ks(Z{}, O{}, BOUNDS);
    if (bf == 0) return ks(O{}, Z{}, BOUNDS);
    return ks(O{}, O{}, BOUNDS);
  };
  return bounds ? fmt(std::true_type{}) : fmt(std::false_type{});
}

hipError_t launch_fp8_kk(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                         hipStream_t s);
hipError_t launch_fp8_km(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                         hipStream_t s);
hipError_t launch_fp8_mk(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                         hipStream_t s);
hipError_t launch_fp8_mm(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                         hipStream_t s);
hipError_t launch_mx_kk(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                         hipStream_t s);
hipError_t launch_mx_km(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                         hipStream_t s);
hipError_t launch_mx_mk(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                         hipStream_t s);
hipError_t launch_mx_mm(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                         hipStream_t s);

}  // namespace tg
