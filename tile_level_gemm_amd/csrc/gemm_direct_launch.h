// Host launch of the 16-bit instantiations of the direct-load GEMM template for shapes that
// are not whole 256x256 blocks with K a multiple of 128, and for 128x128 blocks: ragged M or N
// (BOUNDS), a stage count of any parity and a partial last stage (kTail).  One operand orientation per translation unit
// (gemm_direct_*.hip) so that they compile in parallel.  Internal header.
#pragma once

#include "direct_gemm.h"

namespace tg {

// A_MN: A stored [K][M]; B_MN: B stored [K][N].  dtype: TG_F16 or TG_BF16.  bs: block size,
// 256 or 128.
template <bool A_MN, bool B_MN>
hipError_t launch_direct16_layout(const GemmArgs& g, int64_t grid, int dtype, bool bounds, int bs,
                                  hipStream_t s) {
  auto go = [&](auto DT, auto BOUNDS, auto KS) {
    constexpr int dt = decltype(DT)::value, ks = decltype(KS)::value | kTail;
    constexpr bool b = decltype(BOUNDS)::value;
    // both block sizes: 8 waves in a 2 x 4 grid (on 128x128 blocks measured within a few per
    // cent of 4 waves of 64 x 64: ahead for long K, behind at 3072^3)
    if (bs == 128)
      hipLaunchKernelGGL((gemm_direct128<A_MN, B_MN, dt, 2, 4, b, ks>), dim3((unsigned)grid),
                         dim3(512), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_direct<A_MN, B_MN, dt, 2, 4, b, ks>), dim3((unsigned)grid), dim3(512),
                         0, s, g);
    return hipGetLastError();
  };
  auto ks = [&](auto DT, auto BOUNDS) {
    const int kt = (g.K + Elem<TG_F16>::kBK - 1) / Elem<TG_F16>::kBK;
    if (kt == 1) return go(DT, BOUNDS, std::integral_constant<int, kSingle>{});
    if (kt & 1) return go(DT, BOUNDS, std::integral_constant<int, kOdd>{});
    return go(DT, BOUNDS, std::integral_constant<int, kEven>{});
  };
  auto dt = [&](auto BOUNDS) {
    if (dtype == TG_F16) return ks(std::integral_constant<int, TG_F16>{}, BOUNDS);
    return ks(std::integral_constant<int, TG_BF16>{}, BOUNDS);
  };
  return bounds ? dt(std::true_type{}) : dt(std::false_type{});
}

hipError_t launch_direct16_kk(const GemmArgs& g, int64_t grid, int dtype, bool bounds, int bs,
                              hipStream_t s);
hipError_t launch_direct16_km(const GemmArgs& g, int64_t grid, int dtype, bool bounds, int bs,
                              hipStream_t s);
hipError_t launch_direct16_mk(const GemmArgs& g, int64_t grid, int dtype, bool bounds, int bs,
                              hipStream_t s);
hipError_t launch_direct16_mm(const GemmArgs& g, int64_t grid, int dtype, bool bounds, int bs,
                              hipStream_t s);

}  // namespace tg
