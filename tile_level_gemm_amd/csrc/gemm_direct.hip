// Large-tile GEMM on gfx950 with direct global -> LDS operand loads: the f16 / bf16
// instantiations of the kernel template in direct_gemm.h for whole 256x256 blocks and K a
// multiple of 128, and the host dispatch (ragged shapes: gemm_direct_*.hip).
#include "gemm_direct_launch.h"

namespace tg {
namespace {

// LDS swizzles: both operands use variant 1 (conflict-free for 64-bank reads; measured
// zero SQ_LDS_BANK_CONFLICT on gfx950, against 50 % of LDS-active cycles with variant 0).
// Wave grid 2 x 4 (8 waves, 128 x 64 each, 2 per SIMD): measured 1-2 % ahead of 2 x 2
// (4 waves of 128 x 128) on the same box; 4 x 2 spills.
template <bool A_MN, bool B_MN, int DT>
hipError_t launch_direct_dt(const GemmArgs& g, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_direct<A_MN, B_MN, DT, 2, 4, false, kEven>), dim3((unsigned)grid), dim3(512), 0, s, g);
  return hipGetLastError();
}

}  // namespace

// Each operand, with K rounded up to whole 64-K stages, under 2 GiB: the DMA of an M/N-major
// operand addresses k-rows up to the end of the last stage (those past K are range-checked
// to zero), and every buffer offset (per-lane plus per-stage, and the out-of-range 2^31 of a
// partial last stage plus the stage offset) must fit the 32-bit fields without wrapping back
// into the operand.
bool direct_gemm_fits(int64_t M, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t kp = (K + 63) / 64 * 64;
  return M > 0 && N > 0 && K > 0 && M * kp * 2 < lim && kp * N * 2 < lim;
}

hipError_t launch_gemm_direct(const GemmArgs& g, int64_t grid, int trans_a, int trans_b, int dtype,
                              int bs, hipStream_t s) {
  // A is M/N-major when stored [K][M] (transA); B is M/N-major when stored [K][N] (!transB).
  const bool amn = trans_a != 0, bmn = trans_b == 0;
  const bool exact = bs == 256 && g.M % bs == 0 && g.N % bs == 0 &&
                     g.K % (2 * Elem<TG_F16>::kBK) == 0;
  if (!exact) {
    const bool bounds = g.M % bs != 0 || g.N % bs != 0;
    if (amn && bmn) return launch_direct16_mm(g, grid, dtype, bounds, bs, s);
    if (amn) return launch_direct16_mk(g, grid, dtype, bounds, bs, s);
    if (bmn) return launch_direct16_km(g, grid, dtype, bounds, bs, s);
    return launch_direct16_kk(g, grid, dtype, bounds, bs, s);
  }
  if (dtype == TG_F16) {
    if (amn && bmn) return launch_direct_dt<true, true, TG_F16>(g, grid, s);
    if (amn) return launch_direct_dt<true, false, TG_F16>(g, grid, s);
    if (bmn) return launch_direct_dt<false, true, TG_F16>(g, grid, s);
    return launch_direct_dt<false, false, TG_F16>(g, grid, s);
  }
  if (amn && bmn) return launch_direct_dt<true, true, TG_BF16>(g, grid, s);
  if (amn) return launch_direct_dt<true, false, TG_BF16>(g, grid, s);
  if (bmn) return launch_direct_dt<false, true, TG_BF16>(g, grid, s);
  return launch_direct_dt<false, false, TG_BF16>(g, grid, s);
}

}  // namespace tg
