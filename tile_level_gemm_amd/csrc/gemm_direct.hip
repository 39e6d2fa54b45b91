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

// Each operand under 2 GiB (its byte count is the 32-bit num_records of its buffer
// descriptor), and no 32-bit buffer offset may wrap: a wrapped offset lands back inside the
// operand instead of past its end, where the range check returns zeros.  A K-major operand
// addresses its own rows only (a partial last stage masks the chunks past K per lane with the
// offset 2^31, and 2^31 plus a stage offset stays below 2^32).  The DMA of an M/N-major
// operand addresses k-rows up to the end of its last 64-K stage, so whole stages of it must
// span at most 2^32 bytes; the k-rows past K then lie between the operand's end and 2^32 and
// read as zero.
bool direct_gemm_fits(int64_t M, int64_t N, int64_t K, int trans_a, int trans_b) {
  const int64_t lim = (int64_t)1 << 31, wrap = (int64_t)1 << 32;
  const int64_t kp = (K + 63) / 64 * 64;
  if (M <= 0 || N <= 0 || K <= 0 || M * K * 2 >= lim || K * N * 2 >= lim) return false;
  if (trans_a && kp * M * 2 > wrap) return false;    // A stored [K][M]
  if (!trans_b && kp * N * 2 > wrap) return false;   // B stored [K][N]
  return true;
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
