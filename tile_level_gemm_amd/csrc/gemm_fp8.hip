// fp8 GEMM ([SYNC-GEMM] 七: fp8 operands of the asynchronous GEMM, A and B staged in shared
// memory, fp32 accumulation): dispatch over operand orientation and format, and the
// K-contiguous instantiations (A [M,K], B [N,K]) of the kernel template in direct_gemm.h —
// 256x256 blocks of 8 waves, v_mfma_f32_32x32x64_f8f6f4.
#include "gemm_fp8_launch.h"

namespace tg {

hipError_t launch_fp8_kk(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                         hipStream_t s) {
  return launch_fp8_layout<false, false>(g, grid, af, bf, bounds, bs, s);
}

// MFMA operand format code of a tg_dtype: 0 = e4m3, 1 = e5m2.
static int fp8_format(int dtype) { return dtype == TG_FP8_E5M2 ? 1 : 0; }

hipError_t launch_gemm_fp8(const GemmArgs& g, int64_t grid, int trans_a, int trans_b, int a_dtype,
                           int b_dtype, bool bounds, bool scaled, int bs, hipStream_t s) {
  const int af = fp8_format(a_dtype), bf = fp8_format(b_dtype);
  // A is M-contiguous when stored [K][M] (transA); B is N-contiguous when stored [K][N] (!transB)
  const bool amn = trans_a != 0, bmn = trans_b == 0;
  if (scaled) {
    if (amn && bmn) return launch_mx_mm(g, grid, af, bf, bounds, bs, s);
    if (amn) return launch_mx_mk(g, grid, af, bf, bounds, bs, s);
    if (bmn) return launch_mx_km(g, grid, af, bf, bounds, bs, s);
    return launch_mx_kk(g, grid, af, bf, bounds, bs, s);
  }
  if (amn && bmn) return launch_fp8_mm(g, grid, af, bf, bounds, bs, s);
  if (amn) return launch_fp8_mk(g, grid, af, bf, bounds, bs, s);
  if (bmn) return launch_fp8_km(g, grid, af, bf, bounds, bs, s);
  return launch_fp8_kk(g, grid, af, bf, bounds, bs, s);
}

}  // namespace tg
