// fp8 GEMM ([SYNC-GEMM] 七: fp8 operands of the asynchronous GEMM, A and B staged in shared
// memory, fp32 accumulation): the fp8 instantiations of the kernel template in
// direct_gemm.h — K-contiguous A [M,K] and B [N,K], 256x256 blocks of 8 waves,
// v_mfma_f32_32x32x64_f8f6f4 — and their host dispatch.
#include "direct_gemm.h"

namespace tg {
namespace {

template <int AF, int BF, bool BOUNDS, int KS>
hipError_t launch_fp8(const GemmArgs& g, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_direct<false, false, fp8_code(AF, BF), 2, 4, BOUNDS, KS>),
                     dim3((unsigned)grid), dim3(512), 0, s, g);
  return hipGetLastError();
}

template <bool BOUNDS, int KS>
hipError_t launch_fp8_b(const GemmArgs& g, int64_t grid, int af, int bf, hipStream_t s) {
  if (af == 0 && bf == 0) return launch_fp8<0, 0, BOUNDS, KS>(g, grid, s);
  if (af == 0) return launch_fp8<0, 1, BOUNDS, KS>(g, grid, s);
  if (bf == 0) return launch_fp8<1, 0, BOUNDS, KS>(g, grid, s);
  return launch_fp8<1, 1, BOUNDS, KS>(g, grid, s);
}

}  // namespace

// MFMA operand format code of a tg_dtype: 0 = e4m3, 1 = e5m2.
static int fp8_format(int dtype) { return dtype == TG_FP8_E5M2 ? 1 : 0; }

hipError_t launch_gemm_fp8(const GemmArgs& g, int64_t grid, int a_dtype, int b_dtype, bool bounds,
                           hipStream_t s) {
  const int af = fp8_format(a_dtype), bf = fp8_format(b_dtype);
  // the shape of the kernel's stage count (K / 128) is fixed at compile time
  const int kt = g.K / Elem<kF8>::kBK;
  const int ks = kt == 1 ? kSingle : (kt & 1) ? kOdd : kEven;
  if (bounds) {
    if (ks == kEven) return launch_fp8_b<true, kEven>(g, grid, af, bf, s);
    if (ks == kOdd) return launch_fp8_b<true, kOdd>(g, grid, af, bf, s);
    return launch_fp8_b<true, kSingle>(g, grid, af, bf, s);
  }
  if (ks == kEven) return launch_fp8_b<false, kEven>(g, grid, af, bf, s);
  if (ks == kOdd) return launch_fp8_b<false, kOdd>(g, grid, af, bf, s);
  return launch_fp8_b<false, kSingle>(g, grid, af, bf, s);
}

}  // namespace tg
