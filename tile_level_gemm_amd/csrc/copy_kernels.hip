// Tile copy on gfx950: global -> LDS -> global, bit exact.
//
// [VEC-AUTO] ("TVM TIRx CUDA 向量化内存拷贝实战：vec_auto 变体的 global↔shared 实现路径
// （gmem_smem）深度解析"): a copy between global and shared memory has no register side
// to lend it a thread partition, so one is synthesised from the execution scope as
// [outer, threads, vec] (算法核心 step 1); round f of thread t moves the fused
// elements [(f*threads + t)*vec, +vec) with one vector load and one vector store,
// through a register container that only carries bits (生成的 TIRx IR / PTX).
//
// gfx950 design: a workgroup owns one tile at a time (grid-stride over tiles).
// The load direction issues up to kBatch vector loads per thread before the first
// LDS write, so every wave keeps kBatch x 16 bytes in flight to HBM; the LDS tile
// is XOR-swizzled on 16-byte chunks (lds_layout.h); the store direction reads LDS
// and writes global with the same vector rule, driven by the destination's order.
// The vector widths of both directions are template parameters (16/8/4/2/1 bytes),
// chosen on the host by the width rule; there is no scalar fallback path.
#include <hip/hip_runtime.h>

#include "lds_layout.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kBatch = 8;

template <int VB>
struct VecT;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
template <>
struct VecT<16> { using T = u32x4; };
template <>
struct VecT<8> { using T = u32x2; };
template <>
struct VecT<4> { using T = uint32_t; };
template <>
struct VecT<2> { using T = uint16_t; };
template <>
struct VecT<1> { using T = uint8_t; };

// Element offset of logical (r, c) of the full tensor on a global side.
__device__ __forceinline__ int64_t global_elem(int kind, int64_t ld, int64_t r, int64_t c,
                                               int32_t cols, int32_t eb, int32_t mask) {
  if (kind == TG_COL_MAJOR) return c * ld + r;
  if (kind == TG_ROW_MAJOR) return r * ld + c;
  // one-tile XOR-swizzled tensor
  return (int64_t)xor_swizzle_bytes((uint32_t)r, (uint32_t)(c * eb), (uint32_t)(cols * eb),
                                    (uint32_t)mask) / eb;
}

__device__ __forceinline__ uint32_t lds_byte(const CopyArgs& a, uint32_t r, uint32_t c) {
  const uint32_t pitch = (uint32_t)(a.tile_cols * a.eb);
  const uint32_t cb = c * (uint32_t)a.eb;
  return a.lds_xor ? xor_swizzle_bytes(r, cb, pitch, (uint32_t)a.xor_mask) : r * pitch + cb;
}

// Tile-local (r, c) of the first element of the transfer of round f, thread t.
__device__ __forceinline__ void coords(const CopyPhase& p, int threads, int f, int t, uint32_t* r,
                                       uint32_t* c) {
  const uint32_t x = ((uint32_t)f * (uint32_t)threads + (uint32_t)t) * (uint32_t)p.vec;
  uint32_t o, i;
  if (p.inner_log2 >= 0) {
    o = x >> p.inner_log2;
    i = x & ((1u << p.inner_log2) - 1u);
  } else {
    o = x / (uint32_t)p.inner;
    i = x - o * (uint32_t)p.inner;
  }
  if (p.row_order) {
    *r = o;
    *c = i;
  } else {
    *r = i;
    *c = o;
  }
}

template <int VL, int VS>
__global__ __launch_bounds__(1024) void tile_copy_kernel(CopyArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  using TL = typename VecT<VL>::T;
  using TS = typename VecT<VS>::T;
  const int t = threadIdx.x;
  const int T = a.threads;
  for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int64_t r0 = (tile / a.tiles_c) * a.tile_rows;
    const int64_t c0 = (tile % a.tiles_c) * a.tile_cols;
    // global -> LDS, kBatch loads in flight per thread
    for (int f0 = 0; f0 < a.load.outer; f0 += kBatch) {
      TL v[kBatch];
      uint32_t lo[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (f0 + j < a.load.outer) {
          uint32_t r, c;
          coords(a.load, T, f0 + j, t, &r, &c);
          const int64_t e = global_elem(a.src_kind, a.src_ld, r0 + r, c0 + c, a.tile_cols, a.eb,
                                        a.xor_mask);
          v[j] = __builtin_nontemporal_load((const TL*)(a.src + e * a.eb));
          lo[j] = lds_byte(a, r, c);
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (f0 + j < a.load.outer) *(TL*)(lds + lo[j]) = v[j];
    }
    __syncthreads();
    // LDS -> global
    for (int f0 = 0; f0 < a.store.outer; f0 += kBatch) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (f0 + j < a.store.outer) {
          uint32_t r, c;
          coords(a.store, T, f0 + j, t, &r, &c);
          const TS v = *(const TS*)(lds + lds_byte(a, r, c));
          const int64_t e = global_elem(a.dst_kind, a.dst_ld, r0 + r, c0 + c, a.tile_cols, a.eb,
                                        a.xor_mask);
          __builtin_nontemporal_store(v, (TS*)(a.dst + e * a.eb));
        }
      }
    }
    __syncthreads();
  }
}

template <int VL>
hipError_t launch_vs(const CopyArgs& a, int vs, dim3 grid, dim3 block, int lds, hipStream_t s) {
  switch (vs) {
    case 16: hipLaunchKernelGGL((tile_copy_kernel<VL, 16>), grid, block, lds, s, a); break;
    case 8: hipLaunchKernelGGL((tile_copy_kernel<VL, 8>), grid, block, lds, s, a); break;
    case 4: hipLaunchKernelGGL((tile_copy_kernel<VL, 4>), grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((tile_copy_kernel<VL, 2>), grid, block, lds, s, a); break;
    case 1: hipLaunchKernelGGL((tile_copy_kernel<VL, 1>), grid, block, lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int launch_tile_copy(const CopyArgs& a, int vl, int vs, int lds_bytes, void* stream) {
  // One workgroup per tile up to a cap; the kernel strides over the rest.
  const int64_t grid = a.ntiles < (1 << 20) ? a.ntiles : (1 << 20);
  const dim3 g((unsigned)grid), b((unsigned)a.threads);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (vl) {
    case 16: e = launch_vs<16>(a, vs, g, b, lds_bytes, s); break;
    case 8: e = launch_vs<8>(a, vs, g, b, lds_bytes, s); break;
    case 4: e = launch_vs<4>(a, vs, g, b, lds_bytes, s); break;
    case 2: e = launch_vs<2>(a, vs, g, b, lds_bytes, s); break;
    case 1: e = launch_vs<1>(a, vs, g, b, lds_bytes, s); break;
    default: e = hipErrorInvalidValue;
  }
  if (e != hipSuccess) return fail(TG_E_HIP, std::string("tile_copy launch: ") + hipGetErrorString(e));
  return TG_OK;
}

}  // namespace tg
