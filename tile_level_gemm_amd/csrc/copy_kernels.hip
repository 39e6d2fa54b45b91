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

// XCD-aware block order.  Workgroups are dealt round-robin to the 8 XCDs (each with its own
// L2), so block b runs on XCD b % 8.  Renumbering b -> (b % 8)·(grid / 8) + b / 8 gives each
// XCD a contiguous range of tiles: the workgroups resident on one XCD at a time then cover
// neighbouring tiles, whose row segments join into long contiguous runs in HBM.
__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t grid) {
  return grid % 8 ? b : (b % 8) * (grid / 8) + b / 8;
}

template <int VL, int VS>
__global__ __launch_bounds__(1024) void tile_copy_kernel(CopyArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  using TL = typename VecT<VL>::T;
  using TS = typename VecT<VS>::T;
  const int t = threadIdx.x;
  const int T = a.threads;
  for (int64_t tile = xcd_block(blockIdx.x, gridDim.x); tile < a.ntiles; tile += gridDim.x) {
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

// Row-major fast path: both global sides row-major, one vector width VB for both directions,
// and each round covers whole tile rows (threads·VB is a multiple of the tile's row bytes).
// Then the element a thread moves in round f sits at row r_t + f·rpr, byte column cb_t,
// where (r_t, cb_t) come from the thread index once; with rpr a multiple of the XOR period
// the swizzled LDS offset only advances by rpr rows per round.  Same partition and result
// as tile_copy_kernel, with the per-round divisions and layout switches folded away.
//
// A workgroup moves TPB horizontally adjacent tiles at once, each in its own LDS tile with the
// same partition, issuing round f of every tile before round f + 1: a wave's consecutive
// loads then walk along the same rows, TPB·(row bytes) of each row per workgroup.  On MI355X
// HBM rewards such runs: 16384 x 16384 fp16 in 128x64 tiles moves at about 5.5 TB/s with one
// tile per workgroup and about 6.4 TB/s with four.  ROWB = 128 fixes the tile's row bytes at
// compile time (the default tile: 128-byte rows for every element size): the tiles of a group
// are then immediate offsets of one address per round, which measured about 3 % faster than
// computing all ROUNDS x TPB addresses.
template <int VB, int ROUNDS, int TPB, int ROWB>
__global__ __launch_bounds__(1024) void tile_copy_rows(CopyArgs a, int32_t rpr) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  using TV = typename VecT<VB>::T;
  const uint32_t rowb = ROWB ? (uint32_t)ROWB : (uint32_t)(a.tile_cols * a.eb);
  const uint32_t tile_lds = rowb * (uint32_t)a.tile_rows;
  const uint32_t xb = (uint32_t)threadIdx.x * VB;
  const uint32_t r_t = xb / rowb, cb_t = xb - r_t * rowb;
  const uint32_t lds_t = a.lds_xor ? xor_swizzle_bytes(r_t, cb_t, rowb, (uint32_t)a.xor_mask)
                                   : r_t * rowb + cb_t;
  const uint32_t lds_step = (uint32_t)rpr * rowb;
  const int64_t src_step = (int64_t)rpr * a.src_ld * a.eb;
  const int64_t dst_step = (int64_t)rpr * a.dst_ld * a.eb;
  const int64_t groups = a.ntiles / TPB;   // tiles_c % TPB == 0: a group stays in one tile row
  const int64_t first = TPB == 1 ? xcd_block(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
  for (int64_t grp = first; grp < groups; grp += gridDim.x) {
    const int64_t tile = grp * TPB;
    // tile row / column: 32-bit division when the indices fit (the usual case), 64-bit otherwise
    int64_t tr, tc;
    if (a.ntiles < ((int64_t)1 << 32)) {
      const uint32_t t32 = (uint32_t)tile, n32 = (uint32_t)a.tiles_c;
      tr = t32 / n32;
      tc = t32 - (uint32_t)tr * n32;
    } else {
      tr = tile / a.tiles_c;
      tc = tile - tr * a.tiles_c;
    }
    const int64_t r0 = tr * a.tile_rows + r_t;
    const int64_t c0 = tc * a.tile_cols;
    const uint8_t* sp = a.src + (r0 * a.src_ld + c0) * a.eb + cb_t;
    uint8_t* dp = a.dst + (r0 * a.dst_ld + c0) * a.eb + cb_t;
    // all ROUNDS x TPB loads are in flight before the first LDS write
    TV v[ROUNDS][TPB];
#pragma unroll
    for (int f = 0; f < ROUNDS; ++f)
#pragma unroll
      for (int k = 0; k < TPB; ++k)
        v[f][k] = __builtin_nontemporal_load((const TV*)(sp + f * src_step + k * (int64_t)rowb));
    // The previous group's LDS reads must be done before these writes.  The barrier sits
    // here, not after the stores, so a workgroup's last stores are never waited for.
    if (grp != first) __syncthreads();
#pragma unroll
    for (int f = 0; f < ROUNDS; ++f)
#pragma unroll
      for (int k = 0; k < TPB; ++k) *(TV*)(lds + k * tile_lds + lds_t + (uint32_t)f * lds_step) = v[f][k];
    __syncthreads();
#pragma unroll
    for (int f = 0; f < ROUNDS; ++f)
#pragma unroll
      for (int k = 0; k < TPB; ++k)
        __builtin_nontemporal_store(*(const TV*)(lds + k * tile_lds + lds_t + (uint32_t)f * lds_step),
                                    (TV*)(dp + f * dst_step + k * (int64_t)rowb));
  }
}

template <int VB, int ROUNDS, int TPB>
hipError_t launch_rows_one(const CopyArgs& a, int32_t rpr, dim3 g, dim3 b, int lds, hipStream_t s) {
  if constexpr (ROUNDS * TPB > 16) {
    return hipErrorInvalidValue;   // more than 16 vectors per thread: never chosen
  } else {
    if (a.tile_cols * a.eb == 128)
      hipLaunchKernelGGL((tile_copy_rows<VB, ROUNDS, TPB, 128>), g, b, lds, s, a, rpr);
    else
      hipLaunchKernelGGL((tile_copy_rows<VB, ROUNDS, TPB, 0>), g, b, lds, s, a, rpr);
    return hipGetLastError();
  }
}

template <int VB, int TPB>
hipError_t launch_rows_t(const CopyArgs& a, int32_t rpr, int rounds, dim3 g, dim3 b, int lds,
                         hipStream_t s) {
  switch (rounds) {
    case 1: return launch_rows_one<VB, 1, TPB>(a, rpr, g, b, lds, s);
    case 2: return launch_rows_one<VB, 2, TPB>(a, rpr, g, b, lds, s);
    case 4: return launch_rows_one<VB, 4, TPB>(a, rpr, g, b, lds, s);
    case 8: return launch_rows_one<VB, 8, TPB>(a, rpr, g, b, lds, s);
    default: return hipErrorInvalidValue;
  }
}

template <int VB>
hipError_t launch_rows(const CopyArgs& a, int32_t rpr, int rounds, int tpb, dim3 g, dim3 b, int lds,
                       hipStream_t s) {
  switch (tpb) {
    case 1: return launch_rows_t<VB, 1>(a, rpr, rounds, g, b, lds, s);
    case 2: return launch_rows_t<VB, 2>(a, rpr, rounds, g, b, lds, s);
    case 4: return launch_rows_t<VB, 4>(a, rpr, rounds, g, b, lds, s);
    default: return hipErrorInvalidValue;
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
  const int64_t rowb = (int64_t)a.tile_cols * a.eb;
  const int64_t round_bytes = (int64_t)a.threads * vl;
  const int rounds = a.load.outer;
  const bool rows_fast = a.src_kind == TG_ROW_MAJOR && a.dst_kind == TG_ROW_MAJOR && vl == vs &&
                         (vl == 16 || vl == 8 || vl == 4) && round_bytes % rowb == 0 &&
                         (!a.lds_xor || ((round_bytes / rowb) % (a.xor_mask + 1)) == 0) &&
                         a.load.outer == a.store.outer && a.load.row_order && a.store.row_order &&
                         (rounds == 1 || rounds == 2 || rounds == 4 || rounds == 8);
  if (rows_fast) {
    const int32_t rpr = (int32_t)(round_bytes / rowb);
    // Tiles per workgroup: up to 4 horizontally adjacent tiles, within 64 KiB of LDS and 16
    // vectors of registers per thread.
    int tpb = 4;
    while (tpb > 1 && (a.tiles_c % tpb || (int64_t)tpb * lds_bytes > 65536 || rounds * tpb > 16))
      tpb /= 2;
    const int64_t groups = a.ntiles / tpb;
    const dim3 gr((unsigned)(groups < (1 << 20) ? groups : (1 << 20)));
    if (vl == 16) e = launch_rows<16>(a, rpr, rounds, tpb, gr, b, tpb * lds_bytes, s);
    else if (vl == 8) e = launch_rows<8>(a, rpr, rounds, tpb, gr, b, tpb * lds_bytes, s);
    else e = launch_rows<4>(a, rpr, rounds, tpb, gr, b, tpb * lds_bytes, s);
    if (e != hipSuccess) return fail(TG_E_HIP, std::string("tile_copy launch: ") + hipGetErrorString(e));
    return TG_OK;
  }
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
