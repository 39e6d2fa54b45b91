// Asynchronous tile copy: issue-only global -> LDS transfers whose completion the issuing code
// owns ([TCGEN05-CP] 一个算子、六个变体 and 与其他异步变体的协作关系: a copy_async variant only
// issues the transfer; the caller commits and waits before it uses the data).
//
// On gfx950 the issue is buffer_load_dwordx4 ... lds (or _dword): lane i of a wave sends its
// chunk from HBM to LDS at the wave's base + i·size, without passing through VGPRs, and the
// transfer counts in the wave's vmcnt.  (The buffer form, not global_load_lds: for it the
// compiler tracks which LDS array a transfer writes, and does not make reads of the other
// stages wait for it.)  The wait is the issuing wave's s_waitcnt vmcnt(n), where n is the
// number of its transfers issued after the tile it needs (vector loads complete in order), and
// then a workgroup barrier so that every wave's part of the tile has landed.
//
// A workgroup streams tiles_per_wg consecutive tiles through DEPTH LDS stages: tile k + DEPTH - 1
// is issued before tile k is waited for, so DEPTH tiles are in flight.  Each stage is its own
// named LDS array and the loop is unrolled over the stages, so the compiler sees which stage a
// read touches and does not wait for transfers into the other stages.
#include <hip/hip_runtime.h>

#include "lds_layout.h"
#include "tg_internal.h"

namespace tg {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(3))) void lds_void;

__shared__ __attribute__((aligned(1024))) uint8_t g_stage0[kAsyncStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage1[kAsyncStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage2[kAsyncStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage3[kAsyncStageBytes];

template <int J>
__device__ __forceinline__ uint8_t* stage() {
  if constexpr (J == 0) return g_stage0;
  else if constexpr (J == 1) return g_stage1;
  else if constexpr (J == 2) return g_stage2;
  else return g_stage3;
}

template <int VB>
struct Vec;
template <> struct Vec<16> { typedef u32x4 T; };
template <> struct Vec<4> { typedef uint32_t T; };

// Wait until at most N of this wave's vector memory operations are outstanding (expcnt and
// lgkmcnt left at their maxima: no wait on them).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070 | 0x0F00);
}

// Workgroup barrier without a memory fence: a fence would wait for every outstanding
// transfer, the newer tiles' included.  The memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int VB, int R, int DEPTH>
struct AsyncCopy {
  const CopyArgs& a;
  int64_t first;      // first tile of this workgroup
  int n;              // tiles of this workgroup
  uint32_t rowb, tile_bytes;
  uint32_t src_span;  // bytes of the source a tile spans (the buffer range of its transfers)
  uint32_t lds_wave;  // byte offset of this wave's first slot within a round
  uint32_t goff[R];   // per round: source byte offset (from the tile origin) of this lane's chunk
  uint32_t loff[R];   // per round: LDS byte offset of the chunk this thread stores
  uint32_t doff[R];   // per round: destination byte offset (from the tile origin)
  bool dst_image;     // destination is the one-tile LDS image

  // Byte offset of tile `tile`'s origin on a side with leading dimension ld.
  __device__ __forceinline__ int64_t origin(int64_t tile, int64_t ld) const {
    const int64_t tr = tile / a.tiles_c, tc = tile - tr * a.tiles_c;
    return (tr * a.tile_rows * ld + tc * a.tile_cols) * a.eb;
  }

  // Issue tile k into stage J: R transfers per lane, no wait.
  template <int J>
  __device__ __forceinline__ void issue(int k) const {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.src + origin(first + k, a.src_ld)), (short)0, (int)src_span, 0x00020000);
    uint8_t* base = stage<J>() + lds_wave;
#pragma unroll
    for (int f = 0; f < R; ++f) {
      lds_void* l = (lds_void*)(base + (uint32_t)f * (uint32_t)a.threads * VB);
      const int voff = (int)goff[f];
      if constexpr (VB == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, l, 16, voff, 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, l, 4, voff, 0, 0, 0);
    }
  }

  // Store tile k from stage J.
  template <int J>
  __device__ __forceinline__ void consume(int k) const {
    typedef typename Vec<VB>::T T;
    uint8_t* dst = a.dst + (dst_image ? 0 : origin(first + k, a.dst_ld));
#pragma unroll
    for (int f = 0; f < R; ++f)
      __builtin_nontemporal_store(*(const T*)(stage<J>() + loff[f]), (T*)(dst + doff[f]));
  }

  // Wait for tile k when `newer` of its successors have been issued after it.
  __device__ __forceinline__ void wait_for(int newer) const {
    if constexpr (DEPTH >= 4) { if (newer == 3) { wait_vm<3 * R>(); return; } }
    if constexpr (DEPTH >= 3) { if (newer == 2) { wait_vm<2 * R>(); return; } }
    if constexpr (DEPTH >= 2) { if (newer == 1) { wait_vm<R>(); return; } }
    wait_vm<0>();
  }

  // Tile k sits in stage J; tile k + DEPTH - 1 goes to stage (J + DEPTH - 1) % DEPTH.
  // Steady state: the next tile exists, so DEPTH - 1 newer tiles are in flight at the wait.
  template <int J>
  __device__ __forceinline__ void step_full(int k) const {
    issue<(J + DEPTH - 1) % DEPTH>(k + DEPTH - 1);
    wait_vm<(DEPTH - 1) * R>();
    barrier();          // every wave's part of tile k is in LDS
    consume<J>(k);
    barrier();          // stage J is read out before a later issue refills it
  }

  // General step (the last tiles): issue only what exists, wait for what was issued after k.
  template <int J>
  __device__ __forceinline__ void step(int k) const {
    if (k >= n) return;
    const int next = k + DEPTH - 1;
    if (next < n) issue<(J + DEPTH - 1) % DEPTH>(next);
    const int newer = (n - 1 - k) < (DEPTH - 1) ? (n - 1 - k) : (DEPTH - 1);
    wait_for(newer);
    barrier();
    consume<J>(k);
    barrier();
  }

  __device__ __forceinline__ void run() const {
    // the first DEPTH - 1 tiles go out before any wait
    if constexpr (DEPTH > 1) { if (n > 0) issue<0>(0); }
    if constexpr (DEPTH > 2) { if (n > 1) issue<1>(1); }
    if constexpr (DEPTH > 3) { if (n > 2) issue<2>(2); }
    int k = 0;
    // whole rounds of DEPTH steps whose next tiles all exist: no branches inside
    for (; k + 2 * DEPTH - 1 <= n; k += DEPTH) {
      step_full<0>(k);
      if constexpr (DEPTH > 1) step_full<1>(k + 1);
      if constexpr (DEPTH > 2) step_full<2>(k + 2);
      if constexpr (DEPTH > 3) step_full<3>(k + 3);
    }
    for (; k < n; k += DEPTH) {
      step<0>(k);
      if constexpr (DEPTH > 1) step<1>(k + 1);
      if constexpr (DEPTH > 2) step<2>(k + 2);
      if constexpr (DEPTH > 3) step<3>(k + 3);
    }
  }
};

template <int VB, int R, int DEPTH>
__global__ __launch_bounds__(1024) void tile_copy_async_kernel(CopyArgs a, int32_t tiles_per_wg) {
  AsyncCopy<VB, R, DEPTH> c{a};
  c.first = (int64_t)blockIdx.x * tiles_per_wg;
  const int64_t left = a.ntiles - c.first;
  c.n = (int)(left < tiles_per_wg ? left : tiles_per_wg);
  c.rowb = (uint32_t)(a.tile_cols * a.eb);
  c.tile_bytes = c.rowb * (uint32_t)a.tile_rows;
  c.src_span = (uint32_t)((int64_t)(a.tile_rows - 1) * a.src_ld * a.eb + c.rowb);
  const uint32_t t = threadIdx.x;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
  c.lds_wave = wave * 64u * VB;
  c.dst_image = a.dst_kind == TG_XOR_SWIZZLE;
  const uint32_t mask = (uint32_t)a.xor_mask;
#pragma unroll
  for (int f = 0; f < R; ++f) {
    // Load: this lane's LDS slot is chunk p = f·threads + t of the stage (physical order); it
    // fetches the logical chunk that the tile layout puts there.
    const uint32_t x = ((uint32_t)f * (uint32_t)a.threads + t) * VB;
    const uint32_t r = x / c.rowb, pc = x - r * c.rowb;
    const uint32_t lc = a.lds_xor ? ((((pc >> 4) ^ (r & mask)) << 4) | (pc & 15u)) : pc;
    c.goff[f] = (uint32_t)(r * (uint32_t)a.src_ld * (uint32_t)a.eb) + lc;
    // Store: round f of thread t moves logical chunk f·threads + t.
    c.loff[f] = a.lds_xor ? xor_swizzle_bytes(r, pc, c.rowb, mask) : x;
    c.doff[f] = c.dst_image ? c.loff[f] : (uint32_t)(r * (uint32_t)a.dst_ld * (uint32_t)a.eb) + pc;
  }
  c.run();
}

template <int VB, int R>
hipError_t launch_vr(const CopyArgs& a, int depth, int32_t tpw, dim3 g, dim3 b, hipStream_t s) {
  switch (depth) {
    case 1: hipLaunchKernelGGL((tile_copy_async_kernel<VB, R, 1>), g, b, 0, s, a, tpw); break;
    case 2: hipLaunchKernelGGL((tile_copy_async_kernel<VB, R, 2>), g, b, 0, s, a, tpw); break;
    case 3: hipLaunchKernelGGL((tile_copy_async_kernel<VB, R, 3>), g, b, 0, s, a, tpw); break;
    case 4: hipLaunchKernelGGL((tile_copy_async_kernel<VB, R, 4>), g, b, 0, s, a, tpw); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int VB>
hipError_t launch_v(const CopyArgs& a, int rounds, int depth, int32_t tpw, dim3 g, dim3 b,
                    hipStream_t s) {
  switch (rounds) {
    case 1: return launch_vr<VB, 1>(a, depth, tpw, g, b, s);
    case 2: return launch_vr<VB, 2>(a, depth, tpw, g, b, s);
    case 4: return launch_vr<VB, 4>(a, depth, tpw, g, b, s);
    case 8: return launch_vr<VB, 8>(a, depth, tpw, g, b, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_tile_copy_async(const CopyArgs& a, int vec_bytes, int rounds, int depth,
                                  int32_t tiles_per_wg, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid), b((unsigned)a.threads);
  if (vec_bytes == 16) return launch_v<16>(a, rounds, depth, tiles_per_wg, g, b, s);
  if (vec_bytes == 4) return launch_v<4>(a, rounds, depth, tiles_per_wg, g, b, s);
  return hipErrorInvalidValue;
}

}  // namespace tg
