// Device-side LDS tile layout shared by the copy and GEMM kernels.
//
// A tile row is cut into 16-byte chunks; in the XOR-swizzled layout the chunk
// index is XOR-ed with the low bits of the row index (mask = min(8, chunks per
// row) - 1).  For the 128-byte rows the GEMM uses (64 fp16/bf16 of K) this is
// the address form x ^ ((x & 0x380) >> 3): chunk bits 4..6 XOR row bits 7..9,
// the swizzle family of [TCGEN05-CP] 调度算法 step 2 ("TVM Blackwell tcgen05.cp
// 全解析…") with 16-byte atoms and an 8-row (1 KiB) period.  The bytes inside a
// chunk are never permuted, so a 128-bit vector stays whole ([VEC-AUTO]
// "swizzled shared 布局": the vector may not leave one swizzle chunk).
//
// Why on gfx950: a wave reading one 16-byte chunk per lane down a column of
// 128-byte rows (the MFMA fragment pattern) would hit the same four banks in
// every row; XOR-ing the chunk with the row spreads eight consecutive rows
// over all eight chunk positions, i.e. over every bank.
#pragma once

#include <stdint.h>

namespace tg {

// Byte offset of byte `cb` of tile row `r` (row pitch `pitch` bytes) in the
// XOR-swizzled layout.
__device__ __forceinline__ uint32_t xor_swizzle_bytes(uint32_t r, uint32_t cb, uint32_t pitch,
                                                      uint32_t mask) {
  return r * pitch + ((((cb >> 4) ^ (r & mask)) << 4) | (cb & 15u));
}

// 128-byte rows (the GEMM stage layout): chunk index kc of row r.
__device__ __forceinline__ uint32_t swz128(uint32_t r, uint32_t kc) {
  return (r << 7) | (((kc ^ r) & 7u) << 4);
}

}  // namespace tg
