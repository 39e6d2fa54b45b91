// Large-tile GEMM on gfx950 with direct global -> LDS operand loads (kernel template).
//
// Same contract as gemm_tiled ([SYNC-GEMM] "TVM TIRx 同步 GEMM 深度解析…": D = A·B (+C),
// fp32 accumulation in place over K, 二 / 四 step 3), for 256x256 or 128x128 blocks.  The
// template serves the 16-bit operands of the synchronous GEMM and the fp8 operands of the
// asynchronous GEMM's precision family (七: A and B staged in shared memory, fp8 among the
// operand formats), with or without block scales.  What the kernel does:
//
//  * global -> LDS with buffer_load_dwordx4 ... lds: each instruction moves 64 lanes x 16 bytes
//    and lane i's bytes land at LDS base + 16·i, so no VGPR staging and no ds_write.  The
//    LDS swizzle is applied on the global side: lane i fetches the logical 16-byte chunk
//    that belongs at physical slot i.
//  * one K stage is one 128-byte row of K per operand row: 64 K of a 16-bit operand, 128 K of
//    an fp8 operand, 256 K of a packed e2m1 operand.  All formats therefore share the LDS
//    geometry, the DMA pattern and the bytes per stage; a stage is 4 MFMA K steps of 16
//    (v_mfma_f32_32x32x16_{f16,bf16}), 2 of 64 (v_mfma_f32_32x32x64_f8f6f4, fp8) or 4 of 64
//    (the same instruction with e2m1 operands, which takes half the fp8 cycles), the same MFMA
//    cycles per stage in every case.  An e2m1 lane carries 16 bytes (32 K) per step, like a
//    16-bit lane, so e2m1 stages take the 16-bit fragment reads.  A 6-bit operand (e2m3, e3m2)
//    fills 96 bytes of the row with 128 K: its stages take the fp8 schedule (2 steps of 64 K,
//    MFMAs at the e2m1 rate), the row's last two chunks are zeros (the lanes that would fetch
//    them get an out-of-range offset), and a lane's 24 bytes per step are three 8-byte reads.
//  * K-contiguous operands (A without transA, B with transB) keep [rows][128 bytes] stages
//    (chunk XOR row bits) and are read as fragments with ds_read_b128: one per 16-bit
//    fragment, two per fp8 fragment (32 bytes of K per lane).
//  * M/N-contiguous 16-bit operands (A with transA, B without transB) keep the global
//    orientation, [64 k][256 mn] stages of 512-byte rows (256 bytes on 128-wide blocks), and
//    are read with
//    ds_read_b64_tr_b16: within each 16-lane group, lane j receives element j%4 of the 8-byte
//    reads of lanes 4q + j/4 (q = 0..3), so if lane i reads 4 consecutive mn at k-row
//    k0 + i/4 and column block i%4, lane j receives k0..k0+3 at mn0 + j — four K-consecutive
//    values, half of an MFMA fragment.
//  * the K loop is unrolled by two so each half names its LDS stage at compile time; the
//    next stage's loads are issued at the top of an iteration and the next K step's
//    fragments are read while the current step's MFMAs run.
//  * ragged shapes: the buffer range check compares the whole offset (VGPR + SGPR +
//    immediate) with num_records and returns zeros past it without touching memory (measured
//    on gfx950 for the register and the LDS forms), so operand rows past M or N, and k-rows
//    of an M/N-major operand past K, read as zero.  A K-major operand's last stage when K is
//    not a whole number of stages would read the next row's K instead: there the lanes whose
//    chunk lies past K get a VGPR offset of 2^31, out of range whatever else is added.
//
// Internal header: included through gemm_direct_launch.h (16-bit instantiations) and
// gemm_fp8_launch.h (fp8 and block-scaled fp8).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "tg_internal.h"

namespace tg {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) uint32_t u32x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int BM = 256, BN = 256;
constexpr int kRowBytes = 128;   // bytes of K per operand row and stage
constexpr int kGroupM = 8;       // tile-rows per scheduling group (measured: 8 beats 2, 4, 16)

// Format codes of the template's DT parameter: TG_F16 / TG_BF16, an fp8 pair kF8 + 2·a + b,
// or a block-scaled fp8 pair kMX + 2·a + b, with a, b the MFMA's operand format codes
// (0 = e4m3, 1 = e5m2); kP4: a block-scaled e2m1 pair, both operands K-contiguous packed rows
// (value k of a row at bits [4k, 4k + 4) of its bytes); kP6 + 2·(a − 2) + (b − 2): a block-scaled
// pair of 6-bit operands (format codes a, b: 2 = e2m3, 3 = e3m2), K-contiguous packed rows
// (value k at bits [6k, 6k + 6)).
constexpr int kF8 = 16, kMX = 32, kP4 = 64, kP6 = 96;
constexpr int p6_code(int a_fmt, int b_fmt) { return kP6 + 2 * (a_fmt - 2) + (b_fmt - 2); }
constexpr int fp8_code(int a_fmt, int b_fmt) { return kF8 + 2 * a_fmt + b_fmt; }
constexpr int mx_code(int a_fmt, int b_fmt) { return kMX + 2 * a_fmt + b_fmt; }

// Addressing unit: one element of a 16-bit or fp8 operand, one byte of a packed operand.
// kFp8: the two-step (64-K) stage schedule, which 6-bit operands share.
template <int DT>
struct Elem {
  static constexpr bool kFp4 = DT == kP4;
  static constexpr bool kFp6 = DT >= kP6;
  static constexpr bool kFp8 = DT >= kF8 && !kFp4;
  static constexpr bool kScaled = DT >= kMX;      // E8M0 scale per 32 K of each row / column
  static constexpr int kBytes = kFp8 || kFp4 ? 1 : 2;   // bytes per addressing unit
  static constexpr int kPer = kFp4 ? 2 : 1;        // K values per addressing unit (not 6-bit)
  static constexpr int kBK = kRowBytes / kBytes;   // addressing units per stage
  static constexpr int kStageBytes = kFp6 ? 96 : kRowBytes;   // bytes of a K row per stage
  static constexpr int kSteps = kFp8 ? 2 : 4;      // MFMA K steps per stage
  static constexpr int kParts = kFp6 ? 3 : kFp8 ? 2 : 1;   // K-major reads per fragment
  using Frag = typename std::conditional<kFp8, u32x8, u32x4>::type;
};

template <int DT, class F>
__device__ __forceinline__ f32x16 mfma32(F a, F b, f32x16 c) {
  if constexpr (DT == TG_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else if constexpr (DT == TG_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    // cbsz / blgp name A's and B's formats; no block scales (scale operands 0).  Lane l
    // carries 32 bytes of K of row / column l % 32; A and B put the same K in the same byte.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        __builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b), c, (DT & 3) >> 1, DT & 1, 0,
        0, 0, 0);
}
// Block-scaled fp8 MFMA: the unit's 32-K block q of the 64-K step is bytes 16q .. 16q+15 of
// both lane halves (lanes n and n + 32 of row / column n); its scale is the byte OPSEL selects
// from the scale register of lane n + 32q.
// A 6-bit pair (DT kP6 + …) takes format codes 2 / 3 and its six low operand registers; lane
// half h carries block h of the step, whose scale is the lane's own register, so the same
// byte selection serves it.
template <int DT, int OPSEL, class F>
__device__ __forceinline__ f32x16 mfma32s(F a, F b, f32x16 c, uint32_t sa, uint32_t sb) {
  constexpr int fa = DT >= kP6 ? 2 + ((DT - kP6) >> 1) : (DT & 3) >> 1;
  constexpr int fb = DT >= kP6 ? 2 + ((DT - kP6) & 1) : DT & 1;
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      __builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b), c, fa, fb, OPSEL, (int)sa,
      OPSEL, (int)sb);
}

// Block-scaled e2m1 MFMA (format code 4 for both operands): lane l carries the 32
// consecutive K of block l / 32 of the 64-K step for row / column l % 32, as 16 packed bytes
// in the low half of the 8-register operand, and that block's scale is the byte OPSEL selects
// from the lane's own scale register (measured on gfx950 with an in-bounds probe).  The
// compiler passes only the four low registers for this format.
template <int OPSEL>
__device__ __forceinline__ f32x16 mfma32p4(u32x4 a, u32x4 b, f32x16 c, uint32_t sa, uint32_t sb) {
  const i32x8 a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 b8 = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, OPSEL, (int)sa, OPSEL,
                                                         (int)sb);
}

// ---- LDS layouts --------------------------------------------------------------------
// K-major stage: BS rows (256 or 128) x 128 bytes; physical chunk = kc ^ sk(row).
//   SK 0: row & 7 — eight consecutive rows hit eight chunks (32 four-byte banks);
//   SK 1: (row & 7) ^ ((row >> 3) & 1) — also sixteen consecutive rows hit sixteen distinct
//         (row parity, chunk) pairs, i.e. distinct banks if the LDS has 64 banks.
template <int SK>
__device__ __forceinline__ uint32_t sk(uint32_t r) {
  if constexpr (SK == 0) return r & 7u;
  else return (r & 7u) ^ ((r >> 3) & 1u);
}
// M/N-major stage: 64 k-rows x 512 bytes (32 chunks) for 256-wide blocks, x 256 bytes (16
// chunks) for 128-wide ones; physical chunk = c ^ sm(k).  A transposing read touches 32
// bytes (2 chunks) in each of 4 consecutive k-rows per 16 lanes.
//   SM 0: 2(k & 3) — the four rows land in four distinct 32-byte bank slots of 128 bytes;
//   SM 1: 2(k & 3) ^ 8(k & 1) — additionally, two adjacent 16-lane groups (mn + 16) land
//         in eight distinct slots of 256 bytes.
template <int SM>
__device__ __forceinline__ uint32_t sm(uint32_t k) {
  if constexpr (SM == 0) return (k & 3u) << 1;
  else return ((k & 3u) << 1) ^ ((k & 1u) << 3);
}

// M/N-major fp8 stage: 128 k-rows x ROWB bytes (256: 16 chunks, 128: 8 chunks); physical
// chunk = c ^ s8(k).  A transposing read (ds_read_b64_tr_b8) of 32 lanes touches two adjacent
// chunks (an even one and the next) in each of 8 consecutive k-rows; the swizzle sends the 16
// of them to 16 distinct 16-byte bank slots of 256 bytes: 2(k & 7) with 256-byte rows; with
// 128-byte rows a row pair fills 256 bytes, so the four even (odd) rows need four distinct
// chunk pairs, 2((k >> 1) & 3).
template <int ROWB>
__device__ __forceinline__ uint32_t s8(uint32_t k) {
  static_assert(ROWB == 256 || ROWB == 128, "fp8 M/N-major rows");
  if constexpr (ROWB == 256) return (k & 7u) << 1;
  else return ((k >> 1) & 3u) << 1;
}

// ---- per-lane offsets, computed once ---------------------------------------------------
// Every address below is a per-lane offset computed before the K loop plus compile-time
// immediates (tile, K step, stage), so the loop keeps few address registers.
constexpr int SKV = 1, SMV = 1;   // swizzle variants in use (see sk / sm)

// DMA (global -> LDS) for a K-major operand: PER instructions per wave per stage; instruction
// i writes 1 KiB block b = PER·wave + i = rows 8b .. 8b+7.  Lane l fills physical slot l%8
// of row 8b + l/8 and so fetches logical chunk (l%8) ^ sk(row).  sk(row) depends on the
// lane and on i's parity only (PER is even), so two byte offsets cover all instructions.
// kbyte[p]: the byte of the 128-byte K row where that chunk starts (parity p).
template <int PER, int E>
__device__ __forceinline__ void km_dma_offsets(int64_t ld, int wave, int lane, uint32_t (&off)[2],
                                               uint32_t (&kbyte)[2]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t r = (uint32_t)(8 * PER * wave + 8 * p + (lane >> 3));
    const uint32_t kc = ((uint32_t)lane & 7u) ^ sk<SKV>(r);
    kbyte[p] = kc * 16u;
    if constexpr (E == 2) off[p] = (r * (uint32_t)ld + kc * 8u) * 2u;   // bytes; < 256·K·2 < 2^32
    else off[p] = r * (uint32_t)ld + kc * 16u;                          // bytes; < 256·K < 2^32
  }
}
// DMA for an M/N-major 16-bit operand with ROWB-byte k-rows (CH = ROWB/16 chunks, RPB =
// 1024/ROWB k-rows per 1 KiB block): instruction i writes block b = PER·wave + i = k-rows
// RPB·b .. RPB·b + RPB-1; lane l fills slot l%CH of k-row RPB·b + l/CH, logical chunk
// (l%CH) ^ sm(k); sm depends on k & 3, i.e. on the lane and i's parity.
template <int PER, int ROWB>
__device__ __forceinline__ void mn_dma_offsets(int64_t ld, int wave, int lane, uint32_t (&off)[2]) {
  constexpr uint32_t CH = ROWB / 16, RPB = 1024 / ROWB;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t k = RPB * (uint32_t)(PER * wave + p) + (uint32_t)lane / CH;
    const uint32_t c = ((uint32_t)lane % CH) ^ sm<SMV>(k);
    off[p] = (k * (uint32_t)ld + c * 8u) * 2u;    // bytes; < 64·ld·2 <= 2^32 (whole stages span at most 2^32 bytes)
  }
}

// DMA for an M/N-major fp8 operand with ROWB-byte k-rows (CH = ROWB/16 chunks, RPB =
// 1024/ROWB k-rows per 1 KiB block): instruction i writes block b = PER·wave + i = k-rows RPB·b
// .. RPB·b + RPB-1; lane l fills slot l%CH of k-row RPB·b + l/CH, logical chunk (l%CH) ^ s8(k);
// s8 depends on the lane and i's parity.
template <int PER, int ROWB>
__device__ __forceinline__ void mn8_dma_offsets(int64_t ld, int wave, int lane, uint32_t (&off)[2]) {
  constexpr uint32_t CH = ROWB / 16, RPB = 1024 / ROWB;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t k = RPB * (uint32_t)(PER * wave + p) + (uint32_t)lane / CH;
    const uint32_t c = ((uint32_t)lane % CH) ^ s8<ROWB>(k);
    off[p] = k * (uint32_t)ld + c * 16u;   // bytes; < 128·ld < 2^31 (K % 128 == 0, operand under 2 GiB)
  }
}

// K-major fragment reads (ds_read_b128) of 32-row tile t: lane l reads row base + 32t + l%32.
// 16-bit, K step s: chunk 2s + l/32 (offset u = s).  fp8, K step s: chunks 4s + 2q + l/32
// for q = 0, 1 (offsets u = 2s + q) — 32 bytes of K per lane.  The fp8 order follows the
// unit's 32-K blocks: block q of a 64-K step is bytes 16q .. 16q+15 of both lane halves
// (measured with per-half scales), so lane half h holds K 16h .. 16h+15 of each block.
// sk(row) depends on the lane only (32t is a multiple of 16), the chunk term on u: one byte
// offset per u; tiles are +4096-byte immediates.
template <bool FP8>
__device__ __forceinline__ void km_frag_offsets(int row_base, int lane, uint32_t (&off)[4]) {
  const uint32_t r = (uint32_t)(row_base + (lane & 31));
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t kc = FP8 ? (uint32_t)(4 * (u >> 1) + 2 * (u & 1) + (lane >> 5))
                            : (uint32_t)(2 * u + (lane >> 5));
    off[u] = r * 128u + ((kc ^ sk<SKV>(r)) << 4);
  }
}
// 6-bit K-major fragments of 32-row tile t: lane l reads row base + 32t + l%32, and in K step s
// the 24 bytes 48s + 24h .. +23 of the row (h = l/32), as three 8-byte reads u = 3s + p at
// logical byte x = 48s + 24h + 8p: chunk x/16, swizzled, plus x%16.  Tiles are +4096 bytes.
__device__ __forceinline__ void km6_frag_offsets(int row_base, int lane, uint32_t (&off)[6]) {
  const uint32_t r = (uint32_t)(row_base + (lane & 31));
  const uint32_t h = (uint32_t)lane >> 5;
#pragma unroll
  for (int u = 0; u < 6; ++u) {
    const uint32_t x = 48u * (uint32_t)(u / 3) + 24u * h + 8u * (uint32_t)(u % 3);
    off[u] = r * 128u + (((x >> 4) ^ sk<SKV>(r)) << 4) + (x & 15u);
  }
}
// M/N-major fragment of 32-column tile t, K step s, half h (two ds_read_b64_tr_b16): lane
// l = 16g + j supplies k-row 16s + 8(g/2) + 4h + j/4 and columns mn_base + 32t + 16(g&1) +
// 4(j&3) .. +3.  sm(k) depends on j only; its bits 2-3 XOR with the tile index, so one byte
// offset per tile t; s and h are immediates (16s + 4h rows of ROWB bytes).
template <int T, int ROWB>
__device__ __forceinline__ void mn_frag_offsets(int mn_base, int lane, uint32_t (&off)[4]) {
  const uint32_t g = (uint32_t)lane >> 4, j = (uint32_t)lane & 15u;
  const uint32_t krow = 8u * (g >> 1) + (j >> 2);
  const uint32_t x = sm<SMV>(krow);
  const uint32_t mn_lane = 16u * (g & 1u) + 4u * (j & 3u);
  const uint32_t byte = (mn_lane & 7u) * 2u;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t c = ((uint32_t)mn_base + 32u * (uint32_t)(t < T ? t : 0) + mn_lane) >> 3;
    off[t] = krow * (uint32_t)ROWB + ((c ^ x) << 4) + byte;
  }
}

// M/N-major fp8 fragment of 32-column tile t, K step s (64 k), read u = 0..3 (four
// ds_read_b64_tr_b8): within each 16-lane group g, lane j receives byte j%8 of the 8-byte
// reads of lanes 2k + j/8 (k = 0..7).  So lane l = 16g + j reads k-row 64s + kr(u) + 16(g/2)
// + j/2, kr(u) = 32(u/2) + 8(u%2), at columns mn_base + 32t + 16(g&1) + 8(j&1) .. +7, and
// receives its bytes 8u .. 8u+7 = k kr(u) + 16(g/2) .. +7 of column mn_base + 32t + l%32 —
// the K order of the K-major fp8 fragment.  s8 depends on j only (s, u and g/2 add multiples
// of 8 rows); the chunk of tile t is kept per t (2t carries into the swizzled bits), s and u
// are immediates (rows of ROWB bytes).
template <int T, int ROWB>
__device__ __forceinline__ void mn8_frag_offsets(int mn_base, int lane, uint32_t (&off)[4]) {
  const uint32_t g = (uint32_t)lane >> 4, j = (uint32_t)lane & 15u;
  const uint32_t krow = 16u * (g >> 1) + (j >> 1);
  const uint32_t x = s8<ROWB>(krow);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t c = ((uint32_t)mn_base + 32u * (uint32_t)(t < T ? t : 0)) / 16u + (g & 1u);
    off[t] = krow * (uint32_t)ROWB + ((c ^ x) << 4) + 8u * (j & 1u);
  }
}

// One operand of one wave: T fragments of 32 rows/columns per K step, PER DMA instructions
// per stage; BS rows (K-major) or columns (M/N-major) per block.
template <bool MN, int T, int PER, int DT, int BS>
struct Operand {
  using EL = Elem<DT>;
  using Frag = typename EL::Frag;
  static constexpr int kRowB = BS * EL::kBytes;   // M/N-major: bytes per k-row
  uint32_t dma[2];   // byte offsets of the two DMA parities
  uint32_t kbyte[2]; // K-major: first byte within the K row of each parity's chunk
  uint32_t frag[EL::kFp6 ? 6 : 4];   // byte offsets: per K-major read slot, or per M/N-major tile

  // LDS read instructions per fragment and per K step
  static constexpr int kTileReads = MN ? (EL::kFp8 ? 4 : 2) : EL::kParts;
  static constexpr int kReads = T * kTileReads;

  __device__ __forceinline__ void init(int64_t ld, int base, int wave, int lane) {
    if constexpr (MN && EL::kFp8) {
      mn8_dma_offsets<PER, kRowB>(ld, wave, lane, dma);
      mn8_frag_offsets<T, kRowB>(base, lane, frag);
    } else if constexpr (MN) {
      mn_dma_offsets<PER, kRowB>(ld, wave, lane, dma);
      mn_frag_offsets<T, kRowB>(base, lane, frag);
    } else if constexpr (EL::kFp6) {
      static_assert(!MN, "6-bit operands are K-contiguous");
      km_dma_offsets<PER, EL::kBytes>(ld, wave, lane, dma, kbyte);
      km6_frag_offsets(base, lane, frag);
    } else {
      km_dma_offsets<PER, EL::kBytes>(ld, wave, lane, dma, kbyte);
      km_frag_offsets<EL::kFp8>(base, lane, frag);
    }
  }
  // Buffer descriptor of this operand's panel: base = the block's first element at K stage
  // 0, num_records = bytes from there to the end of the operand (reads past it return 0).
  __amdgpu_buffer_rsrc_t rsrc;

  __device__ __forceinline__ void bind(const uint8_t* panel, int64_t bytes_left) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)panel, (short)0, (int)bytes_left, 0x00020000);
  }
  // Issue the PER DMA instructions of one stage (buffer_load_dwordx4 ... lds): per-lane byte
  // offset `dma[i & 1]` (VGPR), stage and instruction offset `soff` (SGPR), LDS block address
  // in M0 — no per-instruction vector arithmetic.  `wave` is wave-uniform.  TAIL: only the
  // first `lim` bytes of each K row are valid in this stage; a K-major lane whose chunk
  // starts at or past them reads zeros (M/N-major k-rows past K are past the operand's end).
  template <bool TAIL = false>
  __device__ __forceinline__ void load(uint32_t stage_off, int64_t ld, uint8_t* stage, int wave,
                                       uint32_t lim = kRowBytes) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      uint32_t v = dma[i & 1];
      if constexpr ((TAIL || EL::kFp6) && !MN) v = kbyte[i & 1] < lim ? v : 0x80000000u;
      // K-major: +8 rows per instruction pair; M/N-major: +1024/kRowB k-rows
      const uint32_t step = MN ? (uint32_t)((1024 / kRowB) * (i & ~1)) * (uint32_t)ld * (uint32_t)EL::kBytes
                               : (uint32_t)(8 * (i & ~1)) * (uint32_t)ld * (uint32_t)EL::kBytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + (wave * PER + i) * 1024),
                                               16, v, stage_off + step, 0, 0);
    }
  }
  __device__ __forceinline__ void frags(const uint8_t* stage, int s, Frag (&f)[T]) const {
    if constexpr (MN && EL::kFp8) {
#pragma unroll
      for (int t = 0; t < T; ++t) frag_tile(stage, s, t, f[t]);
    } else if constexpr (MN) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        u32x4 out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint8_t* p = stage + frag[t] + (16 * s + 4 * h) * kRowB;
          const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
          out[2 * h] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
          out[2 * h + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
        }
        f[t] = out;
      }
    } else if constexpr (EL::kFp6) {
#pragma unroll
      for (int t = 0; t < T; ++t) frag_tile(stage, s, t, f[t]);
    } else if constexpr (EL::kFp8) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const u32x4 lo = *(const u32x4*)(stage + frag[2 * s] + t * 4096);
        const u32x4 hi = *(const u32x4*)(stage + frag[2 * s + 1] + t * 4096);
        f[t] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t) f[t] = *(const u32x4*)(stage + frag[s] + t * 4096);
    }
  }
  // One fp8 fragment (tile t, K step s): two ds_read_b128 (K-major) or four
  // ds_read_b64_tr_b8 (M/N-major); a 6-bit one: three ds_read_b64 (its top two registers 0).
  __device__ __forceinline__ void frag_tile(const uint8_t* stage, int s, int t, Frag& f) const {
    static_assert(EL::kFp8, "per-tile reads are used for fp8 and 6-bit operands");
    if constexpr (EL::kFp6) {
      u32x8 out = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const u32x2 v = *(const u32x2*)(stage + frag[3 * s + p] + t * 4096);
        out[2 * p] = v[0];
        out[2 * p + 1] = v[1];
      }
      f = out;
    } else if constexpr (MN) {
      u32x8 out;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint8_t* p = stage + frag[t] + (64 * s + 32 * (u >> 1) + 8 * (u & 1)) * kRowB;
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
        out[2 * u] = (uint32_t)v[0];
        out[2 * u + 1] = (uint32_t)v[1];
      }
      f = out;
    } else {
      const u32x4 lo = *(const u32x4*)(stage + frag[2 * s] + t * 4096);
      const u32x4 hi = *(const u32x4*)(stage + frag[2 * s + 1] + t * 4096);
      f = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
};

// Scheduling hints for one K step of NM MFMAs carrying NR LDS reads and ND DMA instructions.
// The next step's fragment reads go out in the first RS slots (so they have almost a whole
// step of MFMAs to land before the next step's first MFMA waits for them); the DMA
// instructions are spread evenly over all slots.
template <int NM, int NR, int ND, int RS, int Q>
__device__ __forceinline__ void interleave_slot() {
  constexpr int r = (NR * (Q + 1)) / RS - (NR * Q) / RS;
  constexpr int d = (ND * (Q + 1)) / NM - (ND * Q) / NM;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
  if constexpr (Q < RS && r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);   // LDS reads
  if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x020, d, 0);   // DMA (VMEM read)
}
template <int NM, int NR, int ND, int RS, int... Q>
__device__ __forceinline__ void interleave_seq(std::integer_sequence<int, Q...>) {
  (interleave_slot<NM, NR, ND, RS, Q>(), ...);
}
template <int NM, int NR, int ND>
__device__ __forceinline__ void interleave() {
  constexpr int rs = NM >= 4 ? NM / 4 : 1;   // read slots: first quarter of the step
  interleave_seq<NM, NR, ND, rs>(std::make_integer_sequence<int, NM>{});
}

// Scheduling hints for one in-place K step (fp8): MFMAs run A-tile by A-tile (TN each); the
// next step's B fragments (NRB reads) go out after the first MFMA into spare registers, and
// A tile i's next fragment (NRA reads) right after the last MFMA that reads tile i, into the
// same registers.  ND DMA instructions are spread evenly.
template <int TN, int NM, int NRA, int NRB, int ND, int Q>
__device__ __forceinline__ void inplace_slot() {
  constexpr int d = (ND * (Q + 1)) / NM - (ND * Q) / NM;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  // MFMA
  if constexpr (Q == 0 && NRB > 0) __builtin_amdgcn_sched_group_barrier(0x100, NRB, 0);  // B reads
  if constexpr (Q % TN == TN - 1 && NRA > 0) __builtin_amdgcn_sched_group_barrier(0x100, NRA, 0);
  if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x020, d, 0);             // DMA
}
template <int TN, int NM, int NRA, int NRB, int ND, int... Q>
__device__ __forceinline__ void inplace_seq(std::integer_sequence<int, Q...>) {
  (inplace_slot<TN, NM, NRA, NRB, ND, Q>(), ...);
}
template <int TN, int NM, int NRA, int NRB, int ND>
__device__ __forceinline__ void interleave_inplace() {
  inplace_seq<TN, NM, NRA, NRB, ND>(std::make_integer_sequence<int, NM>{});
}

// Number of K stages a kernel serves: even, odd and at least 3, or exactly one.  Each shape
// has its own peeled tail, so every LDS address is a compile-time immediate and no
// accumulator state merges across branches.  kTail (added to a shape, 16-bit operands): the
// last stage may hold fewer than 64 K, stages = ceil(K / 64).
enum KStages { kEven = 0, kOdd = 1, kSingle = 2, kTail = 4 };

// WGM x WGN waves on a BS x BS block (256 or 128); wave tile
// (BS/WGM) x (BS/WGN).  BOUNDS: M or N is not a whole number of blocks; operand rows past the end read as zero (buffer range check) and the epilogue skips
// rows and columns past M and N.  An operand row past M or N only feeds outputs that are
// never stored, so the data there need not be zero, only never fetched from outside the
// operand.  KS: the KStages shape of the stage count, plus kTail.
template <bool A_MN, bool B_MN, int DT, int WGM, int WGN, bool BOUNDS, int KS, int BS>
__device__ __forceinline__ void direct_body(const GemmArgs& g) {
  using EL = Elem<DT>;
  using Frag = typename EL::Frag;
  constexpr int NW = WGM * WGN;
  constexpr int WM = BS / WGM, WN = BS / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int PER = BS / 8 / NW;   // DMA blocks (1 KiB) per operand per wave per stage
  constexpr int E = EL::kBytes, BK = EL::kBK, NS = EL::kSteps;
  constexpr int KSH = KS & 3;
  constexpr bool TAIL = (KS & kTail) != 0;
  static_assert(PER % 2 == 0 && TM >= 1 && TN >= 1 && TM <= 4 && TN <= 4, "wave grid");
  static_assert(!TAIL || !EL::kFp8, "a partial last stage is served for 16-bit operands");
  static_assert(!TAIL || !EL::kFp4, "a partial last stage is served for 16-bit operands");
  static_assert(!EL::kFp4 || (!A_MN && !B_MN), "e2m1 operands are K-contiguous");
  static_assert(BS == 256 || BS == 128, "block size");
  // block-scaled fp8 (e2m1): a group of four (two) stages' scales holds BS rows x 16 bytes per operand in
  // blocks of 16 rows, each block 4 bytes longer than its 256 bytes (QB), so that rows r and
  // r + 16 start in different banks; QH: B's offset in a group; QG: a group's bytes; QR: rows
  // per operand in a quarter of a group
  constexpr uint32_t QB = 260u, QH = QB * (BS / 16), QG = 2u * QH, QR = BS / 4;
  __shared__ __attribute__((aligned(1024))) uint8_t sa0[BS * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sb0[BS * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sa1[BS * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sb1[BS * kRowBytes];
  // block scales (scaled fp8 only): a ring of three groups of four stages, each A's BS rows
  // x 16 bytes, then B's
  __shared__ __attribute__((aligned(1024))) uint8_t qg[EL::kScaled ? 3 * QG : 1];

  // tile scheduler: XCD-contiguous ranges, grouped tile-rows (as gemm_tiled)
  const int nb = (int)gridDim.x;
  int bid = (int)blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int group = kGroupM * g.tiles_n;
  const int first_m = (bid / group) * kGroupM;
  const int gsz = min(g.tiles_m - first_m, kGroupM);
  const int tm = first_m + (bid % group) % gsz;
  const int tn = (bid % group) / gsz;
  const int m0 = tm * BS, n0 = tn * BS;

  const int tid = (int)threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = (wave / WGN) * WM, wn = (wave % WGN) * WN;

  // K in addressing units (bytes of a packed e2m1 row)
  const int64_t Kx = EL::kFp6 ? (int64_t)g.K / 4 * 3 : (int64_t)g.K / EL::kPer;
  const int64_t lda = A_MN ? g.M : Kx;
  const int64_t ldb = B_MN ? g.N : Kx;
  using OA = Operand<A_MN, TM, PER, DT, BS>;
  using OB = Operand<B_MN, TN, PER, DT, BS>;
  OA oa;
  OB ob;
  oa.init(lda, wm, wave, lane);
  ob.init(ldb, wn, wave, lane);
  // operand panels of this block at K stage 0, and the per-stage advance in bytes
  const int64_t a0 = A_MN ? (int64_t)m0 : (int64_t)m0 * Kx;
  const int64_t b0 = B_MN ? (int64_t)n0 : (int64_t)n0 * Kx;
  oa.bind((const uint8_t*)g.A + a0 * E, ((int64_t)g.M * Kx - a0) * E);
  ob.bind((const uint8_t*)g.B + b0 * E, (Kx * g.N - b0) * E);
  const uint32_t adv_a = A_MN ? (uint32_t)(BK * g.M * E) : (uint32_t)EL::kStageBytes;
  const uint32_t adv_b = B_MN ? (uint32_t)(BK * g.N * E) : (uint32_t)EL::kStageBytes;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  auto mfmas = [&](const Frag (&a)[TM], const Frag (&b)[TN]) {
    if constexpr (!EL::kFp4) {   // e2m1 stages use mfmas_p4
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32<DT>(a[i], b[j], acc[i][j]);
    }
  };

  // Pipeline (K stage kt in buffer `cur`, kt+1 already loading into `nxt`):
  //   steps 0..NS-2: read step s+1's fragments while step s's MFMAs run;
  //   wait for this wave's DMA and LDS reads, barrier: stage kt+1 is complete in `nxt` and no
  //   wave reads `cur` any more;
  //   then step NS-1's MFMAs (operands already in registers) overlap the reads of stage
  //   kt+1's first fragments and the DMA of stage kt+2 into `cur`.
  // The last two stages are peeled off the loop so the steady-state body is branch free.
  const int KT = TAIL ? (int)((Kx + BK - 1) / BK)
                      : (int)(EL::kFp6 ? g.K / 128 : Kx / BK);   // >= 1, of shape KSH
  // valid bytes of each K row in stage s: all 128 but in a partial last stage
  const uint32_t krem = (uint32_t)(Kx - (int64_t)(KT - 1) * BK) * E;
  auto lim = [&](int s) -> uint32_t {
    if constexpr (EL::kFp6) return (uint32_t)EL::kStageBytes;   // chunks 6, 7 of every row: zeros
    return s == KT - 1 ? krem : (uint32_t)kRowBytes;
  };
  auto load_ab = [&](uint32_t s, uint8_t* stage_a, uint8_t* stage_b) {
    oa.template load<TAIL>(s * adv_a, lda, stage_a, wave, lim((int)s));
    ob.template load<TAIL>(s * adv_b, ldb, stage_b, wave, lim((int)s));
  };

  // Block scales (scaled fp8): K/32 bytes per row, 4 per 128-K stage.  They travel in groups
  // of four stages, 16 bytes per row, into a ring of three LDS group buffers ([row][16 bytes],
  // A's BS rows then B's).  (e2m1: 8 bytes per 256-K stage, groups of two stages; stage kt
  // loads quarters 2(kt % 2) and 2(kt % 2) + 1 of group kt/2 + 2, and the timing argument
  // below holds with stages counted in pairs.)  Stage kt loads quarter kt % 4 of group kt/4 + 2: rows QR·q ..
  // QR·q + QR-1 of A (waves 0-3, 16 rows each) and of B (waves 4-7), four lanes per row with
  // 4 bytes each, so the lanes of a row share one cache line — 128 lines per stage on 256-wide
  // blocks, where one 4-byte load per row and stage took 512.  On 128-wide blocks a quarter
  // is 32 rows, and waves 2-3 (6-7) repeat the transfers of waves 0-1 (4-5): the same bytes
  // to the same place, which keeps the loop free of branches.  Group G is complete four
  // stages before its first read, and its buffer last held group G - 3, read out two stages
  // before.  Groups 0 and 1 load before the K loop.  Rows past M or N read as zero.
  __amdgpu_buffer_rsrc_t qrsrc;
  uint32_t qvoff = 0, qlds = 0, qkb = 0;
  if constexpr (EL::kScaled) {
    const int kb = g.K / 32;
    const bool is_a = wave < 4;
    const int row0 = is_a ? m0 : n0, rows = is_a ? g.M : g.N;
    const uint8_t* qbase = (is_a ? g.SA : g.SB) + (int64_t)row0 * kb;
    qrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)qbase, (short)0, (rows - row0) * kb, 0x00020000);
    const uint32_t wq = (uint32_t)(wave & 3) % (QR / 16);   // this wave's 16 rows of a quarter
    qvoff = (16u * wq + (uint32_t)(lane >> 2)) * (uint32_t)kb + 4u * (uint32_t)(lane & 3);
    qlds = (is_a ? 0u : QH) + QB * wq;
    qkb = (uint32_t)kb;
  }
  // quarter q of group G (G % 3 is the ring slot)
  auto qload_part = [&](uint32_t G, uint32_t q) {
    if constexpr (EL::kScaled)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrsrc, (lds_void*)(qg + (G % 3u) * QG + qlds + QB * (QR / 16) * q),
                                               4, qvoff, QR * q * qkb + 16u * G, 0, 0);
  };
  auto qroll = [&](int kt) {
    if constexpr (EL::kFp4) {
      qload_part((uint32_t)(kt >> 1) + 2u, 2u * (uint32_t)(kt & 1));
      qload_part((uint32_t)(kt >> 1) + 2u, 2u * (uint32_t)(kt & 1) + 1u);
    } else {
      qload_part((uint32_t)(kt >> 2) + 2u, (uint32_t)(kt & 3));
    }
  };
  // stage kt's scale bytes (4, e2m1: 8) of row 0 in the ring
  auto qstage = [&](int kt) -> const uint8_t* {
    if constexpr (EL::kFp4) return qg + ((uint32_t)(kt >> 1) % 3u) * QG + 8u * (uint32_t)(kt & 1);
    else return qg + ((uint32_t)(kt >> 2) % 3u) * QG + 4u * (uint32_t)(kt & 3);
  };
  // This lane's scales of one stage for A tile i / B tile j, shifted so that byte 2s holds
  // the block of K step s this lane supplies (K half lane / 32).  One per-lane LDS offset per
  // operand; tiles are immediates.
  uint32_t qa[TM], qb[TN], qbn[TN];
  uint32_t qan[TM], qbn2[TN];   // e2m1: the next stage's scales, read one step before its barrier
  const uint32_t qsh = 8u * (uint32_t)(lane >> 5);
  // row r of an operand's group: block r / 16, 16 bytes per row within it; tiles are 32 rows
  // (two blocks) apart
  auto qrow = [&](uint32_t r) -> uint32_t { return QB * (r >> 4) + 16u * (r & 15u); };
  const uint32_t qoa = qrow((uint32_t)(wm + (lane & 31))), qob = QH + qrow((uint32_t)(wn + (lane & 31)));
  auto qread_a = [&](const uint8_t* q, int i) -> uint32_t {
    return *(const uint32_t*)(q + qoa + 2 * QB * i) >> qsh;
  };
  auto qread_b = [&](const uint8_t* q, int j) -> uint32_t {
    return *(const uint32_t*)(q + qob + 2 * QB * j) >> qsh;
  };
  auto qread = [&](const uint8_t* q) {
    if constexpr (EL::kScaled) {
#pragma unroll
      for (int i = 0; i < TM; ++i) qa[i] = qread_a(q, i);
#pragma unroll
      for (int j = 0; j < TN; ++j) qb[j] = qread_b(q, j);
    }
  };
  // e2m1: a stage holds blocks 0..7 of each row (8 bytes); lane half h supplies block 2s + h
  // in K step s, so one register per tile carries this lane's four (bytes h, 2+h, 4+h, 6+h,
  // gathered with v_perm) and step s's MFMA selects byte s.
  const uint32_t psel = (lane >> 5) ? 0x07050301u : 0x06040200u;
  auto qread_p4 = [&](const uint8_t* q, uint32_t (&xa)[TM], uint32_t (&xb)[TN]) {
    if constexpr (EL::kFp4) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint8_t* p = q + qoa + 2 * QB * i;
        xa[i] = __builtin_amdgcn_perm(*(const uint32_t*)(p + 4), *(const uint32_t*)p, psel);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint8_t* p = q + qob + 2 * QB * j;
        xb[j] = __builtin_amdgcn_perm(*(const uint32_t*)(p + 4), *(const uint32_t*)p, psel);
      }
    }
  };

  load_ab(0u, sa0, sb0);
  if constexpr (EL::kScaled) {
#pragma unroll
    for (uint32_t G = 0; G < 2; ++G)
#pragma unroll
      for (uint32_t q = 0; q < 4; ++q) qload_part(G, q);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  Frag a[TM], b[TN], an[TM], bn[TN];
  oa.frags(sa0, 0, a);
  ob.frags(sb0, 0, b);
  if constexpr (EL::kFp4) qread_p4(qstage(0), qa, qb);
  else qread(qstage(0));
  if constexpr (KSH != kSingle) load_ab(1u, sa1, sb1);

  constexpr int kMfma = TM * TN;
  constexpr int kReads = OA::kReads + OB::kReads;
  constexpr int kDma = 2 * PER + (EL::kFp4 ? 2 : EL::kScaled ? 1 : 0);

  // e2m1 MFMAs of K step S: scale byte S of the gathered registers
  auto mfmas_p4 = [&](auto S) {
    constexpr int st = decltype(S)::value;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32p4<st>(a[i], b[j], acc[i][j], qa[i], qb[j]);
  };

  // fp8 K step in place: this step's MFMAs, tile by tile of A, while the next step's
  // fragments (K step `sn` of stages `xa` / `xb`) are read — B's into bn, A tile i's into
  // a[i] once its MFMAs are issued.  READ false: last step of the last stage.
  // MS: the K step of the MFMAs issued (selects the scale byte); XQ: the next stage's scales
  // to read (nullptr: none).
  auto step_inplace = [&](const uint8_t* xa, const uint8_t* xb, int sn, auto read, auto dma,
                          auto MS, const uint8_t* xq) {
    constexpr bool kRead = decltype(read)::value;
    constexpr int ms = decltype(MS)::value;
    // the next stage's scales: B's into qbn now, A tile i's into qa[i] after its MFMAs
    constexpr bool kQ = EL::kScaled && kRead && ms == NS - 1;
    if constexpr (kRead) ob.frags(xb, sn, bn);
    if constexpr (kQ) {
#pragma unroll
      for (int j = 0; j < TN; ++j) qbn[j] = qread_b(xq, j);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (EL::kScaled) acc[i][j] = mfma32s<DT, 2 * ms>(a[i], b[j], acc[i][j], qa[i], qb[j]);
        else acc[i][j] = mfma32<DT>(a[i], b[j], acc[i][j]);
      }
      if constexpr (kRead) oa.frag_tile(xa, sn, i, a[i]);
      if constexpr (kQ) qa[i] = qread_a(xq, i);
    }
    constexpr int nra = kRead ? OA::kTileReads + (kQ ? 1 : 0) : 0;
    constexpr int nrb = kRead ? OB::kReads + (kQ ? TN : 0) : 0;
    if constexpr (decltype(dma)::value) interleave_inplace<TN, kMfma, nra, nrb, kDma>();
    else interleave_inplace<TN, kMfma, nra, nrb, 0>();
    if constexpr (kRead) {
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = bn[j];
    }
    if constexpr (kQ) {
#pragma unroll
      for (int j = 0; j < TN; ++j) qb[j] = qbn[j];
    }
  };

  // One K stage.  DMA: also load stage kt+2 into the buffer this stage frees; NEXT: read
  // the next stage's first fragments (false only for the last stage).
  auto stage = [&](uint8_t* ca, uint8_t* cb, const uint8_t* na, const uint8_t* nb_, int kt, auto dma,
                   auto next) {
    if constexpr (EL::kFp4) {
      // steps 0..2 read step s+1's fragments, step 2 also the next stage's scales (its group
      // landed stages ago); the last step, after the barrier, reads the next stage's first
      // fragments.  Reading the scales after the barrier instead left them on the path to the
      // next stage's first MFMAs: 8 % slower at 8192^3.
      constexpr bool kNext = decltype(next)::value;
      auto step = [&](auto S) {
        constexpr int st = decltype(S)::value;
        oa.frags(ca, st + 1, an);
        ob.frags(cb, st + 1, bn);
        mfmas_p4(S);
        if constexpr (st == 2 && kNext) qread_p4(qstage(kt + 1), qan, qbn2);
        interleave<kMfma, kReads + (st == 2 && kNext ? 2 * (TM + TN) : 0), 0>();
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = an[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = bn[j];
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if constexpr (kNext) {
        oa.frags(na, 0, an);
        ob.frags(nb_, 0, bn);
      }
      if constexpr (decltype(dma)::value) {
        load_ab((uint32_t)(kt + 2), ca, cb);
        qroll(kt);
      }
      mfmas_p4(std::integral_constant<int, 3>{});
      constexpr int nr = kNext ? kReads : 0;
      if constexpr (decltype(dma)::value) interleave<kMfma, nr, kDma>();
      else if constexpr (kNext) interleave<kMfma, nr, 0>();
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = an[i];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = bn[j];
      if constexpr (kNext) {
#pragma unroll
        for (int i = 0; i < TM; ++i) qa[i] = qan[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) qb[j] = qbn2[j];
      }
      return;
    }
    if constexpr (EL::kFp8) {
      static_assert(NS == 2, "fp8 stages are two 64-K steps");
      step_inplace(ca, cb, 1, std::true_type{}, std::false_type{}, std::integral_constant<int, 0>{},
                   nullptr);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if constexpr (decltype(dma)::value) {
        load_ab((uint32_t)(kt + 2), ca, cb);
        qroll(kt);
      }
      step_inplace(na, nb_, 0, next, dma, std::integral_constant<int, 1>{},
                   EL::kScaled ? qstage(kt + 1) : nullptr);
      return;
    }
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      oa.frags(ca, s + 1, an);
      ob.frags(cb, s + 1, bn);
      mfmas(a, b);
      interleave<kMfma, kReads, 0>();
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = an[i];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = bn[j];
    }
    __builtin_amdgcn_sched_barrier(0);   // keep step NS-2's MFMAs ahead of the wait
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (decltype(next)::value) {
      oa.frags(na, 0, an);
      ob.frags(nb_, 0, bn);
    }
    if constexpr (decltype(dma)::value) load_ab((uint32_t)(kt + 2), ca, cb);
    mfmas(a, b);
    if constexpr (decltype(dma)::value) interleave<kMfma, kReads, kDma>();
    else if constexpr (decltype(next)::value) interleave<kMfma, kReads, 0>();
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = an[i];
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = bn[j];
  };

  // epilogue: lane holds column n = lane%32 of each tile, rows 8(r/4) + 4(lane/32) + r%4.
  // D is written with nontemporal stores: it is not read again here, and streaming it past
  // the L2 keeps the operand panels of the blocks that follow resident (measured 8-14 %
  // faster at 8192^3 than ordinary stores).  C is read with nontemporal loads for the same
  // reason (8192^3 fp16 transA beta 1: 925 -> 891 us).
  auto epilogue = [&]() {
    const int lrow = lane & 31, khalf = lane >> 5;
    float* dbase = g.D + (int64_t)(m0 + wm + 4 * khalf) * g.N + (n0 + wn + lrow);
    if constexpr (BOUNDS) {
      // ragged block: per-element range check (C read only where D is written)
      const int row0 = m0 + wm + 4 * khalf, col0 = n0 + wn + lrow;
      const float* cbase = g.C + (int64_t)row0 * g.N + col0;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int dr = 32 * i + 8 * (r >> 2) + (r & 3);
            if (row0 + dr < g.M && col0 + 32 * j < g.N) {
              const int64_t o = (int64_t)dr * g.N + 32 * j;
              const float c = g.use_c ? __builtin_nontemporal_load(&cbase[o]) : 0.0f;
              __builtin_nontemporal_store(g.use_c ? acc[i][j][r] + c : acc[i][j][r], &dbase[o]);
            }
          }
    } else if (g.use_c) {
      // C may be exactly D, so the compiler may not move a C load above an earlier D store.
      // Loads are therefore issued in program order one batch (one 32-row band) ahead of the
      // stores: every element is still read before it is written, and each batch costs one
      // memory round trip instead of one per element.
      const float* cbase = g.C + (int64_t)(m0 + wm + 4 * khalf) * g.N + (n0 + wn + lrow);
      float cv[2][TN][16];
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          cv[0][j][r] =
              __builtin_nontemporal_load(&cbase[(int64_t)(8 * (r >> 2) + (r & 3)) * g.N + 32 * j]);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (i + 1 < TM) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              cv[(i + 1) & 1][j][r] =
                  __builtin_nontemporal_load(
                      &cbase[(int64_t)(32 * (i + 1) + 8 * (r >> 2) + (r & 3)) * g.N + 32 * j]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t o = (int64_t)(32 * i + 8 * (r >> 2) + (r & 3)) * g.N + 32 * j;
            __builtin_nontemporal_store(acc[i][j][r] + cv[i & 1][j][r], &dbase[o]);
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t o = (int64_t)(32 * i + 8 * (r >> 2) + (r & 3)) * g.N + 32 * j;
            __builtin_nontemporal_store(acc[i][j][r], &dbase[o]);
          }
    }
  };

  // Steady state: stages kt, kt+1 while both issue DMA (kt + 3 < KT, one more stage kept
  // for an odd count); then the last two (or three, or the only one).
  using T_ = std::true_type;
  using F_ = std::false_type;
  if constexpr (KSH == kSingle) {
    stage(sa0, sb0, sa1, sb1, 0, F_{}, F_{});
  } else {
    constexpr int odd = KSH == kOdd ? 1 : 0;
    int kt = 0;
    for (; kt + 2 + odd < KT; kt += 2) {
      stage(sa0, sb0, sa1, sb1, kt, T_{}, T_{});
      stage(sa1, sb1, sa0, sb0, kt + 1, T_{}, T_{});
    }
    if constexpr (KSH == kEven) {
      stage(sa0, sb0, sa1, sb1, kt, F_{}, T_{});
      stage(sa1, sb1, sa0, sb0, kt + 1, F_{}, F_{});
    } else {
      stage(sa0, sb0, sa1, sb1, kt, T_{}, T_{});
      stage(sa1, sb1, sa0, sb0, kt + 1, F_{}, T_{});
      stage(sa0, sb0, sa1, sb1, kt + 2, F_{}, F_{});
    }
  }
  epilogue();
}

// 256x256 blocks (fp8, block-scaled fp8 and 16-bit operands)
template <bool A_MN, bool B_MN, int DT, int WGM, int WGN, bool BOUNDS, int KS>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_direct(GemmArgs g) {
  direct_body<A_MN, B_MN, DT, WGM, WGN, BOUNDS, KS, 256>(g);
}

// 128x128 blocks: 64 KiB of LDS stages (76 KiB with block scales), so two workgroups share a
// CU; for problems with too few 256x256 blocks to fill the chip.
template <bool A_MN, bool B_MN, int DT, int WGM, int WGN, bool BOUNDS, int KS>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_direct128(GemmArgs g) {
  direct_body<A_MN, B_MN, DT, WGM, WGN, BOUNDS, KS, 128>(g);
}

}  // namespace
}  // namespace tg
