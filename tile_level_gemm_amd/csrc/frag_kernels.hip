// Register fragment kernels: matrix <-> matrix-instruction registers, and the register-level
// gemm over register images.
//
// [SYNC-GEMM] 一 and 四: the register-level gemm keeps A / B fragments and the C / D accumulator
// in registers and issues one matrix instruction per output tile and K atom, accumulating in
// place; the caller fills the fragments first with a copy of the ldstmatrix kind ([VEC-AUTO]
// closing reading list: the register path and the warp-collective ldstmatrix copy).
//
// Every lane's registers are runs of RB bytes along one axis of its tile (G runs of R elements):
// 16 bytes, or 8 for the K = 8 / 16 atoms whose lanes hold four 16-bit values.
// Memory is seen as lines (row-major: rows; column-major: columns); a run either lies along a
// memory line or crosses lines ("transposed").
//
//  * direct route: each lane moves its runs between memory and its VGPRs itself — VB-byte
//    transfers along a line (VB from the widest-first width rule), one element per transfer
//    across lines — and writes / reads its registers to / from the register image.
//  * LDS route: a workgroup stages a block of 64 memory lines x 256 bytes (loads) or 512 bytes
//    (stores) through LDS with
//    128-bit global transfers; lanes then read their runs with ds_read_b128 along a line or
//    with the transposing reads across lines: ds_read_b64_tr_b16 (within each 16-lane group,
//    lane j receives element j%4 of the 8-byte reads of lanes 4q + j/4, q = 0..3) and
//    ds_read_b64_tr_b8 (lane j receives byte j%8 of the reads of lanes 2k + j/8, k = 0..7).
//    Stores write runs with ds_write_b128 along a line and element by element across lines.
//    LDS lines are 16 or 32 chunks of 16 bytes; chunk x of line q sits at x ^ swz(q), swz(q) =
//    2(q & 7) ^ ((q >> 3) & 1): sixteen consecutive lines reading one logical chunk hit sixteen
//    distinct chunks, and the two-chunk spans of four (tr_b16) or the chunks of eight (tr_b8)
//    consecutive lines land apart.
#include <hip/hip_runtime.h>

#include "tg_internal.h"

namespace tg {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Fragment kind traits: tile extent TR x TC, element bytes EB, E elements per lane in G runs
// of R (RB bytes each); RUN_ROWS: runs go along the tile's rows.
template <int KIND>
struct FK {
  static constexpr bool k8 = KIND == TG_FRAG_A8_32x32x64 || KIND == TG_FRAG_B8_32x32x64;
  static constexpr bool kAcc = KIND == TG_FRAG_C32_32x32 || KIND == TG_FRAG_C32_16x16;
  static constexpr bool kShortK = KIND == TG_FRAG_A16_32x32x8 || KIND == TG_FRAG_B16_32x32x8 ||
                                  KIND == TG_FRAG_A16_16x16x16 || KIND == TG_FRAG_B16_16x16x16;
  static constexpr int EB = k8 ? 1 : kAcc ? 4 : 2;
  static constexpr int E = k8 ? 32 : KIND == TG_FRAG_C32_32x32 ? 16
                         : (KIND == TG_FRAG_C32_16x16 || kShortK) ? 4 : 8;
  static constexpr int RB = E * EB < 16 ? E * EB : 16;
  static constexpr int R = RB / EB;
  static constexpr int G = E / R;
  static constexpr bool RUN_ROWS = !(KIND == TG_FRAG_A16_32x32x16 || KIND == TG_FRAG_A16_16x16x32 ||
                                     KIND == TG_FRAG_A8_32x32x64 || KIND == TG_FRAG_A16_32x32x8 ||
                                     KIND == TG_FRAG_A16_16x16x16);
  static constexpr int TR = KIND == TG_FRAG_A16_32x32x16 ? 32 : KIND == TG_FRAG_B16_32x32x16 ? 16
                          : KIND == TG_FRAG_A16_16x16x32 ? 16 : KIND == TG_FRAG_B16_16x16x32 ? 32
                          : KIND == TG_FRAG_A8_32x32x64 ? 32 : KIND == TG_FRAG_B8_32x32x64 ? 64
                          : KIND == TG_FRAG_C32_32x32 ? 32 : KIND == TG_FRAG_A16_32x32x8 ? 32
                          : KIND == TG_FRAG_B16_32x32x8 ? 8 : 16;
  static constexpr int TC = KIND == TG_FRAG_A16_32x32x16 ? 16 : KIND == TG_FRAG_B16_32x32x16 ? 32
                          : KIND == TG_FRAG_A16_16x16x32 ? 32 : KIND == TG_FRAG_B16_16x16x32 ? 16
                          : KIND == TG_FRAG_A8_32x32x64 ? 64 : KIND == TG_FRAG_B8_32x32x64 ? 32
                          : KIND == TG_FRAG_C32_32x32 ? 32 : KIND == TG_FRAG_A16_32x32x8 ? 8
                          : KIND == TG_FRAG_B16_32x32x8 ? 32 : 16;
  static_assert(TR * TC == 64 * E, "a fragment tile holds 64 lanes x E elements");

  // Tile coordinates of the first element of run g of lane l.
  __device__ static __forceinline__ void origin(int l, int g, int& r, int& c) {
    if constexpr (KIND == TG_FRAG_A16_32x32x16) { r = l & 31; c = 8 * (l >> 5); }
    else if constexpr (KIND == TG_FRAG_B16_32x32x16) { r = 8 * (l >> 5); c = l & 31; }
    else if constexpr (KIND == TG_FRAG_A16_16x16x32) { r = l & 15; c = 8 * (l >> 4); }
    else if constexpr (KIND == TG_FRAG_B16_16x16x32) { r = 8 * (l >> 4); c = l & 15; }
    else if constexpr (KIND == TG_FRAG_A8_32x32x64) { r = l & 31; c = 32 * g + 16 * (l >> 5); }
    else if constexpr (KIND == TG_FRAG_B8_32x32x64) { r = 32 * g + 16 * (l >> 5); c = l & 31; }
    else if constexpr (KIND == TG_FRAG_C32_32x32) { r = 8 * g + 4 * (l >> 5); c = l & 31; }
    else if constexpr (KIND == TG_FRAG_A16_32x32x8) { r = l & 31; c = 4 * (l >> 5); }
    else if constexpr (KIND == TG_FRAG_B16_32x32x8) { r = 4 * (l >> 5); c = l & 31; }
    else if constexpr (KIND == TG_FRAG_A16_16x16x16) { r = l & 15; c = 4 * (l >> 4); }
    else if constexpr (KIND == TG_FRAG_B16_16x16x16) { r = 4 * (l >> 4); c = l & 15; }
    else { r = 4 * (l >> 4); c = l & 15; }
  }
};

// Tiles per wave on the direct route: 4 KiB of registers.
template <int KIND>
constexpr int tiles_per_wave() { return 4096 / (64 * FK<KIND>::E * FK<KIND>::EB); }

union Run {
  u32x4 v;
  uint64_t d[2];
  uint32_t w[4];
  uint16_t h[8];
  uint8_t b[16];
};

template <int W>
struct Word;
template <> struct Word<16> { typedef u32x4 T; };
template <> struct Word<8> { typedef uint64_t T; };
template <> struct Word<4> { typedef uint32_t T; };
template <> struct Word<2> { typedef uint16_t T; };
template <> struct Word<1> { typedef uint8_t T; };

// Register type of one run.
template <int RB>
struct RunT;
template <> struct RunT<16> { typedef u32x4 T; };
template <> struct RunT<8> { typedef u32x2 T; };

// One run between memory and registers.  Along a line: 16 / VB transfers of VB bytes; across
// lines: R transfers of one element, `pitch` bytes apart.
template <int VB, bool TRANS, int EB, int RB>
__device__ __forceinline__ typename RunT<RB>::T load_run(const uint8_t* p, int64_t pitch) {
  Run r;
  if constexpr (!TRANS) {
    typedef typename Word<VB>::T T;
#pragma unroll
    for (int s = 0; s < RB / VB; ++s) {
      const T x = ((const T*)p)[s];
      __builtin_memcpy(&r.b[s * VB], &x, VB);
    }
  } else {
    typedef typename Word<EB>::T T;
#pragma unroll
    for (int e = 0; e < RB / EB; ++e) {
      const T x = *(const T*)(p + e * pitch);
      __builtin_memcpy(&r.b[e * EB], &x, EB);
    }
  }
  typename RunT<RB>::T out;
  __builtin_memcpy(&out, r.b, RB);
  return out;
}

template <int VB, bool TRANS, int EB, int RB>
__device__ __forceinline__ void store_run(uint8_t* p, int64_t pitch, typename RunT<RB>::T v) {
  Run r;
  __builtin_memcpy(r.b, &v, RB);
  if constexpr (!TRANS) {
    typedef typename Word<VB>::T T;
#pragma unroll
    for (int s = 0; s < RB / VB; ++s) {
      T x;
      __builtin_memcpy(&x, &r.b[s * VB], VB);
      ((T*)p)[s] = x;
    }
  } else {
    typedef typename Word<EB>::T T;
#pragma unroll
    for (int e = 0; e < RB / EB; ++e) {
      T x;
      __builtin_memcpy(&x, &r.b[e * EB], EB);
      *(T*)(p + e * pitch) = x;
    }
  }
}

// Image side: a lane's registers are LANE_BYTES contiguous bytes, so with 8 or 16 bytes per
// lane one instruction moves 512 bytes or 1 KiB of the image contiguously and streams past the
// caches; with 32 or 64 bytes per lane each instruction covers every second or fourth 16-byte
// chunk, and plain accesses let the L2 merge the chunks of one line before it is written back.
template <int LANE_BYTES, class V>
__device__ __forceinline__ void img_store(uint8_t* p, int g, V v) {
  if constexpr (LANE_BYTES <= 16) __builtin_nontemporal_store(v, (V*)p + g);
  else ((V*)p)[g] = v;
}
template <int LANE_BYTES, class V>
__device__ __forceinline__ V img_load(const uint8_t* p, int g) {
  if constexpr (LANE_BYTES <= 16) return __builtin_nontemporal_load((const V*)p + g);
  else return ((const V*)p)[g];
}

// ------------------------------------------------------------------------ direct route ---
// Wave w moves tiles w·TPW .. w·TPW + TPW - 1 of the work order, which walks along memory
// lines (row-major tile order for row-major memory, column-major for column-major) so that
// neighbouring waves share memory lines; the image index is always the row-major tile index.
template <int KIND, bool STORE, bool TRANS, int VB>
__global__ __launch_bounds__(kFragThreads) void frag_direct(FragArgs a) {
  using K = FK<KIND>;
  constexpr bool CM = K::RUN_ROWS != TRANS;   // memory is column-major
  constexpr int TPW = tiles_per_wave<KIND>();
  constexpr int LANE_BYTES = K::E * K::EB;
  typedef typename RunT<K::RB>::T V;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kFragThreads / 64) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t pitch = a.ld * K::EB;
  int64_t off[K::G];   // byte offset of each run's first element from the tile's origin
#pragma unroll
  for (int g = 0; g < K::G; ++g) {
    int r, c;
    K::origin(lane, g, r, c);
    off[g] = (CM ? (int64_t)c * a.ld + r : (int64_t)r * a.ld + c) * K::EB;
  }
  V regs[TPW][K::G];
  int64_t mem_at[TPW], img_at[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int64_t w = wave * TPW + u;
    const int64_t ti = CM ? w % a.tiles_r : w / a.tiles_c;
    const int64_t tj = CM ? w / a.tiles_r : w % a.tiles_c;
    const int64_t q0 = CM ? tj * K::TC : ti * K::TR, p0 = CM ? ti * K::TR : tj * K::TC;
    mem_at[u] = (q0 * a.ld + p0) * K::EB;
    img_at[u] = ((ti * a.tiles_c + tj) * 64 + lane) * LANE_BYTES;
  }
  if constexpr (!STORE) {
#pragma unroll
    for (int u = 0; u < TPW; ++u)
      if (wave * TPW + u < a.ntiles)
#pragma unroll
        for (int g = 0; g < K::G; ++g)
          regs[u][g] = load_run<VB, TRANS, K::EB, K::RB>(a.mem + mem_at[u] + off[g], pitch);
#pragma unroll
    for (int u = 0; u < TPW; ++u)
      if (wave * TPW + u < a.ntiles)
#pragma unroll
        for (int g = 0; g < K::G; ++g)
          img_store<LANE_BYTES, V>(a.img + img_at[u], g, regs[u][g]);
  } else {
#pragma unroll
    for (int u = 0; u < TPW; ++u)
      if (wave * TPW + u < a.ntiles)
#pragma unroll
        for (int g = 0; g < K::G; ++g)
          regs[u][g] = img_load<LANE_BYTES, V>(a.img + img_at[u], g);
#pragma unroll
    for (int u = 0; u < TPW; ++u)
      if (wave * TPW + u < a.ntiles)
#pragma unroll
        for (int g = 0; g < K::G; ++g)
          store_run<VB, TRANS, K::EB, K::RB>(a.mem + mem_at[u] + off[g], pitch, regs[u][g]);
  }
}

// --------------------------------------------------------------------------- LDS route ---
__device__ __forceinline__ uint32_t swz(uint32_t q) { return ((q & 7u) << 1) ^ ((q >> 3) & 1u); }
// LDS byte address of byte `byte` of line q of a block with LB-byte lines.
template <int LB>
__device__ __forceinline__ uint32_t lds_at(uint32_t q, uint32_t byte) {
  return q * LB + (((byte >> 4) ^ swz(q)) << 4) + (byte & 15u);
}

// Run of a lane whose first element sits at LDS line q, element p (block coordinates).
template <int EB, bool TRANS, int RB, int LB>
__device__ __forceinline__ typename RunT<RB>::T lds_read_run(const uint8_t* lds, int q, int p,
                                                             int lane) {
  typedef typename RunT<RB>::T V;
  Run r;
  if constexpr (!TRANS) {
    const V v = *(const V*)(lds + lds_at<LB>(q, p * EB));
    __builtin_memcpy(r.b, &v, RB);
  } else if constexpr (EB == 2) {
    // Lanes of a 16-lane group hold consecutive p and the same q: lane i reads 4 elements at
    // line q + 4s + i/4, element p - i + 4(i%4), and receives (q + 4s .. +3, p).
    const int i = lane & 15;
#pragma unroll
    for (int s = 0; s < RB / 8; ++s) {
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(lds + lds_at<LB>(q + 4 * s + (i >> 2), 2 * (p - i + 4 * (i & 3)))));
      __builtin_memcpy(&r.b[8 * s], &v, 8);
    }
  } else if constexpr (EB == 1) {
    // lane i reads 8 bytes at line q + 8s + i/2, element p - i + 8(i%2); receives (q + 8s .. +7, p)
    const int i = lane & 15;
#pragma unroll
    for (int s = 0; s < RB / 8; ++s) {
      const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_i32x2*)(lds + lds_at<LB>(q + 8 * s + (i >> 1), p - i + 8 * (i & 1))));
      __builtin_memcpy(&r.b[8 * s], &v, 8);
    }
  } else {
#pragma unroll
    for (int e = 0; e < RB / 4; ++e) r.w[e] = *(const uint32_t*)(lds + lds_at<LB>(q + e, 4 * p));
  }
  V out;
  __builtin_memcpy(&out, r.b, RB);
  return out;
}

template <int EB, bool TRANS, int RB, int LB>
__device__ __forceinline__ void lds_write_run(uint8_t* lds, int q, int p, typename RunT<RB>::T v) {
  typedef typename RunT<RB>::T V;
  Run r;
  __builtin_memcpy(r.b, &v, RB);
  if constexpr (!TRANS) {
    *(V*)(lds + lds_at<LB>(q, p * EB)) = v;
  } else {
    typedef typename Word<EB>::T T;
#pragma unroll
    for (int e = 0; e < RB / EB; ++e) {
      T x;
      __builtin_memcpy(&x, &r.b[e * EB], EB);
      *(T*)(lds + lds_at<LB>(q + e, p * EB)) = x;
    }
  }
}

// One workgroup per NB blocks of 64 lines x LB bytes, adjacent along the lines (groups walk
// along the lines first); each block's tiles are shared out over the four waves.  Stores use
// one block of 512-byte lines (each workgroup writes runs of 512 bytes of every line: 5.6-6.2
// TB/s against 5.5-6.1 with 256), loads four blocks of 256-byte lines (with one block, 512-byte
// lines read at 3.2-3.8 TB/s against 5.0-6.0 with 256): every load of all four blocks is in
// flight before the first LDS write, so a workgroup reads 1 KiB runs of each line.
template <int KIND, bool STORE, bool TRANS>
__global__ __launch_bounds__(kFragThreads) void frag_lds(FragArgs a) {
  constexpr int LB = frag_lds_line_bytes(STORE);
  constexpr int NB = frag_lds_blocks(STORE);
  constexpr int BLK = kFragLdsLines * LB;   // LDS bytes of one block
  constexpr int kLineChunks = LB / 16;   // 16-byte chunks per block line
  using K = FK<KIND>;
  constexpr bool CM = K::RUN_ROWS != TRANS;
  constexpr int TQ = CM ? K::TC : K::TR;            // tile extent across lines
  constexpr int TP = CM ? K::TR : K::TC;            // tile extent along a line (elements)
  constexpr int LINE = LB / K::EB;   // elements per block line
  constexpr int NTQ = kFragLdsLines / TQ, NTP = LINE / TP;
  constexpr int CHUNKS = kFragLdsLines * LB / 16 / kFragThreads;
  constexpr int LANE_BYTES = K::E * K::EB;
  typedef typename RunT<K::RB>::T V;
  static_assert(NTQ * TQ == kFragLdsLines && NTP * TP == LINE, "whole tiles per block");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NB * BLK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nbp = (a.line_len + LINE - 1) / LINE;   // blocks along a line
  const int64_t ngp = (nbp + NB - 1) / NB;               // groups of NB blocks along a line
  const int64_t q0 = (int64_t)(blockIdx.x / ngp) * kFragLdsLines;
  const int64_t p0 = (int64_t)(blockIdx.x % ngp) * NB * LINE;   // the group's first element
  const int qn = (int)(a.lines - q0 < kFragLdsLines ? a.lines - q0 : kFragLdsLines);
  // elements of block k along the line: a multiple of TP, 0 past the end
  auto pn_of = [&](int k) -> int {
    const int64_t left = a.line_len - p0 - (int64_t)k * LINE;
    return (int)(left <= 0 ? 0 : (left < LINE ? left : LINE));
  };
  const int64_t pitch = a.ld * K::EB;
  uint8_t* gblock = a.mem + (q0 * a.ld + p0) * K::EB;

  // tile b of block k
  auto tile_of = [&](int k, int b, int& tq, int& tp, int64_t& img) -> bool {
    tq = b / NTP;
    tp = b % NTP;
    const int pn = pn_of(k);
    if (tq * TQ >= qn || tp * TP >= pn) return false;
    const int64_t qt = q0 + tq * TQ, pt = p0 + (int64_t)k * LINE + tp * TP;
    const int64_t ti = CM ? pt / K::TR : qt / K::TR, tj = CM ? qt / K::TC : pt / K::TC;
    img = ((ti * a.tiles_c + tj) * 64 + lane) * LANE_BYTES;
    return true;
  };

  if constexpr (!STORE) {
    int pnb[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) pnb[k] = pn_of(k) * K::EB;   // bytes of block k's lines
    u32x4 v[CHUNKS][NB];
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + kFragThreads * i, q = c / kLineChunks, x = c % kLineChunks;
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (q < qn && 16 * x < pnb[k])
          v[i][k] = __builtin_nontemporal_load((const u32x4*)(gblock + q * pitch + k * LB + 16 * x));
    }
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + kFragThreads * i, q = c / kLineChunks, x = c % kLineChunks;
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (q < qn && 16 * x < pnb[k]) *(u32x4*)(lds + k * BLK + lds_at<LB>(q, 16 * x)) = v[i][k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      for (int b = wave; b < NTQ * NTP; b += kFragThreads / 64) {
        int tq, tp;
        int64_t img;
        if (!tile_of(k, b, tq, tp, img)) continue;
        V regs[K::G];
#pragma unroll
        for (int g = 0; g < K::G; ++g) {
          int r, c;
          K::origin(lane, g, r, c);
          regs[g] = lds_read_run<K::EB, TRANS, K::RB, LB>(lds + k * BLK, tq * TQ + (CM ? c : r),
                                                      tp * TP + (CM ? r : c), lane);
        }
#pragma unroll
        for (int g = 0; g < K::G; ++g)
          img_store<LANE_BYTES, V>(a.img + img, g, regs[g]);
      }
    }
  } else {
    int pnb[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) pnb[k] = pn_of(k) * K::EB;   // bytes of block k's lines
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      for (int b = wave; b < NTQ * NTP; b += kFragThreads / 64) {
        int tq, tp;
        int64_t img;
        if (!tile_of(k, b, tq, tp, img)) continue;
        V regs[K::G];
#pragma unroll
        for (int g = 0; g < K::G; ++g)
          regs[g] = img_load<LANE_BYTES, V>(a.img + img, g);
#pragma unroll
        for (int g = 0; g < K::G; ++g) {
          int r, c;
          K::origin(lane, g, r, c);
          lds_write_run<K::EB, TRANS, K::RB, LB>(lds + k * BLK, tq * TQ + (CM ? c : r),
                                            tp * TP + (CM ? r : c), regs[g]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + kFragThreads * i, q = c / kLineChunks, x = c % kLineChunks;
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (q < qn && 16 * x < pnb[k])
          __builtin_nontemporal_store(*(const u32x4*)(lds + k * BLK + lds_at<LB>(q, 16 * x)),
                                      (u32x4*)(gblock + q * pitch + k * LB + 16 * x));
    }
  }
}

// ------------------------------------------------------------------ register-level gemm ---
template <int SHAPE, int ADT, int BDT>
__device__ __forceinline__ void mma_step(const uint8_t* a, const uint8_t* b, float* acc) {
  if constexpr (SHAPE == TG_MMA_32x32x8 || SHAPE == TG_MMA_16x16x16) {
    // four 16-bit values per lane (the bf16 forms take them as shorts)
    const u32x2 x = *(const u32x2*)a, y = *(const u32x2*)b;
    if constexpr (SHAPE == TG_MMA_32x32x8) {
      f32x16 c;
      __builtin_memcpy(&c, acc, 64);
      if constexpr (ADT == TG_F16)
        c = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(f16x4, x),
                                                 __builtin_bit_cast(f16x4, y), c, 0, 0, 0);
      else
        c = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(s16x4, x),
                                                     __builtin_bit_cast(s16x4, y), c, 0, 0, 0);
      __builtin_memcpy(acc, &c, 64);
    } else {
      f32x4 c;
      __builtin_memcpy(&c, acc, 16);
      if constexpr (ADT == TG_F16)
        c = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, x),
                                                  __builtin_bit_cast(f16x4, y), c, 0, 0, 0);
      else
        c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, x),
                                                      __builtin_bit_cast(s16x4, y), c, 0, 0, 0);
      __builtin_memcpy(acc, &c, 16);
    }
  } else if constexpr (SHAPE == TG_MMA_32x32x16 || SHAPE == TG_MMA_16x16x32) {
    const u32x4 x = *(const u32x4*)a, y = *(const u32x4*)b;
    if constexpr (SHAPE == TG_MMA_32x32x16) {
      f32x16 c;
      __builtin_memcpy(&c, acc, 64);
      if constexpr (ADT == TG_F16)
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x),
                                                   __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
      else
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                    __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
      __builtin_memcpy(acc, &c, 64);
    } else {
      f32x4 c;
      __builtin_memcpy(&c, acc, 16);
      if constexpr (ADT == TG_F16)
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x),
                                                   __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
      else
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                    __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
      __builtin_memcpy(acc, &c, 16);
    }
  } else {
    // fp8: the format operands name A's and B's encodings (0 = e4m3, 1 = e5m2); no block
    // scales.  Each lane's 32 bytes are two 32-K blocks of 16 bytes per lane half.
    i32x8 x, y;
    __builtin_memcpy(&x, a, 32);
    __builtin_memcpy(&y, b, 32);
    f32x16 c;
    __builtin_memcpy(&c, acc, 64);
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, ADT == TG_FP8_E5M2 ? 1 : 0,
                                                        BDT == TG_FP8_E5M2 ? 1 : 0, 0, 0, 0, 0);
    __builtin_memcpy(acc, &c, 64);
  }
}

// One wave per output tile; every wave of a launch is whole (the tile index is wave-uniform),
// so the matrix instructions always run with all 64 lanes.
template <int SHAPE, int ADT, int BDT>
__global__ __launch_bounds__(kFragThreads) void frag_mma(FragMmaArgs g) {
  constexpr bool F8 = SHAPE == TG_MMA_32x32x64_F8;
  constexpr bool SHORT_K = SHAPE == TG_MMA_32x32x8 || SHAPE == TG_MMA_16x16x16;
  constexpr int AB_BYTES = F8 ? 32 : SHORT_K ? 8 : 16;         // operand bytes per lane
  constexpr int ACC = (SHAPE == TG_MMA_16x16x32 || SHAPE == TG_MMA_16x16x16) ? 4 : 16;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * (kFragThreads / 64) +
                    __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w >= (int64_t)g.tiles_m * g.tiles_n) return;
  const int64_t i = w / g.tiles_n, j = w % g.tiles_n;
  float acc[ACC];
  const int64_t cd = (w * 64 + lane) * ACC;
  if (g.use_c) {
#pragma unroll
    for (int r = 0; r < ACC; r += 4) *(f32x4*)&acc[r] = *(const f32x4*)(g.c + cd + r);
  } else {
#pragma unroll
    for (int r = 0; r < ACC; ++r) acc[r] = 0.0f;
  }
  const uint8_t* pa = g.a + (i * g.tiles_k * 64 + lane) * AB_BYTES;
  const uint8_t* pb = g.b + (j * 64 + lane) * AB_BYTES;
  const int64_t b_step = (int64_t)g.tiles_n * 64 * AB_BYTES;
  for (int kk = 0; kk < g.tiles_k; ++kk) {
    mma_step<SHAPE, ADT, BDT>(pa, pb, acc);
    pa += 64 * AB_BYTES;
    pb += b_step;
  }
#pragma unroll
  for (int r = 0; r < ACC; r += 4) *(f32x4*)(g.d + cd + r) = *(const f32x4*)&acc[r];
}

// ------------------------------------------------------------------------- dispatch ---
template <int KIND, bool STORE, bool TRANS>
hipError_t launch_direct(const FragArgs& a, int vb, int64_t grid, hipStream_t s) {
  constexpr int EB = FK<KIND>::EB;
  const dim3 gd((unsigned)grid), bd(kFragThreads);
  if constexpr (TRANS) {
    hipLaunchKernelGGL((frag_direct<KIND, STORE, true, EB>), gd, bd, 0, s, a);
  } else {
    switch (vb) {
      case 16: hipLaunchKernelGGL((frag_direct<KIND, STORE, false, (FK<KIND>::RB >= 16 ? 16 : FK<KIND>::RB)>), gd, bd, 0, s, a); break;
      case 8: hipLaunchKernelGGL((frag_direct<KIND, STORE, false, (EB <= 8 ? 8 : 16)>), gd, bd, 0, s, a); break;
      case 4: hipLaunchKernelGGL((frag_direct<KIND, STORE, false, (EB <= 4 ? 4 : 16)>), gd, bd, 0, s, a); break;
      case 2: hipLaunchKernelGGL((frag_direct<KIND, STORE, false, (EB <= 2 ? 2 : 16)>), gd, bd, 0, s, a); break;
      default: hipLaunchKernelGGL((frag_direct<KIND, STORE, false, (EB <= 1 ? 1 : 16)>), gd, bd, 0, s, a); break;
    }
  }
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(const FragArgs& a, bool store, bool trans, int route, int vb, int64_t grid,
                       hipStream_t s) {
  const dim3 gd((unsigned)grid), bd(kFragThreads);
  if (route == TG_FRAG_LDS) {
    if (store && trans) hipLaunchKernelGGL((frag_lds<KIND, true, true>), gd, bd, 0, s, a);
    else if (store) hipLaunchKernelGGL((frag_lds<KIND, true, false>), gd, bd, 0, s, a);
    else if (trans) hipLaunchKernelGGL((frag_lds<KIND, false, true>), gd, bd, 0, s, a);
    else hipLaunchKernelGGL((frag_lds<KIND, false, false>), gd, bd, 0, s, a);
    return hipGetLastError();
  }
  if (store) return trans ? launch_direct<KIND, true, true>(a, vb, grid, s)
                          : launch_direct<KIND, true, false>(a, vb, grid, s);
  return trans ? launch_direct<KIND, false, true>(a, vb, grid, s)
               : launch_direct<KIND, false, false>(a, vb, grid, s);
}

}  // namespace

int frag_tiles_per_wave(int kind) {
  switch (kind) {
    case TG_FRAG_A16_32x32x16: return tiles_per_wave<TG_FRAG_A16_32x32x16>();
    case TG_FRAG_B16_32x32x16: return tiles_per_wave<TG_FRAG_B16_32x32x16>();
    case TG_FRAG_A16_16x16x32: return tiles_per_wave<TG_FRAG_A16_16x16x32>();
    case TG_FRAG_B16_16x16x32: return tiles_per_wave<TG_FRAG_B16_16x16x32>();
    case TG_FRAG_A8_32x32x64: return tiles_per_wave<TG_FRAG_A8_32x32x64>();
    case TG_FRAG_B8_32x32x64: return tiles_per_wave<TG_FRAG_B8_32x32x64>();
    case TG_FRAG_C32_32x32: return tiles_per_wave<TG_FRAG_C32_32x32>();
    case TG_FRAG_A16_32x32x8: return tiles_per_wave<TG_FRAG_A16_32x32x8>();
    case TG_FRAG_B16_32x32x8: return tiles_per_wave<TG_FRAG_B16_32x32x8>();
    case TG_FRAG_A16_16x16x16: return tiles_per_wave<TG_FRAG_A16_16x16x16>();
    case TG_FRAG_B16_16x16x16: return tiles_per_wave<TG_FRAG_B16_16x16x16>();
    default: return tiles_per_wave<TG_FRAG_C32_16x16>();
  }
}

hipError_t launch_frag(const FragArgs& a, int kind, bool store, bool transposed, int route,
                       int vec_bytes, int64_t grid, hipStream_t s) {
  switch (kind) {
    case TG_FRAG_A16_32x32x16: return launch_kind<TG_FRAG_A16_32x32x16>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_B16_32x32x16: return launch_kind<TG_FRAG_B16_32x32x16>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_A16_16x16x32: return launch_kind<TG_FRAG_A16_16x16x32>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_B16_16x16x32: return launch_kind<TG_FRAG_B16_16x16x32>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_A8_32x32x64: return launch_kind<TG_FRAG_A8_32x32x64>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_B8_32x32x64: return launch_kind<TG_FRAG_B8_32x32x64>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_C32_32x32: return launch_kind<TG_FRAG_C32_32x32>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_C32_16x16: return launch_kind<TG_FRAG_C32_16x16>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_A16_32x32x8: return launch_kind<TG_FRAG_A16_32x32x8>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_B16_32x32x8: return launch_kind<TG_FRAG_B16_32x32x8>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_A16_16x16x16: return launch_kind<TG_FRAG_A16_16x16x16>(a, store, transposed, route, vec_bytes, grid, s);
    case TG_FRAG_B16_16x16x16: return launch_kind<TG_FRAG_B16_16x16x16>(a, store, transposed, route, vec_bytes, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_frag_mma(const FragMmaArgs& g, int shape, int a_dtype, int b_dtype, int64_t grid,
                           hipStream_t s) {
  const dim3 gd((unsigned)grid), bd(kFragThreads);
  const bool a5 = a_dtype == TG_FP8_E5M2, b5 = b_dtype == TG_FP8_E5M2;
  switch (shape) {
    case TG_MMA_32x32x16:
      if (a_dtype == TG_F16) hipLaunchKernelGGL((frag_mma<TG_MMA_32x32x16, TG_F16, TG_F16>), gd, bd, 0, s, g);
      else hipLaunchKernelGGL((frag_mma<TG_MMA_32x32x16, TG_BF16, TG_BF16>), gd, bd, 0, s, g);
      break;
    case TG_MMA_16x16x32:
      if (a_dtype == TG_F16) hipLaunchKernelGGL((frag_mma<TG_MMA_16x16x32, TG_F16, TG_F16>), gd, bd, 0, s, g);
      else hipLaunchKernelGGL((frag_mma<TG_MMA_16x16x32, TG_BF16, TG_BF16>), gd, bd, 0, s, g);
      break;
    case TG_MMA_32x32x8:
      if (a_dtype == TG_F16) hipLaunchKernelGGL((frag_mma<TG_MMA_32x32x8, TG_F16, TG_F16>), gd, bd, 0, s, g);
      else hipLaunchKernelGGL((frag_mma<TG_MMA_32x32x8, TG_BF16, TG_BF16>), gd, bd, 0, s, g);
      break;
    case TG_MMA_16x16x16:
      if (a_dtype == TG_F16) hipLaunchKernelGGL((frag_mma<TG_MMA_16x16x16, TG_F16, TG_F16>), gd, bd, 0, s, g);
      else hipLaunchKernelGGL((frag_mma<TG_MMA_16x16x16, TG_BF16, TG_BF16>), gd, bd, 0, s, g);
      break;
    case TG_MMA_32x32x64_F8:
      if (!a5 && !b5) hipLaunchKernelGGL((frag_mma<TG_MMA_32x32x64_F8, TG_FP8_E4M3, TG_FP8_E4M3>), gd, bd, 0, s, g);
      else if (!a5) hipLaunchKernelGGL((frag_mma<TG_MMA_32x32x64_F8, TG_FP8_E4M3, TG_FP8_E5M2>), gd, bd, 0, s, g);
      else if (!b5) hipLaunchKernelGGL((frag_mma<TG_MMA_32x32x64_F8, TG_FP8_E5M2, TG_FP8_E4M3>), gd, bd, 0, s, g);
      else hipLaunchKernelGGL((frag_mma<TG_MMA_32x32x64_F8, TG_FP8_E5M2, TG_FP8_E5M2>), gd, bd, 0, s, g);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tg
