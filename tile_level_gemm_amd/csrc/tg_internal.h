// Internal declarations shared by the C-ABI layer (abi.cpp), the host planner
// (plan.cpp) and the HIP kernels (copy_kernels.hip, gemm_kernels.hip).
// Not part of the public ABI: include/tilegemm.h is.
#pragma once

#include <stdint.h>
#include <string>

#include <hip/hip_runtime.h>

#include "../../include/tilegemm.h"

namespace tg {

// ---------------------------------------------------------------- errors ---
// Sets the thread-local reason string and returns `code`.
int fail(int code, const std::string& why);
void clear_error();

// --------------------------------------------------------------- planner ---
// One side of a copy region: layout kind, resolved leading dimension (never 0)
// and the element offset of the region's first element.
struct Side {
  int kind;
  int64_t ld;
  int64_t base;
};

int elem_bytes(int dtype);  // 0 for an unknown dtype

// The vec_auto partition of one rows x cols region (see tile_copy_partition).
// Returns TG_OK or a status with *why set.
int partition(int64_t rows, int64_t cols, int eb, int threads, const Side& drive,
              const Side& other, tg_copy_phase* out, std::string* why);

// Extra alignment rule of a tiled tensor side: every tile's base must stay
// aligned to `vec` (tile steps tile_rows*row_stride and tile_cols*col_stride).
bool tile_steps_aligned(const Side& s, int64_t tile_rows, int64_t tile_cols, int64_t tiles_r,
                        int64_t tiles_c, int64_t vec);

// --------------------------------------------------------- launch structs ---
struct CopyPhase {
  int32_t outer;       // rounds per thread
  int32_t vec;         // elements per transfer
  int32_t row_order;   // 1: fused order is row-major over the tile, 0: column-major
  int32_t inner;       // extent of the fused order's inner dimension
  int32_t inner_log2;  // log2(inner) when a power of two, else -1
};

struct CopyArgs {
  const uint8_t* src;
  uint8_t* dst;
  int64_t src_ld, dst_ld;     // elements
  int32_t src_kind, dst_kind; // tg_layout_kind (XOR only for one-tile tensors)
  int32_t tile_rows, tile_cols;
  int64_t tiles_c;            // tiles along the column dimension
  int64_t ntiles;
  int32_t eb;                 // element bytes
  int32_t lds_xor;            // LDS tile layout: 1 = XOR swizzle, 0 = packed row-major
  int32_t xor_mask;           // (min(8, 16-byte chunks per tile row) - 1) for XOR layouts
  int32_t threads;
  CopyPhase load, store;
};

int launch_tile_copy(const CopyArgs& a, int vec_bytes_load, int vec_bytes_store, int lds_bytes,
                     void* stream);

// Asynchronous tile copy: vec_bytes 16 or 4 on both sides, rounds 1/2/4/8 per thread (the same
// for both sides), depth 1..4 stages, tiles_per_wg consecutive tiles per workgroup.
constexpr int kAsyncStageBytes = 16384;
hipError_t launch_tile_copy_async(const CopyArgs& a, int vec_bytes, int rounds, int depth,
                                  int32_t tiles_per_wg, int64_t grid, hipStream_t s);

struct GemmArgs {
  const uint16_t* A;   // operand base addresses (fp8 kernels read them as bytes)
  const uint16_t* B;
  const float* C;
  float* D;
  int32_t M, N, K;
  int32_t use_c;
  int32_t tiles_m, tiles_n;
  const uint8_t* SA;   // block-scaled fp8: E8M0 scales of A [M][K/32] and B [N][K/32]
  const uint8_t* SB;
};

struct GemmConfig {
  int kernel;          // tg_gemm_kernel
  int bm, bn, bk, wm, wn, threads;
  int bounds;          // ragged tiles present
  int lds_bytes;
  int64_t grid;
  int direct;          // 1: gemm_direct (global -> LDS loads, whole 256x256 tiles, K % 128 == 0)
  int atom;            // TG_GEMM_ATOM: the matrix instruction (tg_mma_shape)
};

// The register kernel's matrix instruction for a problem: the candidates widest first; one is
// admissible when its K depth divides K; the least work after padding M and N up to it wins,
// then the fewest global loads per multiply-add for the stored layouts, then the widest.
// Returns a tg_mma_shape, or 0 when none is admissible (K <= 0 or K % 8 != 0).
int gemm_atom_choice(int64_t M, int64_t N, int64_t K, int trans_a, int trans_b);

// Host-side kernel choice for a validated problem (the transposes decide which operand extents
// the direct kernel's 32-bit offsets must cover).
GemmConfig choose_gemm(int64_t M, int64_t N, int64_t K, int trans_a, int trans_b);

int launch_gemm(const GemmArgs& g, const GemmConfig& cfg, int trans_a, int trans_b, int dtype,
                void* stream);

bool direct_gemm_fits(int64_t M, int64_t N, int64_t K, int trans_a, int trans_b);

// fp8 GEMM (any operand orientation): 256x256 blocks (128x128 when there are fewer than 256 of
// the larger and at most 512 of the smaller), 512 threads, grid = ceil(M/bm)·ceil(N/bn);
// bounds = M or N not a multiple of the block.  scaled: block-scaled fp8.
GemmConfig choose_gemm_fp8(int64_t M, int64_t N, int64_t K, bool scaled);
// scaled: block-scaled fp8 (E8M0 scales in g.SA, g.SB).  bs: block size (cfg.bm).
hipError_t launch_gemm_fp8(const GemmArgs& g, int64_t grid, int trans_a, int trans_b, int a_dtype,
                           int b_dtype, bool bounds, bool scaled, int bs, hipStream_t s);
// Block-scaled GEMM with 6- and 4-bit packed K-contiguous operands (MFMA format codes
// a_fmt, b_fmt: 2 = e2m3, 3 = e3m2, 4 = e2m1) on bs x bs blocks (128: 256 threads, 256: 512);
// grid = ceil(M/bs)·ceil(N/bs); bounds: M or N not a multiple of bs.
hipError_t launch_gemm_mx_packed(const GemmArgs& g, int64_t grid, int a_fmt, int b_fmt, bool bounds,
                                 int bs, hipStream_t s);
int packed_lds_bytes(int a_fmt, int b_fmt, int bs);
// Block-scaled e2m1 x e2m1 GEMM on the direct-load kernel (A [M][K/2], B [N][K/2] packed rows,
// K % 256 == 0), bs x bs blocks (256 or 128) of 512 threads; grid = ceil(M/bs)·ceil(N/bs).
hipError_t launch_fp4_direct(const GemmArgs& g, int64_t grid, bool bounds, int bs, hipStream_t s);
// Block-scaled 6-bit GEMM on the direct-load kernel (A [M][3K/4], B [N][3K/4] packed rows, K % 128
// == 0; af, bf: 2 = e2m3, 3 = e3m2), bs x bs blocks (256 or 128) of 512 threads.
hipError_t launch_fp6_direct(const GemmArgs& g, int64_t grid, int af, int bf, bool bounds, int bs,
                             hipStream_t s);

// 16-bit direct-load GEMM on bs x bs blocks (256 or 128).
hipError_t launch_gemm_direct(const GemmArgs& g, int64_t grid, int trans_a, int trans_b, int dtype,
                              int bs, hipStream_t s);

// ------------------------------------------------------------ fragments ---
// Register fragment copies (tile_frag_load / tile_frag_store).  Memory is seen as lines: Q
// lines of LN elements (row-major: Q = rows, LN = cols; column-major: Q = cols, LN = rows).
struct FragArgs {
  uint8_t* mem;         // src of a load, dst of a store
  uint8_t* img;         // register image: dst of a load, src of a store
  int64_t ld;           // elements between memory lines
  int64_t lines, line_len;   // Q and LN
  int64_t tiles_r, tiles_c;  // fragment tiles along the matrix rows / columns
  int64_t ntiles;
};

constexpr int kFragThreads = 256;          // four waves per workgroup
constexpr int kFragLdsLines = 64;          // LDS route: a block of 64 lines x line bytes
// bytes per block line: 256 for loads, 512 for stores (measured per direction)
constexpr int frag_lds_line_bytes(bool store) { return store ? 512 : 256; }
// LDS route: blocks per workgroup, adjacent along the lines.  Loads take 4, so that a workgroup
// reads 1 KiB runs of every line while each block keeps its 256-byte lines; stores take 1
// (measured: two blocks of 512-byte lines per workgroup dropped most kinds from about 6.0 to
// 4.4 TB/s).
constexpr int frag_lds_blocks(bool store) { return store ? 1 : 4; }

// Tiles one wave moves per direct-route launch iteration (4 KiB of registers per wave).
int frag_tiles_per_wave(int kind);

// route: TG_FRAG_DIRECT or TG_FRAG_LDS; vec_bytes: direct-route transfer width.
hipError_t launch_frag(const FragArgs& a, int kind, bool store, bool transposed, int route,
                       int vec_bytes, int64_t grid, hipStream_t s);

struct FragMmaArgs {
  const uint8_t* a;     // images
  const uint8_t* b;
  const float* c;
  float* d;
  int32_t tiles_m, tiles_n, tiles_k;
  int32_t use_c;
};

hipError_t launch_frag_mma(const FragMmaArgs& a, int shape, int a_dtype, int b_dtype, int64_t grid,
                           hipStream_t s);

}  // namespace tg
