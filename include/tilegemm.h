/*
 * tilegemm.h — C ABI of the MI355X (gfx950) tile GEMM and tile copy library.
 *
 * Sources (cited by page title and section):
 *   [SYNC-GEMM]  "TVM TIRx 同步 GEMM 深度解析：warp 级 mma.sync 的寄存器碎片排布与完整下放链路"
 *                (trdm.cn/news/580350), sections 一 … 八 and the closing test-coverage part.
 *   [VEC-AUTO]   "TVM TIRx CUDA 向量化内存拷贝实战：vec_auto 变体的 global↔shared 实现路径（gmem_smem）
 *                深度解析" (0539edu.com/news/4886382).
 *   [TCGEN05-CP] "TVM Blackwell tcgen05.cp 全解析：shared→tmem 异步拷贝的形状选择、矩阵描述符与调度算法"
 *                (pnsm.cn/news/1939927).
 *
 * Conventions shared by every entry point:
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     allocates no device memory and keeps no pointer after a call returns.
 *   - Device pointers: A, B, C, D, src and dst are device (HBM) pointers of the
 *     current HIP device.  Host-only entry points (the *_plan functions and
 *     tile_copy_partition) take addresses only to test alignment and never
 *     dereference them; they need no GPU.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *     stream).  Launches are asynchronous on that stream; the library creates
 *     no stream and never synchronises.  A call issues kernel launches only (no
 *     allocation, memset or copy), so it may be recorded into a HIP graph; each
 *     replay reads the buffers' contents at that time.
 *   - Errors: every argument is validated before anything is launched, so a
 *     rejected call writes nothing.  The return value is a tg_status; the
 *     reason of the last failure on the calling thread is tile_last_error().
 *     A HIP launch failure returns TG_E_HIP with the HIP error text.
 *   - Rejection, never masking: a call the kernels cannot serve exactly is
 *     refused with a reason rather than run on a slow scalar path
 *     ([VEC-AUTO] 接受什么输入; [SYNC-GEMM] 测试覆盖, rejection tests).
 */
#ifndef TILEGEMM_H
#define TILEGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats.  tile_gemm operands take TG_F16 or TG_BF16, tile_gemm_fp8 operands
 * TG_FP8_E4M3 or TG_FP8_E5M2, tile_gemm_mx those two or the 6- and 4-bit formats; copies move
 * the whole-byte formats as raw bits (a packed 6- or 4-bit matrix copies as TG_U8 bytes). */
typedef enum tg_dtype {
  TG_F16 = 1,       /* IEEE binary16 */
  TG_BF16 = 2,      /* bfloat16 */
  TG_F32 = 3,       /* IEEE binary32 */
  TG_U8 = 4,        /* uint8 */
  TG_I8 = 5,        /* int8 */
  TG_FP8_E4M3 = 6,  /* float8 e4m3fn */
  TG_FP8_E5M2 = 7,  /* float8 e5m2 */
  TG_FP6_E2M3 = 8,  /* 6-bit e2m3 (bias 1, largest 7.5), packed rows: tile_gemm_mx only */
  TG_FP6_E3M2 = 9,  /* 6-bit e3m2 (bias 3, largest 28), packed rows: tile_gemm_mx only */
  TG_FP4_E2M1 = 10  /* 4-bit e2m1 (bias 1, largest 6), packed rows: tile_gemm_mx only */
} tg_dtype;

typedef enum tg_status {
  TG_OK = 0,
  TG_E_NULL = -1,     /* a required pointer is NULL */
  TG_E_SHAPE = -2,    /* extents: negative, M%16, N%8, K%8, or not a whole number of tiles */
  TG_E_DTYPE = -3,    /* unsupported element format */
  TG_E_BETA = -4,     /* beta not exactly 0.0 or 1.0 */
  TG_E_ALIAS = -5,    /* an output overlaps an input other than the allowed C == D */
  TG_E_ALIGN = -6,    /* a GEMM operand cannot be read with 128-bit vectors */
  TG_E_THREADS = -7,  /* thread count <= 0, > 1024, or not dividing the tile's elements */
  TG_E_LAYOUT = -8,   /* layout kind / leading dimension not usable */
  TG_E_HIP = -9,      /* HIP runtime or launch error */
  TG_E_ARG = -10      /* any other invalid argument (flags, transpose values, NULL out-params) */
} tg_status;

/* Layout of a rows x cols matrix in memory ([VEC-AUTO] 算法核心 step 1: a
 * copy is described by the layouts of its two sides). */
typedef enum tg_layout_kind {
  TG_ROW_MAJOR = 0,    /* element (r, c) at r*ld + c; ld >= cols, 0 = packed (cols) */
  TG_COL_MAJOR = 1,    /* element (r, c) at c*ld + r; ld >= rows, 0 = packed (rows) */
  TG_XOR_SWIZZLE = 2   /* packed row-major tile, each row cut into 16-byte chunks whose
                          index is XOR-ed with (r mod min(8, chunks per row)); rows must be a
                          power-of-two number of chunks.  For 128-byte rows this is
                          x ^ ((x & 0x380) >> 3) on the byte offset x — the swizzle family
                          of [TCGEN05-CP] 调度算法 step 2 with 16-byte atoms. */
} tg_layout_kind;

typedef struct tg_layout {
  int32_t kind;      /* tg_layout_kind */
  int32_t reserved;  /* must be 0 */
  int64_t ld;        /* leading dimension in elements; 0 = packed; at most 2^40 (else
                        TG_E_LAYOUT) */
} tg_layout;

/* How tile_copy_ex stages a tensor: it is cut into tile_rows x tile_cols
 * tiles; a workgroup of `threads` threads moves one tile global -> LDS
 * (laid out as lds_kind: TG_ROW_MAJOR or TG_XOR_SWIZZLE), synchronises, then
 * LDS -> global. */
typedef struct tg_copy_opts {
  int32_t tile_rows;
  int32_t tile_cols;
  int32_t threads;   /* 1 .. 1024 */
  int32_t lds_kind;  /* TG_ROW_MAJOR or TG_XOR_SWIZZLE */
  int32_t flags;     /* must be 0 */
} tg_copy_opts;

/* One direction of a tile copy as the vec_auto partition [outer, threads,
 * vec]: round f of thread t moves the fused elements
 * [(f*threads + t)*vec, +vec) of the tile in the driving (global) side's order
 * ([VEC-AUTO] 算法核心 steps 1–2 and 生成的 TIRx IR). */
typedef struct tg_copy_phase {
  int32_t outer;     /* rounds per thread */
  int32_t threads;
  int32_t vec;       /* elements per vector transfer */
  int32_t vec_bits;  /* vec * element bits: 128, 64, 32, 16 or 8 */
} tg_copy_phase;

typedef struct tg_copy_plan {
  tg_copy_phase load;   /* global (src) -> LDS, driven by the src layout's order */
  tg_copy_phase store;  /* LDS -> global (dst), driven by the dst layout's order */
  int32_t tile_rows, tile_cols, lds_kind, lds_bytes;
  int64_t tiles;        /* number of tiles = workgroup-iterations */
} tg_copy_plan;

/* Kernel choice of tile_gemm, reported by tile_gemm_plan. */
typedef enum tg_gemm_kernel {
  TG_GEMM_NONE = 0,     /* nothing to launch (M == 0 or N == 0) */
  TG_GEMM_ATOM = 1,     /* register kernel: one wave per output tile of one matrix instruction
                           (tg_gemm_plan.atom; tile_gemm_atom_select says which) */
  TG_GEMM_TILED = 2,    /* LDS double-buffered kernel, v_mfma_f32_32x32x16 (fp8:
                           v_mfma_f32_32x32x64_f8f6f4) */
  TG_GEMM_FILL = 3      /* K == 0: D = beta*C without a product */
} tg_gemm_kernel;

typedef struct tg_gemm_plan {
  int32_t kernel;                 /* tg_gemm_kernel */
  int32_t block_m, block_n, block_k;
  int32_t wave_m, wave_n;         /* output tile of one wavefront */
  int32_t threads;                /* per workgroup */
  int32_t bounds_checked;         /* 1 when some tile is ragged (masked loads and stores) */
  int32_t lds_bytes;
  int64_t grid;                   /* workgroups */
  int32_t loader;                 /* 0: operands staged through VGPRs, 1: direct global -> LDS */
  int32_t atom;                   /* TG_GEMM_ATOM: the tg_mma_shape it runs (else 0) */
} tg_gemm_plan;

/*
 * tile_gemm — D = A·B + beta·C   ([SYNC-GEMM] 一, 二, 四 step 3).
 *
 *   A      device, dtype (TG_F16 or TG_BF16).  Stored row-major [M,K] when transA == 0,
 *          [K,M] when transA == 1.  Packed (leading dimension K or M).
 *   B      device, same dtype.  Stored row-major [K,N] when transB == 0, [N,K] when transB == 1.
 *   C      device fp32 [M,N] row-major packed; read only when beta == 1 (may be NULL when
 *          beta == 0).  C may be exactly D (in-place D += A·B); any other overlap with D is
 *          rejected.
 *   D      device fp32 [M,N] row-major packed; written.  Must not overlap A or B.
 *   M,N,K  M % 16 == 0, N % 8 == 0, K % 8 == 0, all >= 0 ([SYNC-GEMM] 二).  M == 0 or N == 0 is
 *          a no-op; K == 0 gives D = beta·C.
 *   transA, transB   0 or 1; they only describe the stored orientation, the product is
 *          always A[M,K]·B[K,N] ([SYNC-GEMM] 二 and 四 step 1).
 *   beta   exactly 0.0 (D = A·B, C never read) or 1.0 (D = A·B + C).  alpha is fixed at 1
 *          ([SYNC-GEMM] 二: alpha = 1.0, beta ∈ {0.0, 1.0}).
 *   dtype  TG_F16 or TG_BF16 for both A and B; C and D are fp32.  Products are formed
 *          exactly and accumulated in fp32 in place over K by MFMA.
 *   Alignment: A and B 16-byte aligned (128-bit loads), C and D 4-byte aligned; otherwise
 *          TG_E_ALIGN.
 * Returns TG_OK or a tg_status; asynchronous on `stream`.
 */
int tile_gemm(const void* A, const void* B, const float* C, float* D,
              int64_t M, int64_t N, int64_t K, int transA, int transB,
              float beta, int dtype, void* stream);

/*
 * tile_gemm_plan — host-only validation and kernel choice of tile_gemm for the same
 * arguments (pointers are only tested for NULL, alignment and overlap).  Returns what
 * tile_gemm would return before launching, and fills *out on TG_OK.  Needs no GPU.
 */
int tile_gemm_plan(const void* A, const void* B, const float* C, const float* D,
                   int64_t M, int64_t N, int64_t K, int transA, int transB,
                   float beta, int dtype, tg_gemm_plan* out);

/*
 * tile_gemm_fp8 — D = A·B + beta·C with 8-bit floating-point operands: the fp8 member of the
 * asynchronous GEMM's precision family ([SYNC-GEMM] 七: besides f16/bf16 it takes fp8 and
 * fp4 operands, with A and B staged in shared memory and the product accumulated in fp32).
 *
 *   A      device, OCP fp8 of format a_dtype, stored row-major [M,K] (transA == 0) or [K,M]
 *          (transA == 1).
 *   B      device, OCP fp8 of format b_dtype, stored row-major [K,N] (transB == 0) or [N,K]
 *          (transB == 1).  As for tile_gemm the flags only describe the stored orientation.
 *   C, D   as tile_gemm: fp32 [M,N] row-major packed, C read only when beta == 1, C may be
 *          exactly D, D must not overlap A or B.
 *   M,N,K  M % 16 == 0, N % 16 == 0, K % 128 == 0, all >= 0, and each operand under 2 GiB;
 *          otherwise TG_E_SHAPE.  M == 0 or N == 0 is a no-op; K == 0 gives D = beta·C.
 *   beta   exactly 0.0 or 1.0 (alpha is fixed at 1); otherwise TG_E_BETA.
 *   a_dtype, b_dtype   each TG_FP8_E4M3 (e4m3fn: bias 7, largest finite 448, no infinities,
 *          S.1111.111 is NaN) or TG_FP8_E5M2 (bias 15, IEEE-style infinities and NaNs); the
 *          two may differ.  Anything else -> TG_E_DTYPE.  Every product of two fp8 values is
 *          exact.  The matrix unit does not add them one by one in fp32: each aligned group
 *          of 8 consecutive K products is summed on a fixed-point grid of 2^-13 times the
 *          group's largest |product|, and the group sum is added to the fp32 accumulator.
 *          A product that lies within 2^6 of its group's largest is on that grid and kept
 *          exactly; one further below can lose its low bits (and one more than 2^13 below
 *          can be lost).  No block scales (the block-scaled mode is tile_gemm_mx).
 *   Alignment: A and B 16-byte aligned, C and D 4-byte aligned; otherwise TG_E_ALIGN.
 * Returns TG_OK or a tg_status; asynchronous on `stream`.
 */
int tile_gemm_fp8(const void* A, const void* B, const float* C, float* D,
                  int64_t M, int64_t N, int64_t K, int transA, int transB,
                  float beta, int a_dtype, int b_dtype, void* stream);

/* tile_gemm_fp8_plan — host-only validation and kernel choice of tile_gemm_fp8 (as
 * tile_gemm_plan).  Needs no GPU. */
int tile_gemm_fp8_plan(const void* A, const void* B, const float* C, const float* D,
                       int64_t M, int64_t N, int64_t K, int transA, int transB,
                       float beta, int a_dtype, int b_dtype, tg_gemm_plan* out);

/*
 * tile_gemm_mx — block-scaled fp8 GEMM: the block-scaled mode of the asynchronous GEMM
 * ([SYNC-GEMM] 七: scale factors SFA for A and SFB for B), in the OCP microscaling form:
 *
 *   D[m][n] = sum_k (SA[m][k/32]·A[m][k]) · (SB[n][k/32]·B[k][n])  + beta·C[m][n]
 *
 *   A, B, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype, stream: as tile_gemm_fp8.
 *   SA     device, E8M0 scale bytes of A, [M][K/32] row-major whatever A's orientation: byte
 *          SA[m][kb] scales A[m][32kb .. 32kb+31] by 2^(SA[m][kb] - 127).  255 is NaN.
 *   SB     device, E8M0 scale bytes of B, [N][K/32] row-major: SB[n][kb] scales B[32kb ..][n].
 *          SA and SB are read only when K > 0; they must then be non-NULL (TG_E_NULL), 4-byte
 *          aligned (TG_E_ALIGN) and must not overlap D (TG_E_ALIAS).
 *   The scales are applied by the matrix unit per 32-K block (exact: powers of two); the
 *   scaled products are summed in aligned groups of 8 on the grid tile_gemm_fp8 describes, and
 *   the group sums accumulated in fp32.
 *
 *   6- and 4-bit operands ([SYNC-GEMM] 七 names fp4 among the operand precisions):
 *   a_dtype and b_dtype each TG_FP6_E2M3, TG_FP6_E3M2 or TG_FP4_E2M1 (any pair of the three;
 *   a mix with an fp8 operand is TG_E_DTYPE).  The OCP microscaling element types: sign,
 *   exponent and fraction fields of 1+2+3, 1+3+2 and 1+2+1 bits, biases 1, 3 and 1, subnormals
 *   at a zero exponent field, no infinities or NaNs.  Both operands are stored K-contiguous as
 *   packed rows — A [M][K·w/8] bytes (transA == 0) and B [N][K·w/8] bytes (transB == 1), w the
 *   operand's bits — with code k of a row at bits [w·k, w·k + w) of that row's little-endian bit
 *   stream (fp4: two codes per byte, the even one in the low nibble; fp6: four codes in every
 *   three bytes).  Any other orientation is TG_E_LAYOUT.  Shapes, scales, C, D, beta and
 *   alignment as above; each packed operand under 2 GiB.  The direct-load kernel
 *   (tile_gemm_mx_plan reports loader 1) runs e2m1 x e2m1 with K % 256 == 0 (block_k 256: 256 K
 *   per 128-byte stage row) and every pair of 6-bit operands (block_k 128: 96 bytes of each
 *   128-byte stage row); an e2m1 operand with a 6-bit one, or e2m1 x e2m1 with K % 256 != 0,
 *   runs the packed kernel (loader 0, 128-K stages).
 * Returns TG_OK or a tg_status; asynchronous on `stream`.
 */
int tile_gemm_mx(const void* A, const void* B, const uint8_t* SA, const uint8_t* SB,
                 const float* C, float* D, int64_t M, int64_t N, int64_t K, int transA,
                 int transB, float beta, int a_dtype, int b_dtype, void* stream);

/* tile_gemm_mx_plan — host-only validation and kernel choice of tile_gemm_mx.  Needs no GPU. */
int tile_gemm_mx_plan(const void* A, const void* B, const uint8_t* SA, const uint8_t* SB,
                      const float* C, const float* D, int64_t M, int64_t N, int64_t K,
                      int transA, int transB, float beta, int a_dtype, int b_dtype,
                      tg_gemm_plan* out);

/*
 * tile_copy — bit-exact copy of a shape[0] x shape[1] matrix from src to dst, staged
 * global -> LDS -> global by workgroups with the default options below
 * ([VEC-AUTO]: copy is a synchronous element copy; the gmem_smem path).
 *
 *   src, dst    device buffers of dtype elements; dst must not overlap src.
 *   shape       {rows, cols}, both >= 0; an empty shape is a no-op.
 *   dtype       any tg_dtype (moved as bits; both sides have the same dtype).
 *   src_layout, dst_layout   TG_ROW_MAJOR or TG_COL_MAJOR with ld (0 = packed); a global side
 *               may be TG_XOR_SWIZZLE only when the whole matrix is one tile (it then
 *               exposes the LDS image: the tile written in LDS physical order).
 * Default options: tile_cols = min(cols, 128 bytes / element size), tile_rows =
 * min(rows, 128); threads = 256 when the tile holds a multiple of 256 elements, else 64,
 * else the largest power of two dividing the tile's elements; lds_kind = TG_XOR_SWIZZLE
 * when the tile's rows are a power-of-two number of 16-byte chunks, else TG_ROW_MAJOR.
 * The vector width of each direction is the widest of 128/64/32/16/8 bits that keeps every
 * transfer contiguous and aligned on both of its sides, for every tile ([VEC-AUTO] 算法核心
 * step 2; 对齐约束的兜底: misalignment narrows the width, down to one element).
 * Rejections: the thread count must divide the tile's elements ([VEC-AUTO] 接受什么输入,
 * _divides_thread_cnt) -> TG_E_THREADS; the tensor must be a whole number of tiles ->
 * TG_E_SHAPE.
 */
int tile_copy(const void* src, void* dst, const int64_t shape[2], int dtype,
              const tg_layout* src_layout, const tg_layout* dst_layout, void* stream);

/* tile_copy_ex — tile_copy with explicit staging options (opts != NULL): the tile and the
 * thread count that run one tile, as the demo programs fix them ([VEC-AUTO] 演示程序: one
 * 32x32 tile moved by one group of threads).  Rejections as tile_copy; opts->threads outside
 * 1 .. 1024 or not dividing the tile's elements -> TG_E_THREADS ([VEC-AUTO] 接受什么输入). */
int tile_copy_ex(const void* src, void* dst, const int64_t shape[2], int dtype,
                 const tg_layout* src_layout, const tg_layout* dst_layout,
                 const tg_copy_opts* opts, void* stream);

/*
 * tile_copy_plan — host-only: the plan tile_copy_ex would run (opts may be NULL for the
 * defaults), for the whole tiled tensor: each direction's [outer, threads, vec] partition is
 * the one that every tile accepts.  src and dst are used only for their alignment.  Returns
 * the same status, and the same readable reason, the copy would return before launching
 * ([VEC-AUTO] 接受什么输入: a rejected copy names its reason instead of running masked).
 * Needs no GPU.  The plan of ONE region from (shape, element width, threads, the two layouts
 * and their base addresses) to (outer, vec) is tile_copy_partition below.
 */
int tile_copy_plan(const void* src, const void* dst, const int64_t shape[2], int dtype,
                   const tg_layout* src_layout, const tg_layout* dst_layout,
                   const tg_copy_opts* opts, tg_copy_plan* out);

/*
 * tile_copy_partition — host-only: the vec_auto partition of ONE rows x cols region copied
 * between a driving (global) side and another side ([VEC-AUTO] 接受什么输入 and 算法核心
 * steps 1–2).  Bases are element offsets of the region's first element on each side
 * (pointer address / element size plus region offset).  threads <= 0 or not dividing
 * rows*cols -> TG_E_THREADS.  elem_bits is 8, 16, 32 or 64.  Needs no GPU.
 */
int tile_copy_partition(int64_t rows, int64_t cols, int elem_bits, int threads,
                        const tg_layout* drive, int64_t drive_base,
                        const tg_layout* other, int64_t other_base,
                        tg_copy_phase* out);

/* ---------------------------------------------------------------------------------------
 * Asynchronous tile copy ([TCGEN05-CP] 一个算子、六个变体 and 与其他异步变体的协作关系: every
 * copy_async variant, the per-thread vectorised global -> shared one among them, only issues the
 * transfer, and the code that issued it owns the completion, waiting when it needs the data).
 * On gfx950 the issue is buffer_load_dwordx4 ... lds / buffer_load_dword ... lds (the buffer
 * form of the direct-to-LDS load): each lane's chunk goes from HBM straight to LDS without
 * passing through registers, and completion is the issuing wave's own s_waitcnt vmcnt
 * followed by a workgroup barrier.
 * ------------------------------------------------------------------------------------- */
typedef struct tg_async_opts {
  int32_t tile_rows, tile_cols;  /* one LDS stage holds one tile (at most 16 KiB) */
  int32_t threads;               /* 64 .. 1024, a multiple of 64 (a wave issues together) */
  int32_t lds_kind;              /* TG_ROW_MAJOR or TG_XOR_SWIZZLE */
  int32_t depth;                 /* LDS stages, i.e. tiles in flight per workgroup: 1 .. 4 */
  int32_t tiles_per_workgroup;   /* consecutive tiles a workgroup streams: 1 .. 64, or 0 for the
                                    default (up to 4, keeping 2048 workgroups or more) */
  int32_t flags;                 /* must be 0 */
} tg_async_opts;

typedef struct tg_async_plan {
  tg_copy_plan copy;             /* load = the issue-only DMA partition, store = LDS -> dst;
                                    lds_bytes = depth stages */
  int32_t depth;
  int32_t tiles_per_workgroup;   /* consecutive tiles one workgroup streams through its stages */
  int64_t grid;                  /* workgroups */
} tg_async_plan;

/*
 * tile_copy_async — bit-exact copy of a shape[0] x shape[1] matrix like tile_copy_ex, with the
 * global -> LDS half issued asynchronously: each workgroup keeps `depth` tiles in flight, and
 * before it reads a tile from LDS it waits only until that tile's own transfers have landed
 * (the newer ones stay in flight), then synchronises the workgroup.
 *
 *   src, dst, shape, dtype   as tile_copy.
 *   src_layout   TG_ROW_MAJOR (any ld).  dst_layout   TG_ROW_MAJOR (any ld), or TG_XOR_SWIZZLE for
 *                a one-tile tensor (the LDS image of the tile).  Other layouts: TG_E_LAYOUT.
 *   opts         required (see tg_async_opts).
 * The partition is that of tile_copy: round f of thread t moves chunk f·threads + t of the
 * tile, in the tile's row-major order.  With an XOR-swizzled LDS tile, a lane's LDS slot is
 * fixed by the transfer (lane i of a wave writes 16 or 4 bytes at the wave's base + i·size), so
 * the lane fetches the chunk whose swizzled position is that slot: the chunks of each tile row
 * are assigned to threads in swizzled order.  Transfers are 128 or 32 bits (the widths the
 * hardware's global -> LDS loads have): the width is the widest of those that the width rule
 * accepts on both sides; a copy whose rows admit neither is rejected (TG_E_ALIGN).  Rounds per
 * thread must be 1, 2, 4 or 8 (TG_E_THREADS otherwise), a tile at most 16 KiB (TG_E_SHAPE).
 */
int tile_copy_async(const void* src, void* dst, const int64_t shape[2], int dtype,
                    const tg_layout* src_layout, const tg_layout* dst_layout,
                    const tg_async_opts* opts, void* stream);

/* tile_copy_async_plan — host-only: the plan tile_copy_async would run, with the same status.
 * Needs no GPU. */
int tile_copy_async_plan(const void* src, const void* dst, const int64_t shape[2], int dtype,
                         const tg_layout* src_layout, const tg_layout* dst_layout,
                         const tg_async_opts* opts, tg_async_plan* out);

/* ---------------------------------------------------------------------------------------
 * Register fragments ([SYNC-GEMM] 一 and 四: the register-level gemm takes its A / B fragments
 * and its C / D accumulator in registers, which the caller fills first — typically by a copy
 * of the ldstmatrix kind; [VEC-AUTO] closing reading list: vec_auto's register path, whose
 * partition comes from the register layout's thread axis, and the warp-collective ldstmatrix
 * copy).  On gfx950 those registers are the operands and accumulator of the matrix
 * instructions.  A fragment kind is a tile_rows x tile_cols tile and the map
 * (lane l < 64, register element e < elems) -> (row, col) of the tile below.
 *
 * A register image holds what the wavefront's registers hold: for each tile, in row-major
 * tile order over the matrix, 64 lanes x elems elements, each lane's elements contiguous in
 * register order (tile t, lane l, element e at (t*64 + l)*elems + e).  Every lane's
 * registers are groups of 16 bytes (8 bytes for the K = 8 / 16 atoms) that run along one axis
 * of the tile (a "run").
 * ------------------------------------------------------------------------------------- */
typedef enum tg_frag_kind {
  TG_FRAG_A16_32x32x16 = 1,  /* 32 x 16, 16-bit, 8 per lane: (l%32, 8(l/32) + e)        */
  TG_FRAG_B16_32x32x16 = 2,  /* 16 x 32, 16-bit, 8 per lane: (8(l/32) + e, l%32)        */
  TG_FRAG_A16_16x16x32 = 3,  /* 16 x 32, 16-bit, 8 per lane: (l%16, 8(l/16) + e)        */
  TG_FRAG_B16_16x16x32 = 4,  /* 32 x 16, 16-bit, 8 per lane: (8(l/16) + e, l%16)        */
  TG_FRAG_A8_32x32x64 = 5,   /* 32 x 64, 8-bit, 32 per lane: (l%32, 32(e/16) + 16(l/32) + e%16) */
  TG_FRAG_B8_32x32x64 = 6,   /* 64 x 32, 8-bit, 32 per lane: (32(e/16) + 16(l/32) + e%16, l%32) */
  TG_FRAG_C32_32x32 = 7,     /* 32 x 32 fp32 accumulator, 16 per lane: (8(e/4) + 4(l/32) + e%4, l%32) */
  TG_FRAG_C32_16x16 = 8,     /* 16 x 16 fp32 accumulator, 4 per lane: (4(l/16) + e, l%16) */
  TG_FRAG_A16_32x32x8 = 9,   /* 32 x 8, 16-bit, 4 per lane: (l%32, 4(l/32) + e)          */
  TG_FRAG_B16_32x32x8 = 10,  /* 8 x 32, 16-bit, 4 per lane: (4(l/32) + e, l%32)          */
  TG_FRAG_A16_16x16x16 = 11, /* 16 x 16, 16-bit, 4 per lane: (l%16, 4(l/16) + e)         */
  TG_FRAG_B16_16x16x16 = 12  /* 16 x 16, 16-bit, 4 per lane: (4(l/16) + e, l%16)         */
} tg_frag_kind;

typedef enum tg_frag_route {
  TG_FRAG_AUTO = 0,    /* LDS when the memory lines are 16-byte aligned, else DIRECT */
  TG_FRAG_DIRECT = 1,  /* global <-> registers; the width rule on the registers' runs */
  TG_FRAG_LDS = 2      /* global <-> LDS with 128-bit transfers, LDS <-> registers with
                          ds_read_b128 / ds_write_b128 along memory lines, and
                          ds_read_b64_tr_b16 / ds_read_b64_tr_b8 across them */
} tg_frag_route;

typedef struct tg_frag_plan {
  int32_t route;           /* TG_FRAG_DIRECT or TG_FRAG_LDS */
  int32_t vec;             /* elements per global transfer */
  int32_t vec_bits;        /* vec * element bits: 128, 64, 32, 16 or 8 */
  int32_t transposed;      /* 1 when each run crosses memory lines */
  int32_t tile_rows, tile_cols, elems, elem_bits;
  int32_t threads;         /* per workgroup */
  int32_t lds_bytes;       /* per workgroup (0 on the direct route) */
  int64_t tiles;
  int64_t grid;            /* workgroups */
} tg_frag_plan;

/*
 * tile_frag_load — fill a register image from a matrix (the ldstmatrix direction: memory ->
 * registers), then write the registers to `image`.  Bit-exact.
 *
 *   src     device, shape[0] x shape[1] elements of dtype laid out as src_layout
 *           (TG_ROW_MAJOR or TG_COL_MAJOR, ld 0 = packed); element aligned.
 *   image   device, shape[0]*shape[1] elements, 16-byte aligned; must not overlap src.
 *   shape   whole tiles of the kind: rows % tile_rows == 0, cols % tile_cols == 0 (else
 *           TG_E_SHAPE); an empty shape is a no-op.
 *   dtype   of the kind's width: 16-bit kinds TG_F16 / TG_BF16, 8-bit kinds TG_U8 / TG_I8 /
 *           TG_FP8_E4M3 / TG_FP8_E5M2, accumulator kinds TG_F32 (else TG_E_DTYPE).
 *   kind    tg_frag_kind; route   tg_frag_route (else TG_E_ARG).
 * The direct route moves each run with the widest of 128/64/32/16/8-bit transfers that keep
 * every transfer of every lane contiguous and aligned ([VEC-AUTO] 算法核心 step 2, the register
 * layout as the driving side): 128-bit along memory lines when lines and base are 16-byte
 * aligned, one element at a time when the run crosses lines.  TG_FRAG_LDS needs 16-byte
 * aligned memory lines (base and ld*element size), else TG_E_ALIGN.
 */
int tile_frag_load(const void* src, void* image, const int64_t shape[2], int dtype,
                   const tg_layout* src_layout, int kind, int route, void* stream);

/*
 * tile_frag_store — write a register image back to a matrix (registers -> memory): each lane
 * first loads its own registers from `image`, then the fragments are stored through the route.
 * Arguments as tile_frag_load with the roles of the buffers exchanged; elements of dst outside
 * the matrix (the gaps of ld) are not written.
 */
int tile_frag_store(const void* image, void* dst, const int64_t shape[2], int dtype,
                    const tg_layout* dst_layout, int kind, int route, void* stream);

/*
 * tile_frag_plan — host-only: the plan tile_frag_load (store == 0) or tile_frag_store
 * (store == 1) would run, with the same status.  mem and image are used for their alignment
 * only.  Needs no GPU.
 */
int tile_frag_plan(int store, const void* mem, const void* image, const int64_t shape[2],
                   int dtype, const tg_layout* layout, int kind, int route, tg_frag_plan* out);

/* Matrix-instruction shapes of tile_frag_mma: the A, B and accumulator kinds they use. */
typedef enum tg_mma_shape {
  TG_MMA_32x32x16 = 1,     /* v_mfma_f32_32x32x16_{f16,bf16}: A16_32x32x16, B16_32x32x16, C32_32x32 */
  TG_MMA_16x16x32 = 2,     /* v_mfma_f32_16x16x32_{f16,bf16}: A16_16x16x32, B16_16x16x32, C32_16x16 */
  TG_MMA_32x32x64_F8 = 3,  /* v_mfma_f32_32x32x64_f8f6f4 (fp8): A8_32x32x64, B8_32x32x64, C32_32x32 */
  TG_MMA_32x32x8 = 4,      /* v_mfma_f32_32x32x8_{f16,bf16}: A16_32x32x8, B16_32x32x8, C32_32x32 */
  TG_MMA_16x16x16 = 5      /* v_mfma_f32_16x16x16_{f16,bf16}: A16_16x16x16, B16_16x16x16, C32_16x16 */
} tg_mma_shape;

/*
 * tile_mma_select — host-only: the widest matrix-instruction shape whose atom divides
 * (M, N, K) exactly, for the operand formats ([TCGEN05-CP] 形状选择: candidates from the widest
 * down, the first that fits wins; [SYNC-GEMM] 二: the k16 atom when K allows, else k8).  Width is
 * the multiply-adds of one instruction; 16-bit candidates in order 32x32x16, 16x16x32, 32x32x8,
 * 16x16x16; fp8: 32x32x64.  *shape receives the choice.  Returns TG_E_SHAPE when no atom
 * divides the problem (the caller then pads), TG_E_DTYPE for formats no shape takes, TG_E_ARG
 * for a NULL shape or negative extents.  Needs no GPU.
 */
int tile_mma_select(int64_t M, int64_t N, int64_t K, int a_dtype, int b_dtype, int* shape);

/*
 * tile_frag_mma — the register-level gemm over register images ([SYNC-GEMM] 一 and 四 step 3):
 * D = A·B (+ C) where each output tile runs one matrix instruction per K atom, accumulating
 * in place.
 *
 *   a_image  device, A [M, K] as a register image of the shape's A kind (16-byte aligned).
 *   b_image  device, B [K, N] as an image of the B kind.
 *   c_image  device fp32, C [M, N] as an image of the accumulator kind; read only when
 *            beta == 1 (may be NULL when beta == 0); may be exactly d_image.
 *   d_image  device fp32, D [M, N] as an image of the accumulator kind; written; must not
 *            overlap a_image or b_image.
 *   M, N, K  whole atoms of the shape (32x32x16: M%32, N%32, K%16; 16x16x32: M%16, N%16,
 *            K%32; 32x32x64: M%32, N%32, K%64; 32x32x8: M%32, N%32, K%8; 16x16x16: M%16, N%16,
 *            K%16), else TG_E_SHAPE; M == 0 or N == 0 is a no-op,
 *            K == 0 gives D = beta·C.
 *   beta     exactly 0.0 or 1.0 (alpha is 1), else TG_E_BETA.
 *   a_dtype, b_dtype  TG_F16 or TG_BF16 (equal) for the 16-bit shapes; TG_FP8_E4M3 or
 *            TG_FP8_E5M2 (each) for the fp8 shape; else TG_E_DTYPE.
 *   shape    tg_mma_shape, else TG_E_ARG.
 * Products are exact.  The 16-bit shapes accumulate them in fp32; the fp8 shape sums them in
 * aligned groups of 8 on the grid tile_gemm_fp8 describes before the fp32 accumulation.
 */
int tile_frag_mma(const void* a_image, const void* b_image, const float* c_image, float* d_image,
                  int64_t M, int64_t N, int64_t K, float beta, int a_dtype, int b_dtype,
                  int shape, void* stream);

/*
 * tile_gemm_atom_select — host-only: the matrix instruction tile_gemm's register kernel runs for
 * a problem (tile_gemm takes that kernel when M·N <= 4096).  [TCGEN05-CP] 形状选择 tries the
 * candidate shapes from the widest down against the operands' layouts; [SYNC-GEMM] 二 takes the
 * k16 atom when K allows it and the k8 atom otherwise.  Here the candidates are 32x32x16,
 * 16x16x32, 32x32x8 and 16x16x16 (widest first); one is admissible when its K depth divides K
 * (K is never padded); M and N are padded up to it (MFMA has no 8-wide N; padded rows and
 * columns are zero and never stored).  The admissible shape with the least work after padding
 * wins; ties go to the fewest global loads per multiply-add for the stored layouts (a lane's
 * run of K values is one vector load from a K-contiguous operand — A with transA == 0, B with
 * transB == 1 — and one load per value otherwise), then to the wider shape.  16x8x16 takes
 * 16x16x16; K = 8 or 24 takes 32x32x8.
 *   M, N, K  > 0 and K % 8 == 0 (else TG_E_SHAPE); dtype TG_F16 or TG_BF16 (else TG_E_DTYPE);
 *   transA, transB 0 or 1 (else TG_E_ARG); *shape receives a tg_mma_shape (NULL: TG_E_ARG).
 * Needs no GPU.
 */
int tile_gemm_atom_select(int64_t M, int64_t N, int64_t K, int dtype, int transA, int transB,
                          int* shape);

/* Reason for the last failure on the calling thread ("" after a success): the readable
 * reason a call was refused, as the dispatcher reports why no variant accepts a call
 * ([SYNC-GEMM] 二, the failure reasons of the dispatch; [VEC-AUTO] 接受什么输入).  The
 * string stays valid until the next call on the same thread. */
const char* tile_last_error(void);

/* Library ABI version (this header: 7; 2 added tile_gemm_fp8 and tile_gemm_fp8_plan, 3 added
 * tile_gemm_mx and tile_gemm_mx_plan, 4 the register fragment calls tile_frag_*, 5
 * tile_copy_async and tile_copy_async_plan, 6 the K = 8 / 16 atoms and tile_mma_select, 7
 * tile_gemm_atom_select and tg_gemm_plan.atom). */
int tile_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TILEGEMM_H */
