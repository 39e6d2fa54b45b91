// C-ABI entry points: argument validation, planning and launch.
//
// Validation follows [SYNC-GEMM] 二 ("What it accepts": M%16, N%8, K%8; A and B
// both f16 or both bf16; C and D fp32; alpha = 1; beta in {0, 1}; transposes
// normalised to A[M,K], B[K,N]) and [VEC-AUTO] 接受什么输入 (the copy's element
// count must divide over its threads; equal dtype on both sides).  Every check
// runs before any HIP call, so a rejected call writes nothing and the host-only
// entry points need no GPU.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>

#include "tg_internal.h"

namespace tg {

static thread_local std::string g_last_error;

int fail(int code, const std::string& why) {
  g_last_error = why;
  return code;
}

void clear_error() { g_last_error.clear(); }

}  // namespace tg

using namespace tg;

namespace {

const int64_t kMaxDim = (int64_t)1 << 30;
const int64_t kMaxLd = (int64_t)1 << 40;   // keeps every element offset far inside int64

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

std::string fmt(const char* f, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c);
  return buf;
}

int validate_gemm(const void* A, const void* B, const float* C, const float* D, int64_t M,
                  int64_t N, int64_t K, int transA, int transB, float beta, int dtype) {
  if (M < 0 || N < 0 || K < 0)
    return fail(TG_E_SHAPE, fmt("negative extent (M=%lld, N=%lld, K=%lld)", M, N, K));
  if (M % 16 || N % 8 || K % 8)
    return fail(TG_E_SHAPE,
                fmt("gemm needs M %% 16 == 0, N %% 8 == 0, K %% 8 == 0 (got M=%lld, N=%lld, K=%lld)",
                    M, N, K));
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(TG_E_SHAPE, "extent above 2^30");
  if (dtype != TG_F16 && dtype != TG_BF16)
    return fail(TG_E_DTYPE, fmt("gemm operands must be TG_F16 or TG_BF16 (got dtype %lld); C and D "
                                "are fp32", dtype));
  if (transA != 0 && transA != 1) return fail(TG_E_ARG, "transA must be 0 or 1");
  if (transB != 0 && transB != 1) return fail(TG_E_ARG, "transB must be 0 or 1");
  if (!(beta == 0.0f || beta == 1.0f))
    return fail(TG_E_BETA, "beta must be exactly 0.0 or 1.0 (alpha is fixed at 1)");
  if (M == 0 || N == 0) return TG_OK;
  if (!D) return fail(TG_E_NULL, "D is NULL");
  if (beta == 1.0f && !C) return fail(TG_E_NULL, "beta == 1 needs C");
  if (K > 0 && (!A || !B)) return fail(TG_E_NULL, "A or B is NULL");
  const int64_t dbytes = M * N * 4;
  if (K > 0) {
    if (overlaps(D, dbytes, A, M * K * 2) || overlaps(D, dbytes, B, K * N * 2))
      return fail(TG_E_ALIAS, "D overlaps A or B");
    if ((uintptr_t)A % 16 || (uintptr_t)B % 16)
      return fail(TG_E_ALIGN, "A and B must be 16-byte aligned for 128-bit operand loads");
  }
  if (beta == 1.0f && C != D && overlaps(D, dbytes, C, dbytes))
    return fail(TG_E_ALIAS, "C overlaps D without being exactly D");
  if ((uintptr_t)D % 4 || (beta == 1.0f && (uintptr_t)C % 4))
    return fail(TG_E_ALIGN, "C and D must be 4-byte aligned");
  return TG_OK;
}

bool is_fp8(int dtype) { return dtype == TG_FP8_E4M3 || dtype == TG_FP8_E5M2; }

// tile_gemm_fp8 ([SYNC-GEMM] 七, the fp8 operands of the asynchronous GEMM): same checks
// and order as validate_gemm, with the fp8 shape rule (M % 16, N % 16, K % 128), the fp8
// formats and one-byte operand elements.
int validate_gemm_fp8(const void* A, const void* B, const float* C, const float* D, int64_t M,
                      int64_t N, int64_t K, int transA, int transB, float beta, int a_dtype,
                      int b_dtype) {
  if (M < 0 || N < 0 || K < 0)
    return fail(TG_E_SHAPE, fmt("negative extent (M=%lld, N=%lld, K=%lld)", M, N, K));
  if (M % 16 || N % 16 || K % 128)
    return fail(TG_E_SHAPE,
                fmt("fp8 gemm needs M %% 16 == 0, N %% 16 == 0, K %% 128 == 0 (got M=%lld, N=%lld, "
                    "K=%lld)", M, N, K));
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(TG_E_SHAPE, "extent above 2^30");
  if (M * K >= ((int64_t)1 << 31) || N * K >= ((int64_t)1 << 31))
    return fail(TG_E_SHAPE, "fp8 gemm needs each operand under 2 GiB (32-bit buffer offsets)");
  if (!is_fp8(a_dtype) || !is_fp8(b_dtype))
    return fail(TG_E_DTYPE, fmt("fp8 gemm operands must be TG_FP8_E4M3 or TG_FP8_E5M2 (got a_dtype "
                                "%lld, b_dtype %lld); C and D are fp32", a_dtype, b_dtype));
  if (transA != 0 && transA != 1) return fail(TG_E_ARG, "transA must be 0 or 1");
  if (transB != 0 && transB != 1) return fail(TG_E_ARG, "transB must be 0 or 1");
  if (!(beta == 0.0f || beta == 1.0f))
    return fail(TG_E_BETA, "beta must be exactly 0.0 or 1.0 (alpha is fixed at 1)");
  if (M == 0 || N == 0) return TG_OK;
  if (!D) return fail(TG_E_NULL, "D is NULL");
  if (beta == 1.0f && !C) return fail(TG_E_NULL, "beta == 1 needs C");
  if (K > 0 && (!A || !B)) return fail(TG_E_NULL, "A or B is NULL");
  const int64_t dbytes = M * N * 4;
  if (K > 0) {
    if (overlaps(D, dbytes, A, M * K) || overlaps(D, dbytes, B, K * N))
      return fail(TG_E_ALIAS, "D overlaps A or B");
    if ((uintptr_t)A % 16 || (uintptr_t)B % 16)
      return fail(TG_E_ALIGN, "A and B must be 16-byte aligned for 128-bit operand loads");
  }
  if (beta == 1.0f && C != D && overlaps(D, dbytes, C, dbytes))
    return fail(TG_E_ALIAS, "C overlaps D without being exactly D");
  if ((uintptr_t)D % 4 || (beta == 1.0f && (uintptr_t)C % 4))
    return fail(TG_E_ALIGN, "C and D must be 4-byte aligned");
  return TG_OK;
}

bool is_packed(int d) { return d == TG_FP6_E2M3 || d == TG_FP6_E3M2 || d == TG_FP4_E2M1; }
int packed_bits(int d) { return d == TG_FP4_E2M1 ? 4 : 6; }
// MFMA format code of a packed operand (2 = e2m3, 3 = e3m2, 4 = e2m1)
int packed_fmt(int d) { return d == TG_FP6_E2M3 ? 2 : d == TG_FP6_E3M2 ? 3 : 4; }

// 6- and 4-bit operands: both packed, stored K-contiguous (A [M][K·w/8], B [N][K·w/8]), the fp8
// shape rules, each packed operand under 2 GiB.
int validate_gemm_packed(const void* A, const void* B, const float* C, const float* D, int64_t M,
                         int64_t N, int64_t K, int transA, int transB, float beta, int a_dtype,
                         int b_dtype) {
  if (M < 0 || N < 0 || K < 0)
    return fail(TG_E_SHAPE, fmt("negative extent (M=%lld, N=%lld, K=%lld)", M, N, K));
  if (M % 16 || N % 16 || K % 128)
    return fail(TG_E_SHAPE,
                fmt("block-scaled gemm needs M %% 16 == 0, N %% 16 == 0, K %% 128 == 0 (got M=%lld, "
                    "N=%lld, K=%lld)", M, N, K));
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(TG_E_SHAPE, "extent above 2^30");
  if (!is_packed(a_dtype) || !is_packed(b_dtype))
    return fail(TG_E_DTYPE, fmt("6- and 4-bit operands pair only with each other (got a_dtype %lld, "
                                "b_dtype %lld)", a_dtype, b_dtype));
  const int64_t abytes = M * K * packed_bits(a_dtype) / 8, bbytes = N * K * packed_bits(b_dtype) / 8;
  if (abytes >= ((int64_t)1 << 31) || bbytes >= ((int64_t)1 << 31))
    return fail(TG_E_SHAPE, "each packed operand must be under 2 GiB");
  if (transA != 0 && transA != 1) return fail(TG_E_ARG, "transA must be 0 or 1");
  if (transB != 0 && transB != 1) return fail(TG_E_ARG, "transB must be 0 or 1");
  if (transA != 0 || transB != 1)
    return fail(TG_E_LAYOUT, "6- and 4-bit operands are packed along K: A stored [M][K] (transA = 0) "
                             "and B stored [N][K] (transB = 1)");
  if (!(beta == 0.0f || beta == 1.0f))
    return fail(TG_E_BETA, "beta must be exactly 0.0 or 1.0 (alpha is fixed at 1)");
  if (M == 0 || N == 0) return TG_OK;
  if (!D) return fail(TG_E_NULL, "D is NULL");
  if (beta == 1.0f && !C) return fail(TG_E_NULL, "beta == 1 needs C");
  if (K > 0 && (!A || !B)) return fail(TG_E_NULL, "A or B is NULL");
  const int64_t dbytes = M * N * 4;
  if (K > 0) {
    if (overlaps(D, dbytes, A, abytes) || overlaps(D, dbytes, B, bbytes))
      return fail(TG_E_ALIAS, "D overlaps A or B");
    if ((uintptr_t)A % 16 || (uintptr_t)B % 16)
      return fail(TG_E_ALIGN, "A and B must be 16-byte aligned for 128-bit operand loads");
  }
  if (beta == 1.0f && C != D && overlaps(D, dbytes, C, dbytes))
    return fail(TG_E_ALIAS, "C overlaps D without being exactly D");
  if ((uintptr_t)D % 4 || (beta == 1.0f && (uintptr_t)C % 4))
    return fail(TG_E_ALIGN, "C and D must be 4-byte aligned");
  return TG_OK;
}

// tile_gemm_mx: the fp8 (or packed 6- / 4-bit) checks plus the block scales SA [M][K/32] and
// SB [N][K/32] (present when K > 0, 4-byte aligned for the 4-byte scale loads, not overlapping D).
int validate_gemm_mx(const void* A, const void* B, const uint8_t* SA, const uint8_t* SB,
                     const float* C, const float* D, int64_t M, int64_t N, int64_t K, int transA,
                     int transB, float beta, int a_dtype, int b_dtype) {
  int st = (is_packed(a_dtype) || is_packed(b_dtype))
               ? validate_gemm_packed(A, B, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype)
               : validate_gemm_fp8(A, B, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype);
  if (st || M == 0 || N == 0 || K == 0) return st;
  if (!SA || !SB) return fail(TG_E_NULL, "SA or SB is NULL");
  if ((uintptr_t)SA % 4 || (uintptr_t)SB % 4)
    return fail(TG_E_ALIGN, "SA and SB must be 4-byte aligned");
  const int64_t dbytes = M * N * 4;
  if (overlaps(D, dbytes, SA, M * (K / 32)) || overlaps(D, dbytes, SB, N * (K / 32)))
    return fail(TG_E_ALIAS, "D overlaps SA or SB");
  return TG_OK;
}

// 6- / 4-bit block-scaled GEMM.  The direct-load kernel (DMA into LDS, block size as for fp8)
// takes e2m1 x e2m1 with K a multiple of 256 (256-K stages of 128-byte rows) and every pair of
// 6-bit operands (128-K stages of 96-byte rows).  The packed kernel takes the rest (a 6-bit
// operand with an e2m1 one, e2m1 with K % 256 != 0), 128-K stages: 256x256 blocks of 512
// threads (8 waves of 128x64) when there are at least 256 of them (as for the 16-bit kernel),
// else 128x128 blocks of 256 threads (4 waves of 64x64).
GemmConfig choose_gemm_packed(int64_t M, int64_t N, int64_t K, int a_dtype, int b_dtype) {
  GemmConfig c{};
  if (M == 0 || N == 0) {
    c.kernel = TG_GEMM_NONE;
    return c;
  }
  if (K == 0) {
    c.kernel = TG_GEMM_FILL;
    c.threads = 256;
    c.grid = std::min<int64_t>((M * N + 1023) / 1024, 65536);
    return c;
  }
  auto blocks = [&](int64_t b) { return ((M + b - 1) / b) * ((N + b - 1) / b); };
  if (a_dtype == TG_FP4_E2M1 && b_dtype == TG_FP4_E2M1 && K % 256 == 0) {
    c = choose_gemm_fp8(M, N, K, true);
    c.bk = 256;
    return c;
  }
  if (a_dtype != TG_FP4_E2M1 && b_dtype != TG_FP4_E2M1) return choose_gemm_fp8(M, N, K, true);
  const int bs = blocks(256) >= 256 ? 256 : 128;
  c.kernel = TG_GEMM_TILED;
  c.bm = c.bn = bs;
  c.bk = 128;
  c.wm = bs / 2;
  c.wn = 64;
  c.threads = bs == 256 ? 512 : 256;
  c.bounds = (M % bs) != 0 || (N % bs) != 0;
  c.lds_bytes = packed_lds_bytes(packed_fmt(a_dtype), packed_fmt(b_dtype), bs);
  c.grid = blocks(bs);
  c.direct = 0;
  return c;
}

void fill_plan(const GemmConfig& c, tg_gemm_plan* out) {
  out->kernel = c.kernel;
  out->block_m = c.bm;
  out->block_n = c.bn;
  out->block_k = c.bk;
  out->wave_m = c.wm;
  out->wave_n = c.wn;
  out->threads = c.threads;
  out->bounds_checked = c.bounds;
  out->lds_bytes = c.lds_bytes;
  out->grid = c.grid;
  out->loader = c.direct;
  out->atom = c.kernel == TG_GEMM_ATOM ? c.atom : 0;
}

bool valid_kind(int k) { return k == TG_ROW_MAJOR || k == TG_COL_MAJOR || k == TG_XOR_SWIZZLE; }

// Validates a copy and fills the plan and launch arguments.
int plan_copy(const void* src, const void* dst, const int64_t shape[2], int dtype,
              const tg_layout* sl, const tg_layout* dl, const tg_copy_opts* opts,
              tg_copy_plan* plan, CopyArgs* args) {
  if (!shape) return fail(TG_E_NULL, "shape is NULL");
  if (!sl || !dl) return fail(TG_E_NULL, "src_layout or dst_layout is NULL");
  const int64_t rows = shape[0], cols = shape[1];
  if (rows < 0 || cols < 0) return fail(TG_E_SHAPE, "negative extent");
  if (rows > kMaxDim || cols > kMaxDim) return fail(TG_E_SHAPE, "extent above 2^30");
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(TG_E_DTYPE, fmt("unknown dtype %lld", dtype));
  if (!valid_kind(sl->kind) || !valid_kind(dl->kind) || sl->reserved || dl->reserved)
    return fail(TG_E_LAYOUT, "unknown layout kind or nonzero reserved field");
  if (sl->ld < 0 || dl->ld < 0) return fail(TG_E_LAYOUT, "negative leading dimension");
  if (sl->ld > kMaxLd || dl->ld > kMaxLd)
    return fail(TG_E_LAYOUT, "leading dimension above 2^40 elements");
  if (opts && opts->flags) return fail(TG_E_ARG, "opts->flags must be 0");

  std::memset(plan, 0, sizeof *plan);
  std::memset(args, 0, sizeof *args);
  if (rows == 0 || cols == 0) {
    const int t = opts ? opts->threads : 256;
    if (t <= 0 || t > 1024) return fail(TG_E_THREADS, "threads must be in 1..1024");
    plan->load = plan->store = tg_copy_phase{0, t, 1, 8 * eb};
    return TG_OK;
  }
  if (!src || !dst) return fail(TG_E_NULL, "src or dst is NULL");

  // Tile and workgroup choice.
  tg_copy_opts o{};
  if (opts) {
    o = *opts;
  } else {
    o.tile_cols = (int32_t)std::min<int64_t>(cols, 128 / eb);
    o.tile_rows = (int32_t)std::min<int64_t>(rows, 128);
    const int64_t te = (int64_t)o.tile_rows * o.tile_cols;
    if (te % 256 == 0) o.threads = 256;
    else if (te % 64 == 0) o.threads = 64;
    else { o.threads = 1; while (o.threads < 64 && te % (2 * o.threads) == 0) o.threads *= 2; }
    const int64_t rb = (int64_t)o.tile_cols * eb;
    o.lds_kind = (rb % 16 == 0 && ((rb / 16) & (rb / 16 - 1)) == 0) ? TG_XOR_SWIZZLE : TG_ROW_MAJOR;
  }
  if (o.threads <= 0 || o.threads > 1024) return fail(TG_E_THREADS, "threads must be in 1..1024");
  if (o.tile_rows <= 0 || o.tile_cols <= 0) return fail(TG_E_SHAPE, "tile extents must be positive");
  if (o.lds_kind != TG_ROW_MAJOR && o.lds_kind != TG_XOR_SWIZZLE)
    return fail(TG_E_LAYOUT, "the LDS layout must be TG_ROW_MAJOR or TG_XOR_SWIZZLE");
  if (rows % o.tile_rows || cols % o.tile_cols)
    return fail(TG_E_SHAPE, fmt("a %lld x %lld tensor is not a whole number of %lld-row tiles", rows,
                                cols, o.tile_rows) + fmt(" x %lld-col tiles", o.tile_cols));
  const int64_t lds_bytes = (int64_t)o.tile_rows * o.tile_cols * eb;
  if (lds_bytes > 65536) return fail(TG_E_SHAPE, "a tile may hold at most 64 KiB of LDS");
  const int64_t tiles_r = rows / o.tile_rows, tiles_c = cols / o.tile_cols;

  // Global sides, with leading dimensions resolved.
  auto resolve = [&](const tg_layout* l, const void* p, Side* s, const char* name) -> int {
    s->kind = l->kind;
    if (l->kind == TG_ROW_MAJOR) {
      s->ld = l->ld ? l->ld : cols;
      if (s->ld < cols) return fail(TG_E_LAYOUT, std::string(name) + ": row-major ld < cols");
    } else if (l->kind == TG_COL_MAJOR) {
      s->ld = l->ld ? l->ld : rows;
      if (s->ld < rows) return fail(TG_E_LAYOUT, std::string(name) + ": column-major ld < rows");
    } else {
      if (tiles_r != 1 || tiles_c != 1)
        return fail(TG_E_LAYOUT, std::string(name) + ": an XOR-swizzled global side must be one tile");
      if (l->ld != 0 && l->ld != cols)
        return fail(TG_E_LAYOUT, std::string(name) + ": an XOR-swizzled side is packed");
      s->ld = cols;
    }
    if ((uintptr_t)p % eb) return fail(TG_E_ALIGN, std::string(name) + ": not element aligned");
    s->base = (int64_t)((uintptr_t)p / eb);
    return TG_OK;
  };
  Side ss, ds;
  int st = resolve(sl, src, &ss, "src");
  if (st) return st;
  st = resolve(dl, dst, &ds, "dst");
  if (st) return st;
  const int64_t extent_s = (ss.kind == TG_COL_MAJOR ? (cols - 1) * ss.ld + rows
                                                    : (rows - 1) * ss.ld + cols) * eb;
  const int64_t extent_d = (ds.kind == TG_COL_MAJOR ? (cols - 1) * ds.ld + rows
                                                    : (rows - 1) * ds.ld + cols) * eb;
  if (overlaps(src, extent_s, dst, extent_d)) return fail(TG_E_ALIAS, "dst overlaps src");

  const Side lds{o.lds_kind, o.tile_cols, 0};
  std::string why;
  tg_copy_phase lp, sp;
  // Per direction: the widest width that the region and every tile step accept.
  auto phase = [&](const Side& g, tg_copy_phase* out, const char* dir) -> int {
    int r = partition(o.tile_rows, o.tile_cols, eb, o.threads, g, lds, out, &why);
    if (r) return fail(r, std::string(dir) + ": " + why);
    // Every width below an accepted one is accepted too (all conditions are
    // divisibilities by a power of two), so halving finds the widest width
    // that also keeps every tile's base aligned.
    while (out->vec > 1 && !tile_steps_aligned(g, o.tile_rows, o.tile_cols, tiles_r, tiles_c, out->vec)) {
      out->vec /= 2;
      out->vec_bits /= 2;
      out->outer *= 2;
    }
    return TG_OK;
  };
  st = phase(ss, &lp, "load");
  if (st) return st;
  st = phase(ds, &sp, "store");
  if (st) return st;

  plan->load = lp;
  plan->store = sp;
  plan->tile_rows = o.tile_rows;
  plan->tile_cols = o.tile_cols;
  plan->lds_kind = o.lds_kind;
  plan->lds_bytes = (int32_t)lds_bytes;
  plan->tiles = tiles_r * tiles_c;

  args->src = (const uint8_t*)src;
  args->dst = (uint8_t*)dst;
  args->src_ld = ss.ld;
  args->dst_ld = ds.ld;
  args->src_kind = ss.kind;
  args->dst_kind = ds.kind;
  args->tile_rows = o.tile_rows;
  args->tile_cols = o.tile_cols;
  args->tiles_c = tiles_c;
  args->ntiles = plan->tiles;
  args->eb = eb;
  args->lds_xor = o.lds_kind == TG_XOR_SWIZZLE;
  {
    const int64_t chunks = (int64_t)o.tile_cols * eb / 16;
    args->xor_mask = (int32_t)(std::min<int64_t>(8, std::max<int64_t>(chunks, 1)) - 1);
  }
  args->threads = o.threads;
  auto fill = [&](const Side& g, const tg_copy_phase& p, CopyPhase* c) {
    c->outer = p.outer;
    c->vec = p.vec;
    c->row_order = g.kind != TG_COL_MAJOR;
    c->inner = c->row_order ? o.tile_cols : o.tile_rows;
    c->inner_log2 = -1;
    for (int s = 0; s < 31; ++s)
      if ((1 << s) == c->inner) c->inner_log2 = s;
  };
  fill(ss, lp, &args->load);
  fill(ds, sp, &args->store);
  return TG_OK;
}

// tile_copy_async: the copy's checks and partition (plan_copy), then the asynchronous
// variant's own limits.  Both sides move the same width: the widest of 128 / 32 bits (the
// global -> LDS load widths) that the width rule accepts for both directions.
int plan_async(const void* src, const void* dst, const int64_t shape[2], int dtype,
               const tg_layout* sl, const tg_layout* dl, const tg_async_opts* ao,
               tg_async_plan* plan, CopyArgs* args) {
  if (!ao) return fail(TG_E_ARG, "opts is NULL (tile_copy_async takes explicit options)");
  if (ao->flags) return fail(TG_E_ARG, "opts->flags must be 0");
  if (ao->depth < 1 || ao->depth > 4) return fail(TG_E_ARG, "depth must be 1 .. 4");
  if (ao->tiles_per_workgroup < 0 || ao->tiles_per_workgroup > 64)
    return fail(TG_E_ARG, "tiles_per_workgroup must be 0 (default) or 1 .. 64");
  if (!sl || !dl) return fail(TG_E_NULL, "src_layout or dst_layout is NULL");
  if (sl->kind != TG_ROW_MAJOR)
    return fail(TG_E_LAYOUT, "tile_copy_async reads a row-major source (each chunk lands whole in LDS)");
  if (dl->kind != TG_ROW_MAJOR && dl->kind != TG_XOR_SWIZZLE)
    return fail(TG_E_LAYOUT, "tile_copy_async writes a row-major destination (or the one-tile LDS image)");
  tg_copy_opts o{ao->tile_rows, ao->tile_cols, ao->threads, ao->lds_kind, 0};
  {
    const int eb0 = elem_bytes(dtype);
    if (eb0 && o.tile_rows > 0 && o.tile_cols > 0 &&
        (int64_t)o.tile_rows * o.tile_cols * eb0 > kAsyncStageBytes)
      return fail(TG_E_SHAPE, "an asynchronous stage holds at most 16 KiB");
  }
  std::memset(plan, 0, sizeof *plan);
  int st = plan_copy(src, dst, shape, dtype, sl, dl, &o, &plan->copy, args);
  if (st) return st;
  plan->depth = ao->depth;
  if (plan->copy.tiles == 0) return TG_OK;
  if (o.threads % 64) return fail(TG_E_THREADS, "tile_copy_async needs whole waves (threads % 64 == 0)");
  const int eb = args->eb;
  const int64_t tile_bytes = (int64_t)o.tile_rows * o.tile_cols * eb;
  // per-thread offsets inside a tile are 32-bit
  if ((int64_t)(o.tile_rows - 1) * args->src_ld * eb + (int64_t)o.tile_cols * eb >= ((int64_t)1 << 32) ||
      (int64_t)(o.tile_rows - 1) * args->dst_ld * eb + (int64_t)o.tile_cols * eb >= ((int64_t)1 << 32))
    return fail(TG_E_SHAPE, "a tile of tile_copy_async must span under 4 GiB of either side");
  const int wl = plan->copy.load.vec * eb, ws = plan->copy.store.vec * eb;
  const int w = std::min(wl, ws) >= 16 ? 16 : std::min(wl, ws) >= 4 ? 4 : 0;
  if (!w)
    return fail(TG_E_ALIGN, "tile_copy_async moves 128- or 32-bit chunks; the rows admit neither");
  const int64_t rounds = tile_bytes / ((int64_t)o.threads * w);
  if (rounds != 1 && rounds != 2 && rounds != 4 && rounds != 8)
    return fail(TG_E_THREADS, fmt("tile_copy_async runs 1, 2, 4 or 8 rounds per thread (got %lld); "
                                  "change threads or the tile", rounds));
  for (tg_copy_phase* ph : {&plan->copy.load, &plan->copy.store}) {
    ph->vec = w / eb;
    ph->vec_bits = 8 * w;
    ph->outer = (int32_t)rounds;
  }
  args->load.vec = args->store.vec = w / eb;
  args->load.outer = args->store.outer = (int32_t)rounds;
  plan->copy.lds_bytes = (int32_t)(ao->depth * kAsyncStageBytes);
  // Consecutive tiles per workgroup (row-major tile order keeps them side by side along a tile
  // row).  Default: up to 4 while at least 2048 workgroups remain (on 16384^2 fp16 in 128x64
  // tiles, 4 ran 5-15 % faster than 8 or 16 at every depth, and 16 % faster than 1 at depth 4).
  int32_t tpw = ao->tiles_per_workgroup;
  if (!tpw) {
    tpw = 1;
    while (tpw < 4 && plan->copy.tiles / (2 * tpw) >= 2048) tpw *= 2;
  }
  plan->tiles_per_workgroup = tpw;
  plan->grid = (plan->copy.tiles + tpw - 1) / tpw;
  return TG_OK;
}

}  // namespace

extern "C" {

const char* tile_last_error(void) { return g_last_error.c_str(); }

int tile_abi_version(void) { return 7; }

int tile_gemm_plan(const void* A, const void* B, const float* C, const float* D, int64_t M,
                   int64_t N, int64_t K, int transA, int transB, float beta, int dtype,
                   tg_gemm_plan* out) {
  clear_error();
  if (!out) return fail(TG_E_ARG, "out is NULL");
  int st = validate_gemm(A, B, C, D, M, N, K, transA, transB, beta, dtype);
  if (st) return st;
  fill_plan(choose_gemm(M, N, K, transA, transB), out);
  return TG_OK;
}

int tile_gemm(const void* A, const void* B, const float* C, float* D, int64_t M, int64_t N,
              int64_t K, int transA, int transB, float beta, int dtype, void* stream) {
  clear_error();
  int st = validate_gemm(A, B, C, D, M, N, K, transA, transB, beta, dtype);
  if (st) return st;
  const GemmConfig cfg = choose_gemm(M, N, K, transA, transB);
  if (cfg.kernel == TG_GEMM_NONE) return TG_OK;
  if (cfg.kernel == TG_GEMM_FILL && beta == 1.0f && C == D) return TG_OK;
  GemmArgs g{};
  g.A = (const uint16_t*)A;
  g.B = (const uint16_t*)B;
  g.C = beta == 1.0f ? C : nullptr;
  g.D = D;
  g.M = (int32_t)M;
  g.N = (int32_t)N;
  g.K = (int32_t)K;
  g.use_c = beta == 1.0f;
  if (cfg.bm) {
    g.tiles_m = (int32_t)((M + cfg.bm - 1) / cfg.bm);
    g.tiles_n = (int32_t)((N + cfg.bn - 1) / cfg.bn);
  }
  return launch_gemm(g, cfg, transA, transB, dtype, stream);
}

int tile_gemm_fp8_plan(const void* A, const void* B, const float* C, const float* D, int64_t M,
                       int64_t N, int64_t K, int transA, int transB, float beta, int a_dtype,
                       int b_dtype, tg_gemm_plan* out) {
  clear_error();
  if (!out) return fail(TG_E_ARG, "out is NULL");
  int st = validate_gemm_fp8(A, B, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype);
  if (st) return st;
  fill_plan(choose_gemm_fp8(M, N, K, false), out);
  return TG_OK;
}

static int run_gemm_fp8(const void* A, const void* B, const uint8_t* SA, const uint8_t* SB,
                        const float* C, float* D, int64_t M, int64_t N, int64_t K, int transA,
                        int transB, float beta, int a_dtype, int b_dtype, bool scaled,
                        void* stream) {
  const GemmConfig cfg = choose_gemm_fp8(M, N, K, scaled);
  if (cfg.kernel == TG_GEMM_NONE) return TG_OK;
  if (cfg.kernel == TG_GEMM_FILL && beta == 1.0f && C == D) return TG_OK;
  GemmArgs g{};
  g.A = (const uint16_t*)A;
  g.B = (const uint16_t*)B;
  g.C = beta == 1.0f ? C : nullptr;
  g.D = D;
  g.M = (int32_t)M;
  g.N = (int32_t)N;
  g.K = (int32_t)K;
  g.use_c = beta == 1.0f;
  if (cfg.kernel == TG_GEMM_FILL) return launch_gemm(g, cfg, 0, 0, TG_BF16, stream);
  g.tiles_m = (int32_t)((M + cfg.bm - 1) / cfg.bm);
  g.tiles_n = (int32_t)((N + cfg.bn - 1) / cfg.bn);
  g.SA = SA;
  g.SB = SB;
  const hipError_t e = launch_gemm_fp8(g, cfg.grid, transA, transB, a_dtype, b_dtype,
                                       cfg.bounds != 0, scaled, cfg.bm, (hipStream_t)stream);
  if (e != hipSuccess)
    return fail(TG_E_HIP, std::string(scaled ? "tile_gemm_mx launch: " : "tile_gemm_fp8 launch: ") +
                              hipGetErrorString(e));
  return TG_OK;
}

int tile_gemm_fp8(const void* A, const void* B, const float* C, float* D, int64_t M, int64_t N,
                  int64_t K, int transA, int transB, float beta, int a_dtype, int b_dtype,
                  void* stream) {
  clear_error();
  int st = validate_gemm_fp8(A, B, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype);
  if (st) return st;
  return run_gemm_fp8(A, B, nullptr, nullptr, C, D, M, N, K, transA, transB, beta, a_dtype,
                      b_dtype, false, stream);
}

int tile_gemm_mx_plan(const void* A, const void* B, const uint8_t* SA, const uint8_t* SB,
                      const float* C, const float* D, int64_t M, int64_t N, int64_t K, int transA,
                      int transB, float beta, int a_dtype, int b_dtype, tg_gemm_plan* out) {
  clear_error();
  if (!out) return fail(TG_E_ARG, "out is NULL");
  int st = validate_gemm_mx(A, B, SA, SB, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype);
  if (st) return st;
  fill_plan(is_packed(a_dtype) ? choose_gemm_packed(M, N, K, a_dtype, b_dtype)
                                : choose_gemm_fp8(M, N, K, true), out);
  return TG_OK;
}

int tile_gemm_mx(const void* A, const void* B, const uint8_t* SA, const uint8_t* SB,
                 const float* C, float* D, int64_t M, int64_t N, int64_t K, int transA, int transB,
                 float beta, int a_dtype, int b_dtype, void* stream) {
  clear_error();
  int st = validate_gemm_mx(A, B, SA, SB, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype);
  if (st) return st;
  if (!is_packed(a_dtype))
    return run_gemm_fp8(A, B, SA, SB, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype, true,
                        stream);
  const GemmConfig cfg = choose_gemm_packed(M, N, K, a_dtype, b_dtype);
  if (cfg.kernel == TG_GEMM_NONE) return TG_OK;
  if (cfg.kernel == TG_GEMM_FILL && beta == 1.0f && C == D) return TG_OK;
  GemmArgs g{};
  g.A = (const uint16_t*)A;
  g.B = (const uint16_t*)B;
  g.C = beta == 1.0f ? C : nullptr;
  g.D = D;
  g.M = (int32_t)M;
  g.N = (int32_t)N;
  g.K = (int32_t)K;
  g.use_c = beta == 1.0f;
  if (cfg.kernel == TG_GEMM_FILL) return launch_gemm(g, cfg, 0, 0, TG_BF16, stream);
  g.tiles_m = (int32_t)((M + cfg.bm - 1) / cfg.bm);
  g.tiles_n = (int32_t)((N + cfg.bn - 1) / cfg.bn);
  g.SA = SA;
  g.SB = SB;
  const int af = packed_fmt(a_dtype), bf = packed_fmt(b_dtype);
  const hipError_t e =
      !cfg.direct ? launch_gemm_mx_packed(g, cfg.grid, af, bf, cfg.bounds != 0, cfg.bm,
                                          (hipStream_t)stream)
      : af == 4   ? launch_fp4_direct(g, cfg.grid, cfg.bounds != 0, cfg.bm, (hipStream_t)stream)
                  : launch_fp6_direct(g, cfg.grid, af, bf, cfg.bounds != 0, cfg.bm,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail(TG_E_HIP, std::string("tile_gemm_mx launch: ") + hipGetErrorString(e));
  return TG_OK;
}

int tile_copy_plan(const void* src, const void* dst, const int64_t shape[2], int dtype,
                   const tg_layout* src_layout, const tg_layout* dst_layout,
                   const tg_copy_opts* opts, tg_copy_plan* out) {
  clear_error();
  if (!out) return fail(TG_E_ARG, "out is NULL");
  CopyArgs args;
  return plan_copy(src, dst, shape, dtype, src_layout, dst_layout, opts, out, &args);
}

int tile_copy_ex(const void* src, void* dst, const int64_t shape[2], int dtype,
                 const tg_layout* src_layout, const tg_layout* dst_layout,
                 const tg_copy_opts* opts, void* stream) {
  clear_error();
  if (!opts) return fail(TG_E_ARG, "opts is NULL (use tile_copy for the defaults)");
  tg_copy_plan plan;
  CopyArgs args;
  int st = plan_copy(src, dst, shape, dtype, src_layout, dst_layout, opts, &plan, &args);
  if (st) return st;
  if (plan.tiles == 0) return TG_OK;
  return launch_tile_copy(args, plan.load.vec * args.eb, plan.store.vec * args.eb, plan.lds_bytes,
                          stream);
}

int tile_copy(const void* src, void* dst, const int64_t shape[2], int dtype,
              const tg_layout* src_layout, const tg_layout* dst_layout, void* stream) {
  clear_error();
  tg_copy_plan plan;
  CopyArgs args;
  int st = plan_copy(src, dst, shape, dtype, src_layout, dst_layout, nullptr, &plan, &args);
  if (st) return st;
  if (plan.tiles == 0) return TG_OK;
  return launch_tile_copy(args, plan.load.vec * args.eb, plan.store.vec * args.eb, plan.lds_bytes,
                          stream);
}

int tile_copy_async_plan(const void* src, const void* dst, const int64_t shape[2], int dtype,
                         const tg_layout* src_layout, const tg_layout* dst_layout,
                         const tg_async_opts* opts, tg_async_plan* out) {
  clear_error();
  if (!out) return fail(TG_E_ARG, "out is NULL");
  CopyArgs args;
  return plan_async(src, dst, shape, dtype, src_layout, dst_layout, opts, out, &args);
}

int tile_copy_async(const void* src, void* dst, const int64_t shape[2], int dtype,
                    const tg_layout* src_layout, const tg_layout* dst_layout,
                    const tg_async_opts* opts, void* stream) {
  clear_error();
  tg_async_plan plan;
  CopyArgs args;
  int st = plan_async(src, dst, shape, dtype, src_layout, dst_layout, opts, &plan, &args);
  if (st || plan.copy.tiles == 0) return st;
  const hipError_t e = launch_tile_copy_async(args, plan.copy.load.vec * args.eb, plan.copy.load.outer,
                                              plan.depth, plan.tiles_per_workgroup, plan.grid,
                                              (hipStream_t)stream);
  if (e != hipSuccess) return fail(TG_E_HIP, std::string("tile_copy_async launch: ") + hipGetErrorString(e));
  return TG_OK;
}

int tile_copy_partition(int64_t rows, int64_t cols, int elem_bits, int threads,
                        const tg_layout* drive, int64_t drive_base, const tg_layout* other,
                        int64_t other_base, tg_copy_phase* out) {
  clear_error();
  if (!drive || !other || !out) return fail(TG_E_NULL, "NULL argument");
  if (elem_bits != 8 && elem_bits != 16 && elem_bits != 32 && elem_bits != 64)
    return fail(TG_E_DTYPE, "elem_bits must be 8, 16, 32 or 64");
  if (!valid_kind(drive->kind) || !valid_kind(other->kind))
    return fail(TG_E_LAYOUT, "unknown layout kind");
  if (drive->kind == TG_XOR_SWIZZLE)
    return fail(TG_E_LAYOUT, "the driving (global) side cannot be XOR-swizzled");
  auto side = [&](const tg_layout* l, int64_t base) {
    Side s{l->kind, l->ld, base};
    if (!s.ld) s.ld = l->kind == TG_COL_MAJOR ? rows : cols;
    if (l->kind == TG_XOR_SWIZZLE) s.ld = cols;
    return s;
  };
  const Side d = side(drive, drive_base), o = side(other, other_base);
  if ((d.kind == TG_ROW_MAJOR && d.ld < cols) || (d.kind == TG_COL_MAJOR && d.ld < rows) ||
      (o.kind == TG_ROW_MAJOR && o.ld < cols) || (o.kind == TG_COL_MAJOR && o.ld < rows))
    return fail(TG_E_LAYOUT, "leading dimension smaller than the region");
  if (other->kind == TG_XOR_SWIZZLE && other->ld != 0 && other->ld != cols)
    return fail(TG_E_LAYOUT, "an XOR-swizzled side is packed");
  std::string why;
  int st = partition(rows, cols, elem_bits / 8, threads, d, o, out, &why);
  if (st) return fail(st, why);
  return TG_OK;
}

}  // extern "C"
