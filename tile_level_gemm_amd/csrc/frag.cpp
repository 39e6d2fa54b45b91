// C-ABI entry points of the register fragment calls: validation, planning and launch.
//
// The fragment maps are the matrix instructions' operand and accumulator registers on gfx950
// ([SYNC-GEMM] 一: the register-level gemm takes fragments and accumulators in registers,
// loaded first by the caller; [VEC-AUTO] closing reading list: the register path of vec_auto
// and the ldstmatrix copy).  The register path's transfer width is the page's widest-first
// rule ([VEC-AUTO] 算法核心 step 2) with the register layout as the driving side: every lane
// holds runs of 16 bytes along one tile axis, so a run along memory lines moves with the
// widest 128/64/32/16/8-bit transfer that the base and the line pitch keep aligned, and a run
// across lines moves one element at a time.  Every check runs before any HIP call.
#include <cstdio>
#include <cstring>
#include <string>

#include "tg_internal.h"

using namespace tg;

namespace {

const int64_t kMaxDim = (int64_t)1 << 30;

struct KindInfo {
  int tr, tc;      // tile extent
  int eb;          // element bytes
  int elems;       // register elements per lane
  bool run_rows;   // every run goes along the tile's rows (else along its columns)
  int run_bytes() const { return elems * eb < 16 ? elems * eb : 16; }
};

bool kind_info(int kind, KindInfo* k) {
  switch (kind) {
    case TG_FRAG_A16_32x32x16: *k = {32, 16, 2, 8, false}; return true;
    case TG_FRAG_B16_32x32x16: *k = {16, 32, 2, 8, true}; return true;
    case TG_FRAG_A16_16x16x32: *k = {16, 32, 2, 8, false}; return true;
    case TG_FRAG_B16_16x16x32: *k = {32, 16, 2, 8, true}; return true;
    case TG_FRAG_A8_32x32x64: *k = {32, 64, 1, 32, false}; return true;
    case TG_FRAG_B8_32x32x64: *k = {64, 32, 1, 32, true}; return true;
    case TG_FRAG_C32_32x32: *k = {32, 32, 4, 16, true}; return true;
    case TG_FRAG_C32_16x16: *k = {16, 16, 4, 4, true}; return true;
    case TG_FRAG_A16_32x32x8: *k = {32, 8, 2, 4, false}; return true;
    case TG_FRAG_B16_32x32x8: *k = {8, 32, 2, 4, true}; return true;
    case TG_FRAG_A16_16x16x16: *k = {16, 16, 2, 4, false}; return true;
    case TG_FRAG_B16_16x16x16: *k = {16, 16, 2, 4, true}; return true;
    default: return false;
  }
}

bool dtype_fits(int dtype, int eb) {
  switch (dtype) {
    case TG_F16: case TG_BF16: return eb == 2;
    case TG_U8: case TG_I8: case TG_FP8_E4M3: case TG_FP8_E5M2: return eb == 1;
    case TG_F32: return eb == 4;
    default: return false;
  }
}

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

// Validates a fragment copy and fills the plan and the launch arguments.
int plan_frag(bool store, const void* mem, const void* image, const int64_t shape[2], int dtype,
              const tg_layout* layout, int kind, int route, tg_frag_plan* plan, FragArgs* args) {
  if (!shape) return fail(TG_E_NULL, "shape is NULL");
  if (!layout) return fail(TG_E_NULL, "layout is NULL");
  KindInfo k;
  if (!kind_info(kind, &k)) return fail(TG_E_ARG, fmt("unknown fragment kind %lld", kind));
  if (route != TG_FRAG_AUTO && route != TG_FRAG_DIRECT && route != TG_FRAG_LDS)
    return fail(TG_E_ARG, fmt("unknown route %lld", route));
  if (!dtype_fits(dtype, k.eb))
    return fail(TG_E_DTYPE, fmt("dtype %lld does not have the fragment kind's %lld-bit elements",
                                dtype, 8 * k.eb));
  const int64_t rows = shape[0], cols = shape[1];
  if (rows < 0 || cols < 0) return fail(TG_E_SHAPE, "negative extent");
  if (rows > kMaxDim || cols > kMaxDim) return fail(TG_E_SHAPE, "extent above 2^30");
  if (rows % k.tr || cols % k.tc)
    return fail(TG_E_SHAPE, fmt("a %lld x %lld matrix is not a whole number of ", rows, cols) +
                                fmt("%lld x %lld fragment tiles", k.tr, k.tc));
  if (layout->kind != TG_ROW_MAJOR && layout->kind != TG_COL_MAJOR)
    return fail(TG_E_LAYOUT, "register copies take row- or column-major memory");
  if (layout->reserved) return fail(TG_E_LAYOUT, "nonzero reserved field");
  const bool col_major = layout->kind == TG_COL_MAJOR;
  const int64_t lines = col_major ? cols : rows, line_len = col_major ? rows : cols;
  const int64_t ld = layout->ld ? layout->ld : line_len;
  if (layout->ld < 0 || ld < line_len) return fail(TG_E_LAYOUT, "leading dimension below the line length");
  if (ld > ((int64_t)1 << 40)) return fail(TG_E_LAYOUT, "leading dimension above 2^40 elements");

  std::memset(plan, 0, sizeof *plan);
  std::memset(args, 0, sizeof *args);
  plan->tile_rows = k.tr;
  plan->tile_cols = k.tc;
  plan->elems = k.elems;
  plan->elem_bits = 8 * k.eb;
  plan->threads = kFragThreads;
  // A run crosses memory lines when it goes along the axis memory does not keep contiguous.
  plan->transposed = k.run_rows != col_major;
  if (rows == 0 || cols == 0) {
    plan->route = route == TG_FRAG_LDS ? TG_FRAG_LDS : TG_FRAG_DIRECT;
    plan->vec = 1;
    plan->vec_bits = 8 * k.eb;
    return TG_OK;
  }
  if (!mem || !image) return fail(TG_E_NULL, store ? "image or dst is NULL" : "src or image is NULL");
  if ((uintptr_t)mem % k.eb) return fail(TG_E_ALIGN, "the matrix is not element aligned");
  if ((uintptr_t)image % 16) return fail(TG_E_ALIGN, "the register image must be 16-byte aligned");
  const int64_t mem_bytes = ((lines - 1) * ld + line_len) * k.eb;
  const int64_t img_bytes = rows * cols * k.eb;
  if (overlaps(mem, mem_bytes, image, img_bytes))
    return fail(TG_E_ALIAS, "the register image overlaps the matrix");

  // Direct-route width: the widest transfer every run keeps contiguous and aligned.
  int vb = k.eb;
  if (!plan->transposed)
    for (int w = k.run_bytes(); w > k.eb; w /= 2)
      if ((uintptr_t)mem % w == 0 && (ld * k.eb) % w == 0) { vb = w; break; }
  const bool lds_ok = (uintptr_t)mem % 16 == 0 && (ld * k.eb) % 16 == 0;
  int r = route;
  // Measured on MI355X: the LDS route matches or beats the direct route for every kind,
  // orientation and direction, 128-bit direct transfers included.
  if (r == TG_FRAG_AUTO) r = lds_ok ? TG_FRAG_LDS : TG_FRAG_DIRECT;
  if (r == TG_FRAG_LDS && !lds_ok)
    return fail(TG_E_ALIGN, "the LDS route needs 16-byte aligned memory lines (base and ld)");

  const int64_t tiles_r = rows / k.tr, tiles_c = cols / k.tc;
  plan->route = r;
  plan->tiles = tiles_r * tiles_c;
  if (r == TG_FRAG_LDS) {
    plan->vec = 16 / k.eb;
    plan->vec_bits = 128;
    const int nb = frag_lds_blocks(store);
    plan->lds_bytes = kFragLdsLines * frag_lds_line_bytes(store) * nb;
    const int64_t per_line = frag_lds_line_bytes(store) / k.eb;
    const int64_t nbp = (line_len + per_line - 1) / per_line;   // blocks along a line
    plan->grid = ((lines + kFragLdsLines - 1) / kFragLdsLines) * ((nbp + nb - 1) / nb);
  } else {
    plan->vec = vb / k.eb;
    plan->vec_bits = 8 * vb;
    const int64_t per_wg = (int64_t)(kFragThreads / 64) * frag_tiles_per_wave(kind);
    plan->grid = (plan->tiles + per_wg - 1) / per_wg;
  }
  if (plan->grid >= ((int64_t)1 << 31)) return fail(TG_E_SHAPE, "too many workgroups for one launch");

  args->mem = (uint8_t*)mem;
  args->img = (uint8_t*)image;
  args->ld = ld;
  args->lines = lines;
  args->line_len = line_len;
  args->tiles_r = tiles_r;
  args->tiles_c = tiles_c;
  args->ntiles = plan->tiles;
  return TG_OK;
}

int run_frag(bool store, const void* mem, const void* image, const int64_t shape[2], int dtype,
             const tg_layout* layout, int kind, int route, void* stream) {
  tg_frag_plan plan;
  FragArgs args;
  int st = plan_frag(store, mem, image, shape, dtype, layout, kind, route, &plan, &args);
  if (st || plan.tiles == 0) return st;
  const hipError_t e = launch_frag(args, kind, store, plan.transposed != 0, plan.route,
                                   plan.vec * plan.elem_bits / 8, plan.grid, (hipStream_t)stream);
  if (e != hipSuccess)
    return fail(TG_E_HIP, std::string(store ? "tile_frag_store" : "tile_frag_load") + " launch: " +
                              hipGetErrorString(e));
  return TG_OK;
}

// tile_frag_mma's shapes: atom extents and operand element bytes.
bool mma_info(int shape, int* am, int* an, int* ak, int* eb) {
  switch (shape) {
    case TG_MMA_32x32x16: *am = 32; *an = 32; *ak = 16; *eb = 2; return true;
    case TG_MMA_16x16x32: *am = 16; *an = 16; *ak = 32; *eb = 2; return true;
    case TG_MMA_32x32x64_F8: *am = 32; *an = 32; *ak = 64; *eb = 1; return true;
    case TG_MMA_32x32x8: *am = 32; *an = 32; *ak = 8; *eb = 2; return true;
    case TG_MMA_16x16x16: *am = 16; *an = 16; *ak = 16; *eb = 2; return true;
    default: return false;
  }
}

// Candidates from the widest atom down (multiply-adds per instruction; at equal width the
// longer K first).
const int kCandidates16[] = {TG_MMA_32x32x16, TG_MMA_16x16x32, TG_MMA_32x32x8, TG_MMA_16x16x16};
const int kCandidates8[] = {TG_MMA_32x32x64_F8};

}  // namespace

extern "C" {

int tile_mma_select(int64_t M, int64_t N, int64_t K, int a_dtype, int b_dtype, int* shape) {
  clear_error();
  if (!shape) return fail(TG_E_ARG, "shape is NULL");
  if (M < 0 || N < 0 || K < 0) return fail(TG_E_ARG, "negative extent");
  const bool f16 = (a_dtype == TG_F16 || a_dtype == TG_BF16) && a_dtype == b_dtype;
  const bool f8 = (a_dtype == TG_FP8_E4M3 || a_dtype == TG_FP8_E5M2) &&
                  (b_dtype == TG_FP8_E4M3 || b_dtype == TG_FP8_E5M2);
  if (!f16 && !f8)
    return fail(TG_E_DTYPE, "no matrix-instruction shape takes these operand formats");
  const int* cand = f16 ? kCandidates16 : kCandidates8;
  const int n = f16 ? 4 : 1;
  for (int i = 0; i < n; ++i) {
    int am, an, ak, eb;
    mma_info(cand[i], &am, &an, &ak, &eb);
    if (M % am == 0 && N % an == 0 && K % ak == 0) {
      *shape = cand[i];
      return TG_OK;
    }
  }
  return fail(TG_E_SHAPE, fmt("no atom divides M=%lld, N=%lld, K=%lld", M, N, K));
}

int tile_gemm_atom_select(int64_t M, int64_t N, int64_t K, int dtype, int transA, int transB,
                          int* shape) {
  clear_error();
  if (!shape) return fail(TG_E_ARG, "shape is NULL");
  if (transA != 0 && transA != 1) return fail(TG_E_ARG, "transA must be 0 or 1");
  if (transB != 0 && transB != 1) return fail(TG_E_ARG, "transB must be 0 or 1");
  if (dtype != TG_F16 && dtype != TG_BF16)
    return fail(TG_E_DTYPE, "the register GEMM takes TG_F16 or TG_BF16 operands");
  if (M <= 0 || N <= 0 || K <= 0 || K % 8 != 0)
    return fail(TG_E_SHAPE, fmt("need M, N, K > 0 and K %% 8 == 0 (got M=%lld, N=%lld, K=%lld)", M, N, K));
  *shape = gemm_atom_choice(M, N, K, transA, transB);
  return TG_OK;
}

int tile_frag_plan(int store, const void* mem, const void* image, const int64_t shape[2],
                   int dtype, const tg_layout* layout, int kind, int route, tg_frag_plan* out) {
  clear_error();
  if (!out) return fail(TG_E_ARG, "out is NULL");
  if (store != 0 && store != 1) return fail(TG_E_ARG, "store must be 0 or 1");
  FragArgs args;
  return plan_frag(store != 0, mem, image, shape, dtype, layout, kind, route, out, &args);
}

int tile_frag_load(const void* src, void* image, const int64_t shape[2], int dtype,
                   const tg_layout* src_layout, int kind, int route, void* stream) {
  clear_error();
  return run_frag(false, src, image, shape, dtype, src_layout, kind, route, stream);
}

int tile_frag_store(const void* image, void* dst, const int64_t shape[2], int dtype,
                    const tg_layout* dst_layout, int kind, int route, void* stream) {
  clear_error();
  return run_frag(true, dst, image, shape, dtype, dst_layout, kind, route, stream);
}

int tile_frag_mma(const void* a_image, const void* b_image, const float* c_image, float* d_image,
                  int64_t M, int64_t N, int64_t K, float beta, int a_dtype, int b_dtype,
                  int shape, void* stream) {
  clear_error();
  int am, an, ak, eb;
  if (!mma_info(shape, &am, &an, &ak, &eb)) return fail(TG_E_ARG, fmt("unknown shape %lld", shape));
  if (M < 0 || N < 0 || K < 0) return fail(TG_E_SHAPE, "negative extent");
  if (M % am || N % an || K % ak)
    return fail(TG_E_SHAPE, fmt("the shape needs M %% %lld == 0, N %% %lld == 0, ", am, an) +
                                fmt("K %% %lld == 0", ak));
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(TG_E_SHAPE, "extent above 2^30");
  if (eb == 2 ? !((a_dtype == TG_F16 || a_dtype == TG_BF16) && a_dtype == b_dtype)
              : !((a_dtype == TG_FP8_E4M3 || a_dtype == TG_FP8_E5M2) &&
                  (b_dtype == TG_FP8_E4M3 || b_dtype == TG_FP8_E5M2)))
    return fail(TG_E_DTYPE, eb == 2 ? "16-bit shapes take TG_F16 or TG_BF16 for both operands"
                                    : "the fp8 shape takes TG_FP8_E4M3 or TG_FP8_E5M2 operands");
  if (!(beta == 0.0f || beta == 1.0f))
    return fail(TG_E_BETA, "beta must be exactly 0.0 or 1.0 (alpha is fixed at 1)");
  if (M == 0 || N == 0) return TG_OK;
  if (!d_image) return fail(TG_E_NULL, "d_image is NULL");
  if (beta == 1.0f && !c_image) return fail(TG_E_NULL, "beta == 1 needs c_image");
  if (K > 0 && (!a_image || !b_image)) return fail(TG_E_NULL, "a_image or b_image is NULL");
  const int64_t dbytes = M * N * 4;
  if (K > 0 && (overlaps(d_image, dbytes, a_image, M * K * eb) ||
                overlaps(d_image, dbytes, b_image, K * N * eb)))
    return fail(TG_E_ALIAS, "d_image overlaps a_image or b_image");
  if (beta == 1.0f && c_image != d_image && overlaps(d_image, dbytes, c_image, dbytes))
    return fail(TG_E_ALIAS, "c_image overlaps d_image without being exactly d_image");
  if ((uintptr_t)a_image % 16 || (uintptr_t)b_image % 16 || (uintptr_t)d_image % 16 ||
      (beta == 1.0f && (uintptr_t)c_image % 16))
    return fail(TG_E_ALIGN, "register images must be 16-byte aligned");
  FragMmaArgs g{};
  g.a = (const uint8_t*)a_image;
  g.b = (const uint8_t*)b_image;
  g.c = beta == 1.0f ? c_image : nullptr;
  g.d = d_image;
  g.tiles_m = (int32_t)(M / am);
  g.tiles_n = (int32_t)(N / an);
  g.tiles_k = (int32_t)(K / ak);
  g.use_c = beta == 1.0f;
  const int64_t tiles = (int64_t)g.tiles_m * g.tiles_n;
  const int64_t grid = (tiles + kFragThreads / 64 - 1) / (kFragThreads / 64);
  if (grid >= ((int64_t)1 << 31)) return fail(TG_E_SHAPE, "too many workgroups for one launch");
  const hipError_t e = launch_frag_mma(g, shape, a_dtype, b_dtype, grid, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TG_E_HIP, std::string("tile_frag_mma launch: ") + hipGetErrorString(e));
  return TG_OK;
}

}  // extern "C"
