// Host planner: the vec_auto copy partition and the GEMM kernel choice.
//
// Copy partition, from [VEC-AUTO] ("TVM TIRx CUDA 向量化内存拷贝实战：vec_auto 变体的
// global↔shared 实现路径（gmem_smem）深度解析"):
//   * 接受什么输入 — the thread count must be positive and divide the region's
//     element count; the copy is rejected, never masked by a scalar path.
//   * 算法核心 step 1 — the region becomes [outer, threads, vec] in the global
//     side's canonical order; thread t of round f owns fused elements
//     [(f*threads + t)*vec, +vec) (the IR of the demo: f*128 + tid*4).
//   * 算法核心 step 2 — widths of 128/64/32/16/8 bits, widest first; accept when
//     the contiguous tail divides by the width and every non-vector stride and
//     both base offsets are multiples of it.
//   * 对齐约束的兜底 — misaligned strides or bases narrow the width, to 1 element.
// Readings where the page is silent: widths below or not a multiple of the
// element size are skipped; the width must divide elements/threads; a side
// stored in the other order than the fused one only takes 1-element vectors
// (unless the fused order's inner extent is 1: then both orders visit the same
// sequence); a vector may cross a row only where the whole region is one
// contiguous run.
#include <algorithm>
#include <cstdio>

#include "tg_internal.h"

namespace tg {

int elem_bytes(int dtype) {
  switch (dtype) {
    case TG_F16:
    case TG_BF16:
      return 2;
    case TG_F32:
      return 4;
    case TG_U8:
    case TG_I8:
    case TG_FP8_E4M3:
    case TG_FP8_E5M2:
      return 1;
    default:
      return 0;
  }
}

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Row and column strides (elements) of a side.
void strides(const Side& s, int64_t cols, int64_t* sr, int64_t* sc) {
  if (s.kind == TG_COL_MAJOR) {
    *sr = 1;
    *sc = s.ld;
  } else if (s.kind == TG_XOR_SWIZZLE) {
    *sr = cols;
    *sc = 1;
  } else {
    *sr = s.ld;
    *sc = 1;
  }
}

// Can every v-element run of the fused order be moved as one aligned vector on
// side `s`?  `row_order` is the fused order; the run starting at fused index x
// (a multiple of v) covers (outer, inner) = divmod(x .. x+v-1, inner extent).
bool side_takes(const Side& s, int64_t rows, int64_t cols, bool row_order, int64_t v, int eb) {
  if (s.kind == TG_XOR_SWIZZLE && v * eb > 16) return false;  // one swizzle chunk at most
  if (v == 1) return true;
  // A fused order whose inner extent is 1 visits the region in the other order's sequence
  // (one row in column order is that row, left to right).
  if ((row_order ? cols : rows) == 1) row_order = !row_order;
  int64_t sr, sc;
  strides(s, cols, &sr, &sc);
  const int64_t inner = row_order ? cols : rows;
  const int64_t outer_ext = row_order ? rows : cols;
  const int64_t s_in = row_order ? sc : sr;
  const int64_t s_out = row_order ? sr : sc;
  if (s.kind == TG_XOR_SWIZZLE && !row_order) return false;
  if (inner % v == 0) {
    if (s_in != 1) return false;                         // run inside one row
    if (outer_ext > 1 && s_out % v != 0) return false;   // every row start aligned
  } else {
    if (s.kind == TG_XOR_SWIZZLE) return false;          // chunks are not contiguous
    if (inner > 1 && s_in != 1) return false;
    if (s_out != inner) return false;                    // the region is one run
  }
  return s.base % v == 0;
}

}  // namespace

int partition(int64_t rows, int64_t cols, int eb, int threads, const Side& drive,
              const Side& other, tg_copy_phase* out, std::string* why) {
  char buf[192];
  if (threads <= 0) {
    *why = "thread count must be positive";
    return TG_E_THREADS;
  }
  if (rows < 0 || cols < 0) {
    *why = "negative extent";
    return TG_E_SHAPE;
  }
  const int64_t n = rows * cols;
  if (n % threads != 0) {
    std::snprintf(buf, sizeof buf,
                  "%lld elements do not divide over %d threads (rejected, not masked)",
                  (long long)n, threads);
    *why = buf;
    return TG_E_THREADS;
  }
  for (const Side* s : {&drive, &other}) {
    if (s->kind == TG_XOR_SWIZZLE) {
      const int64_t row_bytes = cols * eb;
      if (row_bytes % 16 != 0 || !is_pow2(row_bytes / 16)) {
        *why = "an XOR-swizzled side needs rows of a power-of-two number of 16-byte chunks";
        return TG_E_LAYOUT;
      }
    }
  }
  const bool row_order = drive.kind != TG_COL_MAJOR;
  const int elem_bits = 8 * eb;
  out->threads = threads;
  if (n == 0) {
    out->outer = 0;
    out->vec = 1;
    out->vec_bits = elem_bits;
    return TG_OK;
  }
  const int64_t per_thread = n / threads;
  static const int kWidths[] = {128, 64, 32, 16, 8};
  for (int bits : kWidths) {
    if (bits < elem_bits || bits % elem_bits != 0) continue;
    const int64_t v = bits / elem_bits;
    if (per_thread % v != 0) continue;
    if (!side_takes(drive, rows, cols, row_order, v, eb)) continue;
    if (!side_takes(other, rows, cols, row_order, v, eb)) continue;
    out->outer = (int32_t)(per_thread / v);
    out->vec = (int32_t)v;
    out->vec_bits = bits;
    return TG_OK;
  }
  *why = "no vector width keeps every transfer contiguous";
  return TG_E_LAYOUT;
}

bool tile_steps_aligned(const Side& s, int64_t tile_rows, int64_t tile_cols, int64_t tiles_r,
                        int64_t tiles_c, int64_t vec) {
  int64_t sr, sc;
  strides(s, tile_cols, &sr, &sc);
  if (tiles_r > 1 && (tile_rows * sr) % vec != 0) return false;
  if (tiles_c > 1 && (tile_cols * sc) % vec != 0) return false;
  return true;
}

// ---------------------------------------------------------------- GEMM ----
// The register kernel's matrix instruction ([TCGEN05-CP] 形状选择: candidates tried from the
// widest down against the operands' layouts; [SYNC-GEMM] 二: k16 when K allows it, else k8).
// Per candidate (M, N, K of one atom; R K values per lane): admissible when K % K_atom == 0;
// cost = (multiply-adds after padding M and N up to the atom, global loads per lane per atom
// step / multiply-adds per atom, candidate order), smallest wins.  A lane's K run is one vector
// load when its operand is stored K-contiguous, R loads when K runs across memory lines.
int gemm_atom_choice(int64_t M, int64_t N, int64_t K, int trans_a, int trans_b) {
  struct Cand { int shape, am, an, ak, r; };
  static const Cand kCands[] = {{TG_MMA_32x32x16, 32, 32, 16, 8}, {TG_MMA_16x16x32, 16, 16, 32, 8},
                                {TG_MMA_32x32x8, 32, 32, 8, 4}, {TG_MMA_16x16x16, 16, 16, 16, 4}};
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  int best = 0;
  int64_t best_work = 0;
  double best_lpm = 0.0;
  for (const Cand& c : kCands) {
    if (K % c.ak != 0) continue;
    const int64_t work = ((M + c.am - 1) / c.am * c.am) * ((N + c.an - 1) / c.an * c.an) * K;
    const int loads = (trans_a ? c.r : 1) + (trans_b ? 1 : c.r);
    const double lpm = (double)loads / (double)(c.am * c.an * c.ak);
    if (best == 0 || work < best_work || (work == best_work && lpm < best_lpm)) {
      best = c.shape;
      best_work = work;
      best_lpm = lpm;
    }
  }
  return best;
}

// Kernel choice.  The page lowers every (m, n) output tile to one atom per K
// step, accumulated in place ([SYNC-GEMM] 四 step 3); on gfx950 a workgroup
// owns a block of output tiles so that operands staged once in LDS feed many
// MFMAs.  The block size is the largest that still gives the chip enough
// workgroups (256 CUs); tiny problems use the register kernel.  256- and 128-wide
// blocks take the direct-load kernel when each operand is under 2 GiB.  Smaller
// blocks only where the larger ones are too few: measured, 128-wide blocks lose to
// 256-wide ones once there are 256 of those (8192^3 bf16: 1082 against 890 us,
// 6000^3: 554 against 435 us).
GemmConfig choose_gemm(int64_t M, int64_t N, int64_t K, int trans_a, int trans_b) {
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
  auto blocks = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (M * N <= 64 * 64) {
    c.kernel = TG_GEMM_ATOM;
    c.atom = gemm_atom_choice(M, N, K, trans_a, trans_b);
    const int am = (c.atom == TG_MMA_32x32x16 || c.atom == TG_MMA_32x32x8) ? 32 : 16;
    c.bm = c.bn = c.wm = c.wn = am;
    c.bk = c.atom == TG_MMA_16x16x32 ? 32 : c.atom == TG_MMA_32x32x8 ? 8 : 16;
    c.threads = 64;
    c.bounds = (M % am) != 0 || (N % am) != 0;
    c.grid = blocks(am, am);
    return c;
  }
  c.kernel = TG_GEMM_TILED;
  c.bk = 64;
  // 128-wide blocks (direct-load kernel only) while they fit one round of two per CU: with
  // more, a CU runs three or more of them one after the other, slower than the one 256-wide
  // block it would get (fp8 3072^3: 41.7 against 35.6 us).  Operands of 2 GiB or more take
  // the VGPR-staged kernel on 256- or 64-wide tiles.
  const bool fits = direct_gemm_fits(M, N, K, trans_a, trans_b);
  if (blocks(256, 256) >= 256 || (fits && blocks(128, 128) > 512)) {
    c.bm = c.bn = 256;
    c.wm = c.wn = 128;
  } else if (fits && blocks(128, 128) >= 128) {
    c.bm = c.bn = 128;
    c.wm = c.wn = 64;
  } else {
    c.bm = c.bn = 64;
    c.wm = c.wn = 32;
  }
  c.threads = (c.bm / c.wm) * (c.bn / c.wn) * 64;
  c.bounds = (M % c.bm) != 0 || (N % c.bn) != 0 || (K % c.bk) != 0;
  c.lds_bytes = 2 * (c.bm + c.bn) * 128;
  c.grid = blocks(c.bm, c.bn);
  // gemm_direct (256x256) and gemm_direct128 (128x128): 8 waves, a 2 x 4 wave grid
  c.direct = c.bm >= 128 && fits;
  if (c.direct) {
    c.wm = c.bm / 2;
    c.wn = c.bn / 4;
    c.threads = 512;
  }
  return c;
}

GemmConfig choose_gemm_fp8(int64_t M, int64_t N, int64_t K, bool scaled) {
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
  // 256x256 blocks; 128x128 when there are fewer than 256 of the larger and at most 512 of the
  // smaller, as for the 16-bit kernel
  auto blocks = [&](int64_t b) { return ((M + b - 1) / b) * ((N + b - 1) / b); };
  const int bs = (blocks(256) < 256 && blocks(128) <= 512) ? 128 : 256;
  c.kernel = TG_GEMM_TILED;
  c.bm = c.bn = bs;
  c.bk = 128;
  c.wm = bs / 2;
  c.wn = bs / 4;
  c.threads = 512;
  c.bounds = (M % bs) != 0 || (N % bs) != 0;
  c.lds_bytes = 4 * bs * 128 + (scaled ? 3 * 2 * 260 * (bs / 16) : 0);   // + the scale ring
  c.grid = blocks(bs);
  c.direct = 1;
  return c;
}

}  // namespace tg
