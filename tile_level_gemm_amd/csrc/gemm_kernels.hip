// Tile GEMM on gfx950: D = A·B (+C), fp16/bf16 operands, fp32 accumulation.
//
// [SYNC-GEMM] ("TVM TIRx 同步 GEMM 深度解析：warp 级 mma.sync 的寄存器碎片排布与完整下放链路"):
//   一    the primitive computes D = alpha·A·B + beta·C as a fully unrolled nest of
//         matrix atoms, one per output tile per K step, accumulated in place;
//   二    alpha = 1, beta in {0, 1}; transposes only describe storage, the product is
//         always A[M,K]·B[K,N];
//   四.3  the emitted nest initialises the accumulator (from C or zero), then runs the
//         K loop of atoms with the accumulator as both input and output;
//   五    the atom's accumulator registers are both its C input and its D output.
// The page's atoms and fragment geometry belong to another instruction set; here the
// atoms are gfx950 MFMAs and the fragments are their lane layouts:
//   v_mfma_f32_32x32x16_{f16,bf16}: lane l supplies A[m = l%32][k = 8(l/32) .. +8] and
//     B[k = 8(l/32) .. +8][n = l%32]; D[m][n] sits in lane n + 32((m/4)%2), accumulator
//     register (m%4) + 4(m/8).
//   v_mfma_f32_16x16x32_{f16,bf16}: lane l supplies A[m = l%16][k = 8(l/16) .. +8] and
//     B[k = 8(l/16) .. +8][n = l%16]; D[m][n] sits in lane n + 16(m/4), register m%4.
// Because the K index is contracted, any lane→k assignment works as long as A and B
// use the same one; only the m and n maps matter for correctness.
//
// Tiled kernel (one workgroup per BM x BN block of D):
//   * operand stages in LDS are [rows][64 k] of 16-bit values, 128-byte rows, XOR
//     swizzled on 16-byte chunks (lds_layout.h), two stages (double buffer);
//   * global -> LDS: K-contiguous operands move as 128-bit vectors in the vec_auto
//     partition (8 consecutive threads cover one 128-byte row); M/N-contiguous operands
//     (A with transA, B without transB) are read as 8x8 blocks of 16-bit values, eight
//     128-bit loads per thread, transposed in registers (16-bit lane shuffles) and written as
//     eight K-contiguous 128-bit LDS rows;
//   * LDS -> registers: one 128-bit read per lane per fragment (ds_read_b128);
//   * MFMA micro-kernel: each wave owns WM x WN of D as (WM/32) x (WN/32) accumulator tiles
//     of 16 fp32 registers, updated in place every 16-wide K step;
//   * epilogue: D = acc (+ C), masked on ragged edges;
//   * tile scheduler: workgroup ids are remapped so that the workgroups one XCD runs
//     (ids congruent mod 8) take a contiguous range of tiles, walked in groups of
//     kGroupM tile-rows, so concurrently running tiles on an XCD share A and B panels
//     in that XCD's L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "lds_layout.h"
#include "tg_internal.h"

namespace tg {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kBK = 64;      // K extent of one LDS stage (128-byte rows)
constexpr int kGroupM = 8;   // tile-rows per scheduling group

template <int DT>
struct Mfma;
template <>
struct Mfma<TG_F16> {
  static __device__ __forceinline__ f32x16 m32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 m16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<TG_BF16> {
  static __device__ __forceinline__ f32x16 m32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 m16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// ------------------------------------------------------------- loaders ----
// Operand stored K-contiguous: rows (m or n) of length ld = K.  The stage holds R rows
// x 64 k; chunk q of the stage is row q/8, k-chunk q%8 (8 consecutive threads = one
// 128-byte row, so each wave reads 8 full rows: coalesced).
template <int R, int NT, bool BOUNDS>
struct KMajorLoader {
  static constexpr int kChunks = R * 8;
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  u32x4 v[kPer];

  __device__ __forceinline__ void load(const uint16_t* X, int64_t ld, int row0, int rows, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int q = p * NT + tid;
      const int row = q >> 3, kc = q & 7;
      const int gr = row0 + row, gk = k0 + kc * 8;
      const bool ok = (kChunks % NT == 0 || q < kChunks) && (!BOUNDS || (gr < rows && gk < K));
      v[p] = ok ? *(const u32x4*)(X + (int64_t)gr * ld + gk) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint8_t* stage, int tid) const {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int q = p * NT + tid;
      if (kChunks % NT == 0 || q < kChunks) {
        const int row = q >> 3, kc = q & 7;
        *(u32x4*)(stage + swz128(row, kc)) = v[p];
      }
    }
  }
};

// Operand stored M/N-contiguous: global is [K][rows] with ld = rows.  The stage (R rows of
// 64 k) is covered by R 8x8 blocks; block b takes k-block kb = b%8 and row-block
// mb = b/8, so the eight threads of one row-block read eight different k rows of the
// same 16-byte column (128 contiguous bytes per k row across a wave) and write eight
// different chunks of the same LDS rows (no bank conflicts).
template <int R, int NT, bool BOUNDS>
struct MNMajorLoader {
  static constexpr int kBlocks = R;
  static constexpr int kPer = (kBlocks + NT - 1) / NT;
  u32x4 v[kPer][8];

  __device__ __forceinline__ void load(const uint16_t* X, int64_t ld, int row0, int rows, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int b = p * NT + tid;
      const int kb = b & 7, mb = b >> 3;
      const int gk = k0 + kb * 8, gr = row0 + mb * 8;
      const bool ok = (kBlocks % NT == 0 || b < kBlocks) && (!BOUNDS || (gk < K && gr < rows));
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[p][i] = ok ? *(const u32x4*)(X + (int64_t)(gk + i) * ld + gr) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint8_t* stage, int tid) const {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int b = p * NT + tid;
      if (kBlocks % NT == 0 || b < kBlocks) {
        const int kb = b & 7, mb = b >> 3;
        // v[p][i] holds 8 consecutive rows (mn) at k = 8kb + i; row j of the
        // transpose holds k = 8kb .. 8kb+7 at mn = 8mb + j.
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u32x4 w;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = v[p][2 * q][j >> 1], hi = v[p][2 * q + 1][j >> 1];
            w[q] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
          }
          *(u32x4*)(stage + swz128(mb * 8 + j, kb)) = w;
        }
      }
    }
  }
};

template <bool MNMAJOR, int R, int NT, bool BOUNDS>
struct LoaderSel {
  using T = KMajorLoader<R, NT, BOUNDS>;
};
template <int R, int NT, bool BOUNDS>
struct LoaderSel<true, R, NT, BOUNDS> {
  using T = MNMajorLoader<R, NT, BOUNDS>;
};

// ------------------------------------------------------- tiled kernel ----
template <int BM, int BN, int WM, int WN, bool TA, bool TB, int DT, bool BOUNDS>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_tiled(GemmArgs g) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int kStage = (BM + BN) * 128;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStage];

  // tile scheduler: XCD-contiguous ranges, grouped tile-rows
  const int nb = (int)gridDim.x;
  int bid = (int)blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int group = kGroupM * g.tiles_n;
  const int first_m = (bid / group) * kGroupM;
  const int gsz = min(g.tiles_m - first_m, kGroupM);
  const int in_group = bid % group;
  const int tm = first_m + in_group % gsz;
  const int tn = in_group / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = (int)threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = (wave / (BN / WN)) * WM;
  const int wn = (wave % (BN / WN)) * WN;

  // TA: A stored [K][M] (M-contiguous); else [M][K].  TB: B stored [N][K]; else [K][N].
  typename LoaderSel<TA, BM, NT, BOUNDS>::T la;
  typename LoaderSel<!TB, BN, NT, BOUNDS>::T lb;
  const int64_t lda = TA ? g.M : g.K;
  const int64_t ldb = TB ? g.K : g.N;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int KT = (g.K + kBK - 1) / kBK;
  la.load(g.A, lda, m0, g.M, 0, g.K, tid);
  lb.load(g.B, ldb, n0, g.N, 0, g.K, tid);
  la.store(smem, tid);
  lb.store(smem + BM * 128, tid);
  __syncthreads();

  // per-lane fragment addressing: row (lane % 32) of each 32-row tile, k-chunk
  // 2s + lane/32 of K step s; swizzle term uses row % 8 == lane % 8.
  const uint32_t lrow = (uint32_t)(lane & 31);
  const uint32_t khalf = (uint32_t)(lane >> 5);

  for (int kt = 0; kt < KT; ++kt) {
    uint8_t* cur = smem + (kt & 1) * kStage;
    if (kt + 1 < KT) {
      la.load(g.A, lda, m0, g.M, (kt + 1) * kBK, g.K, tid);
      lb.load(g.B, ldb, n0, g.N, (kt + 1) * kBK, g.K, tid);
    }
    const uint8_t* sa = cur + (uint32_t)wm * 128;
    const uint8_t* sb = cur + BM * 128 + (uint32_t)wn * 128;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const uint32_t kc = 2u * (uint32_t)s + khalf;
      const uint32_t off = swz128(lrow, kc);
      u32x4 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = *(const u32x4*)(sa + i * 32 * 128 + off);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = *(const u32x4*)(sb + j * 32 * 128 + off);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Mfma<DT>::m32(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < KT) {
      uint8_t* nxt = smem + ((kt + 1) & 1) * kStage;
      la.store(nxt, tid);
      lb.store(nxt + BM * 128, tid);
    }
    __syncthreads();
  }

  // epilogue: lane holds column n = lane%32 of each tile, rows 8(r/4) + 4(lane/32) + r%4.
  // With beta = 1 the C values of a tile are loaded before any of its D stores: C may be
  // exactly D, so program order must already put every load ahead of the store that could
  // overwrite it; batching per tile turns 16 round trips into one.
  auto epilogue = [&](auto use_c) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn + 32 * j + (int)lrow;
        float cv[16];
        if constexpr (decltype(use_c)::value) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (int)khalf + (r & 3);
            cv[r] = (!BOUNDS || (m < g.M && n < g.N)) ? g.C[(int64_t)m * g.N + n] : 0.0f;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (int)khalf + (r & 3);
          if (!BOUNDS || (m < g.M && n < g.N)) {
            float d = acc[i][j][r];
            if constexpr (decltype(use_c)::value) d += cv[r];
            g.D[(int64_t)m * g.N + n] = d;
          }
        }
      }
    }
  };
  if (g.use_c) epilogue(std::true_type{});
  else epilogue(std::false_type{});
}

// --------------------------------------------------------- atom kernel ----
// Register kernel for small problems: one wave per output tile of the chosen matrix instruction
// (its atom), every fragment loaded from global memory straight into the registers the
// instruction reads, one instruction per K step accumulated in place — the page's primitive
// as it stands (一: all fragments in registers, one atom per output tile per K step).  The atom
// is chosen on the host among 32x32x16, 16x16x32, 32x32x8 and 16x16x16: its K depth divides K
// (K is never padded, as the page takes k16 when K allows and k8 otherwise, 二), M and N pad
// up to it (zero fragments, masked stores), and it does the least padded work, then needs the
// fewest loads per multiply-add for the operands' layouts, then is the widest.
//   lane l of an AM x AN x AK atom with R K values per lane supplies A[m0 + l % AM][k0 + R(l / AM)
//   .. + R] and B[k0 + R(l / AN) .. + R][n0 + l % AN]; the 32x32 accumulator holds D[8(e/4) +
//   4(l/32) + e%4][l%32] in register e, the 16x16 one D[4(l/16) + e][l%16].
template <int SHAPE>
struct AtomGeom {
  static constexpr int AM = (SHAPE == TG_MMA_32x32x16 || SHAPE == TG_MMA_32x32x8) ? 32 : 16;
  static constexpr int AK = SHAPE == TG_MMA_16x16x32 ? 32 : SHAPE == TG_MMA_32x32x8 ? 8 : 16;
  static constexpr int R = (SHAPE == TG_MMA_32x32x8 || SHAPE == TG_MMA_16x16x16) ? 4 : 8;
  static constexpr int ACC = AM == 32 ? 16 : 4;
};

typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

template <int SHAPE, int DT, class ACC>
__device__ __forceinline__ ACC atom_mfma(u32x4 a, u32x4 b, ACC c) {
  if constexpr (SHAPE == TG_MMA_32x32x16) return Mfma<DT>::m32(a, b, c);
  else if constexpr (SHAPE == TG_MMA_16x16x32) return Mfma<DT>::m16(a, b, c);
  else {
    const u32x2 a2 = {a[0], a[1]}, b2 = {b[0], b[1]};
    if constexpr (SHAPE == TG_MMA_32x32x8) {
      if constexpr (DT == TG_F16)
        return __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(f16x4, a2),
                                                    __builtin_bit_cast(f16x4, b2), c, 0, 0, 0);
      else
        return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(s16x4, a2),
                                                        __builtin_bit_cast(s16x4, b2), c, 0, 0, 0);
    } else {
      if constexpr (DT == TG_F16)
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a2),
                                                     __builtin_bit_cast(f16x4, b2), c, 0, 0, 0);
      else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a2),
                                                         __builtin_bit_cast(s16x4, b2), c, 0, 0, 0);
    }
  }
}

// R consecutive K values of one row (column) of an operand: one vector load when the operand
// is stored K-contiguous, one 16-bit load per value when K runs across memory lines.  Rows
// (columns) past the matrix and K past its end read as zero.
template <int R, bool KCONTIG>
__device__ __forceinline__ u32x4 atom_run(const uint16_t* p, int64_t line, int64_t ld, int64_t k,
                                          bool in) {
  u32x4 v = {0, 0, 0, 0};
  if (!in) return v;
  if constexpr (KCONTIG) {
    if constexpr (R == 8) {
      v = *(const u32x4*)(p + line * ld + k);
    } else {
      const u32x2 h = *(const u32x2*)(p + line * ld + k);
      v[0] = h[0];
      v[1] = h[1];
    }
  } else {
    uint16_t e[R];
#pragma unroll
    for (int q = 0; q < R; ++q) e[q] = p[(k + q) * ld + line];
#pragma unroll
    for (int q = 0; q < R / 2; ++q) v[q] = (uint32_t)e[2 * q] | ((uint32_t)e[2 * q + 1] << 16);
  }
  return v;
}

template <bool TA, bool TB, int DT, int SHAPE>
__global__ __launch_bounds__(64) void gemm_atom(GemmArgs g) {
  using AG = AtomGeom<SHAPE>;
  constexpr int AM = AG::AM, AN = AG::AM, AK = AG::AK, R = AG::R;
  using Acc = typename std::conditional<AG::ACC == 16, f32x16, f32x4>::type;
  const int tiles_n = (g.N + AN - 1) / AN;
  const int m0 = ((int)blockIdx.x / tiles_n) * AM;
  const int n0 = ((int)blockIdx.x % tiles_n) * AN;
  const int lane = (int)threadIdx.x;
  const int m = m0 + lane % AM, n = n0 + lane % AN;
  const int kl = R * (lane / AM);   // this lane's first K value within an atom step (AM == AN)
  Acc acc = Acc{};
  for (int k0 = 0; k0 < g.K; k0 += AK) {   // AK divides K: every step is whole
    const u32x4 a = atom_run<R, !TA>(g.A, m, TA ? g.M : g.K, k0 + kl, m < g.M);
    const u32x4 b = atom_run<R, TB>(g.B, n, TB ? g.K : g.N, k0 + kl, n < g.N);
    acc = atom_mfma<SHAPE, DT>(a, b, acc);
  }
  if (n < g.N) {
#pragma unroll
    for (int e = 0; e < AG::ACC; ++e) {
      const int mm = AM == 32 ? m0 + 8 * (e / 4) + 4 * (lane / 32) + e % 4 : m0 + 4 * (lane / 16) + e;
      if (mm < g.M) {
        const int64_t o = (int64_t)mm * g.N + n;
        float d = acc[e];
        if (g.use_c) d += g.C[o];
        g.D[o] = d;
      }
    }
  }
}

// K == 0: D = beta·C (an empty product).
__global__ __launch_bounds__(256) void gemm_fill(GemmArgs g) {
  const int64_t total = (int64_t)g.M * g.N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x)
    g.D[i] = g.use_c ? g.C[i] : 0.0f;
}

template <int BM, int BN, int WM, int WN, bool TA, bool TB, int DT>
hipError_t launch_tiled(const GemmArgs& g, const GemmConfig& c, hipStream_t s) {
  const dim3 grid((unsigned)c.grid), block((unsigned)c.threads);
  if (c.bounds)
    hipLaunchKernelGGL((gemm_tiled<BM, BN, WM, WN, TA, TB, DT, true>), grid, block, 0, s, g);
  else
    hipLaunchKernelGGL((gemm_tiled<BM, BN, WM, WN, TA, TB, DT, false>), grid, block, 0, s, g);
  return hipGetLastError();
}

template <bool TA, bool TB, int DT>
hipError_t launch_dt(const GemmArgs& g, const GemmConfig& c, hipStream_t s) {
  if (c.kernel == TG_GEMM_ATOM) {
    const dim3 gd((unsigned)c.grid), bd(64);
    switch (c.atom) {
      case TG_MMA_32x32x16: hipLaunchKernelGGL((gemm_atom<TA, TB, DT, TG_MMA_32x32x16>), gd, bd, 0, s, g); break;
      case TG_MMA_16x16x32: hipLaunchKernelGGL((gemm_atom<TA, TB, DT, TG_MMA_16x16x32>), gd, bd, 0, s, g); break;
      case TG_MMA_32x32x8: hipLaunchKernelGGL((gemm_atom<TA, TB, DT, TG_MMA_32x32x8>), gd, bd, 0, s, g); break;
      case TG_MMA_16x16x16: hipLaunchKernelGGL((gemm_atom<TA, TB, DT, TG_MMA_16x16x16>), gd, bd, 0, s, g); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (c.bm == 256) return launch_tiled<256, 256, 128, 128, TA, TB, DT>(g, c, s);
  if (c.bm == 64) return launch_tiled<64, 64, 32, 32, TA, TB, DT>(g, c, s);
  return hipErrorInvalidValue;   // 128-wide blocks run on the direct-load kernel only
}

template <int DT>
hipError_t launch_trans(const GemmArgs& g, const GemmConfig& c, int ta, int tb, hipStream_t s) {
  if (!ta && !tb) return launch_dt<false, false, DT>(g, c, s);
  if (!ta && tb) return launch_dt<false, true, DT>(g, c, s);
  if (ta && !tb) return launch_dt<true, false, DT>(g, c, s);
  return launch_dt<true, true, DT>(g, c, s);
}

}  // namespace

int launch_gemm(const GemmArgs& g, const GemmConfig& c, int trans_a, int trans_b, int dtype,
                void* stream) {
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (c.kernel == TG_GEMM_TILED && c.direct) {
    e = launch_gemm_direct(g, c.grid, trans_a, trans_b, dtype, c.bm, s);
  } else if (c.kernel == TG_GEMM_FILL) {
    hipLaunchKernelGGL(gemm_fill, dim3((unsigned)c.grid), dim3(256), 0, s, g);
    e = hipGetLastError();
  } else if (dtype == TG_F16) {
    e = launch_trans<TG_F16>(g, c, trans_a, trans_b, s);
  } else {
    e = launch_trans<TG_BF16>(g, c, trans_a, trans_b, s);
  }
  if (e != hipSuccess) return fail(TG_E_HIP, std::string("tile_gemm launch: ") + hipGetErrorString(e));
  return TG_OK;
}

}  // namespace tg
