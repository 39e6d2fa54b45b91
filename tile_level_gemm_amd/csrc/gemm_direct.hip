// Large-tile GEMM on gfx950 with direct global -> LDS operand loads.
//
// Same contract as gemm_tiled ([SYNC-GEMM] "TVM TIRx 同步 GEMM 深度解析…": D = A·B (+C),
// fp32 accumulation in place over K, 二 / 四 step 3), for whole 256x256 blocks and K a
// multiple of 128.  What changes is how operands reach the MFMAs:
//
//  * global -> LDS with buffer_load_dwordx4 ... lds: each instruction moves 64 lanes x 16 bytes
//    and lane i's bytes land at LDS base + 16·i, so no VGPR staging and no ds_write.  The
//    LDS swizzle is applied on the global side: lane i fetches the logical 16-byte chunk
//    that belongs at physical slot i.
//  * K-contiguous operands (A without transA, B with transB) keep [rows][64 k] stages
//    of 128-byte rows (chunk XOR row bits) and are read as fragments with ds_read_b128.
//  * M/N-contiguous operands (A with transA, B without transB) keep the global orientation,
//    [64 k][256 mn] stages of 512-byte rows, and are read with ds_read_b64_tr_b16: within
//    each 16-lane group, lane j receives element j%4 of the 8-byte reads of lanes
//    4q + j/4 (q = 0..3), so if lane i reads 4 consecutive mn at k-row k0 + i/4 and
//    column block i%4, lane j receives k0..k0+3 at mn0 + j — four K-consecutive values,
//    half of an MFMA fragment.
//  * the K loop is unrolled by two so each half names its LDS stage at compile time; the
//    next stage's loads are issued at the top of an iteration and the next K step's
//    fragments are read while the current step's 16 MFMAs run.
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
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGroupM = 8;   // tile-rows per scheduling group (measured: 8 beats 2, 4, 16)

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == TG_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- LDS layouts --------------------------------------------------------------------
// K-major stage: 256 rows x 128 bytes; physical chunk = kc ^ sk(row).
//   SK 0: row & 7 — eight consecutive rows hit eight chunks (32 four-byte banks);
//   SK 1: (row & 7) ^ ((row >> 3) & 1) — also sixteen consecutive rows hit sixteen distinct
//         (row parity, chunk) pairs, i.e. distinct banks if the LDS has 64 banks.
template <int SK>
__device__ __forceinline__ uint32_t sk(uint32_t r) {
  if constexpr (SK == 0) return r & 7u;
  else return (r & 7u) ^ ((r >> 3) & 1u);
}
// M/N-major stage: 64 k-rows x 512 bytes (32 chunks); physical chunk = c ^ sm(k).  A
// transposing read touches 32 bytes (2 chunks) in each of 4 consecutive k-rows per 16 lanes.
//   SM 0: 2(k & 3) — the four rows land in four distinct 32-byte bank slots of 128 bytes;
//   SM 1: 2(k & 3) ^ 8(k & 1) — additionally, two adjacent 16-lane groups (mn + 16) land
//         in eight distinct slots of 256 bytes.
template <int SM>
__device__ __forceinline__ uint32_t sm(uint32_t k) {
  if constexpr (SM == 0) return (k & 3u) << 1;
  else return ((k & 3u) << 1) ^ ((k & 1u) << 3);
}

// ---- per-lane offsets, computed once ---------------------------------------------------
// Every address below is a per-lane offset computed before the K loop plus compile-time
// immediates (tile, K step, stage), so the loop keeps few address registers.
constexpr int SKV = 1, SMV = 1;   // swizzle variants in use (see sk / sm)

// DMA (global -> LDS) for a K-major operand: PER instructions per wave per stage; instruction
// i writes 1 KiB block b = PER·wave + i = rows 8b .. 8b+7.  Lane l fills physical slot l%8
// of row 8b + l/8 and so fetches logical chunk (l%8) ^ sk(row).  sk(row) depends on the
// lane and on i's parity only (PER is even), so two byte offsets cover all instructions.
template <int PER>
__device__ __forceinline__ void km_dma_offsets(int64_t ld, int wave, int lane, uint32_t (&off)[2]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t r = (uint32_t)(8 * PER * wave + 8 * p + (lane >> 3));
    const uint32_t kc = ((uint32_t)lane & 7u) ^ sk<SKV>(r);
    off[p] = (r * (uint32_t)ld + kc * 8u) * 2u;   // bytes; < 256·K·2 < 2^32
  }
}
// DMA for an M/N-major operand: instruction i writes block b = PER·wave + i = k-rows 2b,
// 2b+1; lane l fills slot l%32 of k-row 2b + l/32, logical chunk (l%32) ^ sm(k); sm depends
// on k & 3, i.e. on the lane and i's parity.
template <int PER>
__device__ __forceinline__ void mn_dma_offsets(int64_t ld, int wave, int lane, uint32_t (&off)[2]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t k = (uint32_t)(2 * PER * wave + 2 * p + (lane >> 5));
    const uint32_t c = ((uint32_t)lane & 31u) ^ sm<SMV>(k);
    off[p] = (k * (uint32_t)ld + c * 8u) * 2u;    // bytes; < 64·N·2 < 2^32
  }
}

// K-major fragment (ds_read_b128) of 32-row tile t, K step s: lane l reads row
// base + 32t + l%32, chunk 2s + l/32.  sk(row) depends on the lane only (32t is a multiple
// of 16), the chunk term on s: one byte offset per s; tiles are +4096-byte immediates.
__device__ __forceinline__ void km_frag_offsets(int row_base, int lane, uint32_t (&off)[4]) {
  const uint32_t r = (uint32_t)(row_base + (lane & 31));
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t kc = (uint32_t)(2 * s + (lane >> 5));
    off[s] = r * 128u + ((kc ^ sk<SKV>(r)) << 4);
  }
}
// M/N-major fragment of 32-column tile t, K step s, half h (two ds_read_b64_tr_b16): lane
// l = 16g + j supplies k-row 16s + 8(g/2) + 4h + j/4 and columns mn_base + 32t + 16(g&1) +
// 4(j&3) .. +3.  sm(k) depends on j only; its bits 2-3 XOR with the tile index, so one byte
// offset per tile t; s and h are immediates (16s + 4h rows of 512 bytes).
template <int T>
__device__ __forceinline__ void mn_frag_offsets(int mn_base, int lane, uint32_t (&off)[4]) {
  const uint32_t g = (uint32_t)lane >> 4, j = (uint32_t)lane & 15u;
  const uint32_t krow = 8u * (g >> 1) + (j >> 2);
  const uint32_t x = sm<SMV>(krow);
  const uint32_t mn_lane = 16u * (g & 1u) + 4u * (j & 3u);
  const uint32_t byte = (mn_lane & 7u) * 2u;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t c = ((uint32_t)mn_base + 32u * (uint32_t)(t < T ? t : 0) + mn_lane) >> 3;
    off[t] = krow * 512u + ((c ^ x) << 4) + byte;
  }
}

// One operand of one wave: T fragments of 32 rows/columns per K step, PER DMA instructions
// per stage.
template <bool MN, int T, int PER>
struct Operand {
  uint32_t dma[2];   // byte offsets of the two DMA parities
  uint32_t frag[4];  // byte offsets: per K step (K-major) or per tile (M/N-major)

  static constexpr int kReads = MN ? 2 * T : T;   // LDS read instructions per K step

  __device__ __forceinline__ void init(int64_t ld, int base, int wave, int lane) {
    if constexpr (MN) {
      mn_dma_offsets<PER>(ld, wave, lane, dma);
      mn_frag_offsets<T>(base, lane, frag);
    } else {
      km_dma_offsets<PER>(ld, wave, lane, dma);
      km_frag_offsets(base, lane, frag);
    }
  }
  // Buffer descriptor of this operand's panel: base = the block's first element at K stage
  // 0, num_records = bytes from there to the end of the operand (reads past it return 0).
  __amdgpu_buffer_rsrc_t rsrc;

  __device__ __forceinline__ void bind(const uint16_t* panel, int64_t bytes_left) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)panel, (short)0, (int)bytes_left, 0x00020000);
  }
  // Issue the PER DMA instructions of one stage (buffer_load_dwordx4 ... lds): per-lane byte
  // offset `dma[i & 1]` (VGPR), stage and instruction offset `soff` (SGPR), LDS block address
  // in M0 — no per-instruction vector arithmetic.  `wave` is wave-uniform.
  __device__ __forceinline__ void load(uint32_t stage_off, int64_t ld, uint8_t* stage,
                                       int wave) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      // K-major: +8 rows per instruction pair; M/N-major: +2 k-rows per instruction pair
      const uint32_t step = MN ? (uint32_t)(2 * (i & ~1)) * (uint32_t)ld * 2u
                               : (uint32_t)(8 * (i & ~1)) * (uint32_t)ld * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + (wave * PER + i) * 1024),
                                               16, dma[i & 1], stage_off + step, 0, 0);
    }
  }
  __device__ __forceinline__ void frags(const uint8_t* stage, int s, u32x4 (&f)[T]) const {
    if constexpr (MN) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        u32x4 out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint8_t* p = stage + frag[t] + (16 * s + 4 * h) * 512;
          const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
          out[2 * h] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
          out[2 * h + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
        }
        f[t] = out;
      }
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t) f[t] = *(const u32x4*)(stage + frag[s] + t * 4096);
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

// WGM x WGN waves; wave tile (256/WGM) x (256/WGN).
template <bool A_MN, bool B_MN, int DT, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_direct(GemmArgs g) {
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int PER = 32 / NW;   // DMA blocks per operand per wave per stage
  static_assert(PER % 2 == 0 && TM >= 1 && TN >= 1 && TM <= 4 && TN <= 4, "wave grid");
  __shared__ __attribute__((aligned(1024))) uint8_t sa0[BM * BK * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t sb0[BN * BK * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t sa1[BM * BK * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t sb1[BN * BK * 2];

  // tile scheduler: XCD-contiguous ranges, grouped tile-rows (as gemm_tiled)
  const int nb = (int)gridDim.x;
  int bid = (int)blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int group = kGroupM * g.tiles_n;
  const int first_m = (bid / group) * kGroupM;
  const int gsz = min(g.tiles_m - first_m, kGroupM);
  const int tm = first_m + (bid % group) % gsz;
  const int tn = (bid % group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = (int)threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = (wave / WGN) * WM, wn = (wave % WGN) * WN;

  const int64_t lda = A_MN ? g.M : g.K;
  const int64_t ldb = B_MN ? g.N : g.K;
  using OA = Operand<A_MN, TM, PER>;
  using OB = Operand<B_MN, TN, PER>;
  OA oa;
  OB ob;
  oa.init(lda, wm, wave, lane);
  ob.init(ldb, wn, wave, lane);
  // operand panels of this block at K stage 0, and the per-stage advance in bytes
  const int64_t a0 = A_MN ? (int64_t)m0 : (int64_t)m0 * g.K;
  const int64_t b0 = B_MN ? (int64_t)n0 : (int64_t)n0 * g.K;
  oa.bind(g.A + a0, ((int64_t)g.M * g.K - a0) * 2);
  ob.bind(g.B + b0, ((int64_t)g.K * g.N - b0) * 2);
  const uint32_t adv_a = A_MN ? (uint32_t)(BK * g.M * 2) : (uint32_t)(BK * 2);
  const uint32_t adv_b = B_MN ? (uint32_t)(BK * g.N * 2) : (uint32_t)(BK * 2);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  auto mfmas = [&](const u32x4 (&a)[TM], const u32x4 (&b)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32<DT>(a[i], b[j], acc[i][j]);
  };

  // Pipeline (K stage kt in buffer `cur`, kt+1 already loading into `nxt`):
  //   steps 0..2: read step s+1's fragments while step s's MFMAs run;
  //   wait for this wave's DMA and LDS reads, barrier: stage kt+1 is complete in `nxt` and no
  //   wave reads `cur` any more;
  //   then step 3's MFMAs (operands already in registers) overlap the reads of stage kt+1's
  //   first fragments and the DMA of stage kt+2 into `cur`.
  // The last two stages are peeled off the loop so the steady-state body is branch free.
  const int KT = g.K / BK;   // even and >= 2: K % 128 == 0, K > 0
  oa.load(0u, lda, sa0, wave);
  ob.load(0u, ldb, sb0, wave);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  u32x4 a[TM], b[TN], an[TM], bn[TN];
  oa.frags(sa0, 0, a);
  ob.frags(sb0, 0, b);
  if (KT > 1) {
    oa.load(adv_a, lda, sa1, wave);
    ob.load(adv_b, ldb, sb1, wave);
  }

  constexpr int kMfma = TM * TN;
  constexpr int kReads = OA::kReads + OB::kReads;
  constexpr int kDma = 2 * PER;

  // One K stage.  DMA: also load stage kt+2 into the buffer this stage frees; NEXT: read
  // the next stage's first fragments (false only for the last stage).
  auto stage = [&](uint8_t* ca, uint8_t* cb, const uint8_t* na, const uint8_t* nb_, int kt,
                   auto dma, auto next) {
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      oa.frags(ca, s + 1, an);
      ob.frags(cb, s + 1, bn);
      mfmas(a, b);
      interleave<kMfma, kReads, 0>();
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = an[i];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = bn[j];
    }
    __builtin_amdgcn_sched_barrier(0);   // keep step 2's MFMAs ahead of the wait
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (decltype(next)::value) {
      oa.frags(na, 0, an);
      ob.frags(nb_, 0, bn);
    }
    if constexpr (decltype(dma)::value) {
      oa.load((uint32_t)(kt + 2) * adv_a, lda, ca, wave);
      ob.load((uint32_t)(kt + 2) * adv_b, ldb, cb, wave);
    }
    mfmas(a, b);
    if constexpr (decltype(dma)::value) interleave<kMfma, kReads, kDma>();
    else if constexpr (decltype(next)::value) interleave<kMfma, kReads, 0>();
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = an[i];
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = bn[j];
  };

  // Steady state: stages kt, kt+1 with kt + 3 < KT (both issue DMA); then the last two.
  using T_ = std::true_type;
  using F_ = std::false_type;
  int kt = 0;
  for (; kt + 2 < KT; kt += 2) {
    stage(sa0, sb0, sa1, sb1, kt, T_{}, T_{});
    stage(sa1, sb1, sa0, sb0, kt + 1, T_{}, T_{});
  }
  stage(sa0, sb0, sa1, sb1, kt, F_{}, T_{});
  stage(sa1, sb1, sa0, sb0, kt + 1, F_{}, F_{});

  // epilogue: lane holds column n = lane%32 of each tile, rows 8(r/4) + 4(lane/32) + r%4
  const int lrow = lane & 31, khalf = lane >> 5;
  float* dbase = g.D + (int64_t)(m0 + wm + 4 * khalf) * g.N + (n0 + wn + lrow);
  if (g.use_c) {
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
        cv[0][j][r] = cbase[(int64_t)(8 * (r >> 2) + (r & 3)) * g.N + 32 * j];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i + 1 < TM) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            cv[(i + 1) & 1][j][r] =
                cbase[(int64_t)(32 * (i + 1) + 8 * (r >> 2) + (r & 3)) * g.N + 32 * j];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t o = (int64_t)(32 * i + 8 * (r >> 2) + (r & 3)) * g.N + 32 * j;
          dbase[o] = acc[i][j][r] + cv[i & 1][j][r];
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
          dbase[o] = acc[i][j][r];
        }
  }
}

// LDS swizzles: both operands use variant 1 (conflict-free for 64-bank reads; measured
// zero SQ_LDS_BANK_CONFLICT on gfx950, against 50 % of LDS-active cycles with variant 0).
// Wave grid 2 x 4 (8 waves, 128 x 64 each, 2 per SIMD): measured 1-2 % ahead of 2 x 2
// (4 waves of 128 x 128) on the same box; 4 x 2 spills.
template <bool A_MN, bool B_MN, int DT>
hipError_t launch_direct_dt(const GemmArgs& g, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_direct<A_MN, B_MN, DT, 2, 4>), dim3((unsigned)grid), dim3(512), 0, s, g);
  return hipGetLastError();
}

}  // namespace

// Whole 256x256 tiles, K a multiple of 128, and each operand under 2 GiB so that every
// buffer offset (per-lane plus per-stage) fits the 32-bit offset fields.
bool direct_gemm_fits(int64_t M, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)1 << 31;
  return M % BM == 0 && N % BN == 0 && K % (2 * BK) == 0 && K > 0 && M * K * 2 < lim &&
         K * N * 2 < lim;
}

hipError_t launch_gemm_direct(const GemmArgs& g, int64_t grid, int trans_a, int trans_b, int dtype,
                              hipStream_t s) {
  // A is M/N-major when stored [K][M] (transA); B is M/N-major when stored [K][N] (!transB).
  const bool amn = trans_a != 0, bmn = trans_b == 0;
  if (dtype == TG_F16) {
    if (amn && bmn) return launch_direct_dt<true, true, TG_F16>(g, grid, s);
    if (amn) return launch_direct_dt<true, false, TG_F16>(g, grid, s);
    if (bmn) return launch_direct_dt<false, true, TG_F16>(g, grid, s);
    return launch_direct_dt<false, false, TG_F16>(g, grid, s);
  }
  if (amn && bmn) return launch_direct_dt<true, true, TG_BF16>(g, grid, s);
  if (amn) return launch_direct_dt<true, false, TG_BF16>(g, grid, s);
  if (bmn) return launch_direct_dt<false, true, TG_BF16>(g, grid, s);
  return launch_direct_dt<false, false, TG_BF16>(g, grid, s);
}

}  // namespace tg
