// Block-scaled GEMM with 6- and 4-bit operands on gfx950: D = sum_k (SA·A)(SB·B) (+C).
//
// [SYNC-GEMM] ("TVM TIRx 同步 GEMM 深度解析…") 七: the asynchronous GEMM takes fp4 operands with
// SFA / SFB block scales, A and B staged in shared memory, the product accumulated in fp32.
// Here the operands are the OCP microscaling element types e2m3, e3m2 (6-bit) and e2m1 (4-bit),
// stored K-contiguous as packed rows (code k at bits [w·k, w·k + w) of the row's little-endian
// bit stream), with one E8M0 scale per 32 K of each row of A and of B.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with the 6- / 4-bit format codes (2 = e2m3, 3 = e3m2,
// 4 = e2m1).  An in-bounds probe on gfx950 fixed its operand map for these formats: lane l
// holds row (column) l % 32 and the 32 consecutive K of block l / 32 of the 64-K step, as one
// packed bit stream (slot s at bit w·s of its registers); A and B pair slot for slot, and the
// block's scale is the lane's own scale register.  (The 8-bit formats split a lane's 32
// values over both blocks instead.)  So a lane's operand is one contiguous run of a stored
// row: 16 bytes of fp4 or 24 bytes of fp6.
//
// Kernel: BS x BS blocks, 128 (4 waves of 64x64) or 256 (8 waves of 128x64, for problems with at
// least 256 such blocks: half the operand traffic per flop), 128-K stages.
//  * global -> LDS through registers: a stage row is 64 (fp4) or 96 (fp6) bytes, moved as
//    16-byte chunks (consecutive threads take consecutive chunks of a row: coalesced); rows
//    past M or N are written as zeros;
//  * LDS rows are padded to 80 / 104 bytes so that the 32 rows one fragment read touches start
//    in distinct bank groups (20 and 26 four-byte banks apart, both spread over all 64 banks):
//    one ds_read_b128 per fp4 fragment, three ds_read_b64 per fp6 fragment;
//  * the stage's scales (4 bytes per row for 128 K) go to LDS beside it; a lane reads its row's
//    4 bytes, shifted by 8·(lane / 32) so that op_sel = 2·step picks the byte of its block;
//  * two stages (double buffer), the next stage's loads in flight during the MFMAs, one
//    workgroup barrier per stage;
//  * epilogue D = acc (+ C), masked past M and N.
#include <hip/hip_runtime.h>

#include "tg_internal.h"

namespace tg {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kBK = 128;
constexpr int kGroupM = 8;   // tile-rows per scheduling group

// Per operand format code (2 = e2m3, 3 = e3m2, 4 = e2m1) and block size BS: bits per value,
// bytes of one row per stage, padded LDS pitch, 16-byte chunks per row, and chunks per thread
// (256 threads on 128-wide blocks, 512 on 256-wide ones).
template <int F, int BS>
struct Pk {
  static constexpr int kThreads = BS == 256 ? 512 : 256;
  static constexpr int kBits = F == 4 ? 4 : 6;
  static constexpr int kRow = kBK * kBits / 8;          // 64 or 96
  static constexpr int kPitch = F == 4 ? 80 : 104;
  static constexpr int kChunks = kRow / 16;              // 4 or 6
  static constexpr int kPer = BS * kChunks / kThreads;   // 2 or 3 chunks per thread
};

// One operand's stage: global -> registers -> LDS.
template <int F, int BS, bool BOUNDS>
struct PkLoader {
  using P = Pk<F, BS>;
  u32x4 v[P::kPer];
  __device__ __forceinline__ void load(const uint8_t* base, int64_t row_bytes, int rows_left,
                                       int kt, int tid) {
#pragma unroll
    for (int i = 0; i < P::kPer; ++i) {
      const int c = tid + i * P::kThreads;
      const int r = c / P::kChunks, q = c - r * P::kChunks;
      if (!BOUNDS || r < rows_left)
        v[i] = *(const u32x4*)(base + (int64_t)r * row_bytes + (int64_t)kt * P::kRow + q * 16);
      else
        v[i] = u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < P::kPer; ++i) {
      const int c = tid + i * P::kThreads;
      const int r = c / P::kChunks, q = c - r * P::kChunks;
      uint8_t* p = lds + r * P::kPitch + q * 16;
      if constexpr (P::kPitch % 16 == 0) {
        *(u32x4*)p = v[i];
      } else {
        *(u32x2*)p = u32x2{v[i][0], v[i][1]};
        *(u32x2*)(p + 8) = u32x2{v[i][2], v[i][3]};
      }
    }
  }
};

// This lane's 32 K values of row `row` in 64-K step s: bytes (64s + 32h)·bits/8 of the row.
template <int F>
__device__ __forceinline__ i32x8 pk_frag(const uint8_t* lds, int row, int s, int h) {
  using P = Pk<F, 128>;
  const uint8_t* p = lds + row * P::kPitch + (64 * s + 32 * h) * P::kBits / 8;
  i32x8 f = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (F == 4) {
    const u32x4 x = *(const u32x4*)p;
    f[0] = (int)x[0]; f[1] = (int)x[1]; f[2] = (int)x[2]; f[3] = (int)x[3];
  } else {
    const u32x2 x0 = *(const u32x2*)p, x1 = *(const u32x2*)(p + 8), x2 = *(const u32x2*)(p + 16);
    f[0] = (int)x0[0]; f[1] = (int)x0[1]; f[2] = (int)x1[0]; f[3] = (int)x1[1];
    f[4] = (int)x2[0]; f[5] = (int)x2[1];
  }
  return f;
}

template <int AF, int BF, int OPSEL>
__device__ __forceinline__ f32x16 pk_mfma(i32x8 a, i32x8 b, f32x16 c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, AF, BF, OPSEL, (int)sa, OPSEL,
                                                         (int)sb);
}

template <int AF, int BF, bool BOUNDS, int BS>
__global__ __launch_bounds__(BS == 256 ? 512 : 256) void gemm_mx_packed(GemmArgs g) {
  using PA = Pk<AF, BS>;
  using PB = Pk<BF, BS>;
  constexpr int kBM = BS, kBN = BS;
  constexpr int WGN = BS == 256 ? 4 : 2;                 // waves along N (2 along M)
  constexpr int WM = BS / 2, WN = BS / WGN;              // 128x64 or 64x64
  constexpr int TM = WM / 32, TN = WN / 32;
  __shared__ __attribute__((aligned(16))) uint8_t la[2][kBM * PA::kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t lb[2][kBN * PB::kPitch];
  __shared__ __attribute__((aligned(16))) uint32_t ls[2][kBM + kBN];   // 4 scale bytes per row

  // tile scheduler: XCD-contiguous ranges, groups of kGroupM tile-rows
  const int nb = (int)gridDim.x;
  int bid = (int)blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int group = kGroupM * g.tiles_n;
  const int first_m = (bid / group) * kGroupM;
  const int gsz = min(g.tiles_m - first_m, kGroupM);
  const int m0 = (first_m + (bid % group) % gsz) * kBM;
  const int n0 = ((bid % group) / gsz) * kBN;

  const int tid = (int)threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave / WGN) * WM, wn = (wave % WGN) * WN;
  const int h = lane >> 5, lr = lane & 31;

  const int64_t rowa = (int64_t)g.K * PA::kBits / 8, rowb = (int64_t)g.K * PB::kBits / 8;
  const uint8_t* abase = (const uint8_t*)g.A + (int64_t)m0 * rowa;
  const uint8_t* bbase = (const uint8_t*)g.B + (int64_t)n0 * rowb;
  const int ma = g.M - m0, nbl = g.N - n0;
  const int kb = g.K / 32;   // scale bytes per row
  // scales: threads 0..BS-1 carry A's rows, BS..2BS-1 B's; one 4-byte load per row and stage
  const bool sa_side = tid < kBM;
  const int srow = sa_side ? tid : tid - kBM;
  const bool s_in = !BOUNDS || srow < (sa_side ? ma : nbl);
  const uint8_t* sbase = sa_side ? g.SA + (int64_t)(m0 + srow) * kb : g.SB + (int64_t)(n0 + srow) * kb;

  PkLoader<AF, BS, BOUNDS> lda;
  PkLoader<BF, BS, BOUNDS> ldb;
  uint32_t sv = 0;
  auto gload = [&](int kt) {
    lda.load(abase, rowa, ma, kt, tid);
    ldb.load(bbase, rowb, nbl, kt, tid);
    sv = s_in ? *(const uint32_t*)(sbase + 4 * kt) : 0u;
  };
  auto lstore = [&](int buf) {
    lda.store(la[buf], tid);
    ldb.store(lb[buf], tid);
    ls[buf][tid] = sv;
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  auto compute = [&](int buf) {
    // the scale words of this lane's rows, shifted so that byte 2s is block 2s + h
    uint32_t qa[TM], qb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) qa[i] = ls[buf][wm + 32 * i + lr] >> (8 * h);
#pragma unroll
    for (int j = 0; j < TN; ++j) qb[j] = ls[buf][kBM + wn + 32 * j + lr] >> (8 * h);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      i32x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = pk_frag<AF>(la[buf], wm + 32 * i + lr, s, h);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = pk_frag<BF>(lb[buf], wn + 32 * j + lr, s, h);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if (s == 0) acc[i][j] = pk_mfma<AF, BF, 0>(a[i], b[j], acc[i][j], qa[i], qb[j]);
          else acc[i][j] = pk_mfma<AF, BF, 2>(a[i], b[j], acc[i][j], qa[i], qb[j]);
        }
    }
  };

  const int KT = g.K / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    compute(buf);
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column lr of each tile, rows 8(e/4) + 4h + e%4
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        const int c = n0 + wn + 32 * j + lr;
        if (!BOUNDS || (r < g.M && c < g.N)) {
          const int64_t o = (int64_t)r * g.N + c;
          g.D[o] = g.use_c ? acc[i][j][e] + g.C[o] : acc[i][j][e];
        }
      }
}

template <int AF, int BF, int BS>
hipError_t launch_pk(const GemmArgs& g, int64_t grid, bool bounds, hipStream_t s) {
  const dim3 gd((unsigned)grid), bd(BS == 256 ? 512 : 256);
  if (bounds)
    hipLaunchKernelGGL((gemm_mx_packed<AF, BF, true, BS>), gd, bd, 0, s, g);
  else
    hipLaunchKernelGGL((gemm_mx_packed<AF, BF, false, BS>), gd, bd, 0, s, g);
  return hipGetLastError();
}

template <int AF>
hipError_t launch_pk_b(const GemmArgs& g, int64_t grid, int b_fmt, bool bounds, int bs, hipStream_t s) {
  switch (b_fmt) {
    case 2: return bs == 256 ? launch_pk<AF, 2, 256>(g, grid, bounds, s) : launch_pk<AF, 2, 128>(g, grid, bounds, s);
    case 3: return bs == 256 ? launch_pk<AF, 3, 256>(g, grid, bounds, s) : launch_pk<AF, 3, 128>(g, grid, bounds, s);
    case 4: return bs == 256 ? launch_pk<AF, 4, 256>(g, grid, bounds, s) : launch_pk<AF, 4, 128>(g, grid, bounds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int packed_lds_bytes(int a_fmt, int b_fmt, int bs) {
  auto pitch = [](int f) { return f == 4 ? 80 : 104; };
  return 2 * bs * (pitch(a_fmt) + pitch(b_fmt)) + 2 * 2 * bs * 4;
}

hipError_t launch_gemm_mx_packed(const GemmArgs& g, int64_t grid, int a_fmt, int b_fmt, bool bounds,
                                 int bs, hipStream_t s) {
  switch (a_fmt) {
    case 2: return launch_pk_b<2>(g, grid, b_fmt, bounds, bs, s);
    case 3: return launch_pk_b<3>(g, grid, b_fmt, bounds, bs, s);
    case 4: return launch_pk_b<4>(g, grid, b_fmt, bounds, bs, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tg
