"""GPU parity of tile_gemm against the oracle: |D - D_ref| <= 1e-4·sum|a·b| + 1e-6 per element."""

import numpy as np
import pytest
import torch

import synth
import tile_level_gemm_amd as tg
from oracle import gemm as og
from tests.gpu_util import Guarded, say, upload_bits, upload_f32

pytestmark = pytest.mark.gpu

FMT = {"f16": tg.TG_F16, "bf16": tg.TG_BF16}


def run_gemm(a_bits, b_bits, c, M, N, K, ta, tb, beta, fmt, c_is_d=False):
    A = upload_bits(a_bits)
    B = upload_bits(b_bits)
    D = Guarded(M * N * 4, fill=(c if c_is_d else np.full((M, N), np.nan, np.float32)))
    Cd = None
    if beta == 1.0 and not c_is_d:
        Cd = upload_f32(c)
    cptr = D.ptr if c_is_d else Cd
    tg.tile_gemm(A, B, cptr, D.ptr, M, N, K, ta, tb, beta, FMT[fmt])
    torch.cuda.synchronize()
    return D.host(np.float32).reshape(M, N), D.guards_intact()


def full_check(M, N, K, fmt, ta, tb, beta, seeds, dist="normal", c_is_d=False, scale=1.0):
    a_bits, b_bits, c = synth.gemm_inputs(M, N, K, fmt, ta, tb, beta, seeds, a_scale=scale,
                                          b_scale=scale, dist=dist, c_dist=dist)
    d, guards = run_gemm(a_bits, b_bits, c, M, N, K, ta, tb, beta, fmt, c_is_d=c_is_d)
    ref = og.gemm_ref(a_bits, b_bits, c, M, N, K, ta, tb, beta, fmt)
    bound = og.abs_bound(a_bits, b_bits, M, N, K, ta, tb, fmt)
    ok, worst = og.check(d, ref, bound)
    assert guards, "guard band written"
    assert ok, f"worst |D-D_ref|/tol = {worst}"
    return worst


@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_atom_16x8x16(beta):
    say(f"gemm atom 16x8x16 f16 beta={beta}")
    a_bits, b_bits, c = synth.atom_inputs(beta)
    d, guards = run_gemm(a_bits, b_bits, c, 16, 8, 16, False, False, beta, "f16")
    ref = og.gemm_ref(a_bits, b_bits, c, 16, 8, 16, False, False, beta, "f16")
    bound = og.abs_bound(a_bits, b_bits, 16, 8, 16, False, False, "f16")
    ok, worst = og.check(d, ref, bound)
    assert guards and ok, worst


# The register kernel's atoms: shapes whose choice is each of the four matrix instructions,
# in every stored orientation, with M and N padded up to the atom where they are ragged.
ATOM_SHAPES = [((16, 8, 16), tg.TG_MMA_16x16x16), ((48, 40, 16), tg.TG_MMA_16x16x16),
               ((16, 8, 8), tg.TG_MMA_32x32x8), ((48, 24, 24), tg.TG_MMA_32x32x8),
               ((16, 16, 32), tg.TG_MMA_16x16x32), ((48, 24, 96), tg.TG_MMA_16x16x32),
               ((64, 64, 48), tg.TG_MMA_32x32x16), ((32, 32, 16), tg.TG_MMA_32x32x16)]


@pytest.mark.parametrize("shape,atom", ATOM_SHAPES)
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
@pytest.mark.parametrize("fmt,beta", [("f16", 1.0), ("bf16", 0.0)])
def test_register_kernel_atoms(shape, atom, ta, tb, fmt, beta):
    M, N, K = shape
    code = FMT[fmt]
    plan = tg.tile_gemm_plan(0x100000, 0x40000000, 0x80000000 if beta else None, 0xC0000000,
                             M, N, K, int(ta), int(tb), beta, code)
    assert (plan.kernel, plan.atom) == (tg.TG_GEMM_ATOM, atom)
    say(f"gemm register atom {plan.atom} {M}x{N}x{K} {fmt} transA={ta} transB={tb} beta={beta}")
    full_check(M, N, K, fmt, ta, tb, beta, (M + 21, N + 22, K + 23))


def test_gemm_512x512x256_bf16_transb_beta1():
    say("gemm 512x512x256 bf16 transB beta=1")
    a_bits, b_bits, c = synth.gemm512_inputs()
    d, guards = run_gemm(a_bits, b_bits, c, 512, 512, 256, False, True, 1.0, "bf16")
    ref = og.gemm_ref(a_bits, b_bits, c, 512, 512, 256, False, True, 1.0, "bf16")
    bound = og.abs_bound(a_bits, b_bits, 512, 512, 256, False, True, "bf16")
    ok, worst = og.check(d, ref, bound)
    assert guards and ok, worst


# The page's tiled categories (single tile, one dim multi-tile, all dims, M = 64, K = 8,
# K = 24) plus ragged edges of every kernel configuration.
SHAPES = [(16, 8, 16), (16, 8, 8), (16, 8, 24), (32, 8, 16), (16, 24, 16), (64, 8, 16),
          (64, 64, 24), (80, 72, 40), (128, 128, 64), (192, 136, 72), (320, 264, 200),
          (528, 520, 264), (1536, 1536, 128), (1552, 1544, 136), (4096, 4096, 128),
          (4112, 4104, 72)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fmt,beta", [("f16", 0.0), ("f16", 1.0), ("bf16", 0.0), ("bf16", 1.0)])
def test_tiled_shapes(M, N, K, fmt, beta):
    say(f"gemm {M}x{N}x{K} {fmt} beta={beta}")
    full_check(M, N, K, fmt, False, False, beta, (M + 1, N + 2, K + 3))


@pytest.mark.parametrize("M,N,K", [(48, 24, 40), (320, 192, 128), (1552, 1544, 136), (4096, 4096, 640),
                                   (4112, 4104, 72)])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
def test_transposes(M, N, K, fmt, ta, tb):
    say(f"gemm {M}x{N}x{K} {fmt} transA={ta} transB={tb}")
    full_check(M, N, K, fmt, ta, tb, 1.0, (7, 8, 9))


def test_k_zero_and_empty():
    say("gemm K=0 / M=0")
    c = synth.uniform(5, 32 * 16).reshape(32, 16)
    D = Guarded(32 * 16 * 4, fill=np.full((32, 16), np.nan, np.float32))
    tg.tile_gemm(None, None, upload_f32(c), D.ptr, 32, 16, 0, 0, 0, 1.0, tg.TG_F16)
    torch.cuda.synchronize()
    assert np.array_equal(D.host(np.float32).reshape(32, 16), c) and D.guards_intact()
    tg.tile_gemm(None, None, None, D.ptr, 32, 16, 0, 0, 0, 0.0, tg.TG_BF16)
    torch.cuda.synchronize()
    assert not D.host(np.float32).any() and D.guards_intact()
    E = Guarded(64, fill=np.full(16, 7.0, np.float32))
    tg.tile_gemm(None, None, None, E.ptr, 0, 16, 16, 0, 0, 0.0, tg.TG_F16)
    torch.cuda.synchronize()
    assert np.all(E.host(np.float32) == 7.0) and E.guards_intact()


@pytest.mark.parametrize("M,N,K", [(16, 8, 16), (256, 192, 96), (1552, 1544, 136)])
def test_in_place_c_is_d(M, N, K):
    say(f"gemm in-place C==D {M}x{N}x{K}")
    full_check(M, N, K, "bf16", False, False, 1.0, (11, 12, 13), c_is_d=True)


def test_beta0_ignores_nan_c():
    say("gemm beta=0 with NaN C")
    M, N, K = 320, 264, 200
    a_bits, b_bits, _ = synth.gemm_inputs(M, N, K, "f16", False, False, 0.0, (1, 2, 3))
    A, B = upload_bits(a_bits), upload_bits(b_bits)
    Cn = torch.full((M, N), float("nan"), device="cuda:0")
    D1 = torch.empty((M, N), device="cuda:0")
    D2 = torch.empty((M, N), device="cuda:0")
    tg.tile_gemm(A, B, Cn, D1, M, N, K, 0, 0, 0.0, tg.TG_F16)
    tg.tile_gemm(A, B, None, D2, M, N, K, 0, 0, 0.0, tg.TG_F16)
    torch.cuda.synchronize()
    assert torch.isfinite(D1).all() and torch.equal(D1, D2)


# Shapes the 256x256 direct-load kernel serves without being whole blocks: ragged M and / or
# N, stage counts (64 K each) odd, even and one, and a partial last stage (K % 64 = 8 .. 56);
# M or N below one block.  Every case has at least 256 blocks, so the direct kernel runs.
DIRECT_RAGGED = [(4000, 4008, 8), (4000, 4008, 40), (4112, 4104, 64), (4096, 4096, 192),
                 (4096, 4096, 200), (4000, 4104, 136), (4016, 4000, 256), (4080, 4096, 312),
                 (16, 65544, 24), (65552, 8, 88)]


@pytest.mark.parametrize("M,N,K", DIRECT_RAGGED)
@pytest.mark.parametrize("fmt,beta", [("f16", 0.0), ("bf16", 1.0)])
def test_direct_ragged_shapes(M, N, K, fmt, beta):
    plan = tg.tile_gemm_plan(0x100000, 0x40000000, 0x80000000 if beta else None, 0xC0000000,
                             M, N, K, 0, 0, beta, FMT[fmt])
    assert (plan.block_m, plan.block_n, plan.loader) == (256, 256, 1)
    assert plan.bounds_checked == int(M % 256 != 0 or N % 256 != 0 or K % 64 != 0)
    say(f"gemm direct ragged {M}x{N}x{K} {fmt} beta={beta}")
    full_check(M, N, K, fmt, False, False, beta, (M + 5, N + 6, K + 7))


@pytest.mark.parametrize("M,N,K", [(4000, 4008, 40), (4000, 4104, 136), (16, 65544, 24),
                                   (65552, 8, 88)])
@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_direct_ragged_transposes(M, N, K, ta, tb, fmt):
    say(f"gemm direct ragged {M}x{N}x{K} {fmt} transA={ta} transB={tb}")
    full_check(M, N, K, fmt, ta, tb, 1.0, (17, 18, 19))


# 128x128 direct-load blocks: problems with fewer than 256 blocks of 256x256 but at least 128
# of 128x128; whole and ragged blocks, every stage-count shape, a partial last stage.
DIRECT_128 = [(2048, 2048, 512), (1552, 2056, 200), (128, 16384, 64), (1040, 2064, 8),
              (2048, 1024, 1032), (1536, 1536, 128)]


@pytest.mark.parametrize("M,N,K", DIRECT_128)
@pytest.mark.parametrize("fmt,beta", [("f16", 1.0), ("bf16", 0.0)])
def test_direct128_shapes(M, N, K, fmt, beta):
    plan = tg.tile_gemm_plan(0x100000, 0x40000000, 0x80000000 if beta else None, 0xC0000000,
                             M, N, K, 0, 0, beta, FMT[fmt])
    assert (plan.block_m, plan.block_n, plan.loader) == (128, 128, 1)
    say(f"gemm direct 128 {M}x{N}x{K} {fmt} beta={beta}")
    full_check(M, N, K, fmt, False, False, beta, (M + 8, N + 9, K + 10))


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_direct128_transposes(ta, tb, fmt):
    M, N, K = 1552, 2056, 200
    say(f"gemm direct 128 {M}x{N}x{K} {fmt} transA={ta} transB={tb}")
    full_check(M, N, K, fmt, ta, tb, 1.0, (24, 25, 26))


@pytest.mark.parametrize("ta,tb", [(False, False), (True, True)])
def test_direct_ragged_in_place(ta, tb):
    say(f"gemm direct ragged in-place C==D 4000x4008x136 transA={ta} transB={tb}")
    full_check(4000, 4008, 136, "bf16", ta, tb, 1.0, (21, 22, 23), c_is_d=True)


def _sampled(M, N, K, fmt, ta, tb, beta, inputs, sample_seed, tag, bounds=0, loader=1):
    a_bits, b_bits, c = inputs
    say(f"gemm {tag}: {M}x{N}x{K} {fmt} transA={ta} transB={tb} beta={beta}")
    A, B = upload_bits(a_bits), upload_bits(b_bits)
    Cd = upload_f32(c) if beta == 1.0 else None
    D = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    plan = tg.tile_gemm_plan(A, B, Cd, D, M, N, K, ta, tb, beta, FMT[fmt])
    assert (plan.block_m, plan.block_n, plan.bounds_checked, plan.loader) == (256, 256, bounds, loader)
    tg.tile_gemm(A, B, Cd, D, M, N, K, ta, tb, beta, FMT[fmt])
    D2 = torch.empty_like(D)
    tg.tile_gemm(A, B, Cd, D2, M, N, K, ta, tb, beta, FMT[fmt])
    torch.cuda.synchronize()
    assert torch.equal(D, D2), "two runs differ (no atomics: results must be bitwise repeatable)"
    rows, cols = synth.sample_points(M, N, sample_seed)
    d_gpu = D.cpu().numpy()[rows, cols]
    ref, bound = og.gemm_ref_at(a_bits, b_bits, c, M, N, K, ta, tb, beta, fmt, rows, cols)
    ok, worst = og.check(d_gpu, ref, bound)
    say(f"{tag}: worst |D-D_ref|/tol = {worst:.3g} over {rows.size} samples")
    assert ok, worst
    assert torch.isfinite(D).all()


def test_gemm_8192_bf16_beta0_sampled():
    _sampled(8192, 8192, 8192, "bf16", False, False, 0.0, synth.gemm8k_bf16_inputs(), 53, "8192 bf16")


def test_gemm_8192_f16_transa_beta1_sampled():
    _sampled(8192, 8192, 8192, "f16", True, False, 1.0, synth.gemm8k_f16_inputs(), 57, "8192 f16")


def test_gemm_8000_ragged_sampled():
    # 8000 = 31 blocks + 64 rows; 8000 K = 125 stages (odd), no partial stage
    M = N = K = 8000
    s = float(1.0 / np.sqrt(K))
    inputs = synth.gemm_inputs(M, N, K, "bf16", False, False, 0.0, (61, 62, 63), a_scale=s, b_scale=s)
    _sampled(M, N, K, "bf16", False, False, 0.0, inputs, 59, "8000 bf16", bounds=1)


def test_gemm_ragged_partial_stage_sampled():
    # K = 8008: 126 stages, the last holding 8 K; transA, beta 1
    M, N, K = 8016, 8200, 8008
    s = float(1.0 / np.sqrt(K))
    inputs = synth.gemm_inputs(M, N, K, "f16", True, False, 1.0, (64, 65, 66), a_scale=s, b_scale=s)
    _sampled(M, N, K, "f16", True, False, 1.0, inputs, 67, "ragged partial stage", bounds=1)


# Operands at the direct kernel's limit: its buffer offsets are 32-bit, so it serves operands
# under 2 GiB; from 2 GiB on the 64-bit-indexed tiled kernel takes over.
@pytest.mark.parametrize("ta", [False, True])
def test_gemm_operand_just_under_2gib_sampled(ta):
    # A = 130928 x 8200 f16 = 2 GiB - 256 KiB; ragged M, and a last stage of 8 K
    M, N, K = 130928, 256, 8200
    assert M * K * 2 < 1 << 31
    s = float(1.0 / np.sqrt(K))
    inputs = synth.gemm_inputs(M, N, K, "f16", ta, False, 1.0, (71, 72, 73), a_scale=s, b_scale=s)
    _sampled(M, N, K, "f16", ta, False, 1.0, inputs, 74, "A just under 2 GiB", bounds=1)


def test_gemm_operand_of_2gib_sampled():
    # A = 131072 x 8192 f16 = 2 GiB: the tiled kernel, element offsets past 2^31 bytes
    M, N, K = 131072, 256, 8192
    s = float(1.0 / np.sqrt(K))
    inputs = synth.gemm_inputs(M, N, K, "f16", False, True, 0.0, (75, 76, 0), a_scale=s, b_scale=s)
    _sampled(M, N, K, "f16", False, True, 0.0, inputs, 77, "A of 2 GiB", bounds=0, loader=0)
