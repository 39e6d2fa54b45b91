"""GPU parity of tile_gemm_mx (block-scaled fp8, [SYNC-GEMM] 七: the SFA / SFB scale factors)
against the oracle, with the fp8 bar computed on the scaled products."""

import numpy as np
import pytest
import torch

import synth
import tile_level_gemm_amd as tg
from oracle import gemm as og
from tests.gpu_util import Guarded, say, upload_bits, upload_f32

pytestmark = pytest.mark.gpu

FMT = {"e4m3": tg.TG_FP8_E4M3, "e5m2": tg.TG_FP8_E5M2}


def mx_case(M, N, K, af, bf, ta, tb, beta, seed, lo=117, hi=137):
    a, b, c = synth.gemm_fp8_inputs(M, N, K, af, bf, ta, tb, beta, (seed, seed + 1, seed + 2))
    g = synth.rng(seed + 3)
    sa = g.integers(lo, hi + 1, size=(M, K // 32)).astype(np.uint8)
    sb = g.integers(lo, hi + 1, size=(N, K // 32)).astype(np.uint8)
    return a, b, sa, sb, c


def run_mx(a, b, sa, sb, c, M, N, K, ta, tb, beta, af, bf, c_is_d=False):
    D = Guarded(M * N * 4, fill=(c if c_is_d else np.full((M, N), np.nan, np.float32)))
    Cd = upload_f32(c) if beta == 1.0 and not c_is_d else None
    tg.tile_gemm_mx(upload_bits(a), upload_bits(b), upload_bits(sa), upload_bits(sb),
                    D.ptr if c_is_d else Cd, D.ptr, M, N, K, int(ta), int(tb), beta, FMT[af], FMT[bf])
    torch.cuda.synchronize()
    return D.host(np.float32).reshape(M, N), D.guards_intact()


def full_check(M, N, K, af, bf, ta, tb, beta, seed, c_is_d=False):
    a, b, sa, sb, c = mx_case(M, N, K, af, bf, ta, tb, beta, seed)
    d, guards = run_mx(a, b, sa, sb, c, M, N, K, ta, tb, beta, af, bf, c_is_d)
    ref = og.gemm_mx_ref(a, b, sa, sb, c, M, N, K, ta, tb, beta, af, bf)
    bound = og.abs_bound_mx(a, b, sa, sb, M, N, K, ta, tb, af, bf)
    ok, worst = og.check_fp8(d, ref, bound, a, b, M, N, K, ta, tb, af, bf, sa_bits=sa, sb_bits=sb)
    assert guards, "guard band written"
    assert ok, f"worst |D-D_ref|/tol = {worst}"


# K in stages of 128: one, two, three, five, 11 and 25 (the scales travel in groups of four
# stages through a three-slot ring: partial last groups and several turns of the ring).
@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (48, 32, 128), (256, 256, 256), (272, 528, 384),
                                   (784, 1040, 640), (1024, 1024, 2048), (528, 784, 1408),
                                   (1040, 272, 3200)])
@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_shapes(M, N, K, beta):
    say(f"gemm_mx {M}x{N}x{K} e4m3 x e4m3 beta={beta}")
    full_check(M, N, K, "e4m3", "e4m3", False, True, beta, M + N + K)


@pytest.mark.parametrize("ta,tb", [(False, False), (True, True), (True, False), (False, True)])
@pytest.mark.parametrize("af,bf", [("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")])
def test_layouts_and_formats(ta, tb, af, bf):
    say(f"gemm_mx 528x272x640 {af} x {bf} transA={ta} transB={tb}")
    full_check(528, 272, 640, af, bf, ta, tb, 1.0, 31)


def test_wide_scale_range():
    """Scales over 2^-60 .. 2^60 per block: each block's scale reaches the right products."""
    say("gemm_mx wide scales")
    M, N, K = 256, 256, 512
    a, b, sa, sb, _ = mx_case(M, N, K, "e4m3", "e4m3", False, True, 0.0, 5, lo=67, hi=187)
    d, guards = run_mx(a, b, sa, sb, None, M, N, K, False, True, 0.0, "e4m3", "e4m3")
    ref = og.gemm_mx_ref(a, b, sa, sb, None, M, N, K, False, True, 0.0, "e4m3", "e4m3")
    bound = og.abs_bound_mx(a, b, sa, sb, M, N, K, False, True, "e4m3", "e4m3")
    ok, worst = og.check_fp8(d, ref, bound, a, b, M, N, K, False, True, "e4m3", "e4m3", sa_bits=sa,
                             sb_bits=sb)
    assert guards and ok, worst


def test_nan_scale():
    """E8M0 0xFF is NaN: its row of A (column of B) gives NaN where the block has a nonzero
    product, and every other output stays finite."""
    say("gemm_mx NaN scale")
    M, N, K = 256, 256, 256
    a, b, sa, sb, _ = mx_case(M, N, K, "e4m3", "e4m3", False, True, 0.0, 9)
    a = np.full_like(a, 0x38)
    b = np.full_like(b, 0x38)
    sa[17, 3] = 255
    sb[200, 0] = 255
    d, guards = run_mx(a, b, sa, sb, None, M, N, K, False, True, 0.0, "e4m3", "e4m3")
    ref = og.gemm_mx_ref(a, b, sa, sb, None, M, N, K, False, True, 0.0, "e4m3", "e4m3")
    assert guards
    assert np.array_equal(np.isnan(d), np.isnan(ref))
    # the finite outputs to the fp8 bar (bound and allowance of the scaled products)
    sa_ok, sb_ok = sa.copy(), sb.copy()
    sa_ok[17, 3] = 127
    sb_ok[200, 0] = 127
    bound = og.abs_bound_mx(a, b, sa_ok, sb_ok, M, N, K, False, True, "e4m3", "e4m3")
    finite = ~np.isnan(ref)
    ok, worst = og.check_fp8(np.where(finite, d, 0.0), np.where(finite, ref, 0.0), bound, a, b, M, N,
                             K, False, True, "e4m3", "e4m3", sa_bits=sa_ok, sb_bits=sb_ok)
    assert ok, worst


def test_in_place_and_k_zero():
    say("gemm_mx in place, K = 0")
    full_check(272, 528, 384, "e5m2", "e4m3", True, False, 1.0, 41, c_is_d=True)
    c = synth.uniform(5, 32 * 16).reshape(32, 16)
    D = Guarded(32 * 16 * 4, fill=np.full((32, 16), np.nan, np.float32))
    tg.tile_gemm_mx(None, None, None, None, upload_f32(c), D.ptr, 32, 16, 0, 0, 1, 1.0,
                    tg.TG_FP8_E4M3, tg.TG_FP8_E4M3)
    torch.cuda.synchronize()
    assert np.array_equal(D.host(np.float32).reshape(32, 16), c) and D.guards_intact()


def test_large_sampled():
    """8192^3 e4m3, A [M,K], B [N,K], scales 2^-10 .. 2^10: 4096 sampled outputs, repeatable."""
    M = N = K = 8192
    say("gemm_mx 8192^3 e4m3 sampled")
    a, b, sa, sb, _ = mx_case(M, N, K, "e4m3", "e4m3", False, True, 0.0, 71)
    A, B, SA, SB = upload_bits(a), upload_bits(b), upload_bits(sa), upload_bits(sb)
    D = torch.empty((M, N), device="cuda:0")
    D2 = torch.empty((M, N), device="cuda:0")
    tg.tile_gemm_mx(A, B, SA, SB, None, D, M, N, K, 0, 1, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3)
    tg.tile_gemm_mx(A, B, SA, SB, None, D2, M, N, K, 0, 1, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3)
    torch.cuda.synchronize()
    assert torch.equal(D, D2)
    rows, cols = synth.sample_points(M, N, 72)
    got = D[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    ref, bound = og.gemm_mx_ref_at(a, b, sa, sb, None, M, N, K, False, True, 0.0, "e4m3", "e4m3",
                                   rows, cols)
    ok, worst = og.check_fp8(got, ref, bound, a, b, M, N, K, False, True, "e4m3", "e4m3", rows, cols,
                             sa_bits=sa, sb_bits=sb)
    assert ok, worst


# 256x256 blocks on ragged problems (the shape tests above run on 128x128 blocks): M, N past a
# block edge, stage counts one, odd (with a partial scale group) and even, every orientation.
@pytest.mark.parametrize("M,N,K,ta,tb", [(4000, 4112, 384, False, True), (4112, 4000, 128, True, False),
                                         (4016, 4096, 1408, True, True), (4096, 4016, 1024, False, False)])
def test_ragged_256_sampled(M, N, K, ta, tb):
    say(f"gemm_mx ragged 256 {M}x{N}x{K} e4m3 x e5m2 transA={ta} transB={tb} beta=1 sampled")
    a, b, sa, sb, c = mx_case(M, N, K, "e4m3", "e5m2", ta, tb, 1.0, 91)
    A, B, SA, SB = upload_bits(a), upload_bits(b), upload_bits(sa), upload_bits(sb)
    Cd = upload_f32(c)
    D = torch.empty((M, N), device="cuda:0")
    plan = tg.tile_gemm_mx_plan(A, B, SA, SB, Cd, D, M, N, K, int(ta), int(tb), 1.0, FMT["e4m3"],
                                FMT["e5m2"])
    assert (plan.block_m, plan.bounds_checked) == (256, 1)
    tg.tile_gemm_mx(A, B, SA, SB, Cd, D, M, N, K, int(ta), int(tb), 1.0, FMT["e4m3"], FMT["e5m2"])
    torch.cuda.synchronize()
    rows, cols = synth.sample_points(M, N, 92)
    got = D[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    ref, bound = og.gemm_mx_ref_at(a, b, sa, sb, c, M, N, K, ta, tb, 1.0, "e4m3", "e5m2", rows, cols)
    ok, worst = og.check_fp8(got, ref, bound, a, b, M, N, K, ta, tb, "e4m3", "e5m2", rows, cols,
                             sa_bits=sa, sb_bits=sb)
    assert ok, worst
    assert torch.isfinite(D).all()


def test_128_blocks_long_k_sampled():
    # 2048 x 2064 outputs on 128x128 blocks, 64 stages (16 turns of the scale ring's groups)
    M, N, K = 2048, 2064, 8192
    say(f"gemm_mx 128 blocks {M}x{N}x{K} e4m3 sampled")
    a, b, sa, sb, _ = mx_case(M, N, K, "e4m3", "e4m3", False, True, 0.0, 93)
    A, B, SA, SB = upload_bits(a), upload_bits(b), upload_bits(sa), upload_bits(sb)
    D = torch.empty((M, N), device="cuda:0")
    plan = tg.tile_gemm_mx_plan(A, B, SA, SB, None, D, M, N, K, 0, 1, 0.0, FMT["e4m3"], FMT["e4m3"])
    assert (plan.block_m, plan.bounds_checked) == (128, 1)
    tg.tile_gemm_mx(A, B, SA, SB, None, D, M, N, K, 0, 1, 0.0, FMT["e4m3"], FMT["e4m3"])
    torch.cuda.synchronize()
    rows, cols = synth.sample_points(M, N, 94, tile=(128, 128))
    got = D[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    ref, bound = og.gemm_mx_ref_at(a, b, sa, sb, None, M, N, K, False, True, 0.0, "e4m3", "e4m3",
                                   rows, cols)
    ok, worst = og.check_fp8(got, ref, bound, a, b, M, N, K, False, True, "e4m3", "e4m3", rows, cols,
                             sa_bits=sa, sb_bits=sb)
    assert ok, worst
