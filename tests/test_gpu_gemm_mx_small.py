"""GPU parity of tile_gemm_mx with 6- and 4-bit operands (e2m3, e3m2, e2m1; [SYNC-GEMM] 七: fp4
operands with SFA / SFB block scales) against the oracle, element by element, with the fp8
bar (the unit's grouped-sum allowance on the scaled products) and the plain 16-bit bar
recorded beside it."""

import numpy as np
import pytest
import torch

import synth
import tile_level_gemm_amd as tg
from oracle import gemm as og
from tests.gpu_util import Guarded, say, upload_f32

pytestmark = pytest.mark.gpu

FMT = {"e2m3": tg.TG_FP6_E2M3, "e3m2": tg.TG_FP6_E3M2, "e2m1": tg.TG_FP4_E2M1}


def up8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to("cuda:0")


def run_small(M, N, K, af, bf, beta, seed, dist="codes", c_is_d=False, scale_range=(117, 138)):
    pa, pb, _, _, sa, sb, c = synth.gemm_mx_small_inputs(M, N, K, af, bf, beta,
                                                          (seed, seed + 1, seed + 2), dist=dist,
                                                          scale_range=scale_range)
    D = Guarded(M * N * 4, fill=(c if c_is_d else np.full((M, N), np.nan, np.float32)))
    Cd = upload_f32(c) if beta == 1.0 and not c_is_d else None
    tg.tile_gemm_mx(up8(pa), up8(pb), up8(sa), up8(sb), D.ptr if c_is_d else Cd, D.ptr, M, N, K,
                    0, 1, beta, FMT[af], FMT[bf])
    torch.cuda.synchronize()
    return D.host(np.float32).reshape(M, N), D.guards_intact(), (pa, pb, sa, sb, c)


def full_check(M, N, K, af, bf, beta, seed, **kw):
    d, guards, (pa, pb, sa, sb, c) = run_small(M, N, K, af, bf, beta, seed, **kw)
    ref = og.gemm_mx_ref(pa, pb, sa, sb, c, M, N, K, False, True, beta, af, bf)
    bound = og.abs_bound_mx(pa, pb, sa, sb, M, N, K, False, True, af, bf)
    ok, worst = og.check_fp8(d, ref, bound, pa, pb, M, N, K, False, True, af, bf, sa_bits=sa,
                             sb_bits=sb)
    assert guards, "guard band written"
    assert ok, f"worst |D-D_ref|/tol = {worst}"
    return og.check(d, ref, bound)[1]


PAIRS = [(a, b) for a in FMT for b in FMT]


@pytest.mark.parametrize("af,bf", PAIRS)
def test_format_pairs(af, bf):
    say(f"gemm_mx packed 256x256x384 {af} x {bf}")
    full_check(256, 256, 384, af, bf, 1.0, 7)


# whole and ragged 128x128 blocks, one to many 128-K stages, beta 0 and 1
@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (128, 128, 128), (144, 208, 256), (400, 272, 640),
                                   (1024, 1040, 1152)])
@pytest.mark.parametrize("beta", [0.0, 1.0])
@pytest.mark.parametrize("af,bf", [("e2m1", "e2m1"), ("e3m2", "e2m3")])
def test_shapes(M, N, K, beta, af, bf):
    say(f"gemm_mx packed {M}x{N}x{K} {af} x {bf} beta={beta}")
    full_check(M, N, K, af, bf, beta, M + N + K)


# 256x256 blocks of 512 threads (256 or more of them): whole and ragged, beta 0 and 1
@pytest.mark.parametrize("M,N,K,af,bf,beta", [(4096, 4096, 256, "e2m1", "e2m1", 0.0),
                                              (4096, 4112, 384, "e3m2", "e2m1", 1.0),
                                              (4112, 4096, 256, "e2m3", "e3m2", 1.0),
                                              (4352, 4240, 128, "e2m1", "e2m3", 0.0)])
def test_large_blocks(M, N, K, af, bf, beta):
    say(f"gemm_mx packed {M}x{N}x{K} {af} x {bf} beta={beta} (256x256 blocks)")
    full_check(M, N, K, af, bf, beta, M + K)


# e2m1 x e2m1 with K % 256 == 0 runs the direct-load kernel: one, an even and an odd number of
# 256-K stages, 128- and 256-wide blocks, whole and ragged, beta 0 and 1
@pytest.mark.parametrize("M,N,K,beta", [(144, 208, 256, 1.0), (256, 384, 512, 0.0),
                                        (400, 272, 768, 1.0), (1024, 1040, 1280, 0.0),
                                        (4096, 4096, 512, 0.0), (4112, 4096, 768, 1.0),
                                        (4096, 4352, 256, 1.0), (4352, 4240, 1024, 0.0)])
def test_fp4_direct(M, N, K, beta):
    say(f"gemm_mx e2m1 direct {M}x{N}x{K} beta={beta}")
    full_check(M, N, K, "e2m1", "e2m1", beta, M + N + K, dist="normal", scale_range=(100, 154))


# two 6-bit operands run the direct-load kernel: one, an even and an odd number of 128-K stages,
# 128- and 256-wide blocks, whole and ragged, beta 0 and 1, every pair of the two types
@pytest.mark.parametrize("M,N,K,af,bf,beta", [(144, 208, 128, "e2m3", "e2m3", 1.0),
                                              (256, 384, 256, "e3m2", "e3m2", 0.0),
                                              (400, 272, 384, "e2m3", "e3m2", 1.0),
                                              (1024, 1040, 640, "e3m2", "e2m3", 0.0),
                                              (4096, 4096, 256, "e2m3", "e2m3", 0.0),
                                              (4112, 4096, 384, "e3m2", "e2m3", 1.0),
                                              (4096, 4352, 128, "e2m3", "e3m2", 1.0),
                                              (4352, 4240, 512, "e3m2", "e3m2", 0.0)])
def test_fp6_direct(M, N, K, af, bf, beta):
    say(f"gemm_mx 6-bit direct {M}x{N}x{K} {af} x {bf} beta={beta}")
    full_check(M, N, K, af, bf, beta, M + N + K + 1, dist="normal", scale_range=(100, 154))


def test_fp6_direct_in_place_and_codes():
    say("gemm_mx 6-bit direct in place C == D, every code")
    full_check(512, 768, 1152, "e3m2", "e2m3", 1.0, 57, c_is_d=True)


def test_fp4_direct_in_place_and_codes():
    say("gemm_mx e2m1 direct in place C == D, every code")
    full_check(512, 768, 1536, "e2m1", "e2m1", 1.0, 53, c_is_d=True)


# the packed kernel's pairs (an e2m1 operand with a 6-bit one; e2m1 x e2m1 with K % 256 != 0):
# 128- and 256-wide blocks, whole and ragged, one to many 128-K stages, beta 0 and 1
@pytest.mark.parametrize("M,N,K,af,bf,beta", [(16, 48, 128, "e2m1", "e3m2", 1.0),
                                              (400, 272, 640, "e2m3", "e2m1", 0.0),
                                              (1024, 1040, 1152, "e2m1", "e2m3", 1.0),
                                              (4112, 4096, 384, "e3m2", "e2m1", 0.0),
                                              (4096, 4352, 640, "e2m1", "e2m1", 1.0)])
def test_packed_kernel_pairs(M, N, K, af, bf, beta):
    say(f"gemm_mx packed kernel {M}x{N}x{K} {af} x {bf} beta={beta}")
    full_check(M, N, K, af, bf, beta, M + N + K + 2, dist="normal", scale_range=(100, 154))


@pytest.mark.parametrize("af", ["e2m1", "e2m3"])
def test_normal_data_and_wide_scales(af):
    # N(0,1) rounded to the format, scales over 2^-60 .. 2^60
    say(f"gemm_mx packed 512x512x1024 {af} normal data, wide scales")
    full_check(512, 512, 1024, af, af, 0.0, 41, dist="normal", scale_range=(67, 188))


def test_in_place_c_is_d():
    say("gemm_mx packed in place C == D")
    full_check(272, 144, 384, "e2m1", "e3m2", 1.0, 51, c_is_d=True)


def test_sampled_2048():
    M = N = K = 2048
    say("gemm_mx packed 2048^3 e2m1 sampled")
    d, guards, (pa, pb, sa, sb, c) = run_small(M, N, K, "e2m1", "e2m1", 0.0, 61, dist="normal")
    rows, cols = synth.sample_points(M, N, 64, count=4096, tile=(128, 128))
    ref, bound = og.gemm_mx_ref_at(pa, pb, sa, sb, None, M, N, K, False, True, 0.0, "e2m1", "e2m1",
                                   rows, cols)
    ok, worst = og.check_fp8(d[rows, cols], ref, bound, pa, pb, M, N, K, False, True, "e2m1", "e2m1",
                             rows, cols, sa_bits=sa, sb_bits=sb)
    assert guards and ok, worst


@pytest.mark.parametrize("af,seed", [("e2m1", 65), ("e2m3", 68)])
def test_sampled_8192(af, seed):
    # the 8192^3 timed configuration: same inputs and launch, outputs sampled over every block
    M = N = K = 8192
    say(f"gemm_mx packed 8192^3 {af} sampled")
    d, guards, (pa, pb, sa, sb, c) = run_small(M, N, K, af, af, 0.0, seed, dist="normal")
    rows, cols = synth.sample_points(M, N, 64, count=4096, tile=(256, 256))
    ref, bound = og.gemm_mx_ref_at(pa, pb, sa, sb, None, M, N, K, False, True, 0.0, af, af,
                                   rows, cols)
    ok, worst = og.check_fp8(d[rows, cols], ref, bound, pa, pb, M, N, K, False, True, af, af,
                             rows, cols, sa_bits=sa, sb_bits=sb)
    assert guards and ok, worst


# A packed operand just under 2 GiB on each direct-load path (ragged M, every code equally
# likely, scales over 2^-10 .. 2^10), checked on 4096 sampled outputs
@pytest.mark.parametrize("M,af,bf,beta", [(524272, "e2m1", "e2m1", 0.0), (349520, "e2m3", "e3m2", 1.0)])
def test_direct_operand_just_under_2gib_sampled(M, af, bf, beta):
    N, K = 256, 8192
    wa, wb = synth.SMALL_W[af], synth.SMALL_W[bf]
    abytes = M * K * wa // 8
    assert abytes < 1 << 31 and abytes > (1 << 31) - (1 << 20)
    pa, pb = synth.packed_random(abytes, 81), synth.packed_random(N * K * wb // 8, 82)
    g = synth.rng(83)
    sa = g.integers(117, 138, size=(M, K // 32)).astype(np.uint8)
    sb = g.integers(117, 138, size=(N, K // 32)).astype(np.uint8)
    c = synth.uniform(84, M * N).reshape(M, N) if beta else None
    say(f"gemm_mx {af} x {bf} {M}x{N}x{K}: A of {abytes} bytes (direct-load kernel)")
    A, B, SA, SB = up8(pa), up8(pb), up8(sa), up8(sb)
    D = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    Cd = upload_f32(c) if beta else None
    p = tg.tile_gemm_mx_plan(A, B, SA, SB, Cd, D, M, N, K, 0, 1, beta, FMT[af], FMT[bf])
    assert p.loader == 1 and p.bounds_checked == 1
    tg.tile_gemm_mx(A, B, SA, SB, Cd, D, M, N, K, 0, 1, beta, FMT[af], FMT[bf])
    torch.cuda.synchronize()
    rows, cols = synth.sample_points(M, N, 85, count=4096, tile=(256, 256))
    rows[:8] = M - 1 - np.arange(8)   # the last rows: the far end of A
    ref, bound = og.gemm_mx_ref_at(pa, pb, sa, sb, c, M, N, K, False, True, beta, af, bf, rows, cols)
    got = D.cpu().numpy()[rows, cols]
    ok, worst = og.check_fp8(got, ref, bound, pa, pb, M, N, K, False, True, af, bf, rows, cols,
                             sa_bits=sa, sb_bits=sb)
    assert ok, worst


@pytest.mark.parametrize("af,bf", [("e2m1", "e2m1"), ("e2m3", "e3m2"), ("e2m1", "e2m3")])
def test_empty_and_k_zero(af, bf):
    # M or N = 0: nothing is read or written; K = 0: D = beta·C (beta 1) or 0 (beta 0)
    say(f"gemm_mx {af} x {bf}: M = 0, N = 0, K = 0")
    tg.tile_gemm_mx(None, None, None, None, None, None, 0, 64, 128, 0, 1, 0.0, FMT[af], FMT[bf])
    tg.tile_gemm_mx(None, None, None, None, None, None, 64, 0, 128, 0, 1, 1.0, FMT[af], FMT[bf])
    c = synth.uniform(6, 48 * 32).reshape(48, 32)
    for beta in (1.0, 0.0):
        D = Guarded(48 * 32 * 4, fill=np.full((48, 32), np.nan, np.float32))
        tg.tile_gemm_mx(None, None, None, None, upload_f32(c) if beta else None, D.ptr, 48, 32, 0, 0, 1,
                        beta, FMT[af], FMT[bf])
        torch.cuda.synchronize()
        want = c if beta else np.zeros((48, 32), np.float32)
        assert np.array_equal(D.host(np.float32).reshape(48, 32), want) and D.guards_intact()


def test_one_hot_block_scales_reach_their_block():
    # A = 1.0 everywhere, B one-hot per column in one block, scales 2^(n mod 7) on that block of B:
    # each output is exactly the chosen B scale times the A scale of the block
    M, N, K = 32, 32, 256
    ca = np.full((M, K), 0x2, np.uint8)          # e2m1 1.0
    cb = np.zeros((N, K), np.uint8)
    ks = (np.arange(N) * 37) % K
    cb[np.arange(N), ks] = 0x2
    sa = np.full((M, K // 32), 127, np.uint8)
    sa[:, 3] = 130
    sb = (127 + (np.arange(N)[:, None] % 7) + np.zeros((1, K // 32), int)).astype(np.uint8)
    D = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    say("gemm_mx packed one-hot block scales")
    tg.tile_gemm_mx(up8(synth.pack_rows(ca, 4)), up8(synth.pack_rows(cb, 4)), up8(sa), up8(sb), None,
                    D, M, N, K, 0, 1, 0.0, tg.TG_FP4_E2M1, tg.TG_FP4_E2M1)
    torch.cuda.synchronize()
    want = og.gemm_mx_ref(synth.pack_rows(ca, 4), synth.pack_rows(cb, 4), sa, sb, None, M, N, K,
                          False, True, 0.0, "e2m1", "e2m1")
    assert np.array_equal(D.cpu().numpy(), want.astype(np.float32))


def test_rejections():
    A = torch.zeros(8192, dtype=torch.uint8, device="cuda:0")
    S = torch.zeros(1024, dtype=torch.uint8, device="cuda:0")
    D = torch.zeros(64 * 64, dtype=torch.float32, device="cuda:0")
    for args, status in (((0, 0), tg.TG_E_LAYOUT), ((1, 1), tg.TG_E_LAYOUT),
                         ((0, 1, tg.TG_FP4_E2M1, tg.TG_FP8_E4M3), tg.TG_E_DTYPE)):
        ta, tb = args[:2]
        af, bf = (args[2], args[3]) if len(args) > 2 else (tg.TG_FP4_E2M1, tg.TG_FP4_E2M1)
        with pytest.raises(tg.TileError) as e:
            tg.tile_gemm_mx(A, A, S, S, None, D, 64, 64, 128, ta, tb, 0.0, af, bf)
        assert e.value.status == status
