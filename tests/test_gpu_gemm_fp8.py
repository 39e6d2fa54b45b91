"""GPU parity of tile_gemm_fp8 against the oracle ([SYNC-GEMM] 七: fp8 operands of the
asynchronous GEMM).  Bar per element: |D - D_ref| <= 1e-4·sum|a·b| + T + 1e-6, where T is
the fp8 product unit's allowance (oracle.gemm.fp8_unit_allowance_at: within each aligned
group of 8 K products, what lies below 2^-13 of the group's largest product may be lost).
test_unit_groups_of_eight checks that rule on the device itself."""

import numpy as np
import pytest
import torch

import synth
import tile_level_gemm_amd as tg
from oracle import gemm as og
from tests.gpu_util import Guarded, say, upload_bits, upload_f32

pytestmark = pytest.mark.gpu

FMT = {"e4m3": tg.TG_FP8_E4M3, "e5m2": tg.TG_FP8_E5M2}
PAIRS = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]


def run_fp8(a_bits, b_bits, c, M, N, K, beta, af, bf, c_is_d=False, ta=False, tb=True):
    """A stored [M, K] or [K, M] (ta), B stored [K, N] or [N, K] (tb)."""
    A = upload_bits(a_bits)
    B = upload_bits(b_bits)
    D = Guarded(M * N * 4, fill=(c if c_is_d else np.full((M, N), np.nan, np.float32)))
    Cd = upload_f32(c) if beta == 1.0 and not c_is_d else None
    tg.tile_gemm_fp8(A, B, D.ptr if c_is_d else Cd, D.ptr, M, N, K, int(ta), int(tb), beta, FMT[af],
                     FMT[bf])
    torch.cuda.synchronize()
    return D.host(np.float32).reshape(M, N), D.guards_intact()


def full_check(M, N, K, af, bf, beta, seeds, scale=1.0, c_is_d=False, ta=False, tb=True):
    a_bits, b_bits, c = synth.gemm_fp8_inputs(M, N, K, af, bf, ta, tb, beta, seeds, scale)
    d, guards = run_fp8(a_bits, b_bits, c, M, N, K, beta, af, bf, c_is_d=c_is_d, ta=ta, tb=tb)
    ref = og.gemm_fp8_ref(a_bits, b_bits, c, M, N, K, ta, tb, beta, af, bf)
    bound = og.abs_bound_fp8(a_bits, b_bits, M, N, K, ta, tb, af, bf)
    ok, worst = og.check_fp8(d, ref, bound, a_bits, b_bits, M, N, K, ta, tb, af, bf)
    assert guards, "guard band written"
    assert ok, f"worst |D-D_ref|/tol = {worst}"
    return worst


# Whole blocks and ragged edges, with every shape of the stage count K/128: one stage, even,
# odd >= 3.  These problems have fewer than 256 blocks of 256x256, so they run on 128x128
# blocks; test_ragged_256_sampled covers the 256-wide ones.
SHAPES = [(16, 16, 128), (48, 32, 128), (256, 256, 128), (256, 256, 256), (256, 256, 384),
          (272, 528, 384), (512, 512, 1152), (784, 1040, 640), (1024, 1024, 2048),
          (1296, 1040, 1280)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_shapes_e4m3(M, N, K, beta):
    say(f"gemm_fp8 {M}x{N}x{K} e4m3 x e4m3 beta={beta}")
    full_check(M, N, K, "e4m3", "e4m3", beta, (M + 1, N + 2, K + 3))


@pytest.mark.parametrize("M,N,K", [(48, 32, 128), (256, 256, 384), (784, 1040, 640)])
@pytest.mark.parametrize("af,bf", PAIRS)
def test_format_pairs(M, N, K, af, bf):
    say(f"gemm_fp8 {M}x{N}x{K} {af} x {bf} beta=1")
    full_check(M, N, K, af, bf, 1.0, (5, 6, 7), scale=4.0)


@pytest.mark.parametrize("M,N,K", [(48, 32, 128), (272, 528, 384), (784, 1040, 640),
                                   (1296, 1040, 1280), (512, 768, 2048)])
@pytest.mark.parametrize("ta,tb", [(False, False), (True, True), (True, False), (False, True)])
def test_transposes(M, N, K, ta, tb):
    """Every stored orientation: M/N-contiguous operands go through ds_read_b64_tr_b8."""
    say(f"gemm_fp8 {M}x{N}x{K} e4m3 x e5m2 transA={ta} transB={tb} beta=1")
    full_check(M, N, K, "e4m3", "e5m2", 1.0, (M + 7, N + 8, K + 9), ta=ta, tb=tb)


@pytest.mark.parametrize("ta,tb", [(True, False), (False, False)])
def test_every_finite_code_mn(ta, tb):
    """All finite codes with M/N-contiguous operands: the transposing reads must hand each
    lane the same K order as the K-contiguous path (the fp8 bar's groups of 8 rely on it)."""
    say(f"gemm_fp8 all finite codes e5m2 x e5m2 transA={ta} transB={tb}")
    M, N, K = 256, 256, 512
    a_bits = finite_codes(71, M * K, "e5m2").reshape((K, M) if ta else (M, K))
    b_bits = finite_codes(72, N * K, "e5m2").reshape((N, K) if tb else (K, N))
    d, guards = run_fp8(a_bits, b_bits, None, M, N, K, 0.0, "e5m2", "e5m2", ta=ta, tb=tb)
    ref = og.gemm_fp8_ref(a_bits, b_bits, None, M, N, K, ta, tb, 0.0, "e5m2", "e5m2")
    bound = og.abs_bound_fp8(a_bits, b_bits, M, N, K, ta, tb, "e5m2", "e5m2")
    ok, worst = og.check_fp8(d, ref, bound, a_bits, b_bits, M, N, K, ta, tb, "e5m2", "e5m2")
    assert guards and ok, worst


def finite_codes(seed, n, fmt):
    """n fp8 codes drawn uniformly from every finite code of the format (zeros, subnormals
    and the largest finite values included)."""
    all_codes = np.arange(256, dtype=np.uint8)
    if fmt == "e4m3":
        finite = all_codes[(all_codes & 0x7F) != 0x7F]
    else:
        finite = all_codes[((all_codes >> 2) & 0x1F) != 0x1F]
    return finite[synth.rng(seed).integers(0, finite.size, size=n)]


@pytest.mark.parametrize("af,bf", PAIRS)
def test_every_finite_code(af, bf):
    """Operands drawn from all finite codes: the unit's decode of each code (subnormals,
    signed zeros, the extremes) against the oracle's exact values."""
    say(f"gemm_fp8 all finite codes {af} x {bf}")
    M, N, K = 256, 256, 512
    a_bits = finite_codes(61, M * K, af).reshape(M, K)
    b_bits = finite_codes(62, N * K, bf).reshape(N, K)
    d, guards = run_fp8(a_bits, b_bits, None, M, N, K, 0.0, af, bf)
    ref = og.gemm_fp8_ref(a_bits, b_bits, None, M, N, K, False, True, 0.0, af, bf)
    bound = og.abs_bound_fp8(a_bits, b_bits, M, N, K, False, True, af, bf)
    ok, worst = og.check_fp8(d, ref, bound, a_bits, b_bits, M, N, K, False, True, af, bf)
    assert guards and ok, worst


@pytest.mark.parametrize("af,bf", [("e4m3", "e4m3"), ("e5m2", "e5m2")])
def test_subnormal_products(af, bf):
    """Only subnormal and smallest-normal codes, with an identity-like B, so that D holds the
    subnormal values themselves (a flushed decode would give zeros)."""
    say(f"gemm_fp8 subnormals {af} x {bf}")
    M, N, K = 256, 256, 256
    # exponent field 0 (subnormal) in both formats, plus the smallest normal (0x04 is the
    # smallest e5m2 normal, still subnormal in e4m3)
    small = np.array([0x01, 0x02, 0x03, 0x04, 0x81, 0x82, 0x83], np.uint8)
    a_bits = small[synth.rng(63).integers(0, small.size, size=M * K)].reshape(M, K)
    one = 0x38 if bf == "e4m3" else 0x3C
    b_bits = np.zeros((N, K), np.uint8)
    b_bits[np.arange(N), np.arange(N) % K] = one          # B[k][n] = 1 iff k == n
    d, guards = run_fp8(a_bits, b_bits, None, M, N, K, 0.0, af, bf)
    ref = og.gemm_fp8_ref(a_bits, b_bits, None, M, N, K, False, True, 0.0, af, bf)
    assert guards and np.array_equal(d.astype(np.float64), ref)
    assert np.count_nonzero(ref) == ref.size


def test_k_zero_and_empty():
    say("gemm_fp8 K=0 / M=0")
    c = synth.uniform(5, 32 * 16).reshape(32, 16)
    D = Guarded(32 * 16 * 4, fill=np.full((32, 16), np.nan, np.float32))
    tg.tile_gemm_fp8(None, None, upload_f32(c), D.ptr, 32, 16, 0, 0, 1, 1.0, tg.TG_FP8_E4M3,
                     tg.TG_FP8_E5M2)
    torch.cuda.synchronize()
    assert np.array_equal(D.host(np.float32).reshape(32, 16), c) and D.guards_intact()
    tg.tile_gemm_fp8(None, None, None, D.ptr, 32, 16, 0, 0, 1, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3)
    torch.cuda.synchronize()
    assert not D.host(np.float32).any() and D.guards_intact()
    E = Guarded(64, fill=np.full(16, 7.0, np.float32))
    tg.tile_gemm_fp8(None, None, None, E.ptr, 0, 16, 128, 0, 1, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3)
    torch.cuda.synchronize()
    assert np.all(E.host(np.float32) == 7.0) and E.guards_intact()


@pytest.mark.parametrize("M,N,K", [(48, 32, 128), (512, 256, 384), (784, 1040, 640)])
def test_in_place_c_is_d(M, N, K):
    say(f"gemm_fp8 in-place C==D {M}x{N}x{K}")
    full_check(M, N, K, "e5m2", "e4m3", 1.0, (11, 12, 13), c_is_d=True)


def test_beta0_ignores_nan_c():
    say("gemm_fp8 beta=0 with NaN C")
    M, N, K = 272, 528, 384
    a_bits, b_bits, _ = synth.gemm_fp8_inputs(M, N, K, "e4m3", "e4m3", False, True, 0.0, (1, 2, 3))
    A, B = upload_bits(a_bits), upload_bits(b_bits)
    Cn = torch.full((M, N), float("nan"), device="cuda:0")
    D1 = torch.empty((M, N), device="cuda:0")
    D2 = torch.empty((M, N), device="cuda:0")
    tg.tile_gemm_fp8(A, B, Cn, D1, M, N, K, 0, 1, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3)
    tg.tile_gemm_fp8(A, B, None, D2, M, N, K, 0, 1, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3)
    torch.cuda.synchronize()
    assert torch.isfinite(D1).all() and torch.equal(D1, D2)


@pytest.mark.parametrize("af,bf,K,tb", [("e4m3", "e4m3", 8192, True), ("e5m2", "e4m3", 8064, True),
                                        ("e4m3", "e4m3", 8192, False)])
def test_large_sampled(af, bf, K, tb):
    """The 8192 x 8192 x 8192 e4m3 workload (and a mixed-format one whose stage count is
    odd, and one with B stored [K, N]) in the launch configuration the benchmark times:
    4096 sampled outputs plus tile boundaries against one float64 dot each, and bitwise
    repeatability."""
    M = N = 8192
    say(f"gemm_fp8 {M}x{N}x{K} {af} x {bf} transB={tb} sampled")
    if (af, bf, K, tb) == ("e4m3", "e4m3", 8192, True):
        a_bits, b_bits, c = synth.gemm8k_fp8_inputs()
    else:
        beta_in = 1.0 if af != bf else 0.0
        a_bits, b_bits, c = synth.gemm_fp8_inputs(M, N, K, af, bf, False, tb, beta_in, (64, 65, 66))
    beta = 0.0 if c is None else 1.0
    A, B = upload_bits(a_bits), upload_bits(b_bits)
    plan = tg.tile_gemm_fp8_plan(A, B, None if c is None else 1 << 40, 1 << 41, M, N, K, 0, int(tb),
                                 beta, FMT[af], FMT[bf])
    assert (plan.block_m, plan.block_n, plan.bounds_checked, plan.loader) == (256, 256, 0, 1)
    Cd = upload_f32(c) if c is not None else None
    D = torch.empty((M, N), device="cuda:0")
    tg.tile_gemm_fp8(A, B, Cd, D, M, N, K, 0, int(tb), beta, FMT[af], FMT[bf])
    D2 = torch.empty((M, N), device="cuda:0")
    tg.tile_gemm_fp8(A, B, Cd, D2, M, N, K, 0, int(tb), beta, FMT[af], FMT[bf])
    torch.cuda.synchronize()
    assert torch.equal(D, D2), "not bitwise repeatable"
    rows, cols = synth.sample_points(M, N, 63)
    got = D[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    ref, bound = og.gemm_fp8_ref_at(a_bits, b_bits, c, M, N, K, False, tb, beta, af, bf, rows, cols)
    ok, worst = og.check_fp8(got, ref, bound, a_bits, b_bits, M, N, K, False, tb, af, bf, rows, cols)
    assert ok, worst


def test_unit_groups_of_eight():
    """The rule behind the fp8 bar, on the device: with B = 1, row m of A holds a product
    2^12 at k = kb and one 2^-2 (2^14 below) at k = ks; the small one is lost exactly when
    kb and ks share an aligned group of 8 K.  One 2^-1 below (2^13) is always kept."""
    say("gemm_fp8 unit rule: groups of 8, 13-bit window")
    M, N, K = 256, 16, 128
    m = np.arange(M)
    kb = m % 64
    ks = (m * 37 + 5) % 64
    ks = np.where(ks == kb, (kb + 1) % 64, ks)
    big = synth.fp8_bits(np.float32([2.0 ** 12]), "e5m2")[0]
    b_bits = np.full((N, K), 0x3C, np.uint8)           # e5m2 1.0
    for small, kept_always in ((2.0 ** -2, False), (2.0 ** -1, True)):
        a_bits = np.zeros((M, K), np.uint8)
        a_bits[m, kb] = big
        a_bits[m, ks] = synth.fp8_bits(np.float32([small]), "e5m2")[0]
        d, guards = run_fp8(a_bits, b_bits, None, M, N, K, 0.0, "e5m2", "e5m2")
        same_group = (kb // 8) == (ks // 8)
        want = 4096.0 + np.where(same_group & (not kept_always), 0.0, small)
        assert guards and np.array_equal(d[:, 0], want.astype(np.float32)), small
        assert np.all(d == d[:, :1])
    assert same_group.any() and (~same_group).any()


# 256x256 blocks on ragged problems (at least 256 of them): M, N past a block edge, stage
# counts one, odd and even, every orientation; sampled outputs plus every block edge.
@pytest.mark.parametrize("M,N,K,ta,tb", [(4000, 4112, 384, False, True), (4112, 4000, 128, True, False),
                                         (4016, 4096, 1024, True, True), (4096, 4016, 640, False, False)])
def test_ragged_256_sampled(M, N, K, ta, tb):
    say(f"gemm_fp8 ragged 256 {M}x{N}x{K} e5m2 x e4m3 transA={ta} transB={tb} beta=1 sampled")
    a_bits, b_bits, c = synth.gemm_fp8_inputs(M, N, K, "e5m2", "e4m3", ta, tb, 1.0, (81, 82, 83))
    A, B = upload_bits(a_bits), upload_bits(b_bits)
    Cd = upload_f32(c)
    D = torch.empty((M, N), device="cuda:0")
    plan = tg.tile_gemm_fp8_plan(A, B, Cd, D, M, N, K, int(ta), int(tb), 1.0, FMT["e5m2"], FMT["e4m3"])
    assert (plan.block_m, plan.bounds_checked, plan.loader) == (256, 1, 1)
    tg.tile_gemm_fp8(A, B, Cd, D, M, N, K, int(ta), int(tb), 1.0, FMT["e5m2"], FMT["e4m3"])
    torch.cuda.synchronize()
    rows, cols = synth.sample_points(M, N, 84)
    got = D[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    ref, bound = og.gemm_fp8_ref_at(a_bits, b_bits, c, M, N, K, ta, tb, 1.0, "e5m2", "e4m3", rows, cols)
    ok, worst = og.check_fp8(got, ref, bound, a_bits, b_bits, M, N, K, ta, tb, "e5m2", "e4m3", rows, cols)
    assert ok, worst
    assert torch.isfinite(D).all()


# 128x128 blocks at the size where they replace the 256-wide ones: 2048^2 outputs, long K.
@pytest.mark.parametrize("ta,tb", [(False, True), (True, False)])
def test_128_blocks_long_k_sampled(ta, tb):
    M, N, K = 2048, 2064, 8192
    say(f"gemm_fp8 128 blocks {M}x{N}x{K} e4m3 transA={ta} transB={tb} sampled")
    a_bits, b_bits, c = synth.gemm_fp8_inputs(M, N, K, "e4m3", "e4m3", ta, tb, 0.0, (85, 86, 87))
    A, B = upload_bits(a_bits), upload_bits(b_bits)
    D = torch.empty((M, N), device="cuda:0")
    plan = tg.tile_gemm_fp8_plan(A, B, None, D, M, N, K, int(ta), int(tb), 0.0, FMT["e4m3"], FMT["e4m3"])
    assert (plan.block_m, plan.bounds_checked, plan.loader) == (128, 1, 1)
    tg.tile_gemm_fp8(A, B, None, D, M, N, K, int(ta), int(tb), 0.0, FMT["e4m3"], FMT["e4m3"])
    torch.cuda.synchronize()
    rows, cols = synth.sample_points(M, N, 88, tile=(128, 128))
    got = D[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    ref, bound = og.gemm_fp8_ref_at(a_bits, b_bits, c, M, N, K, ta, tb, 0.0, "e4m3", "e4m3", rows, cols)
    ok, worst = og.check_fp8(got, ref, bound, a_bits, b_bits, M, N, K, ta, tb, "e4m3", "e4m3", rows, cols)
    assert ok, worst
