"""Pins of the 6- and 4-bit block-scaled GEMM oracle ([SYNC-GEMM] 七: fp4 among the operand
precisions, SFA / SFB block scales).  CPU only."""

from fractions import Fraction
from itertools import product

import numpy as np
import pytest

import synth
from oracle import gemm as G
from oracle.numerics import fp8_bits_to_f64, small_bits_to_f64, unpack_rows

FMTS = ("e2m3", "e3m2", "e2m1")
W = {"e2m3": 6, "e3m2": 6, "e2m1": 4}


def test_e2m1_value_table():
    # the eight fp4 magnitudes of the OCP element type, codes 0..7, and their negatives
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    v = small_bits_to_f64(np.arange(16), "e2m1")
    assert list(v[:8]) == want and list(-v[8:]) == want
    assert np.signbit(v[8])   # code 8 is -0


@pytest.mark.parametrize("fmt,top,sub", [("e2m3", 7.5, 0.125), ("e3m2", 28.0, 0.0625), ("e2m1", 6.0, 0.5)])
def test_extremes_monotone_and_symmetric(fmt, top, sub):
    n = 1 << W[fmt]
    v = small_bits_to_f64(np.arange(n), fmt)
    pos = v[: n // 2]
    assert pos.max() == top and pos[1] == sub
    assert np.all(np.diff(pos) > 0)                       # positive codes increase strictly
    assert np.array_equal(v[n // 2:], -pos)               # the sign bit only negates
    assert np.all(np.isfinite(v))                         # no infinities or NaNs


def test_fp4_embeds_in_e2m3():
    # e2m3 is e2m1 with two more fraction bits: s.ee.m -> s.ee.m00 keeps the value
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        assert small_bits_to_f64(np.array([c]), "e2m1")[0] == \
            small_bits_to_f64(np.array([(s << 5) | (e << 3) | (m << 2)]), "e2m3")[0]


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_values_are_e4m3_values(fmt):
    # every fp6 value is exactly an e4m3 value (the fp8 decoder is pinned against torch)
    e4 = set(fp8_bits_to_f64(np.arange(256, dtype=np.uint8), "e4m3")[np.isfinite(
        fp8_bits_to_f64(np.arange(256, dtype=np.uint8), "e4m3"))].tolist())
    for x in small_bits_to_f64(np.arange(64), fmt):
        assert x in e4


def test_unpack_hand_built_bytes():
    # fp4: byte 0x21 holds code 1 (low nibble) then code 2
    assert unpack_rows(np.array([0x21], np.uint8), 1, 2, 4).tolist() == [[1, 2]]
    # fp6: codes 1, 2, 3, 4 -> bit stream 1 | 2<<6 | 3<<12 | 4<<18 = 0x103081
    assert unpack_rows(np.array([0x81, 0x30, 0x10], np.uint8), 1, 4, 6).tolist() == [[1, 2, 3, 4]]
    # two rows are unpacked independently
    two = unpack_rows(np.array([0x21, 0x43], np.uint8), 2, 2, 4)
    assert two.tolist() == [[1, 2], [3, 4]]


@pytest.mark.parametrize("w", [4, 6])
def test_unpack_inverts_the_input_packer(w):
    g = np.random.default_rng(5)
    codes = g.integers(0, 1 << w, size=(7, 64)).astype(np.uint8)
    assert np.array_equal(unpack_rows(synth.pack_rows(codes, w), 7, 64, w), codes)


def _fraction_mx(ca, cb, sa, sb, fa, fb, M, N, K):
    va = small_bits_to_f64(ca, fa)
    vb = small_bits_to_f64(cb, fb)
    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                s = Fraction(2) ** (int(sa[m, k // 32]) - 127) * Fraction(2) ** (int(sb[n, k // 32]) - 127)
                acc += Fraction(va[m, k]) * Fraction(vb[n, k]) * s
            out[m, n] = acc
    return out


@pytest.mark.parametrize("fa,fb", [("e2m1", "e2m1"), ("e2m3", "e3m2"), ("e3m2", "e2m1")])
def test_fraction_brute_force(fa, fb):
    M, N, K = 16, 16, 128
    pa, pb, ca, cb, sa, sb, _ = synth.gemm_mx_small_inputs(M, N, K, fa, fb, 0.0, (1, 2, 3))
    d = G.gemm_mx_ref(pa, pb, sa, sb, None, M, N, K, False, True, 0.0, fa, fb)
    exact = _fraction_mx(ca, cb, sa, sb, fa, fb, M, N, K)
    # every scaled product is a dyadic rational well inside float64: the sum is exact to
    # within K rounding steps of float64
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(d[m, n]) - exact[m, n]) <= abs(exact[m, n]) * K * 2 ** -52 + 2 ** -200


@pytest.mark.parametrize("fmt", FMTS)
def test_ones_times_b_is_column_sums(fmt):
    # A = 1.0 everywhere, unit scales: D[m][n] = sum_k B[k][n], the same for every m
    M, N, K = 16, 32, 128
    one = {"e2m3": 0x08, "e3m2": 0x0C, "e2m1": 0x2}[fmt]
    ca = np.full((M, K), one, np.uint8)
    g = np.random.default_rng(9)
    cb = g.integers(0, 1 << W[fmt], size=(N, K)).astype(np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    d = G.gemm_mx_ref(synth.pack_rows(ca, W[fmt]), synth.pack_rows(cb, W[fmt]), sa, sb, None, M, N,
                      K, False, True, 0.0, fmt, fmt)
    col = small_bits_to_f64(cb, fmt).sum(axis=1)
    assert np.array_equal(d, np.broadcast_to(col, (M, N)))


def test_scale_raises_one_block_by_two():
    M, N, K = 16, 16, 256
    pa, pb, ca, cb, sa, sb, _ = synth.gemm_mx_small_inputs(M, N, K, "e2m1", "e2m3", 0.0, (4, 5, 6))
    d0 = G.gemm_mx_ref(pa, pb, sa, sb, None, M, N, K, False, True, 0.0, "e2m1", "e2m3")
    sa2 = sa.copy()
    sa2[3, 5] += 1                                   # row 3, K 160..191 doubled
    d1 = G.gemm_mx_ref(pa, pb, sa2, sb, None, M, N, K, False, True, 0.0, "e2m1", "e2m3")
    va = small_bits_to_f64(ca, "e2m1") * np.repeat(np.ldexp(1.0, sa.astype(int) - 127), 32, axis=1)
    vb = small_bits_to_f64(cb, "e2m3") * np.repeat(np.ldexp(1.0, sb.astype(int) - 127), 32, axis=1)
    block = (va[3, 160:192][None, :] * vb[:, 160:192]).sum(axis=1)
    assert np.array_equal(np.delete(d1, 3, axis=0), np.delete(d0, 3, axis=0))
    assert np.allclose(d1[3] - d0[3], block, rtol=1e-15, atol=1e-300)


def test_sampled_equals_full_and_beta():
    M, N, K = 48, 32, 256
    pa, pb, _, _, sa, sb, c = synth.gemm_mx_small_inputs(M, N, K, "e3m2", "e2m1", 1.0, (7, 8, 9))
    full = G.gemm_mx_ref(pa, pb, sa, sb, c, M, N, K, False, True, 1.0, "e3m2", "e2m1")
    d0 = G.gemm_mx_ref(pa, pb, sa, sb, None, M, N, K, False, True, 0.0, "e3m2", "e2m1")
    assert np.array_equal(full - d0, np.asarray(c, np.float64)) or np.allclose(full - d0, c, atol=1e-12)
    rows, cols = synth.sample_points(M, N, 3, count=200, tile=(16, 16))
    d, bd = G.gemm_mx_ref_at(pa, pb, sa, sb, c, M, N, K, False, True, 1.0, "e3m2", "e2m1", rows, cols)
    assert np.allclose(d, full[rows, cols], rtol=1e-13, atol=1e-13)
    bound = G.abs_bound_mx(pa, pb, sa, sb, M, N, K, False, True, "e3m2", "e2m1")
    assert np.allclose(bd, bound[rows, cols], rtol=1e-13, atol=0)


@pytest.mark.parametrize("args,category", [
    (dict(M=32, N=32, K=128, a_dtype="e2m1", b_dtype="e2m3"), None),
    (dict(M=0, N=0, K=0, a_dtype="e3m2", b_dtype="e3m2"), None),
    (dict(M=32, N=32, K=64, a_dtype="e2m1", b_dtype="e2m1"), "shape"),
    (dict(M=8, N=32, K=128, a_dtype="e2m1", b_dtype="e2m1"), "shape"),
    (dict(M=32, N=32, K=128, a_dtype="e2m1", b_dtype="e4m3"), "dtype"),
    (dict(M=32, N=32, K=128, a_dtype="e4m3", b_dtype="e3m2"), "dtype"),
    (dict(M=32, N=32, K=128, a_dtype="e2m1", b_dtype="e2m1", trans_a=True), "layout"),
    (dict(M=32, N=32, K=128, a_dtype="e2m1", b_dtype="e2m1", trans_b=False), "layout"),
    (dict(M=32, N=32, K=128, a_dtype="e2m1", b_dtype="e2m1", alpha=0.5), "alpha"),
    (dict(M=32, N=32, K=128, a_dtype="e2m1", b_dtype="e2m1", beta=2.0), "beta"),
    (dict(M=32, N=32, K=128, a_dtype="e4m3", b_dtype="e5m2", trans_a=True, trans_b=False), None),
])
def test_acceptance_table(args, category):
    ok, cat = G.accepts_mx(**args)
    assert ok == (category is None) and cat == category
