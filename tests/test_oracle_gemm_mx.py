"""Pins of the block-scaled (MX) fp8 GEMM oracle ([SYNC-GEMM] 七: block-scaled operands, the
SFA / SFB scale factors): every 32 consecutive K of a row of A / a column of B share one E8M0
scale 2^(e-127)."""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import gemm as G
from tests import pins


def mx_inputs(M, N, K, af, bf, ta, tb, beta, seed, lo=117, hi=137):
    a, b, c = synth.gemm_fp8_inputs(M, N, K, af, bf, ta, tb, beta, (seed, seed + 1, seed + 2))
    g = synth.rng(seed + 3)
    sa = g.integers(lo, hi + 1, size=(M, K // 32)).astype(np.uint8)
    sb = g.integers(lo, hi + 1, size=(N, K // 32)).astype(np.uint8)
    return a, b, sa, sb, c


def exact_mx(a_bits, b_bits, sa, sb, c, M, N, K, ta, tb, af, bf, beta):
    """Fraction brute force: operand values from torch's float8 types, scales 2^(e-127)."""
    av = pins.torch_fp8_values(a_bits, af).reshape((K, M) if ta else (M, K))
    bv = pins.torch_fp8_values(b_bits, bf).reshape((N, K) if tb else (K, N))
    av = av.T if ta else av
    bv = bv.T if tb else bv
    out = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                scale = Fraction(2) ** (int(sa[i, k // 32]) - 127 + int(sb[j, k // 32]) - 127)
                s += Fraction(float(av[i, k])) * Fraction(float(bv[k, j])) * scale
            if beta == 1.0:
                s += Fraction(float(c[i, j]))
            out[i, j] = s
    return out


def pin_mx_exact(fn):
    seed = 900
    cases = [(16, 16, 128, "e4m3", "e5m2", False, True, 0.0), (16, 16, 128, "e5m2", "e4m3", True, False, 1.0),
             (16, 16, 256, "e5m2", "e5m2", True, True, 1.0), (16, 16, 256, "e4m3", "e4m3", False, False, 0.0)]
    for (M, N, K, af, bf, ta, tb, beta) in cases:
        seed += 5
        a, b, sa, sb, c = mx_inputs(M, N, K, af, bf, ta, tb, beta, seed)
        d = fn(a, b, sa, sb, c, M, N, K, ta, tb, beta, af, bf)
        ex = exact_mx(a, b, sa, sb, c, M, N, K, ta, tb, af, bf, beta)
        lim = Fraction(K + 4) * Fraction(2) ** -52 * Fraction(float(np.abs(d).max()) + 1)
        for i in range(M):
            for j in range(N):
                assert abs(Fraction(float(d[i, j])) - ex[i, j]) <= lim, (M, N, K, af, bf, ta, tb, beta, i, j)


def pin_mx_blocks(fn):
    """Doubling one block scale doubles exactly that block's contribution."""
    M, N, K = 16, 16, 256
    a, b, sa, sb, _ = mx_inputs(M, N, K, "e4m3", "e4m3", False, True, 0.0, 77)
    base = fn(a, b, sa, sb, None, M, N, K, False, True, 0.0, "e4m3", "e4m3")
    for kb in range(K // 32):
        a0 = a.copy()
        a0[:, 32 * kb:32 * kb + 32] = 0
        without = fn(a0, b, sa, sb, None, M, N, K, False, True, 0.0, "e4m3", "e4m3")
        sa2 = sa.copy()
        sa2[3, kb] += 1
        d2 = fn(a, b, sa2, sb, None, M, N, K, False, True, 0.0, "e4m3", "e4m3")
        contrib = base - without
        want = base.copy()
        want[3] += contrib[3]
        assert np.allclose(d2, want, rtol=1e-12, atol=1e-12), kb


MX_PINS = (pin_mx_exact, pin_mx_blocks)


def test_exact_fraction_brute_force():
    pin_mx_exact(G.gemm_mx_ref)


def test_block_structure():
    pin_mx_blocks(G.gemm_mx_ref)


def test_unit_scales_reduce_to_fp8_gemm():
    M, N, K = 48, 32, 384
    for ta, tb in ((False, True), (True, False), (True, True), (False, False)):
        a, b, c = synth.gemm_fp8_inputs(M, N, K, "e5m2", "e4m3", ta, tb, 1.0, (4, 5, 6))
        one_a = np.full((M, K // 32), 127, np.uint8)
        one_b = np.full((N, K // 32), 127, np.uint8)
        assert np.array_equal(G.gemm_mx_ref(a, b, one_a, one_b, c, M, N, K, ta, tb, 1.0, "e5m2", "e4m3"),
                              G.gemm_fp8_ref(a, b, c, M, N, K, ta, tb, 1.0, "e5m2", "e4m3"))


def test_nan_scale_poisons_its_row():
    M, N, K = 16, 16, 128
    a, b, sa, sb, _ = mx_inputs(M, N, K, "e4m3", "e4m3", False, True, 0.0, 11)
    a = np.full_like(a, 0x38)                       # 1.0: every product nonzero
    sa[5, 2] = 255
    d = G.gemm_mx_ref(a, b, sa, sb, None, M, N, K, False, True, 0.0, "e4m3", "e4m3")
    assert np.all(np.isnan(d[5])) and np.all(np.isfinite(np.delete(d, 5, axis=0)))


def test_scaled_allowance_matches_unscaled_for_unit_scales():
    M, N, K = 32, 32, 256
    a, b, sa, sb, _ = mx_inputs(M, N, K, "e5m2", "e5m2", False, True, 0.0, 21)
    rows, cols = np.arange(32), np.arange(32)[::-1].copy()
    one_a, one_b = np.full_like(sa, 127), np.full_like(sb, 127)
    t0 = G.fp8_unit_allowance_at(a, b, M, N, K, False, True, "e5m2", "e5m2", rows, cols)
    t1 = G.fp8_unit_allowance_at(a, b, M, N, K, False, True, "e5m2", "e5m2", rows, cols, one_a, one_b)
    assert np.array_equal(t0, t1)
    # a uniform scale 2^s on every block scales the allowance by 2^s exactly
    t2 = G.fp8_unit_allowance_at(a, b, M, N, K, False, True, "e5m2", "e5m2", rows, cols,
                                 one_a + 3, one_b - 1)
    assert np.array_equal(t2, t0 * 4.0)


@pytest.mark.parametrize("kind", ["block16", "scales_transposed", "bias128", "sa_on_columns",
                                  "no_b_scale"])
def test_mx_mutants_are_caught(kind):
    from oracle.numerics import e8m0_bits_to_f64

    def mutant(a_bits, b_bits, sa_bits, sb_bits, c, M, N, K, ta, tb, beta, af, bf):
        a_l, b_l = G.logical_operands(a_bits, b_bits, M, N, K, ta, tb, af, bf)
        blk = 16 if kind == "block16" else 32
        sa = np.asarray(sa_bits, np.uint8).reshape(M, K // 32)
        sb = np.asarray(sb_bits, np.uint8).reshape(N, K // 32)
        if kind == "scales_transposed":
            sa = sa.reshape(K // 32, M).T
        bias = 128 if kind == "bias128" else 127
        fa = np.ldexp(1.0, sa.astype(np.int64) - bias)
        fb = np.ldexp(1.0, sb.astype(np.int64) - bias)
        if kind == "sa_on_columns":
            fa, fb = fb[:M] if N >= M else fa, fa[:N] if M >= N else fb
        if kind == "no_b_scale":
            fb = np.ones_like(fb)
        ka = np.repeat(fa, 32, axis=1)[:, :K] if blk == 32 else np.repeat(fa, 16, axis=1)[:, :K]
        kb = np.repeat(fb, 32, axis=1)[:, :K] if blk == 32 else np.repeat(fb, 16, axis=1)[:, :K]
        d = (a_l * ka) @ (b_l * kb.T)
        if beta == 1.0:
            d = d + np.asarray(c, np.float32).reshape(M, N)
        return d

    def caught(p):
        try:
            p(mutant)
        except (AssertionError, ValueError, IndexError):
            return True
        return False
    assert any(caught(p) for p in MX_PINS)


def test_sampled_equals_full():
    M, N, K = 96, 80, 256
    for ta, tb in ((False, True), (True, False)):
        a, b, sa, sb, c = mx_inputs(M, N, K, "e5m2", "e4m3", ta, tb, 1.0, 55)
        full = G.gemm_mx_ref(a, b, sa, sb, c, M, N, K, ta, tb, 1.0, "e5m2", "e4m3")
        bound = G.abs_bound_mx(a, b, sa, sb, M, N, K, ta, tb, "e5m2", "e4m3")
        rows, cols = synth.sample_points(M, N, 8, count=400, tile=(16, 16))
        d, bd = G.gemm_mx_ref_at(a, b, sa, sb, c, M, N, K, ta, tb, 1.0, "e5m2", "e4m3", rows, cols)
        assert np.allclose(d, full[rows, cols], rtol=1e-13, atol=1e-13)
        assert np.allclose(bd, bound[rows, cols], rtol=1e-13, atol=0)
