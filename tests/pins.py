"""Pin checks for the oracle, parametrised by the function under test.

Each check raises AssertionError when the given implementation disagrees with
something the pages or plain mathematics fix.  tests/test_oracle_*.py run them
against the oracle; tests/test_oracle_mutations.py runs them against copies of
the oracle with a planted mistake and requires that some check fails.
"""

from fractions import Fraction

import numpy as np

import synth

# Shapes of the page's tiled-test categories ([SYNC-GEMM], 测试覆盖): a single
# tile (the 16x8x16 atom), one dimension multi-tile, all dimensions multi-tile,
# M = 64, K = 8 (the k8 instruction) and K = 24 (16 does not divide 24).
SMALL_SHAPES = [(16, 8, 16), (16, 8, 8), (16, 8, 24), (32, 8, 16), (16, 24, 16),
                (32, 16, 32), (64, 8, 16), (16, 16, 40), (48, 24, 8)]


def _exact_gemm(a_l, b_l, c, beta):
    """Exact rational sum_k a_ik b_kj (+ c_ij) with pure-Python loops."""
    M, K = a_l.shape
    N = b_l.shape[1]
    af = [[Fraction(float(a_l[i, k])) for k in range(K)] for i in range(M)]
    bf = [[Fraction(float(b_l[k, j])) for j in range(N)] for k in range(K)]
    out = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += af[i][k] * bf[k][j]
            if beta == 1.0:
                s += Fraction(float(c[i, j]))
            out[i, j] = s
    return out


def _decode_plain(bits, fmt):
    """Independent decode through numpy float16 / a float32 shift (used only to build test operands)."""
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_gemm_brute_force(gemm_fn, shapes=SMALL_SHAPES):
    """Oracle within fp64 rounding of the exact rational result, all transposes, both betas."""
    seed = 100
    for (M, N, K) in shapes:
        for fmt in ("f16", "bf16"):
            for ta in (False, True):
                for tb in (False, True):
                    for beta in (0.0, 1.0):
                        seed += 3
                        a_bits, b_bits, c = synth.gemm_inputs(M, N, K, fmt, ta, tb, beta,
                                                              (seed, seed + 1, seed + 2),
                                                              dist="uniform", c_dist="uniform")
                        a = _decode_plain(a_bits, fmt)
                        b = _decode_plain(b_bits, fmt)
                        a_l = a.T if ta else a
                        b_l = b.T if tb else b
                        exact = _exact_gemm(a_l, b_l, c, beta)
                        d = gemm_fn(a_bits, b_bits, c, M, N, K, ta, tb, beta, fmt)
                        assert d.shape == (M, N)
                        bound = np.abs(a_l) @ np.abs(b_l)
                        for i in range(M):
                            for j in range(N):
                                err = abs(Fraction(float(d[i, j])) - exact[i, j])
                                lim = Fraction(K + 2) * Fraction(2) ** -52 * Fraction(
                                    float(bound[i, j]) + (abs(float(c[i, j])) if beta else 0.0))
                                assert err <= lim, (M, N, K, fmt, ta, tb, beta, i, j)


def pin_gemm_beta(gemm_fn):
    """beta = 0 never reads C; beta = 1 with A = 0 returns C exactly."""
    M, N, K = 32, 16, 24
    a_bits, b_bits, c = synth.gemm_inputs(M, N, K, "f16", False, False, 1.0, (7, 8, 9))
    nan_c = np.full((M, N), np.nan, dtype=np.float32)
    d0 = gemm_fn(a_bits, b_bits, None, M, N, K, False, False, 0.0, "f16")
    d0n = gemm_fn(a_bits, b_bits, nan_c, M, N, K, False, False, 0.0, "f16")
    assert np.all(np.isfinite(d0n))
    assert np.array_equal(d0, d0n)
    zero_a = np.zeros_like(a_bits)
    d1 = gemm_fn(zero_a, b_bits, c, M, N, K, False, False, 1.0, "f16")
    assert np.array_equal(d1, c.astype(np.float64))
    d1 = gemm_fn(a_bits, b_bits, c, M, N, K, False, False, 1.0, "f16")
    assert np.allclose(d1 - d0, c.astype(np.float64), rtol=0, atol=1e-12)


def pin_gemm_transpose(gemm_fn):
    """Storing an operand transposed and setting its flag gives bit-identical results."""
    M, N, K = 48, 24, 40
    for fmt in ("f16", "bf16"):
        a_bits, b_bits, c = synth.gemm_inputs(M, N, K, fmt, False, False, 1.0, (21, 22, 23))
        ref = gemm_fn(a_bits, b_bits, c, M, N, K, False, False, 1.0, fmt)
        for ta in (False, True):
            for tb in (False, True):
                a_st = np.ascontiguousarray(a_bits.T) if ta else a_bits
                b_st = np.ascontiguousarray(b_bits.T) if tb else b_bits
                d = gemm_fn(a_st, b_st, c, M, N, K, ta, tb, 1.0, fmt)
                assert np.array_equal(d, ref), (fmt, ta, tb)


def pin_gemm_identity_zero(gemm_fn):
    """A = I gives B (and B + C); K = 0 gives 0 (and C); M = 0 gives an empty result."""
    one = {"f16": np.uint16(0x3C00), "bf16": np.uint16(0x3F80)}
    for fmt in ("f16", "bf16"):
        M = K = 32
        N = 24
        eye = np.zeros((M, K), dtype=np.uint16)
        eye[np.arange(M), np.arange(K)] = one[fmt]
        _, b_bits, c = synth.gemm_inputs(M, N, K, fmt, False, False, 1.0, (31, 32, 33))
        b = _decode_plain(b_bits, fmt)
        d = gemm_fn(eye, b_bits, None, M, N, K, False, False, 0.0, fmt)
        assert np.array_equal(d, b)
        d = gemm_fn(eye, b_bits, c, M, N, K, False, False, 1.0, fmt)
        assert np.array_equal(d, b + c.astype(np.float64))
        # rectangular identity-like A (M != K) selects the first M rows of B
        eye2 = np.zeros((16, K), dtype=np.uint16)
        eye2[np.arange(16), np.arange(16) + 5] = one[fmt]
        d = gemm_fn(eye2, b_bits, None, 16, N, K, False, False, 0.0, fmt)
        assert np.array_equal(d, b[5:21])
    empty_a = np.zeros((16, 0), dtype=np.uint16)
    empty_b = np.zeros((0, 8), dtype=np.uint16)
    c = np.arange(128, dtype=np.float32).reshape(16, 8)
    assert np.array_equal(gemm_fn(empty_a, empty_b, None, 16, 8, 0, False, False, 0.0, "f16"),
                          np.zeros((16, 8)))
    assert np.array_equal(gemm_fn(empty_a, empty_b, c, 16, 8, 0, False, False, 1.0, "f16"),
                          c.astype(np.float64))
    d = gemm_fn(np.zeros((0, 8), np.uint16), np.zeros((8, 8), np.uint16), None, 0, 8, 8,
                False, False, 0.0, "bf16")
    assert d.shape == (0, 8)


GEMM_PINS = (pin_gemm_brute_force, pin_gemm_beta, pin_gemm_transpose, pin_gemm_identity_zero)


def pin_sampled_matches_exact(gemm_at_fn):
    """The per-output dot path equals the exact rational result at every sampled point."""
    M, N, K = 64, 48, 40
    for fmt, ta, tb, beta in (("bf16", False, True, 1.0), ("f16", True, False, 1.0),
                              ("f16", False, False, 0.0), ("bf16", True, True, 0.0)):
        a_bits, b_bits, c = synth.gemm_inputs(M, N, K, fmt, ta, tb, beta, (41, 42, 43))
        a = _decode_plain(a_bits, fmt)
        b = _decode_plain(b_bits, fmt)
        a_l = a.T if ta else a
        b_l = b.T if tb else b
        exact = _exact_gemm(a_l, b_l, c, beta)
        rows, cols = synth.sample_points(M, N, 44, count=200, tile=(16, 16))
        d, bound = gemm_at_fn(a_bits, b_bits, c, M, N, K, ta, tb, beta, fmt, rows, cols)
        for s in range(rows.size):
            i, j = int(rows[s]), int(cols[s])
            lim = Fraction(K + 2) * Fraction(2) ** -52 * Fraction(
                float(bound[s]) + (abs(float(c[i, j])) if beta else 0.0))
            assert abs(Fraction(float(d[s])) - exact[i, j]) <= lim
            true_bound = sum(abs(Fraction(float(a_l[i, k])) * Fraction(float(b_l[k, j]))) for k in range(K))
            assert abs(Fraction(float(bound[s])) - true_bound) <= Fraction(K) * Fraction(2) ** -52 * true_bound
