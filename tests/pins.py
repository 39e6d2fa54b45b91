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


# ---- fp8 (the asynchronous GEMM's precision family, [SYNC-GEMM] 七) ---------------------
# Every e4m3 value is an integer multiple of 2^-9 and every e5m2 value of 2^-16, so with
# operands scaled to integers every product, and the sum over K of them, is exact in int64
# as long as max|a|·max|b|·K < 2^63 (checked): an exact result that needs neither the
# oracle's decoder nor floating point.  Operand values come from torch's own float8
# conversions.

FP8_PAIRS = (("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2"))
_FP8_QUANTUM_EXP = {"e4m3": 9, "e5m2": 16}


def torch_fp8_values(bits, fmt):
    """float64 values of fp8 bit patterns through torch's float8_e4m3fn / float8_e5m2."""
    import torch
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8))
    return t.view(dt).to(torch.float64).numpy()


def _fp8_ints(bits, fmt):
    v = torch_fp8_values(bits, fmt)
    q = np.ldexp(v, _FP8_QUANTUM_EXP[fmt])
    assert np.all(np.isfinite(q)) and np.array_equal(q, np.rint(q))
    return q.astype(np.int64)


def exact_fp8_gemm(a_bits, b_bits, M, N, K, ta, tb, a_fmt, b_fmt):
    """Exact A·B as (integer matrix, power-of-two exponent): value = ints · 2^-e."""
    ai = _fp8_ints(a_bits, a_fmt).reshape((K, M) if ta else (M, K))
    bi = _fp8_ints(b_bits, b_fmt).reshape((N, K) if tb else (K, N))
    a_l = ai.T if ta else ai
    b_l = bi.T if tb else bi
    if K:
        top = int(np.abs(ai).max()) * int(np.abs(bi).max()) * K
        assert top < 2 ** 63, "operands too large for an exact int64 product"
    return a_l @ b_l, _FP8_QUANTUM_EXP[a_fmt] + _FP8_QUANTUM_EXP[b_fmt]


FP8_SHAPES = [(16, 16, 128), (32, 16, 256), (48, 32, 128), (16, 64, 384)]


def pin_fp8_gemm_exact(fn, shapes=FP8_SHAPES):
    """fp8 GEMM within fp64 rounding of the exact integer result: all format pairs, all
    transposes, both betas; values spread over the whole finite range of each format."""
    seed = 700
    for (M, N, K) in shapes:
        for a_fmt, b_fmt in FP8_PAIRS:
            for ta in (False, True):
                for tb in (False, True):
                    for beta in (0.0, 1.0):
                        seed += 3
                        a_bits, b_bits, c = synth.gemm_fp8_inputs(
                            M, N, K, a_fmt, b_fmt, ta, tb, beta, (seed, seed + 1, seed + 2),
                            scale=4.0)
                        ints, e = exact_fp8_gemm(a_bits, b_bits, M, N, K, ta, tb, a_fmt, b_fmt)
                        exact = np.ldexp(ints.astype(np.float64), -e)   # may round: bound below
                        d = fn(a_bits, b_bits, c, M, N, K, ta, tb, beta, a_fmt, b_fmt)
                        assert d.shape == (M, N)
                        if beta == 1.0:
                            exact = exact + c.astype(np.float64)
                        mag = np.ldexp(np.abs(ints).astype(np.float64), -e)
                        lim = (K + 4) * 2.0 ** -52 * (mag + (np.abs(c) if beta else 0.0)) + 1e-300
                        assert np.all(np.abs(d - exact) <= lim), (M, N, K, a_fmt, b_fmt, ta, tb, beta)


def pin_fp8_gemm_beta(fn):
    """beta = 0 never reads C (NaN C is harmless); beta = 1 with A = 0 returns C exactly."""
    M, N, K = 32, 16, 128
    a_bits, b_bits, c = synth.gemm_fp8_inputs(M, N, K, "e4m3", "e5m2", False, True, 1.0, (81, 82, 83))
    nan_c = np.full((M, N), np.nan, dtype=np.float32)
    d0 = fn(a_bits, b_bits, None, M, N, K, False, True, 0.0, "e4m3", "e5m2")
    d0n = fn(a_bits, b_bits, nan_c, M, N, K, False, True, 0.0, "e4m3", "e5m2")
    assert np.all(np.isfinite(d0n)) and np.array_equal(d0, d0n)
    d1 = fn(np.zeros_like(a_bits), b_bits, c, M, N, K, False, True, 1.0, "e4m3", "e5m2")
    assert np.array_equal(d1, c.astype(np.float64))


def pin_fp8_gemm_transpose(fn):
    """Storing an operand transposed and setting its flag gives bit-identical results."""
    M, N, K = 48, 32, 256
    for a_fmt, b_fmt in FP8_PAIRS:
        a_bits, b_bits, c = synth.gemm_fp8_inputs(M, N, K, a_fmt, b_fmt, False, False, 1.0,
                                                  (91, 92, 93))
        ref = fn(a_bits, b_bits, c, M, N, K, False, False, 1.0, a_fmt, b_fmt)
        for ta in (False, True):
            for tb in (False, True):
                a_st = np.ascontiguousarray(a_bits.T) if ta else a_bits
                b_st = np.ascontiguousarray(b_bits.T) if tb else b_bits
                d = fn(a_st, b_st, c, M, N, K, ta, tb, 1.0, a_fmt, b_fmt)
                assert np.array_equal(d, ref), (a_fmt, b_fmt, ta, tb)


def pin_fp8_gemm_identity(fn):
    """A = I (1.0 is 0x38 in e4m3, 0x3C in e5m2) gives B's values exactly, for B in the other
    format too; K = 0 gives 0 or C."""
    one = {"e4m3": 0x38, "e5m2": 0x3C}
    M = K = 128
    N = 32
    for a_fmt, b_fmt in FP8_PAIRS:
        eye = np.zeros((M, K), dtype=np.uint8)
        eye[np.arange(M), np.arange(K)] = one[a_fmt]
        _, b_bits, _ = synth.gemm_fp8_inputs(16, N, K, a_fmt, b_fmt, False, False, 0.0, (95, 96, 0))
        d = fn(eye, b_bits, None, M, N, K, False, False, 0.0, a_fmt, b_fmt)
        assert np.array_equal(d, torch_fp8_values(b_bits, b_fmt).reshape(K, N)), (a_fmt, b_fmt)
    c = np.arange(16 * 16, dtype=np.float32).reshape(16, 16)
    e_a = np.zeros((16, 0), np.uint8)
    e_b = np.zeros((0, 16), np.uint8)
    assert np.array_equal(fn(e_a, e_b, None, 16, 16, 0, False, False, 0.0, "e4m3", "e4m3"),
                          np.zeros((16, 16)))
    assert np.array_equal(fn(e_a, e_b, c, 16, 16, 0, False, False, 1.0, "e5m2", "e4m3"),
                          c.astype(np.float64))


FP8_GEMM_PINS = (pin_fp8_gemm_exact, pin_fp8_gemm_beta, pin_fp8_gemm_transpose,
                 pin_fp8_gemm_identity)


def pin_fp8_sampled_exact(fn_at):
    """The per-output dot path for fp8 equals the exact integer result at sampled points."""
    M, N, K = 64, 48, 384
    for (a_fmt, b_fmt), ta, tb, beta in ((("e4m3", "e4m3"), False, True, 0.0),
                                         (("e5m2", "e4m3"), True, False, 1.0),
                                         (("e4m3", "e5m2"), True, True, 1.0)):
        a_bits, b_bits, c = synth.gemm_fp8_inputs(M, N, K, a_fmt, b_fmt, ta, tb, beta,
                                                  (97, 98, 99), scale=8.0)
        ints, e = exact_fp8_gemm(a_bits, b_bits, M, N, K, ta, tb, a_fmt, b_fmt)
        rows, cols = synth.sample_points(M, N, 100, count=300, tile=(16, 16))
        d, bound = fn_at(a_bits, b_bits, c, M, N, K, ta, tb, beta, a_fmt, b_fmt, rows, cols)
        want = np.ldexp(ints[rows, cols].astype(np.float64), -e)
        if beta == 1.0:
            want = want + c[rows, cols].astype(np.float64)
        mag = np.ldexp(np.abs(ints[rows, cols]).astype(np.float64), -e)
        assert np.all(np.abs(d - want) <= (K + 4) * 2.0 ** -52 * (mag + 1.0))
        # the bound is sum |a·b| >= |sum a·b|, and at least the magnitude of each term
        assert np.all(bound >= mag * (1 - 1e-12))


def pin_fp8_decode(fn):
    """All 256 patterns of e4m3 and e5m2 against torch's conversions, and the formats'
    closed-form extremes."""
    bits = np.arange(256, dtype=np.uint8)
    for fmt in ("e4m3", "e5m2"):
        got = fn(bits, fmt)
        want = torch_fp8_values(bits, fmt)
        same = (got == want) | (np.isnan(got) & np.isnan(want))
        assert np.all(same), (fmt, np.nonzero(~same)[0][:8])
        assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(want[~np.isnan(want)]))
    e4, e5 = fn(bits, "e4m3"), fn(bits, "e5m2")
    assert e4[0x7E] == 448.0 and np.isnan(e4[0x7F]) and e4[0x01] == 2.0 ** -9 and e4[0x08] == 2.0 ** -6
    assert e4[0x78] == 256.0 and e4[0x38] == 1.0 and np.isnan(e4[0xFF]) and e4[0xFE] == -448.0
    assert e5[0x7B] == 57344.0 and e5[0x7C] == np.inf and e5[0xFC] == -np.inf
    assert e5[0x01] == 2.0 ** -16 and e5[0x04] == 2.0 ** -14 and e5[0x3C] == 1.0
    assert int(np.isnan(e4).sum()) == 2 and int(np.isnan(e5).sum()) == 6
