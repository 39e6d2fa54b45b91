"""Pins of the fp8 GEMM oracle ([SYNC-GEMM] 七: fp8 operands of the asynchronous GEMM)."""

import numpy as np
import pytest

from oracle import gemm as G
from tests import pins
import synth


def test_exact_integer_products():
    pins.pin_fp8_gemm_exact(G.gemm_fp8_ref)


def test_beta_semantics():
    pins.pin_fp8_gemm_beta(G.gemm_fp8_ref)


def test_transpose_equivalence():
    pins.pin_fp8_gemm_transpose(G.gemm_fp8_ref)


def test_identity_and_empty():
    pins.pin_fp8_gemm_identity(G.gemm_fp8_ref)


def test_sampled_path_exact():
    pins.pin_fp8_sampled_exact(G.gemm_fp8_ref_at)


def test_sampled_equals_full():
    M, N, K = 96, 80, 256
    a_bits, b_bits, c = synth.gemm_fp8_inputs(M, N, K, "e5m2", "e4m3", True, False, 1.0, (5, 6, 7))
    full = G.gemm_fp8_ref(a_bits, b_bits, c, M, N, K, True, False, 1.0, "e5m2", "e4m3")
    bound = G.abs_bound_fp8(a_bits, b_bits, M, N, K, True, False, "e5m2", "e4m3")
    rows, cols = synth.sample_points(M, N, 8, count=500, tile=(16, 16))
    d, bd = G.gemm_fp8_ref_at(a_bits, b_bits, c, M, N, K, True, False, 1.0, "e5m2", "e4m3",
                              rows, cols)
    assert np.allclose(d, full[rows, cols], rtol=1e-13, atol=1e-13)
    assert np.allclose(bd, bound[rows, cols], rtol=1e-13, atol=0)


@pytest.mark.parametrize("args,category", [
    (dict(M=16, N=16, K=128, a_dtype="e4m3", b_dtype="e4m3"), None),
    (dict(M=256, N=512, K=384, a_dtype="e5m2", b_dtype="e4m3", beta=1.0), None),
    (dict(M=0, N=0, K=0, a_dtype="e4m3", b_dtype="e5m2"), None),
    (dict(M=8, N=16, K=128, a_dtype="e4m3", b_dtype="e4m3"), "shape"),
    (dict(M=16, N=8, K=128, a_dtype="e4m3", b_dtype="e4m3"), "shape"),
    (dict(M=16, N=16, K=64, a_dtype="e4m3", b_dtype="e4m3"), "shape"),
    (dict(M=16, N=16, K=192, a_dtype="e4m3", b_dtype="e4m3"), "shape"),
    (dict(M=-16, N=16, K=128, a_dtype="e4m3", b_dtype="e4m3"), "shape"),
    (dict(M=16, N=16, K=128, a_dtype="f16", b_dtype="e4m3"), "dtype"),
    (dict(M=16, N=16, K=128, a_dtype="e4m3", b_dtype="bf16"), "dtype"),
    (dict(M=16, N=16, K=128, a_dtype="e4m3", b_dtype="e4m3", c_dtype="f16"), "dtype"),
    (dict(M=16, N=16, K=128, a_dtype="e4m3", b_dtype="e4m3", d_dtype="bf16"), "dtype"),
    (dict(M=16, N=16, K=128, a_dtype="e4m3", b_dtype="e4m3", alpha=2.0), "alpha"),
    (dict(M=16, N=16, K=128, a_dtype="e4m3", b_dtype="e4m3", beta=0.5), "beta"),
    (dict(M=8, N=16, K=128, a_dtype="f16", b_dtype="e4m3", beta=0.5), "shape"),
])
def test_acceptance_table(args, category):
    ok, why = G.accepts_fp8(**args)
    assert ok == (category is None)
    assert why == category


def test_rejected_call_raises():
    a = np.zeros((16, 64), np.uint8)
    with pytest.raises(ValueError):
        G.gemm_fp8_ref(a, a, None, 16, 16, 64, False, True, 0.0, "e4m3", "e4m3")


# ---- the fp8 comparison bar: the unit's allowance ---------------------------------------

def _allowance_loops(a_vals, b_vals, group=8, window=13):
    """Pure-Python restatement for tiny inputs: a_vals [M][K], b_vals [K][N] (floats)."""
    import math
    M, K, N = len(a_vals), len(a_vals[0]), len(b_vals[0])
    out = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            t = 0.0
            for g0 in range(0, K, group):
                ps = [abs(a_vals[i][k] * b_vals[k][j]) for k in range(g0, g0 + group)]
                top = max(ps)
                if top == 0.0:
                    continue
                _, ex = math.frexp(top)          # top = f·2^ex, f in [0.5, 1)
                q = math.ldexp(1.0, ex - 1 - window)
                for p in ps:
                    if math.fmod(p, q) != 0.0:
                        t += min(p, q)
            out[i][j] = t
    return np.array(out)


def allowance_pin(fn):
    """fn(a_bits, b_bits, M, N, K, ta, tb, a_fmt, b_fmt, rows, cols) -> T at the points."""
    from tests.pins import torch_fp8_values
    # brute force on tiny full-range inputs, all format pairs, stored [M,K] / [N,K]
    for s, (af, bf) in enumerate(pins.FP8_PAIRS):
        M, N, K = 4, 3, 32
        a_bits = synth.random_bits(300 + s, M * K, 1).reshape(M, K)
        b_bits = synth.random_bits(400 + s, N * K, 1).reshape(N, K)
        a_bits = np.where(np.isfinite(torch_fp8_values(a_bits, af)), a_bits, 0).astype(np.uint8)
        b_bits = np.where(np.isfinite(torch_fp8_values(b_bits, bf)), b_bits, 0).astype(np.uint8)
        av = torch_fp8_values(a_bits, af).reshape(M, K)
        bv = torch_fp8_values(b_bits, bf).reshape(N, K).T
        want = _allowance_loops(av.tolist(), bv.tolist())
        rr, cc = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        got = fn(a_bits, b_bits, M, N, K, False, True, af, bf, rr.ravel(), cc.ravel()).reshape(M, N)
        assert np.allclose(got, want, rtol=1e-12, atol=0), (af, bf)
    # closed cases, e5m2 x e5m2 with B = 1: D[0][0] = sum_k A[0][k]
    def e5m2(v):
        return synth.fp8_bits(np.array([v], np.float32), "e5m2")[0]

    def one_row(vals):
        K = 16
        a = np.zeros((16, K), np.uint8)
        for k, v in vals.items():
            a[0, k] = e5m2(v)
        b = np.full((16, K), e5m2(1.0), np.uint8)
        return float(fn(a, b, 16, 16, K, False, True, "e5m2", "e5m2", [0], [0])[0])
    assert one_row({0: 2.0 ** 10, 1: 2.0 ** 10, 2: 3.0 * 2 ** 8}) == 0.0        # all on the grid
    assert one_row({0: 2.0 ** 10, 1: 2.0 ** -4}) == 2.0 ** -4                    # q = 2^-3: lost
    assert one_row({0: 2.0 ** 10, 1: 2.0 ** -3}) == 0.0                          # exactly on q
    assert one_row({0: 2.0 ** 10, 1: 2.0 ** -5, 2: -2.0 ** -6}) == 2.0 ** -5 + 2.0 ** -6
    assert one_row({0: 1.5 * 2 ** 10, 1: 2.0 ** -4}) == 2.0 ** -4               # floor(log2 1536) = 10
    assert one_row({0: 2.0 ** 10, 8: 2.0 ** -4}) == 0.0                          # other group of 8
    assert one_row({7: 2.0 ** 10, 8: 2.0 ** -4, 15: 2.0 ** -4}) == 0.0           # groups align to 8
    assert one_row({}) == 0.0


def test_unit_allowance_pins():
    allowance_pin(G.fp8_unit_allowance_at)


@pytest.mark.parametrize("kind", ["window14", "window12", "group16", "group4", "count_on_grid",
                                  "full_product"])
def test_unit_allowance_mutants_are_caught(kind):
    import oracle.gemm as g

    def mutant(a_bits, b_bits, M, N, K, ta, tb, af, bf, rows, cols):
        saved = (g.FP8_GROUP, g.FP8_WINDOW)
        try:
            if kind == "window14":
                g.FP8_WINDOW = 14
            if kind == "window12":
                g.FP8_WINDOW = 12
            if kind == "group16":
                g.FP8_GROUP = 16
            if kind == "group4":
                g.FP8_GROUP = 4
            t = g.fp8_unit_allowance_at(a_bits, b_bits, M, N, K, ta, tb, af, bf, rows, cols)
        finally:
            g.FP8_GROUP, g.FP8_WINDOW = saved
        if kind in ("count_on_grid", "full_product"):
            a = g.decode(np.asarray(a_bits).reshape(M, K)[np.asarray(rows)], af)
            b = g.decode(np.asarray(b_bits).reshape(N, K)[np.asarray(cols)], bf)
            p = np.abs(a * b).reshape(len(rows), K // 8, 8)
            mx = p.max(axis=2, keepdims=True)
            e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
            q = np.ldexp(1.0, (e - 13).astype(np.int64))
            if kind == "full_product":      # a lost product costs all of itself, not < q
                return np.where(np.mod(p, q) != 0, p, 0.0).sum(axis=(1, 2))
            return np.minimum(p, q).sum(axis=(1, 2))   # on-grid products counted too
        return t
    with pytest.raises(AssertionError):
        allowance_pin(mutant)


def test_check_fp8_uses_allowance_only_where_needed():
    # seven products lost within one group (beyond the 16-bit bar) pass; twice that fails
    M, N, K = 16, 16, 128
    a = np.zeros((M, K), np.uint8)
    b = np.full((N, K), 0x3C, np.uint8)           # e5m2 1.0
    a[:, 0] = synth.fp8_bits(np.float32([2.0 ** 10]), "e5m2")[0]
    a[:, 1:8] = synth.fp8_bits(np.float32([2.0 ** -4]), "e5m2")[0]   # q = 2^-3: all lost
    ref = G.gemm_fp8_ref(a, b, None, M, N, K, False, True, 0.0, "e5m2", "e5m2")
    bound = G.abs_bound_fp8(a, b, M, N, K, False, True, "e5m2", "e5m2")
    lost = ref - 7 * 2.0 ** -4
    assert np.all(np.abs(lost - ref) > G.tolerance(bound))
    ok, worst = G.check_fp8(lost, ref, bound, a, b, M, N, K, False, True, "e5m2", "e5m2")
    assert ok and worst <= 1.0
    ok, _ = G.check_fp8(ref - 14 * 2.0 ** -4, ref, bound, a, b, M, N, K, False, True, "e5m2", "e5m2")
    assert not ok
    # sampled form
    rows, cols = np.array([0, 3, 15]), np.array([1, 2, 15])
    ok, _ = G.check_fp8(lost[rows, cols], ref[rows, cols], bound[rows, cols], a, b, M, N, K, False,
                        True, "e5m2", "e5m2", rows, cols)
    assert ok
    ok, worst = G.check_fp8(ref, ref, bound, a, b, M, N, K, False, True, "e5m2", "e5m2")
    assert ok and worst == 0.0


def _fp8_codes_in(fmt, lo, hi):
    """Every finite fp8 code of `fmt` whose magnitude lies in [lo, hi)."""
    from oracle.numerics import fp8_bits_to_f64
    codes = np.arange(256, dtype=np.uint8)
    v = np.abs(fp8_bits_to_f64(codes, fmt))
    return codes[np.isfinite(v) & (v >= lo) & (v < hi)]


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e5m2", "e5m2")])
def test_fp8_bar_is_the_16bit_bar_within_six_binades(fa, fb):
    # An fp8 product carries at most 8 significant bits, so a product within 2^6 of its group's
    # largest lies on the group's 2^-13 grid: the allowance is exactly zero and the fp8 bar is
    # the 16-bit bar (1e-4·sum|a·b| + 1e-6).  Operands drawn from [1, 2) and [2^-2, 2^1) keep
    # every product in [2^-2, 2^2), inside six binades of any group maximum.
    rs = np.random.default_rng(8)
    M, N, K = 32, 48, 256
    ca, cb = _fp8_codes_in(fa, 1.0, 2.0), _fp8_codes_in(fb, 0.25, 2.0)
    a = rs.choice(ca, size=(M, K)) ^ (rs.integers(0, 2, (M, K), dtype=np.uint8) << 7)
    b = rs.choice(cb, size=(K, N)) ^ (rs.integers(0, 2, (K, N), dtype=np.uint8) << 7)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    t = G.fp8_unit_allowance_at(a, b, M, N, K, False, False, fa, fb, rows.ravel(), cols.ravel())
    assert np.all(t == 0.0)
    d = G.gemm_fp8_ref(a, b, None, M, N, K, False, False, 0.0, fa, fb)
    bound = G.abs_bound_fp8(a, b, M, N, K, False, False, fa, fb)
    perturbed = d + 0.9 * G.tolerance(bound)
    assert G.check_fp8(perturbed, d, bound, a, b, M, N, K, False, False, fa, fb) == \
        G.check(perturbed, d, bound)
    over = d + 1.1 * G.tolerance(bound)
    assert not G.check_fp8(over, d, bound, a, b, M, N, K, False, False, fa, fb)[0]


def test_fp8_allowance_appears_only_far_below_the_group_max():
    # One group of 8 products: seven at 1 and one with low bits set 2^-10 below; the low
    # product is off the 2^-13 grid of a group whose largest is 1 (q = 2^-13) only when it has
    # bits below 2^-13.  e4m3 1.125·2^-6 times 1.125·2^-4 = 1.265625·2^-10 = 0b1.010001·2^-10:
    # its last bit is 2^-16, off the grid, so the allowance is min(|p|, 2^-13) = 2^-13.
    from oracle.numerics import fp8_bits_to_f64
    codes = np.arange(256, dtype=np.uint8)
    val = fp8_bits_to_f64(codes, "e4m3")
    one = int(np.nonzero(val == 1.0)[0][0])
    x = int(np.nonzero(val == 1.125 * 2.0 ** -6)[0][0])
    y = int(np.nonzero(val == 1.125 * 2.0 ** -4)[0][0])
    a = np.full((1, 8), one, np.uint8)
    b = np.full((8, 1), one, np.uint8)
    a[0, 7], b[7, 0] = x, y
    t = G.fp8_unit_allowance_at(a, b, 1, 1, 8, False, False, "e4m3", "e4m3", [0], [0])
    assert t[0] == 2.0 ** -13
    # the same low product alone in its group is on its own grid: no allowance
    a2 = np.full((1, 16), x, np.uint8)
    b2 = np.full((16, 1), y, np.uint8)
    a2[0, :8], b2[:8, 0] = one, one
    a2[0, 8:15], b2[8:15, 0] = 0, 0
    t2 = G.fp8_unit_allowance_at(a2, b2, 1, 1, 16, False, False, "e4m3", "e4m3", [0], [0])
    assert t2[0] == 0.0
