"""Planted mistakes in copies of the oracle must be caught by the pins.

Each mutant is a plausible slip (a transposed operand, a wrong sign, a dropped
term, an ignored flag or alignment rule).  The test passes when at least one pin
check fails on the mutant; the real oracle is never modified.
"""

import numpy as np
import pytest

from oracle import gemm as G
from oracle import layout as L
from oracle import planner as P
from oracle.numerics import decode
from tests import pins


def _mut_gemm(kind):
    def fn(a_bits, b_bits, c, M, N, K, ta, tb, beta, dtype):
        a = decode(a_bits, dtype).reshape((K, M) if ta else (M, K))
        b = decode(b_bits, dtype).reshape((N, K) if tb else (K, N))
        a_l = a.T if ta else a
        b_l = b.T if tb else b
        if kind == "ignore_trans_a":
            a_l = decode(a_bits, dtype).reshape(M, K)
        if kind == "ignore_trans_b":
            b_l = decode(b_bits, dtype).reshape(K, N)
        if kind == "abs_a":
            a_l = np.abs(a_l)
        if kind == "drop_last_k" and K:
            a_l = a_l[:, :-1]
            b_l = b_l[:-1, :]
        d = a_l @ b_l if a_l.shape[1] else np.zeros((M, N))
        if kind == "beta_ignored":
            return d
        if kind == "subtract_c" and beta == 1.0:
            return d - np.asarray(c, np.float32).reshape(M, N).astype(np.float64)
        if kind == "read_c_when_beta0" and c is not None:
            return d + beta * np.asarray(c, np.float32).reshape(M, N).astype(np.float64)
        if kind == "c_shifted" and beta == 1.0:
            return d + np.roll(np.asarray(c, np.float32).reshape(M, N), 1, axis=0).astype(np.float64)
        if beta == 1.0:
            d = d + np.asarray(c, np.float32).reshape(M, N).astype(np.float64)
        return d
    return fn


def _caught(check, fn):
    try:
        check(fn)
    except Exception:
        return True
    return False


@pytest.mark.parametrize("kind", ["ignore_trans_a", "ignore_trans_b", "abs_a", "drop_last_k",
                                  "beta_ignored", "subtract_c", "read_c_when_beta0", "c_shifted"])
def test_gemm_mutant_is_caught(kind):
    fn = _mut_gemm(kind)
    shapes = pins.SMALL_SHAPES[:4]
    assert (_caught(lambda f: pins.pin_gemm_brute_force(f, shapes), fn)
            or any(_caught(p, fn) for p in pins.GEMM_PINS[1:]))


def test_acceptance_mutants_are_caught():
    from tests.test_oracle_gemm import test_acceptance_table as t
    import inspect
    params = [m for m in t.pytestmark if m.name == "parametrize"][0].args[1]

    def run(accepts_fn):
        for args, cat in params:
            ok, why = accepts_fn(**args)
            assert ok == (cat is None) and why == cat

    def no_alpha(M, N, K, a_dtype, b_dtype, c_dtype="f32", d_dtype="f32", alpha=1.0, beta=0.0):
        return G.accepts(M, N, K, a_dtype, b_dtype, c_dtype, d_dtype, 1.0, beta)

    def loose_k(M, N, K, a_dtype, b_dtype, c_dtype="f32", d_dtype="f32", alpha=1.0, beta=0.0):
        return G.accepts(M, N, K - K % 8, a_dtype, b_dtype, c_dtype, d_dtype, alpha, beta)

    def mixed_ok(M, N, K, a_dtype, b_dtype, c_dtype="f32", d_dtype="f32", alpha=1.0, beta=0.0):
        return G.accepts(M, N, K, a_dtype, a_dtype, c_dtype, d_dtype, alpha, beta)

    for m in (no_alpha, loose_k, mixed_ok):
        assert _caught(run, m)
    assert inspect.isfunction(t)


def _planner_pins():
    from tests import test_oracle_planner as T
    checks = [T.test_worked_example_32x32_f32_one_warp, T.test_dtype_rounds_table,
              T.test_rejections_and_narrowing, T.test_swizzled_side_caps_vector_at_one_chunk,
              T.test_tiled_plan_is_min_over_tiles]
    cases = list(T._cases())

    def brute(_):
        for case in cases:
            T.test_plan_is_valid_and_widest(case)
    return [lambda _, c=c: c() for c in checks] + [brute]


@pytest.mark.parametrize("kind", ["no_base", "no_ld", "narrow_first", "no_thread_check",
                                  "no_vec_divides"])
def test_planner_mutant_is_caught(kind, monkeypatch):
    orig_width_ok = P._width_ok
    orig_plan = P.plan_region

    def width_ok(side, rows, cols, order, v, eb):
        if kind == "no_base":
            side = L.Layout(side.kind, side.ld, 0)
        if kind == "no_ld" and side.kind != L.XOR:
            ld = side.eff_ld(rows, cols)
            side = L.Layout(side.kind, ld - ld % v if ld % v and ld > v else ld, side.base)
        return orig_width_ok(side, rows, cols, order, v, eb)

    def plan_region(rows, cols, elem_bits, threads, drive, other):
        if kind == "no_thread_check":
            if threads <= 0:
                threads = 1
            if (rows * cols) % threads:
                return P.Plan((rows * cols) // threads, threads, 1, elem_bits)
        if kind == "narrow_first":
            monkeypatch.setattr(P, "WIDTHS_BITS", (8, 16, 32, 64, 128))
        if kind == "no_vec_divides":
            n = rows * cols
            for bits in (128, 64, 32, 16, 8):
                if bits < elem_bits:
                    continue
                v = bits // elem_bits
                if all(orig_width_ok(s, rows, cols, P.fused_order(drive), v, elem_bits // 8) for s in (drive, other)) \
                        and threads > 0 and n % threads == 0:
                    return P.Plan(max(1, n // (threads * v)), threads, v, bits)
        return orig_plan(rows, cols, elem_bits, threads, drive, other)

    monkeypatch.setattr(P, "_width_ok", width_ok)
    monkeypatch.setattr(P, "plan_region", plan_region)
    import tests.test_oracle_planner as T
    monkeypatch.setattr(T, "plan_region", plan_region)
    assert any(_caught(p, None) for p in _planner_pins())


@pytest.mark.parametrize("kind", ["period4", "col_as_row", "xor_whole_row"])
def test_layout_mutant_is_caught(kind, monkeypatch):
    import tests.test_oracle_copy as T
    orig_offsets = L.offsets

    def xor_offset(r, c, cols, eb):
        ce = 16 // eb
        chunks = cols // ce
        r = np.asarray(r, dtype=np.int64)
        c = np.asarray(c, dtype=np.int64)
        if kind == "period4":
            return r * cols + ((c // ce) ^ (r % min(4, chunks))) * ce + c % ce
        if kind == "xor_whole_row":
            return r * cols + (c ^ (r % min(8, cols)))
        return r * cols + ((c // ce) ^ (r % min(8, chunks))) * ce + c % ce

    def offsets(layout, rows, cols, eb):
        if kind == "col_as_row" and layout.kind == L.COL:
            layout = L.Layout(L.ROW, 0, layout.base)
        return orig_offsets(layout, rows, cols, eb)

    monkeypatch.setattr(L, "xor_offset", xor_offset)
    monkeypatch.setattr(L, "offsets", offsets)
    monkeypatch.setattr(T, "offsets", offsets)
    monkeypatch.setattr(T, "xor_offset", xor_offset)
    import oracle.copy as C
    monkeypatch.setattr(C, "offsets", offsets)
    checks = [T.test_xor_matches_byte_address_form_for_128_byte_rows, T.test_copy_row_to_col_is_transpose]
    checks += [lambda a=a: T.test_xor_layout_is_a_bijection_with_whole_chunks(*a) for a in T.TILES]
    checks += [lambda a=a: T.test_xor_layout_is_an_involution(*a) for a in T.TILES]
    assert any(_caught(lambda _: c(), None) for c in checks)


# ---- fp8 GEMM and the 8-bit decoders ---------------------------------------------------

def _mut_fp8_decode(kind):
    from oracle.numerics import fp8_bits_to_f64

    def fn(bits, fmt):
        u = np.asarray(bits, np.uint8).astype(np.int64)
        if kind == "fnuz_bias":            # e4m3 read with the bias of the FNUZ variant
            v = fp8_bits_to_f64(bits, fmt)
            return v / 2.0 if fmt == "e4m3" else v
        if kind == "e4m3_ieee_specials":  # e4m3 given infinities like e5m2
            v = fp8_bits_to_f64(bits, fmt)
            if fmt == "e4m3":
                e, m = (u >> 3) & 15, u & 7
                v = np.where(e == 15, np.where(m == 0, np.where(u >> 7, -np.inf, np.inf), np.nan), v)
            return v
        if kind == "no_subnormals":        # exponent 0 read as a normal number
            ebits, mbits = (4, 3) if fmt == "e4m3" else (5, 2)
            bias = (1 << (ebits - 1)) - 1
            v = fp8_bits_to_f64(bits, fmt)
            e = (u >> mbits) & ((1 << ebits) - 1)
            m = u & ((1 << mbits) - 1)
            sub = np.where(u >> 7, -1.0, 1.0) * np.ldexp((1 << mbits) + m, -bias - mbits)
            return np.where((e == 0) & (m != 0), sub, v)
        if kind == "e5m2_inf_as_nan":
            v = fp8_bits_to_f64(bits, fmt)
            return np.where(np.isinf(v), np.nan, v) if fmt == "e5m2" else v
        if kind == "lost_sign_of_zero":
            v = fp8_bits_to_f64(bits, fmt)
            return np.where(v == 0, 0.0, v)
        raise AssertionError(kind)
    return fn


@pytest.mark.parametrize("kind", ["fnuz_bias", "e4m3_ieee_specials", "no_subnormals",
                                  "e5m2_inf_as_nan", "lost_sign_of_zero"])
def test_fp8_decoder_mutant_is_caught(kind):
    assert _caught(pins.pin_fp8_decode, _mut_fp8_decode(kind))


def _mut_fp8_gemm(kind):
    def fn(a_bits, b_bits, c, M, N, K, ta, tb, beta, a_fmt, b_fmt):
        if kind == "b_in_a_format":
            b_fmt = a_fmt
        if kind == "formats_swapped":
            a_fmt, b_fmt = b_fmt, a_fmt
        a = decode(a_bits, a_fmt).reshape((K, M) if ta else (M, K))
        b = decode(b_bits, b_fmt).reshape((N, K) if tb else (K, N))
        a_l = a.T if ta else a
        b_l = b.T if tb else b
        if kind == "ignore_trans_b":
            b_l = decode(b_bits, b_fmt).reshape(K, N)
        if kind == "half_k" and K:
            a_l = a_l[:, :K // 2]
            b_l = b_l[:K // 2, :]
        d = a_l @ b_l if a_l.shape[1] else np.zeros((M, N))
        if kind == "saturate_products":
            d = np.clip(d, -448.0, 448.0)
        if beta == 1.0 and kind != "beta_ignored":
            d = d + np.asarray(c, np.float32).reshape(M, N).astype(np.float64)
        return d
    return fn


@pytest.mark.parametrize("kind", ["b_in_a_format", "formats_swapped", "ignore_trans_b", "half_k",
                                  "saturate_products", "beta_ignored"])
def test_fp8_gemm_mutant_is_caught(kind):
    fn = _mut_fp8_gemm(kind)
    assert any(_caught(p, fn) for p in pins.FP8_GEMM_PINS)


def test_fp8_acceptance_mutants_are_caught():
    from tests.test_oracle_gemm_fp8 import test_acceptance_table as t
    params = [m for m in t.pytestmark if m.name == "parametrize"][0].args[1]

    def run(accepts_fn):
        for args, cat in params:
            ok, why = accepts_fn(**args)
            assert ok == (cat is None) and why == cat

    def k64(M, N, K, a_dtype, b_dtype, c_dtype="f32", d_dtype="f32", alpha=1.0, beta=0.0):
        return G.accepts_fp8(M, N, K - K % 128 if K % 64 == 0 else K, a_dtype, b_dtype, c_dtype,
                             d_dtype, alpha, beta)

    def n8(M, N, K, a_dtype, b_dtype, c_dtype="f32", d_dtype="f32", alpha=1.0, beta=0.0):
        return G.accepts_fp8(M, N - N % 16 if N % 8 == 0 else N, K, a_dtype, b_dtype, c_dtype,
                             d_dtype, alpha, beta)

    def any16(M, N, K, a_dtype, b_dtype, c_dtype="f32", d_dtype="f32", alpha=1.0, beta=0.0):
        fix = {"f16": "e4m3", "bf16": "e5m2"}
        return G.accepts_fp8(M, N, K, fix.get(a_dtype, a_dtype), fix.get(b_dtype, b_dtype),
                             c_dtype, d_dtype, alpha, beta)

    run(G.accepts_fp8)
    for mutant in (k64, n8, any16):
        assert _caught(run, mutant)


# ---- 6- and 4-bit operands of the block-scaled GEMM --------------------------------------

def _small_pins():
    import tests.test_oracle_gemm_mx_small as T
    checks = [T.test_e2m1_value_table, T.test_fp4_embeds_in_e2m3, T.test_unpack_hand_built_bytes,
              lambda: T.test_unpack_inverts_the_input_packer(4),
              lambda: T.test_unpack_inverts_the_input_packer(6),
              lambda: T.test_fraction_brute_force("e2m1", "e2m1"),
              lambda: T.test_fraction_brute_force("e2m3", "e3m2"),
              T.test_scale_raises_one_block_by_two]
    checks += [lambda f=f: T.test_fp6_values_are_e4m3_values(f) for f in ("e2m3", "e3m2")]
    checks += [lambda f=f, t=t, s=s: T.test_extremes_monotone_and_symmetric(f, t, s)
               for f, t, s in (("e2m3", 7.5, 0.125), ("e3m2", 28.0, 0.0625), ("e2m1", 6.0, 0.5))]
    checks += [lambda f=f: T.test_ones_times_b_is_column_sums(f) for f in ("e2m3", "e3m2", "e2m1")]
    return checks


@pytest.mark.parametrize("kind", ["high_nibble_first", "e2m3_bias_2", "e3m2_subnormal_as_normal",
                                  "fp6_in_bytes", "scale_block_16", "scales_of_b_on_a"])
def test_small_format_mutant_is_caught(kind, monkeypatch):
    import oracle.numerics as Nm
    orig_small, orig_unpack = Nm.small_bits_to_f64, Nm.unpack_rows

    def small(codes, fmt):
        u = np.asarray(codes).astype(np.int64)
        if kind == "e2m3_bias_2" and fmt == "e2m3":
            return orig_small(codes, fmt) / 2.0
        if kind == "e3m2_subnormal_as_normal" and fmt == "e3m2":
            e, f = (u >> 2) & 7, u & 3
            v = orig_small(codes, fmt)
            return np.where((e == 0) & (f != 0), np.where(u >> 5, -1.0, 1.0) * (4 + f) / 16.0, v)
        return orig_small(codes, fmt)

    def unpack(packed, rows, K, width):
        if kind == "high_nibble_first" and width == 4:
            b = np.ascontiguousarray(packed, np.uint8)
            return orig_unpack(((b >> 4) | (b << 4)).astype(np.uint8), rows, K, width)
        if kind == "fp6_in_bytes" and width == 6:
            b = np.ascontiguousarray(packed, np.uint8).reshape(rows, -1)
            out = np.zeros((rows, K), np.int64)
            n = min(K, b.shape[1])
            out[:, :n] = b[:, :n] & 63
            return out
        return orig_unpack(packed, rows, K, width)

    monkeypatch.setattr(Nm, "small_bits_to_f64", small)
    monkeypatch.setattr(Nm, "unpack_rows", unpack)
    monkeypatch.setattr(G, "unpack_rows", unpack)
    import tests.test_oracle_gemm_mx_small as T
    monkeypatch.setattr(T, "small_bits_to_f64", small)
    monkeypatch.setattr(T, "unpack_rows", unpack)
    if kind == "scale_block_16":
        monkeypatch.setattr(G, "MX_BLOCK", 16)
    if kind == "scales_of_b_on_a":
        orig = G._scaled_operands

        def swapped(a_bits, b_bits, sa_bits, sb_bits, M, N, K, ta, tb, af, bf):
            return orig(a_bits, b_bits, sb_bits if M == N else sa_bits, sa_bits if M == N else sb_bits,
                        M, N, K, ta, tb, af, bf)
        monkeypatch.setattr(G, "_scaled_operands", swapped)
    assert any(_caught(lambda _: c(), None) for c in _small_pins())
