"""Pins of the GEMM oracle (CPU only)."""

import numpy as np
import pytest

import synth
from oracle import gemm
from tests import pins


def test_brute_force_small_shapes():
    pins.pin_gemm_brute_force(gemm.gemm_ref)


def test_beta_semantics():
    pins.pin_gemm_beta(gemm.gemm_ref)


def test_transpose_equivalence():
    pins.pin_gemm_transpose(gemm.gemm_ref)


def test_identity_and_zero():
    pins.pin_gemm_identity_zero(gemm.gemm_ref)


def test_sampled_path_matches_exact():
    pins.pin_sampled_matches_exact(gemm.gemm_ref_at)


def test_sampled_equals_full():
    M, N, K = 96, 80, 64
    a_bits, b_bits, c = synth.gemm_inputs(M, N, K, "bf16", True, True, 1.0, (1, 2, 3))
    full = gemm.gemm_ref(a_bits, b_bits, c, M, N, K, True, True, 1.0, "bf16")
    bfull = gemm.abs_bound(a_bits, b_bits, M, N, K, True, True, "bf16")
    rows, cols = synth.sample_points(M, N, 5, count=500, tile=(32, 32))
    d, bound = gemm.gemm_ref_at(a_bits, b_bits, c, M, N, K, True, True, 1.0, "bf16", rows, cols)
    assert np.allclose(d, full[rows, cols], rtol=1e-13, atol=1e-13)
    assert np.allclose(bound, bfull[rows, cols], rtol=1e-13, atol=0)


# The page's acceptance table and its listed rejections ([SYNC-GEMM] 二 and 测试覆盖:
# alpha = 2.0, beta = 0.5, f16 accumulate, mixed A/B, tf32, int8).
@pytest.mark.parametrize("args,category", [
    (dict(M=16, N=8, K=16, a_dtype="f16", b_dtype="f16"), None),
    (dict(M=16, N=8, K=16, a_dtype="bf16", b_dtype="bf16", beta=1.0), None),
    (dict(M=16, N=8, K=16, a_dtype="f16", b_dtype="f16", alpha=2.0), "alpha"),
    (dict(M=16, N=8, K=16, a_dtype="f16", b_dtype="f16", beta=0.5), "beta"),
    (dict(M=16, N=8, K=16, a_dtype="f16", b_dtype="f16", c_dtype="f16", d_dtype="f16"), "dtype"),
    (dict(M=16, N=8, K=16, a_dtype="f16", b_dtype="bf16"), "dtype"),
    (dict(M=16, N=8, K=16, a_dtype="tf32", b_dtype="tf32"), "dtype"),
    (dict(M=16, N=8, K=16, a_dtype="i8", b_dtype="i8"), "dtype"),
    (dict(M=8, N=8, K=16, a_dtype="f16", b_dtype="f16"), "shape"),
    (dict(M=16, N=4, K=16, a_dtype="f16", b_dtype="f16"), "shape"),
    (dict(M=16, N=8, K=12, a_dtype="f16", b_dtype="f16"), "shape"),
    (dict(M=-16, N=8, K=16, a_dtype="f16", b_dtype="f16"), "shape"),
    (dict(M=0, N=8, K=16, a_dtype="f16", b_dtype="f16"), None),
    (dict(M=16, N=8, K=24, a_dtype="f16", b_dtype="f16"), None),
])
def test_acceptance_table(args, category):
    ok, why = gemm.accepts(**args)
    assert ok == (category is None)
    assert why == category


def test_tolerance_formula_values():
    assert gemm.tolerance(0.0) == pytest.approx(1e-6)
    assert gemm.tolerance(10.0) == pytest.approx(1e-3 + 1e-6)
    ok, worst = gemm.check(np.array([1.0 + 5e-5]), np.array([1.0]), np.array([1.0]))
    assert ok and worst < 1.0
    ok, _ = gemm.check(np.array([1.0 + 2e-4]), np.array([1.0]), np.array([1.0]))
    assert not ok
    ok, _ = gemm.check(np.array([np.nan]), np.array([1.0]), np.array([1.0]))
    assert not ok


def test_atom_reference_is_one_tile():
    """The 16x8x16 atom workload through the oracle has the right shape and is finite."""
    for beta in (0.0, 1.0):
        a_bits, b_bits, c = synth.atom_inputs(beta)
        d = gemm.gemm_ref(a_bits, b_bits, c, 16, 8, 16, False, False, beta, "f16")
        assert d.shape == (16, 8) and np.all(np.isfinite(d))
