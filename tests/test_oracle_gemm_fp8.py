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
