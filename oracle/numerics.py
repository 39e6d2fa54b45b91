"""Exact decoding of 16-bit floating-point bit patterns (oracle; test infrastructure).

[SYNC-GEMM] 二 (What it accepts): A and B are both float16 or both bfloat16,
C and D are float32.  The oracle receives A and B as the raw uint16 bit patterns
the GPU receives, and decodes them to float64.  Both formats embed exactly in
float64, so the decode is exact (subnormals included).

Pinned by tests/test_oracle_numerics.py: exhaustive comparison of all 65 536
patterns of each format with a sign/exponent/mantissa formula written in the
test from the IEEE-754 binary16 and the bfloat16 definitions.
"""

import numpy as np


def f16_bits_to_f64(bits):
    """IEEE binary16 bit patterns (uint16 array) -> float64, exact."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16 array) -> float64, exact.

    A bfloat16 value is the upper half of an IEEE binary32 value.
    """
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode(bits, dtype):
    """Decode by format name: 'f16' or 'bf16'."""
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    raise ValueError(f"oracle: unknown 16-bit format {dtype!r}")
