"""Exact decoding of 16- and 8-bit floating-point bit patterns (oracle; test infrastructure).

[SYNC-GEMM] 二 (What it accepts): A and B are both float16 or both bfloat16,
C and D are float32.  The oracle receives A and B as the raw uint16 bit patterns
the GPU receives, and decodes them to float64.  Both formats embed exactly in
float64, so the decode is exact (subnormals included).

Pinned by tests/test_oracle_numerics.py: exhaustive comparison of all 65 536
patterns of each 16-bit format with a sign/exponent/mantissa formula written in
the test from the IEEE-754 binary16 and the bfloat16 definitions, and of all 256
patterns of each 8-bit format with torch's own float8_e4m3fn / float8_e5m2 /
float8_e8m0fnu conversions plus the formats' closed-form extremes.
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
    """Decode by format name: 'f16', 'bf16', 'e4m3', 'e5m2', or the 6- and 4-bit 'e2m3',
    'e3m2', 'e2m1' (codes one per array element, in the low bits)."""
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype in _FP8:
        return fp8_bits_to_f64(bits, dtype)
    if dtype in SMALL:
        return small_bits_to_f64(bits, dtype)
    raise ValueError(f"oracle: unknown format {dtype!r}")


# ---- 8-bit formats of the asynchronous GEMM's precision family ------------------------
# [SYNC-GEMM] 七 lists fp8 (and block-scaled variants with per-block scale factors) among
# the asynchronous GEMM's operand precisions.  The formats are the OCP 8-bit floats:
#
#   e4m3 ("E4M3FN"): sign, 4 exponent bits (bias 7), 3 fraction bits.  No infinities; the
#                    single pattern S.1111.111 is NaN, so the largest finite value is 448.
#   e5m2:            sign, 5 exponent bits (bias 15), 2 fraction bits, IEEE-style: exponent
#                    11111 is infinity (fraction 0) or NaN.
#   e8m0:            the block scale: 8 exponent bits, bias 127, no sign and no fraction;
#                    value 2^(E-127), and E = 255 is NaN.
#
# Every value embeds exactly in float64.

_FP8 = {"e4m3": (4, 3), "e5m2": (5, 2)}


def fp8_bits_to_f64(bits, fmt):
    """OCP fp8 bit patterns (uint8 array) -> float64, exact.  fmt: 'e4m3' or 'e5m2'."""
    if fmt not in _FP8:
        raise ValueError(f"oracle: unknown 8-bit format {fmt!r}")
    ebits, mbits = _FP8[fmt]
    bias = (1 << (ebits - 1)) - 1
    u = np.ascontiguousarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(u >> 7, -1.0, 1.0)
    e = (u >> mbits) & ((1 << ebits) - 1)
    m = u & ((1 << mbits) - 1)
    normal = np.ldexp((1 << mbits) + m, e - bias - mbits)
    sub = np.ldexp(m.astype(np.float64), 1 - bias - mbits)
    v = sign * np.where(e == 0, sub, normal)
    emax = (1 << ebits) - 1
    if fmt == "e4m3":
        v = np.where((e == emax) & (m == (1 << mbits) - 1), np.nan, v)
    else:
        v = np.where(e == emax, np.where(m == 0, sign * np.inf, np.nan), v)
    return v


def e8m0_bits_to_f64(bits):
    """E8M0 block-scale patterns (uint8 array) -> float64: 2^(E-127), E = 255 is NaN."""
    u = np.ascontiguousarray(bits, dtype=np.uint8).astype(np.int64)
    return np.where(u == 255, np.nan, np.ldexp(1.0, u - 127))


# ---- 6- and 4-bit formats of the block-scaled asynchronous GEMM -------------------------
# [SYNC-GEMM] 七 names fp4 among the asynchronous GEMM's operand precisions, with SFA / SFB
# block scales.  The formats here are the OCP microscaling element types, read from their
# definition (sign bit, exponent field, fraction field, exponent bias):
#
#   e2m3 (fp6): 1 + 2 + 3 bits, bias 1;   e3m2 (fp6): 1 + 3 + 2 bits, bias 3;
#   e2m1 (fp4): 1 + 2 + 1 bits, bias 1.
#
# A zero exponent field encodes the subnormals (fraction / 2^f) * 2^(1 - bias); any other
# field e the normals (1 + fraction / 2^f) * 2^(e - bias).  None of the three has infinities
# or NaNs: every code is a finite value, so the largest magnitudes are 7.5, 28 and 6.
#
# Packing (our reading; the page gives none): an operand stored K-contiguous keeps each row's
# K codes as one little-endian bit stream, code k at bits [w·k, w·k + w) of the row, w = 6
# or 4 — for fp4 two codes per byte, the even one in the low nibble; for fp6 four codes in
# every 3 bytes.  A row of K codes is K·w/8 bytes.

SMALL = {"e2m3": (2, 3, 1), "e3m2": (3, 2, 3), "e2m1": (2, 1, 1)}   # exponent bits, fraction bits, bias
SMALL_WIDTH = {"e2m3": 6, "e3m2": 6, "e2m1": 4}


def small_bits_to_f64(codes, fmt):
    """6- or 4-bit codes (an integer array, one code per element) -> float64, exact."""
    if fmt not in SMALL:
        raise ValueError(f"oracle: unknown small format {fmt!r}")
    ebits, fbits, bias = SMALL[fmt]
    u = np.ascontiguousarray(codes).astype(np.int64)
    if np.any((u < 0) | (u >= (1 << (1 + ebits + fbits)))):
        raise ValueError("oracle: code out of range for the format")
    sign = np.where((u >> (ebits + fbits)) & 1, -1.0, 1.0)
    e = (u >> fbits) & ((1 << ebits) - 1)
    f = u & ((1 << fbits) - 1)
    normal = np.ldexp(((1 << fbits) + f).astype(np.float64), e - bias - fbits)
    sub = np.ldexp(f.astype(np.float64), 1 - bias - fbits)
    return sign * np.where(e == 0, sub, normal)


def unpack_rows(packed, rows, K, width):
    """Codes [rows, K] from rows of K·width/8 bytes, code k of a row at bits [width·k, width·k +
    width) of that row's little-endian bit stream."""
    if (K * width) % 8:
        raise ValueError("oracle: a packed row must be a whole number of bytes")
    nb = K * width // 8
    b = np.ascontiguousarray(packed, dtype=np.uint8).reshape(rows, nb)
    bits = np.unpackbits(b, axis=1, bitorder="little")          # [rows, K·width], bit i of the row
    bits = bits.reshape(rows, K, width).astype(np.int64)
    return (bits << np.arange(width, dtype=np.int64)).sum(axis=2)
