"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no GEMM or copy arithmetic: it draws random numbers, rounds
them to the storage formats (round-to-nearest-even, the same bits for the GPU
and the oracle), and picks the seeded sample of output coordinates that the
large GEMM checks compare.  Neither the HIP library nor the oracle is imported.

Workloads (seeds are part of the recipe):

  atom     A f16 [16,16] U[-1,1] (11), B f16 [16,8] U[-1,1] (12), C f32 [16,8] U[-1,1] (13)
  copy32   f32 [32,32] U[-1,1] (21), one 64-lane wavefront, row-major LDS
  copy128  f16 [128,64] U[-1,1] (22), 256 threads, XOR-swizzled LDS
  gemm512  A bf16 [512,256] N(0,1) (31), B stored [N,K]=[512,256] N(0,1) (32),
           C f32 [512,512] N(0,1) (33), beta=1, transB
  stream   f16 16384x16384 U[-1,1] (41), 128x64 tiles, 256 threads, XOR LDS
  gemm8k   A, B bf16 [8192,8192] N(0,1)/sqrt(K) (51, 52), beta=0, sample seed 53
  gemm8kh  A stored [K,M] f16 N(0,1)/sqrt(K) (54), B f16 [K,N] (55), C f32 U[-1,1] (56),
           transA, beta=1, sample seed 57
  gemm8kf8 A e4m3 [8192,8192] N(0,1) (61), B e4m3 stored [N,K] N(0,1) (62), transB,
           beta=0, sample seed 63
  gemm8kf4 A e2m1 [8192,8192] N(0,1) (65), B e2m1 stored [N,K] N(0,1) (66), packed rows,
           E8M0 scales 2^-10..2^10 (67), beta=0 (the e2m3 pair: seeds 68-70; A e2m1 with
           B e2m3: 71-73)

6- and 4-bit operands (e2m3, e3m2, e2m1) are stored K-contiguous as packed rows: code k of a
row at bits [w·k, w·k + w) of the row's little-endian bit stream (w = 6 or 4).
"""

import numpy as np

ELEM_BYTES = {"f16": 2, "bf16": 2, "f32": 4, "u8": 1, "i8": 1, "fp8e4m3": 1, "fp8e5m2": 1}


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def uniform(seed, n, lo=-1.0, hi=1.0):
    """n float32 values, uniform on [lo, hi)."""
    return (rng(seed).random(n, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)


def normal(seed, n, scale=1.0):
    """n float32 values, normal(0, scale)."""
    return (rng(seed).standard_normal(n, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def f16_bits(x):
    """float32 array -> IEEE binary16 bit patterns (round to nearest even)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits(x):
    """float32 array -> bfloat16 bit patterns (round to nearest even; inputs are finite)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


_FP8_FIELDS = {"e4m3": (3, 7, 448.0), "e5m2": (2, 15, 57344.0)}   # fraction bits, bias, max


def fp8_bits(x, fmt):
    """float32 array -> OCP fp8 bit patterns ('e4m3' or 'e5m2'), round to nearest even.

    Inputs must be finite and round to at most the format's largest finite value."""
    mbits, bias, top = _FP8_FIELDS[fmt]
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                                   # a = f·2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, 1 - bias)                      # unbiased exponent, subnormals clamped
    quantum = np.ldexp(1.0, e - mbits)
    r = np.rint(a / quantum) * quantum                    # exact scaling; rint is half-even
    if np.any(r > top):
        raise ValueError(f"synth: value beyond the {fmt} range")
    _, ex2 = np.frexp(r)
    normal = r >= np.ldexp(1.0, 1 - bias)
    e2 = np.where(normal, ex2 - 1, 1 - bias)
    frac = np.where(normal, r / np.ldexp(1.0, e2) - 1.0, r / np.ldexp(1.0, 1 - bias))
    field_e = np.where(normal, e2 + bias, 0).astype(np.int64)
    field_m = np.rint(frac * (1 << mbits)).astype(np.int64)
    sign = np.signbit(x).astype(np.int64)
    return ((sign << 7) | (field_e << mbits) | field_m).astype(np.uint8)


def bits16(x, fmt):
    return f16_bits(x) if fmt == "f16" else bf16_bits(x)


def random_bits(seed, n, elem_bytes):
    """n arbitrary bit patterns of the given width (NaN payloads, -0 and subnormals included)."""
    dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[elem_bytes]
    return rng(seed).integers(0, np.iinfo(dt).max, size=n, dtype=dt, endpoint=True)


def sample_points(M, N, seed, count=4096, tile=(256, 256)):
    """Seeded output coordinates for large-GEMM checks.

    `count` distinct (i, j) drawn without replacement, plus the four corners and
    points on the tile boundaries (first/last row and column of tiles).
    """
    g = rng(seed)
    flat = g.choice(M * N, size=min(count, M * N), replace=False)
    rows, cols = list(flat // N), list(flat % N)
    extra = [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]
    tm, tn = tile
    for k in range(16):
        i = int(g.integers(0, M))
        j = int(g.integers(0, N))
        bi = min(M - 1, (i // tm) * tm + (k % 2) * (tm - 1))
        bj = min(N - 1, (j // tn) * tn + ((k // 2) % 2) * (tn - 1))
        extra += [(bi, j), (i, bj), (bi, bj)]
    for i, j in extra:
        rows.append(i)
        cols.append(j)
    return np.asarray(rows, dtype=np.int64), np.asarray(cols, dtype=np.int64)


# ---- workload recipes -------------------------------------------------------

def gemm_inputs(M, N, K, fmt, trans_a, trans_b, beta, seeds, a_scale=1.0, b_scale=1.0,
                dist="normal", c_dist="normal"):
    """Bits of A (stored orientation), B (stored orientation) and C (float32 or None)."""
    sa, sb, sc = seeds
    draw = normal if dist == "normal" else uniform
    if dist == "normal":
        a = draw(sa, M * K, a_scale)
        b = draw(sb, K * N, b_scale)
    else:
        a = draw(sa, M * K) * np.float32(a_scale)
        b = draw(sb, K * N) * np.float32(b_scale)
    c = None
    if beta == 1.0:
        c = normal(sc, M * N) if c_dist == "normal" else uniform(sc, M * N)
        c = c.reshape(M, N)
    a_bits = bits16(a, fmt).reshape((K, M) if trans_a else (M, K))
    b_bits = bits16(b, fmt).reshape((N, K) if trans_b else (K, N))
    return a_bits, b_bits, c


def atom_inputs(beta):
    return gemm_inputs(16, 8, 16, "f16", False, False, beta, (11, 12, 13), dist="uniform", c_dist="uniform")


def gemm512_inputs():
    return gemm_inputs(512, 512, 256, "bf16", False, True, 1.0, (31, 32, 33))


def gemm8k_bf16_inputs(K=8192):
    s = float(1.0 / np.sqrt(K))
    return gemm_inputs(K, K, K, "bf16", False, False, 0.0, (51, 52, 0), a_scale=s, b_scale=s)


def gemm8k_f16_inputs(K=8192):
    s = float(1.0 / np.sqrt(K))
    return gemm_inputs(K, K, K, "f16", True, False, 1.0, (54, 55, 56), a_scale=s, b_scale=s,
                       c_dist="uniform")


def gemm_fp8_inputs(M, N, K, a_fmt, b_fmt, trans_a, trans_b, beta, seeds, scale=1.0):
    """fp8 bits of A and B (stored orientations), N(0, scale) before rounding, and C
    (float32 U[-1, 1]) or None."""
    sa, sb, sc = seeds
    a = fp8_bits(normal(sa, M * K, scale), a_fmt).reshape((K, M) if trans_a else (M, K))
    b = fp8_bits(normal(sb, K * N, scale), b_fmt).reshape((N, K) if trans_b else (K, N))
    c = uniform(sc, M * N).reshape(M, N) if beta == 1.0 else None
    return a, b, c


def gemm8k_fp8_inputs(K=8192):
    """A e4m3 [M, K] N(0,1) (61), B e4m3 stored [N, K] N(0,1) (62), beta = 0."""
    return gemm_fp8_inputs(K, K, K, "e4m3", "e4m3", False, True, 0.0, (61, 62, 0))


def copy32_input():
    return uniform(21, 32 * 32).view(np.uint32)


def copy128_input():
    return f16_bits(uniform(22, 128 * 64))


def stream_input(rows=16384, cols=16384, seed=41):
    """f16 U[-1,1] bits, generated in row blocks to bound host memory."""
    out = np.empty(rows * cols, dtype=np.uint16)
    g = rng(seed)
    step = 1 << 24
    for s in range(0, out.size, step):
        n = min(step, out.size - s)
        out[s:s + n] = f16_bits(g.random(n, dtype=np.float32) * np.float32(2.0) - np.float32(1.0))
    return out


# ---- 6- and 4-bit operands ------------------------------------------------------------------
# (exponent bits, fraction bits, exponent bias) of the OCP microscaling element types
SMALL_FMT = {"e2m3": (2, 3, 1), "e3m2": (3, 2, 3), "e2m1": (2, 1, 1)}
SMALL_W = {"e2m3": 6, "e3m2": 6, "e2m1": 4}


def small_codes(x, fmt):
    """float array -> codes of a 6- or 4-bit format: round to nearest, ties to the even
    fraction, saturating at the largest finite magnitude (the formats have no infinities)."""
    eb, fb, bias = SMALL_FMT[fmt]
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.int64)
    a = np.abs(x)
    e_max = (1 << eb) - 1 - bias
    top = (2.0 - 2.0 ** -fb) * 2.0 ** e_max
    e_min = 1 - bias
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    e = np.maximum(e, e_min)
    q = np.rint(a / np.ldexp(1.0, e - fb)).astype(np.int64)       # significand in units of 2^(e-fb)
    carry = q >= (2 << fb)
    e = np.where(carry, e + 1, e)
    q = np.where(carry, q >> 1, q)
    normal = q >= (1 << fb)
    field = np.where(normal, e + bias, 0)
    frac = np.where(normal, q - (1 << fb), q)
    code = (field << fb) | frac
    code = np.where(a >= top, (((1 << eb) - 1) << fb) | ((1 << fb) - 1), code)
    return ((sign << (eb + fb)) | code).astype(np.uint8)


def pack_rows(codes, width):
    """codes [rows, K] (one code per element) -> packed rows [rows, K·width/8] (uint8)."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    bits = (codes[:, :, None] >> np.arange(width, dtype=np.uint8)) & 1
    return np.packbits(bits.reshape(rows, K * width), axis=1, bitorder="little")


def packed_random(nbytes, seed):
    """nbytes uniformly random bytes: packed 6- or 4-bit rows in which every code is equally
    likely (no code of these formats is a NaN or an infinity)."""
    return rng(seed).integers(0, 256, size=nbytes, dtype=np.uint8)


def gemm_mx_small_inputs(M, N, K, a_fmt, b_fmt, beta, seeds, dist="codes", scale_range=(117, 138)):
    """Packed A [M, K·wa/8], packed B [N, K·wb/8] (both K-contiguous), their codes, E8M0
    scales SA [M, K/32], SB [N, K/32] and C (float32 U[-1, 1]) or None.

    dist "codes": every code equally likely; "normal": N(0, 1) rounded to the format."""
    sa_, sb_, sc_ = seeds
    ga, gb = rng(sa_), rng(sb_)
    if dist == "codes":
        ca = ga.integers(0, 1 << SMALL_W[a_fmt], size=(M, K)).astype(np.uint8)
        cb = gb.integers(0, 1 << SMALL_W[b_fmt], size=(N, K)).astype(np.uint8)
    else:
        ca = small_codes(ga.standard_normal((M, K), dtype=np.float32), a_fmt)
        cb = small_codes(gb.standard_normal((N, K), dtype=np.float32), b_fmt)
    gs = rng(sc_)
    sa = gs.integers(scale_range[0], scale_range[1], size=(M, K // 32)).astype(np.uint8)
    sb = gs.integers(scale_range[0], scale_range[1], size=(N, K // 32)).astype(np.uint8)
    c = uniform(sc_ + 1000, M * N).reshape(M, N) if beta == 1.0 else None
    return pack_rows(ca, SMALL_W[a_fmt]), pack_rows(cb, SMALL_W[b_fmt]), ca, cb, sa, sb, c
