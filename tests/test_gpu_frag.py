"""GPU parity of the register fragment calls against the oracle: tile_frag_load / tile_frag_store
bit exact (guard bands intact, gaps of ld untouched), tile_frag_mma within the GEMM bars, and the
whole register pipeline (load A and B, product, store D) against the matrix product."""

import numpy as np
import pytest
import torch

import synth
import tile_level_gemm_amd as tg
from oracle import fragment as fr
from oracle.gemm import check, check_fp8
from oracle.layout import Layout
from tests.gpu_util import Guarded, say, upload_bits, upload_f32

pytestmark = pytest.mark.gpu

KIND_CODE = {"a16_32x32x16": tg.TG_FRAG_A16_32x32x16, "b16_32x32x16": tg.TG_FRAG_B16_32x32x16,
             "a16_16x16x32": tg.TG_FRAG_A16_16x16x32, "b16_16x16x32": tg.TG_FRAG_B16_16x16x32,
             "a8_32x32x64": tg.TG_FRAG_A8_32x32x64, "b8_32x32x64": tg.TG_FRAG_B8_32x32x64,
             "c32_32x32": tg.TG_FRAG_C32_32x32, "c32_16x16": tg.TG_FRAG_C32_16x16,
             "a16_32x32x8": tg.TG_FRAG_A16_32x32x8, "b16_32x32x8": tg.TG_FRAG_B16_32x32x8,
             "a16_16x16x16": tg.TG_FRAG_A16_16x16x16, "b16_16x16x16": tg.TG_FRAG_B16_16x16x16}
DTYPES = {8: (tg.TG_U8, tg.TG_FP8_E4M3), 16: (tg.TG_F16, tg.TG_BF16), 32: (tg.TG_F32,)}
UINT = {1: np.uint8, 2: np.uint16, 4: np.uint32}
LK = {"row": tg.TG_ROW_MAJOR, "col": tg.TG_COL_MAJOR}
ROUTES = {"direct": tg.TG_FRAG_DIRECT, "lds": tg.TG_FRAG_LDS, "auto": tg.TG_FRAG_AUTO}


def mem_elems(rows, cols, lk, ld):
    lines, line = (rows, cols) if lk == "row" else (cols, rows)
    ld = ld or line
    return (lines - 1) * ld + line


def run_load(kind, rows, cols, lk, route, ld=0, base=0, seed=1, dtype=None):
    _, _, bits, e = fr.KINDS[kind]
    eb = bits // 8
    dtype = dtype or DTYPES[bits][0]
    n = mem_elems(rows, cols, lk, ld) if rows and cols else 0
    src_bits = synth.random_bits(seed, base + n + 1, eb)
    src = upload_bits(src_bits)
    init = synth.random_bits(seed + 1000, rows * cols, eb)
    img = Guarded(rows * cols * eb, fill=init)
    say(f"frag_load {kind} {rows}x{cols} {lk} ld={ld} base={base} route={route}")
    tg.tile_frag_load(src.data_ptr() + base * eb, img.ptr, (rows, cols), dtype, (LK[lk], ld),
                      KIND_CODE[kind], ROUTES[route])
    torch.cuda.synchronize()
    got = img.host(UINT[eb])
    want = fr.frag_load(src_bits, rows, cols, Layout(lk, ld=ld, base=base), kind).reshape(-1) \
        if rows and cols else init
    return got, want, img.guards_intact()


def run_store(kind, rows, cols, lk, route, ld=0, base=0, seed=2, dtype=None):
    _, _, bits, e = fr.KINDS[kind]
    eb = bits // 8
    dtype = dtype or DTYPES[bits][0]
    n = base + mem_elems(rows, cols, lk, ld) + 3
    img_bits = synth.random_bits(seed, rows * cols, eb)
    init = synth.random_bits(seed + 1000, n, eb)
    dst = Guarded(n * eb, fill=init)
    img = upload_bits(img_bits)
    say(f"frag_store {kind} {rows}x{cols} {lk} ld={ld} base={base} route={route}")
    tg.tile_frag_store(img.data_ptr(), dst.ptr + base * eb, (rows, cols), dtype, (LK[lk], ld),
                       KIND_CODE[kind], ROUTES[route])
    torch.cuda.synchronize()
    want = fr.frag_store(img_bits.reshape(-1, 64, e), init, rows, cols,
                         Layout(lk, ld=ld, base=base), kind)
    return dst.host(UINT[eb]), want, dst.guards_intact()


@pytest.mark.parametrize("route", ["direct", "lds"])
@pytest.mark.parametrize("lk", ["row", "col"])
@pytest.mark.parametrize("kind", list(fr.KINDS))
def test_load_several_tiles_and_blocks(kind, lk, route):
    tr, tc, _, _ = fr.KINDS[kind]
    got, want, guards = run_load(kind, 5 * tr, 7 * tc, lk, route)
    assert guards and np.array_equal(got, want)


@pytest.mark.parametrize("route", ["direct", "lds"])
@pytest.mark.parametrize("lk", ["row", "col"])
@pytest.mark.parametrize("kind", list(fr.KINDS))
def test_store_several_tiles_and_blocks(kind, lk, route):
    tr, tc, _, _ = fr.KINDS[kind]
    got, want, guards = run_store(kind, 5 * tr, 7 * tc, lk, route)
    assert guards and np.array_equal(got, want)


# Narrower direct-route widths: padded lines and offset bases (vec in elements).
NARROW = [
    ("a16_32x32x16", "row", 4, 0, 4), ("a16_32x32x16", "row", 2, 0, 2),
    ("a16_32x32x16", "row", 0, 1, 1), ("a16_32x32x16", "row", 3, 0, 1),
    ("b16_16x16x32", "col", 4, 4, 4), ("a8_32x32x64", "row", 8, 0, 8),
    ("a8_32x32x64", "row", 4, 4, 4), ("b8_32x32x64", "col", 2, 2, 2), ("b8_32x32x64", "col", 1, 3, 1),
    ("c32_32x32", "col", 2, 0, 2), ("c32_16x16", "col", 1, 1, 1),
    ("a16_32x32x16", "col", 5, 1, 1), ("c32_32x32", "row", 1, 3, 1),
    ("a16_32x32x8", "row", 4, 0, 4), ("a16_32x32x8", "row", 2, 0, 2),
    ("b16_16x16x16", "col", 4, 4, 4), ("b16_32x32x8", "col", 1, 0, 1),
]


@pytest.mark.parametrize("kind,lk,pad,base,vec", NARROW)
@pytest.mark.parametrize("store", [False, True])
def test_direct_narrow_widths(kind, lk, pad, base, vec, store):
    tr, tc, bits, _ = fr.KINDS[kind]
    rows, cols = 3 * tr, 2 * tc
    ld = (cols if lk == "row" else rows) + pad
    eb = bits // 8
    # the plan must pick the width under test (checked on the same addresses the call uses)
    probe = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = tg.tile_frag_plan(int(store), probe.data_ptr() + base * eb, 1 << 40, (rows, cols),
                          DTYPES[bits][0], (LK[lk], ld), KIND_CODE[kind], tg.TG_FRAG_DIRECT)
    assert p.vec == vec
    fn = run_store if store else run_load
    got, want, guards = fn(kind, rows, cols, lk, "direct", ld=ld, base=base, seed=5)
    assert guards and np.array_equal(got, want)


@pytest.mark.parametrize("kind,lk", [("a16_32x32x16", "row"), ("a16_32x32x16", "col"),
                                     ("b8_32x32x64", "row"), ("c32_32x32", "row"),
                                     ("c32_16x16", "col"), ("b16_16x16x32", "col")])
@pytest.mark.parametrize("store", [False, True])
def test_lds_route_padded_lines_and_many_blocks(kind, lk, store):
    # 16-byte aligned padding and base; several 512-byte blocks along each line and a ragged
    # last block in both directions.
    tr, tc, bits, _ = fr.KINDS[kind]
    eb = bits // 8
    rows, cols = (3 * tr, 37 * tc) if lk == "row" else (37 * tr, 3 * tc)
    ld = (cols if lk == "row" else rows) + 32 // eb
    fn = run_store if store else run_load
    got, want, guards = fn(kind, rows, cols, lk, "lds", ld=ld, base=48 // eb, seed=7)
    assert guards and np.array_equal(got, want)


@pytest.mark.parametrize("kind", ["a8_32x32x64", "b16_32x32x16", "c32_16x16"])
@pytest.mark.parametrize("dtype_index", [0, 1])
def test_every_dtype_of_the_width(kind, dtype_index):
    _, _, bits, _ = fr.KINDS[kind]
    if dtype_index >= len(DTYPES[bits]):
        pytest.skip("one dtype of this width")
    tr, tc, _, _ = fr.KINDS[kind]
    got, want, guards = run_load(kind, 2 * tr, 2 * tc, "row", "auto",
                                 dtype=DTYPES[bits][dtype_index])
    assert guards and np.array_equal(got, want)


def test_every_16_bit_pattern_survives_both_directions():
    # 65536 patterns (NaN payloads, -0, subnormals) through a transposing load and store.
    bits = np.arange(65536, dtype=np.uint16)
    src = upload_bits(bits)
    img = torch.empty(65536, dtype=torch.int16, device="cuda")
    back = torch.empty(65536, dtype=torch.int16, device="cuda")
    say("frag all 16-bit patterns, a16 col-major, lds route")
    tg.tile_frag_load(src, img, (256, 256), tg.TG_BF16, (tg.TG_COL_MAJOR, 0),
                      tg.TG_FRAG_A16_32x32x16, tg.TG_FRAG_LDS)
    tg.tile_frag_store(img, back, (256, 256), tg.TG_BF16, (tg.TG_COL_MAJOR, 0),
                       tg.TG_FRAG_A16_32x32x16, tg.TG_FRAG_DIRECT)
    torch.cuda.synchronize()
    want = fr.frag_load(bits, 256, 256, Layout("col"), "a16_32x32x16").reshape(-1)
    assert np.array_equal(img.cpu().numpy().view(np.uint16), want)
    assert np.array_equal(back.cpu().numpy().view(np.uint16), bits)


@pytest.mark.parametrize("kind", list(fr.KINDS))
@pytest.mark.parametrize("lk", ["row", "col"])
def test_auto_round_trip(kind, lk):
    tr, tc, bits, _ = fr.KINDS[kind]
    eb = bits // 8
    rows, cols = 4 * tr, 3 * tc
    src_bits = synth.random_bits(9, rows * cols, eb)
    src = upload_bits(src_bits)
    img = torch.empty(rows * cols * eb, dtype=torch.uint8, device="cuda")
    back = Guarded(rows * cols * eb, fill=np.zeros(rows * cols, UINT[eb]))
    say(f"frag round trip {kind} {lk}")
    tg.tile_frag_load(src, img, (rows, cols), DTYPES[bits][0], (LK[lk], 0), KIND_CODE[kind])
    tg.tile_frag_store(img, back.ptr, (rows, cols), DTYPES[bits][0], (LK[lk], 0), KIND_CODE[kind])
    torch.cuda.synchronize()
    assert back.guards_intact() and np.array_equal(back.host(UINT[eb]), src_bits)


def test_empty_shapes_are_no_ops():
    say("frag empty shapes")
    tg.tile_frag_load(None, None, (0, 32), tg.TG_F16, None, tg.TG_FRAG_A16_16x16x32)
    tg.tile_frag_store(None, None, (16, 0), tg.TG_F16, None, tg.TG_FRAG_A16_16x16x32)
    tg.tile_frag_mma(None, None, None, None, 0, 32, 16, 0.0, tg.TG_F16, tg.TG_F16,
                     tg.TG_MMA_32x32x16)
    torch.cuda.synchronize()


# ---- the register-level product --------------------------------------------------------------

SHAPE_CODE = {"32x32x16": tg.TG_MMA_32x32x16, "16x16x32": tg.TG_MMA_16x16x32,
              "32x32x64_f8": tg.TG_MMA_32x32x64_F8, "32x32x8": tg.TG_MMA_32x32x8,
              "16x16x16": tg.TG_MMA_16x16x16}
FMT_CODE = {"f16": tg.TG_F16, "bf16": tg.TG_BF16, "e4m3": tg.TG_FP8_E4M3, "e5m2": tg.TG_FP8_E5M2}


def operands(shape, M, N, K, af, bf, beta, seed):
    """Row-major bits of A [M, K], B [K, N] and float32 C [M, N] (or None)."""
    if shape.endswith("_f8"):
        a, b, c = synth.gemm_fp8_inputs(M, N, K, af, bf, False, False, beta,
                                        (seed, seed + 1, seed + 2))
    else:
        a, b, c = synth.gemm_inputs(M, N, K, af, False, False, beta, (seed, seed + 1, seed + 2))
    return a, b, c


def check_d(shape, d, ref, bound, a, b, M, N, K, af, bf):
    if shape.endswith("_f8"):
        return check_fp8(d, ref, bound, a, b, M, N, K, 0, 0, af, bf)
    return check(d, ref, bound)


MMA_CASES = [("32x32x16", "f16", "f16"), ("32x32x16", "bf16", "bf16"),
             ("16x16x32", "f16", "f16"), ("16x16x32", "bf16", "bf16"),
             ("32x32x64_f8", "e4m3", "e4m3"), ("32x32x64_f8", "e4m3", "e5m2"),
             ("32x32x64_f8", "e5m2", "e4m3"), ("32x32x64_f8", "e5m2", "e5m2"),
             ("32x32x8", "f16", "f16"), ("32x32x8", "bf16", "bf16"),
             ("16x16x16", "f16", "f16"), ("16x16x16", "bf16", "bf16")]


@pytest.mark.parametrize("shape,af,bf", MMA_CASES)
@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_frag_mma_against_the_oracle(shape, af, bf, beta):
    ka, kb, kc, (am, an, ak) = fr.SHAPES[shape]
    M, N, K = 3 * am, 5 * an, 4 * ak
    a, b, c = operands(shape, M, N, K, af, bf, beta, 300)
    row = Layout("row")
    a_img = fr.frag_load(a.reshape(-1), M, K, row, ka)
    b_img = fr.frag_load(b.reshape(-1), K, N, row, kb)
    c_img = fr.frag_load(c.reshape(-1), M, N, row, kc) if beta else None
    d_ref, bound = fr.frag_mma_ref(a_img, b_img, c_img, M, N, K, shape, beta, af, bf)
    d = Guarded(M * N * 4)
    say(f"frag_mma {shape} {af}x{bf} beta={beta} {M}x{N}x{K}")
    tg.tile_frag_mma(upload_bits(a_img.reshape(-1)), upload_bits(b_img.reshape(-1)),
                     upload_f32(c_img.reshape(-1)) if beta else None, d.ptr, M, N, K, beta,
                     FMT_CODE[af], FMT_CODE[bf], SHAPE_CODE[shape])
    torch.cuda.synchronize()
    got = fr.unpack(d.host(np.float32).reshape(-1, 64, fr.KINDS[kc][3]), M, N, kc, np.float32)
    ref = fr.unpack(d_ref, M, N, kc, np.float64)
    bnd = fr.unpack(bound, M, N, kc, np.float64)
    ok, worst = check_d(shape, got, ref, bnd, a, b, M, N, K, af, bf)
    assert d.guards_intact() and ok, worst


@pytest.mark.parametrize("shape,af,bf", [MMA_CASES[0], MMA_CASES[3], MMA_CASES[5]])
def test_frag_mma_in_place_and_k0(shape, af, bf):
    ka, kb, kc, (am, an, ak) = fr.SHAPES[shape]
    M, N, K = 2 * am, 2 * an, 2 * ak
    a, b, c = operands(shape, M, N, K, af, bf, 1.0, 400)
    row = Layout("row")
    a_img = fr.frag_load(a.reshape(-1), M, K, row, ka)
    b_img = fr.frag_load(b.reshape(-1), K, N, row, kb)
    c_img = fr.frag_load(c.reshape(-1), M, N, row, kc)
    cd = upload_f32(c_img.reshape(-1))
    say(f"frag_mma in place {shape}")
    tg.tile_frag_mma(upload_bits(a_img.reshape(-1)), upload_bits(b_img.reshape(-1)), cd, cd, M, N,
                     K, 1.0, FMT_CODE[af], FMT_CODE[bf], SHAPE_CODE[shape])
    torch.cuda.synchronize()
    d_ref, bound = fr.frag_mma_ref(a_img, b_img, c_img, M, N, K, shape, 1.0, af, bf)
    got = fr.unpack(cd.cpu().numpy().reshape(-1, 64, fr.KINDS[kc][3]), M, N, kc, np.float32)
    ok, worst = check_d(shape, got, fr.unpack(d_ref, M, N, kc, np.float64),
                        fr.unpack(bound, M, N, kc, np.float64), a, b, M, N, K, af, bf)
    assert ok, worst
    # K == 0: D = beta·C exactly, C not read when beta == 0 (NaN C)
    d = Guarded(M * N * 4)
    say(f"frag_mma K=0 {shape}")
    tg.tile_frag_mma(None, None, upload_f32(c_img.reshape(-1)), d.ptr, M, N, 0, 1.0,
                     FMT_CODE[af], FMT_CODE[bf], SHAPE_CODE[shape])
    torch.cuda.synchronize()
    assert np.array_equal(d.host(np.float32), c_img.reshape(-1).astype(np.float32))
    nan_c = upload_f32(np.full(M * N, np.nan, np.float32))
    tg.tile_frag_mma(None, None, nan_c, d.ptr, M, N, 0, 0.0, FMT_CODE[af], FMT_CODE[bf],
                     SHAPE_CODE[shape])
    torch.cuda.synchronize()
    assert (d.host(np.float32) == 0).all() and d.guards_intact()


@pytest.mark.parametrize("shape,af,bf", [MMA_CASES[1], MMA_CASES[2], MMA_CASES[4],
                                         MMA_CASES[7], MMA_CASES[8], MMA_CASES[11]])
@pytest.mark.parametrize("a_lk,b_lk", [("row", "row"), ("col", "col"), ("col", "row")])
def test_register_pipeline_equals_the_matrix_product(shape, af, bf, a_lk, b_lk):
    """Load A and B into registers from memory in either orientation, multiply, store D: the
    fragment maps must match what the matrix unit computes."""
    ka, kb, kc, (am, an, ak) = fr.SHAPES[shape]
    M, N, K = 2 * am, 3 * an, 3 * ak
    a, b, c = operands(shape, M, N, K, af, bf, 1.0, 500)
    # memory copies of A and B in the requested orientation
    a_mem = a if a_lk == "row" else np.ascontiguousarray(a.T)
    b_mem = b if b_lk == "row" else np.ascontiguousarray(b.T)
    eb = a.dtype.itemsize
    a_img = torch.empty(M * K * eb, dtype=torch.uint8, device="cuda")
    b_img = torch.empty(K * N * eb, dtype=torch.uint8, device="cuda")
    c_img = torch.empty(M * N, dtype=torch.float32, device="cuda")
    d_out = Guarded(M * N * 4)
    say(f"frag pipeline {shape} {af}x{bf} A {a_lk} B {b_lk}")
    tg.tile_frag_load(upload_bits(a_mem.reshape(-1)), a_img, (M, K), FMT_CODE[af], (LK[a_lk], 0),
                      KIND_CODE[ka])
    tg.tile_frag_load(upload_bits(b_mem.reshape(-1)), b_img, (K, N), FMT_CODE[bf], (LK[b_lk], 0),
                      KIND_CODE[kb])
    tg.tile_frag_load(upload_f32(c.reshape(-1)), c_img, (M, N), tg.TG_F32, (tg.TG_ROW_MAJOR, 0),
                      KIND_CODE[kc])
    tg.tile_frag_mma(a_img, b_img, c_img, c_img, M, N, K, 1.0, FMT_CODE[af], FMT_CODE[bf],
                     SHAPE_CODE[shape])
    tg.tile_frag_store(c_img, d_out.ptr, (M, N), tg.TG_F32, (tg.TG_ROW_MAJOR, 0), KIND_CODE[kc])
    torch.cuda.synchronize()
    from oracle.gemm import logical_operands
    al, bl = logical_operands(a, b, M, N, K, 0, 0, af, bf)
    ref = al @ bl + c.astype(np.float64)
    bound = np.abs(al) @ np.abs(bl)
    got = d_out.host(np.float32).reshape(M, N)
    ok, worst = check_d(shape, got, ref, bound, a, b, M, N, K, af, bf)
    assert d_out.guards_intact() and ok, worst


@pytest.mark.parametrize("M,N,K,fmt", [(64, 96, 64, "bf16"), (48, 32, 96, "f16"), (32, 64, 40, "f16"),
                                       (16, 48, 48, "bf16"), (64, 64, 256, "e4m3")])
def test_selected_atom_runs_the_product(M, N, K, fmt):
    """The widest atom tile_mma_select names, through the whole register pipeline."""
    code = {"f16": tg.TG_F16, "bf16": tg.TG_BF16, "e4m3": tg.TG_FP8_E4M3}[fmt]
    shape_code = tg.tile_mma_select(M, N, K, code, code)
    shape = {v: k for k, v in SHAPE_CODE.items()}[shape_code]
    assert shape == fr.select_mma(M, N, K, fmt, fmt)
    ka, kb, kc, _ = fr.SHAPES[shape]
    a, b, c = operands(shape, M, N, K, fmt, fmt, 0.0, 600)
    eb = a.dtype.itemsize
    a_img = torch.empty(M * K * eb, dtype=torch.uint8, device="cuda")
    b_img = torch.empty(K * N * eb, dtype=torch.uint8, device="cuda")
    d_img = torch.empty(M * N, dtype=torch.float32, device="cuda")
    d_out = Guarded(M * N * 4)
    say(f"frag selected {shape} {M}x{N}x{K} {fmt}")
    tg.tile_frag_load(upload_bits(a.reshape(-1)), a_img, (M, K), code, (tg.TG_ROW_MAJOR, 0),
                      KIND_CODE[ka])
    tg.tile_frag_load(upload_bits(b.reshape(-1)), b_img, (K, N), code, (tg.TG_ROW_MAJOR, 0),
                      KIND_CODE[kb])
    tg.tile_frag_mma(a_img, b_img, None, d_img, M, N, K, 0.0, code, code, shape_code)
    tg.tile_frag_store(d_img, d_out.ptr, (M, N), tg.TG_F32, (tg.TG_ROW_MAJOR, 0), KIND_CODE[kc])
    torch.cuda.synchronize()
    from oracle.gemm import logical_operands
    al, bl = logical_operands(a, b, M, N, K, 0, 0, fmt, fmt)
    ok, worst = check_d(shape, d_out.host(np.float32).reshape(M, N), al @ bl, np.abs(al) @ np.abs(bl),
                        a, b, M, N, K, fmt, fmt)
    assert d_out.guards_intact() and ok, worst


# ---- the measured workloads, at full size ------------------------------------------------------

def sampled_tiles(kind, rows, cols, seed, count=64):
    tr, tc, _, _ = fr.KINDS[kind]
    g = np.random.default_rng(seed)
    tiles_r, tiles_c = rows // tr, cols // tc
    picks = {(0, 0), (tiles_r - 1, tiles_c - 1), (0, tiles_c - 1), (tiles_r - 1, 0)}
    while len(picks) < count:
        picks.add((int(g.integers(tiles_r)), int(g.integers(tiles_c))))
    return sorted(picks)


def tile_ref(mem, kind, lk, ld, ti, tj):
    """Oracle image of one tile: the tile as a matrix of its own inside the same memory."""
    tr, tc, _, _ = fr.KINDS[kind]
    base = ti * tr * ld + tj * tc if lk == "row" else tj * tc * ld + ti * tr
    return fr.frag_load(mem, tr, tc, Layout(lk, ld=ld, base=base), kind)[0]


@pytest.mark.parametrize("lk,route", [("row", "auto"), ("col", "auto"), ("col", "direct")])
def test_full_size_a16_load(lk, route):
    rows = cols = 16384
    kind = "a16_32x32x16"
    src_bits = synth.stream_input(rows, cols)
    src = upload_bits(src_bits)
    img = torch.empty(rows * cols, dtype=torch.int16, device="cuda")
    say(f"frag_load full size a16 {lk} {route}")
    tg.tile_frag_load(src, img, (rows, cols), tg.TG_F16, (LK[lk], 0), KIND_CODE[kind], ROUTES[route])
    torch.cuda.synchronize()
    got = img.view(-1, 64, 8)
    tiles_c = cols // 16
    for ti, tj in sampled_tiles(kind, rows, cols, 77):
        t = ti * tiles_c + tj
        want = tile_ref(src_bits, kind, lk, cols if lk == "row" else rows, ti, tj)
        assert np.array_equal(got[t].cpu().numpy().view(np.uint16), want), (ti, tj)
    # every element arrives exactly once: the image is a permutation of the matrix
    assert torch.equal(torch.sort(img.view(-1))[0], torch.sort(src.view(-1))[0])


def test_full_size_c32_store_row_major():
    rows, cols = 8192, 16384
    kind = "c32_32x32"
    img_bits = synth.uniform(43, rows * cols).view(np.uint32)
    img = upload_bits(img_bits)
    dst = torch.empty(rows * cols, dtype=torch.int32, device="cuda")
    say("frag_store full size c32 row-major auto")
    tg.tile_frag_store(img, dst, (rows, cols), tg.TG_F32, (tg.TG_ROW_MAJOR, 0), KIND_CODE[kind])
    torch.cuda.synchronize()
    host = dst.cpu().numpy().view(np.uint32).reshape(rows, cols)
    r, c = fr.coords(kind)
    tiles_c = cols // 32
    imgv = img_bits.reshape(-1, 64, 16)
    for ti, tj in sampled_tiles(kind, rows, cols, 78):
        t = ti * tiles_c + tj
        assert np.array_equal(host[ti * 32 + r, tj * 32 + c], imgv[t]), (ti, tj)
    assert torch.equal(torch.sort(dst.view(-1))[0], torch.sort(img.view(-1))[0])
