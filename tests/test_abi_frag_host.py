"""Host-only checks of the register fragment calls (no GPU): the plan's transfer width against
the oracle's register-path width rule, the route choice, and every rejection."""

import numpy as np
import pytest

import tile_level_gemm_amd as tg
from oracle import fragment as fr
from oracle.layout import Layout

KIND_CODE = {"a16_32x32x16": tg.TG_FRAG_A16_32x32x16, "b16_32x32x16": tg.TG_FRAG_B16_32x32x16,
             "a16_16x16x32": tg.TG_FRAG_A16_16x16x32, "b16_16x16x32": tg.TG_FRAG_B16_16x16x32,
             "a8_32x32x64": tg.TG_FRAG_A8_32x32x64, "b8_32x32x64": tg.TG_FRAG_B8_32x32x64,
             "c32_32x32": tg.TG_FRAG_C32_32x32, "c32_16x16": tg.TG_FRAG_C32_16x16,
             "a16_32x32x8": tg.TG_FRAG_A16_32x32x8, "b16_32x32x8": tg.TG_FRAG_B16_32x32x8,
             "a16_16x16x16": tg.TG_FRAG_A16_16x16x16, "b16_16x16x16": tg.TG_FRAG_B16_16x16x16}
DTYPE_OF_BITS = {8: tg.TG_FP8_E4M3, 16: tg.TG_BF16, 32: tg.TG_F32}
MEM, IMG = 1 << 32, 1 << 36          # far-apart addresses, only used for alignment


def plan(store, kind, rows, cols, lk, ld=0, mem=MEM, img=IMG, route=tg.TG_FRAG_AUTO, dtype=None):
    bits = fr.KINDS[kind][2]
    return tg.tile_frag_plan(store, mem, img, (rows, cols), dtype or DTYPE_OF_BITS[bits],
                             (tg.TG_ROW_MAJOR if lk == "row" else tg.TG_COL_MAJOR, ld),
                             KIND_CODE[kind], route)


def status(fn):
    try:
        fn()
    except tg.TileError as e:
        return e.status
    return tg.TG_OK


@pytest.mark.parametrize("kind", list(fr.KINDS))
def test_direct_width_matches_the_oracle_rule(kind):
    tr, tc, bits, e = fr.KINDS[kind]
    eb = bits // 8
    rng = np.random.default_rng(3)
    for _ in range(40):
        rows, cols = tr * int(rng.integers(1, 3)), tc * int(rng.integers(1, 3))
        lk = "row" if rng.integers(2) else "col"
        line = cols if lk == "row" else rows
        ld = line + int(rng.integers(0, 20)) * int(rng.integers(0, 2))
        off = eb * int(rng.integers(0, 16))
        p = plan(int(rng.integers(2)), kind, rows, cols, lk, ld, mem=MEM + off,
                 route=tg.TG_FRAG_DIRECT)
        want = fr.reg_vec(kind, rows, cols, Layout(lk, ld=ld), base_addr=MEM + off)
        assert (p.vec, p.vec_bits) == (want, want * bits), (rows, cols, lk, ld, off)
        assert p.route == tg.TG_FRAG_DIRECT
        assert (p.tile_rows, p.tile_cols, p.elems, p.elem_bits) == (tr, tc, e, bits)
        assert p.tiles == (rows // tr) * (cols // tc)
        runs_cross_lines = (lk == "row") == (kind.startswith("b") or kind.startswith("c"))
        assert p.transposed == int(runs_cross_lines)


@pytest.mark.parametrize("kind,lk,route", [
    # 16-byte aligned lines: the LDS route, along lines and across them
    ("a16_32x32x16", "row", tg.TG_FRAG_LDS), ("a16_32x32x16", "col", tg.TG_FRAG_LDS),
    ("b16_32x32x16", "row", tg.TG_FRAG_LDS), ("b16_32x32x16", "col", tg.TG_FRAG_LDS),
    ("a8_32x32x64", "col", tg.TG_FRAG_LDS), ("c32_32x32", "row", tg.TG_FRAG_LDS),
    ("c32_16x16", "col", tg.TG_FRAG_LDS),
])
def test_auto_route(kind, lk, route):
    tr, tc, _, _ = fr.KINDS[kind]
    # blocks of 64 lines: loads 256-byte lines, four blocks per workgroup along the lines;
    # stores 512-byte lines, one block per workgroup
    for store, line_bytes, nb in ((0, 256, 4), (1, 512, 1)):
        p = plan(store, kind, 2 * tr, 4 * tc, lk)
        assert p.route == route
        if route == tg.TG_FRAG_LDS:
            assert (p.vec_bits, p.lds_bytes, p.threads) == (128, 64 * line_bytes * nb, 256)
            lines, line_len = (2 * tr, 4 * tc) if lk == "row" else (4 * tc, 2 * tr)
            per_line = line_bytes // (fr.KINDS[kind][2] // 8)
            assert p.grid == -(-lines // 64) * -(-(-(-line_len // per_line)) // nb)


def test_auto_falls_back_to_direct_when_lines_are_not_16_byte_aligned():
    p = plan(0, "a16_32x32x16", 64, 32, "col", ld=68)      # 136-byte lines
    assert (p.route, p.vec) == (tg.TG_FRAG_DIRECT, 1)
    assert status(lambda: plan(0, "a16_32x32x16", 64, 32, "col", ld=68,
                               route=tg.TG_FRAG_LDS)) == tg.TG_E_ALIGN
    assert status(lambda: plan(0, "a16_32x32x16", 64, 32, "col", mem=MEM + 8,
                               route=tg.TG_FRAG_LDS)) == tg.TG_E_ALIGN


def test_direct_grid_covers_every_tile():
    # 4 waves per workgroup, 4 KiB of registers per wave
    for kind, per_wave in (("a16_32x32x16", 4), ("a8_32x32x64", 2), ("c32_32x32", 1),
                           ("c32_16x16", 4), ("a16_32x32x8", 8), ("b16_16x16x16", 8)):
        tr, tc, _, _ = fr.KINDS[kind]
        p = plan(1, kind, 3 * tr, 5 * tc, "row", route=tg.TG_FRAG_DIRECT)
        assert p.grid == -(-15 // (4 * per_wave))


@pytest.mark.parametrize("mutate,code", [
    (dict(kind=99), tg.TG_E_ARG),
    (dict(route=7), tg.TG_E_ARG),
    (dict(dtype=tg.TG_F32), tg.TG_E_DTYPE),          # 16-bit kind
    (dict(dtype=tg.TG_U8), tg.TG_E_DTYPE),
    (dict(dtype=42), tg.TG_E_DTYPE),
    (dict(shape=(48, 16)), tg.TG_E_SHAPE),            # 32-row tiles
    (dict(shape=(32, 8)), tg.TG_E_SHAPE),
    (dict(shape=(-32, 16)), tg.TG_E_SHAPE),
    (dict(shape=(1 << 31, 16)), tg.TG_E_SHAPE),
    (dict(layout=(tg.TG_XOR_SWIZZLE, 0)), tg.TG_E_LAYOUT),
    (dict(layout=(tg.TG_ROW_MAJOR, 8)), tg.TG_E_LAYOUT),   # ld below the line length
    (dict(layout=(tg.TG_ROW_MAJOR, -1)), tg.TG_E_LAYOUT),
    (dict(mem=None), tg.TG_E_NULL),
    (dict(img=None), tg.TG_E_NULL),
    (dict(mem=MEM + 1), tg.TG_E_ALIGN),                # not element aligned
    (dict(img=IMG + 8), tg.TG_E_ALIGN),                # image must be 16-byte aligned
    (dict(img=MEM + 64), tg.TG_E_ALIAS),
    (dict(store=2), tg.TG_E_ARG),
])
def test_rejections(mutate, code):
    args = dict(store=0, mem=MEM, img=IMG, shape=(64, 32), dtype=tg.TG_F16,
                layout=(tg.TG_ROW_MAJOR, 0), kind=tg.TG_FRAG_A16_32x32x16, route=tg.TG_FRAG_AUTO)
    args.update(mutate)
    st = status(lambda: tg.tile_frag_plan(args["store"], args["mem"], args["img"], args["shape"],
                                          args["dtype"], args["layout"], args["kind"], args["route"]))
    assert st == code
    assert tg.tile_last_error() if code else True


def test_rejected_copy_calls_launch_nothing():
    # The entry points validate first; these return before any HIP call.
    assert status(lambda: tg.tile_frag_load(MEM, IMG, (48, 16), tg.TG_F16, None,
                                            tg.TG_FRAG_A16_32x32x16)) == tg.TG_E_SHAPE
    assert status(lambda: tg.tile_frag_store(IMG, MEM, (32, 16), tg.TG_F32, None,
                                             tg.TG_FRAG_A16_32x32x16)) == tg.TG_E_DTYPE
    # an empty matrix is a no-op
    assert status(lambda: tg.tile_frag_load(None, None, (0, 16), tg.TG_F16, None,
                                            tg.TG_FRAG_A16_32x32x16)) == tg.TG_OK
    assert status(lambda: tg.tile_frag_store(None, None, (32, 0), tg.TG_F16, None,
                                             tg.TG_FRAG_A16_32x32x16)) == tg.TG_OK


@pytest.mark.parametrize("args,code", [
    ((32, 32, 16, 0.0, tg.TG_F16, tg.TG_F16, 9), tg.TG_E_ARG),
    ((16, 32, 16, 0.0, tg.TG_F16, tg.TG_F16, tg.TG_MMA_32x32x16), tg.TG_E_SHAPE),
    ((32, 32, 8, 0.0, tg.TG_F16, tg.TG_F16, tg.TG_MMA_32x32x16), tg.TG_E_SHAPE),
    ((16, 16, 16, 0.0, tg.TG_F16, tg.TG_F16, tg.TG_MMA_16x16x32), tg.TG_E_SHAPE),
    ((32, 32, 32, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3, tg.TG_MMA_32x32x64_F8), tg.TG_E_SHAPE),
    ((32, 32, 16, 0.0, tg.TG_F16, tg.TG_BF16, tg.TG_MMA_32x32x16), tg.TG_E_DTYPE),
    ((32, 32, 16, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3, tg.TG_MMA_32x32x16), tg.TG_E_DTYPE),
    ((32, 32, 64, 0.0, tg.TG_F16, tg.TG_F16, tg.TG_MMA_32x32x64_F8), tg.TG_E_DTYPE),
    ((32, 32, 64, 0.0, tg.TG_FP8_E4M3, tg.TG_U8, tg.TG_MMA_32x32x64_F8), tg.TG_E_DTYPE),
    ((32, 32, 16, 0.5, tg.TG_F16, tg.TG_F16, tg.TG_MMA_32x32x16), tg.TG_E_BETA),
    ((32, 32, 4, 0.0, tg.TG_F16, tg.TG_F16, tg.TG_MMA_32x32x8), tg.TG_E_SHAPE),
    ((16, 16, 8, 0.0, tg.TG_BF16, tg.TG_BF16, tg.TG_MMA_16x16x16), tg.TG_E_SHAPE),
    ((32, 32, 8, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3, tg.TG_MMA_32x32x8), tg.TG_E_DTYPE),
])
def test_mma_rejections_match_the_oracle(args, code):
    M, N, K, beta, ad, bd, shape = args
    st = status(lambda: tg.tile_frag_mma(IMG, IMG + (1 << 30), None, MEM, M, N, K, beta, ad, bd,
                                         shape))
    assert st == code
    names = {tg.TG_MMA_32x32x16: "32x32x16", tg.TG_MMA_16x16x32: "16x16x32",
             tg.TG_MMA_32x32x64_F8: "32x32x64_f8", tg.TG_MMA_32x32x8: "32x32x8",
             tg.TG_MMA_16x16x16: "16x16x16"}
    fmts = {tg.TG_F16: "f16", tg.TG_BF16: "bf16", tg.TG_FP8_E4M3: "e4m3", tg.TG_FP8_E5M2: "e5m2"}
    ok, why = fr.accepts_mma(M, N, K, names.get(shape, "?"), fmts.get(ad, "?"), fmts.get(bd, "?"),
                             beta)
    assert not ok
    assert {"shape": tg.TG_E_ARG, "extent": tg.TG_E_SHAPE, "dtype": tg.TG_E_DTYPE,
            "beta": tg.TG_E_BETA}[why] == code


SHAPE_NAME = {tg.TG_MMA_32x32x16: "32x32x16", tg.TG_MMA_16x16x32: "16x16x32",
              tg.TG_MMA_32x32x64_F8: "32x32x64_f8", tg.TG_MMA_32x32x8: "32x32x8",
              tg.TG_MMA_16x16x16: "16x16x16"}
FMT = {tg.TG_F16: "f16", tg.TG_BF16: "bf16", tg.TG_FP8_E4M3: "e4m3", tg.TG_FP8_E5M2: "e5m2"}


def test_mma_select_matches_the_oracle():
    for ad, bd in ((tg.TG_F16, tg.TG_F16), (tg.TG_BF16, tg.TG_BF16), (tg.TG_FP8_E4M3, tg.TG_FP8_E5M2)):
        for M in (0, 8, 16, 32, 48, 64, 96):
            for N in (0, 8, 16, 32, 48):
                for K in (0, 8, 16, 24, 32, 48, 64, 128, 192):
                    want = fr.select_mma(M, N, K, FMT[ad], FMT[bd])
                    try:
                        got = SHAPE_NAME[tg.tile_mma_select(M, N, K, ad, bd)]
                    except tg.TileError as e:
                        assert e.status == tg.TG_E_SHAPE
                        got = None
                    assert got == want, (M, N, K, ad, bd, got, want)


def test_mma_select_rejections():
    assert status(lambda: tg.tile_mma_select(32, 32, 16, tg.TG_F16, tg.TG_BF16)) == tg.TG_E_DTYPE
    assert status(lambda: tg.tile_mma_select(32, 32, 16, tg.TG_F32, tg.TG_F32)) == tg.TG_E_DTYPE
    assert status(lambda: tg.tile_mma_select(-32, 32, 16, tg.TG_F16, tg.TG_F16)) == tg.TG_E_ARG
    assert status(lambda: tg.tile_mma_select(16, 8, 16, tg.TG_F16, tg.TG_F16)) == tg.TG_E_SHAPE


def test_mma_pointer_checks():
    f16, s = tg.TG_F16, tg.TG_MMA_32x32x16
    assert status(lambda: tg.tile_frag_mma(IMG, IMG + (1 << 30), None, None, 32, 32, 16, 0.0,
                                           f16, f16, s)) == tg.TG_E_NULL
    assert status(lambda: tg.tile_frag_mma(IMG, IMG + (1 << 30), None, MEM, 32, 32, 16, 1.0,
                                           f16, f16, s)) == tg.TG_E_NULL
    assert status(lambda: tg.tile_frag_mma(IMG, IMG + (1 << 30), None, IMG + 512, 32, 32, 16, 0.0,
                                           f16, f16, s)) == tg.TG_E_ALIAS
    assert status(lambda: tg.tile_frag_mma(IMG, IMG + (1 << 30), MEM + 256, MEM, 32, 32, 16, 1.0,
                                           f16, f16, s)) == tg.TG_E_ALIAS
    assert status(lambda: tg.tile_frag_mma(IMG + 4, IMG + (1 << 30), None, MEM, 32, 32, 16, 0.0,
                                           f16, f16, s)) == tg.TG_E_ALIGN
    assert status(lambda: tg.tile_frag_mma(None, None, None, None, 0, 32, 16, 0.0, f16, f16,
                                           s)) == tg.TG_OK


def test_huge_leading_dimensions_are_rejected():
    # offsets must stay far inside 64 bits: ld above 2^40 elements is refused on every call
    big = (1 << 40) + 1
    assert status(lambda: plan(0, "a16_32x32x16", 64, 32, "row", ld=big)) == tg.TG_E_LAYOUT
    assert status(lambda: tg.tile_copy_plan(1 << 20, 1 << 30, (64, 64), tg.TG_F16,
                                            (tg.TG_ROW_MAJOR, big), None)) == tg.TG_E_LAYOUT
    assert status(lambda: tg.tile_copy_async_plan(1 << 20, 1 << 30, (64, 64), tg.TG_F16, None,
                                                  (tg.TG_ROW_MAJOR, big),
                                                  dict(tile_rows=64, tile_cols=64, threads=256,
                                                       depth=2))) == tg.TG_E_LAYOUT
