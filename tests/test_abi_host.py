"""Host-only checks of libtilegemm.so (no GPU): exported symbols, planner and
validation decisions against the oracle, kernel choice.  Integer decisions must
match exactly."""

import itertools
import json
import os
import re

import numpy as np
import pytest

import tile_level_gemm_amd as tg
from oracle import gemm as ogemm
from oracle.layout import COL, ROW, XOR, Layout
from oracle.planner import Plan, Reject, plan_region, plan_tiles

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KIND = {ROW: tg.TG_ROW_MAJOR, COL: tg.TG_COL_MAJOR, XOR: tg.TG_XOR_SWIZZLE}
CATEGORY = {tg.TG_E_THREADS: "threads", tg.TG_E_LAYOUT: "layout", tg.TG_E_SHAPE: "shape",
            tg.TG_E_DTYPE: "dtype", tg.TG_E_BETA: "beta"}


def declared_functions():
    text = open(os.path.join(ROOT, "include", "tilegemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tile_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"tile_gemm", "tile_copy", "tile_copy_ex", "tile_copy_plan", "tile_gemm_plan",
            "tile_gemm_fp8", "tile_gemm_fp8_plan", "tile_gemm_mx", "tile_gemm_mx_plan",
            "tile_copy_partition", "tile_frag_load", "tile_frag_store", "tile_frag_plan",
            "tile_frag_mma", "tile_copy_async", "tile_copy_async_plan", "tile_mma_select",
            "tile_gemm_atom_select",
            "tile_last_error",
            "tile_abi_version"} <= set(names)
    lib = tg.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in tg._SIGS, n   # the binding marshals every declared entry point
    assert tg.tile_abi_version() == 7


# ------------------------------------------------------------- planner ----

def c_partition(rows, cols, eb, threads, drive, other):
    try:
        p = tg.tile_copy_partition(rows, cols, 8 * eb, threads, (KIND[drive.kind], drive.ld), drive.base,
                                   (KIND[other.kind], other.ld), other.base)
        return Plan(p.outer, p.threads, p.vec, p.vec_bits)
    except tg.TileError as e:
        return Reject(CATEGORY[e.status], e.reason)


def same(a, b):
    if isinstance(a, Reject) or isinstance(b, Reject):
        return isinstance(a, Reject) and isinstance(b, Reject) and a.category == b.category
    return a == b


def _partition_cases():
    rs = np.random.default_rng(77)
    shapes = [(8, 16), (16, 16), (4, 24), (32, 32), (16, 8), (6, 40), (1, 64), (8, 64), (3, 5),
              (128, 64), (64, 32), (2, 128), (12, 12)]
    for (rows, cols), eb, threads in itertools.product(shapes, (1, 2, 4, 8), (0, 1, 3, 4, 8, 32, 64, 256)):
        kind = rs.choice([ROW, ROW, COL])
        full = cols if kind == ROW else rows
        ld = int(full + rs.choice([0, 0, 1, 2, 4, 8, 16, 20]))
        base = int(rs.choice([0, 0, 1, 2, 4, 8, 16, 3, 6]))
        okind = rs.choice([ROW, ROW, XOR, COL])
        oful = cols if okind != COL else rows
        old = 0 if okind == XOR else int(oful + rs.choice([0, 0, 8]))
        obase = 0 if okind == XOR else int(rs.choice([0, 0, 4, 2]))
        yield rows, cols, eb, threads, Layout(kind, ld, base), Layout(okind, old, obase)


@pytest.mark.parametrize("case", list(_partition_cases()))
def test_partition_matches_oracle(case):
    rows, cols, eb, threads, drive, other = case
    want = plan_region(rows, cols, 8 * eb, threads, drive, other)
    got = c_partition(rows, cols, eb, threads, drive, other)
    assert same(got, want), (case, got, want)


def _golden(name):
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        return json.load(f)


def test_golden_fixtures_through_the_library():
    g = _golden("planner_worked_example.json")
    p = c_partition(g["rows"], g["cols"], g["elem_bits"] // 8, g["threads"],
                    Layout(ROW, 32, 0), Layout(ROW, 32, 0))
    assert p == Plan(8, 32, 4, 128)
    g = _golden("planner_dtype_rounds.json")
    for case in g["cases"]:
        p = c_partition(32, 32, case["elem_bits"] // 8, 32, Layout(ROW), Layout(ROW))
        assert (p.vec, p.outer) == (case["vec"], case["outer"])
    g = _golden("planner_rejections_and_narrowing.json")
    for case in g["reject"]:
        p = c_partition(case["rows"], case["cols"], case["elem_bits"] // 8, case["threads"],
                        Layout(ROW), Layout(ROW))
        assert isinstance(p, Reject) and p.category == case["category"]
    for case in g["narrow"]:
        s, d = case["src"], case["dst"]
        p = c_partition(case["rows"], case["cols"], case["elem_bits"] // 8, case["threads"],
                        Layout(s["kind"], s["ld"], s["base"]), Layout(d["kind"], d["ld"], d["base"]))
        assert (p.vec, p.outer) == (case["vec"], case["outer"])


def _tiled_cases():
    rs = np.random.default_rng(99)
    for _ in range(300):
        eb = int(rs.choice([1, 2, 4]))
        tr, tc = int(rs.choice([1, 2, 4, 8, 16])), int(rs.choice([2, 4, 8, 16, 32, 64]))
        nr, nc = int(rs.integers(1, 4)), int(rs.integers(1, 4))
        rows, cols = tr * nr, tc * nc
        threads = int(rs.choice([1, 2, 4, 8, 16, 32, 64]))
        skind = rs.choice([ROW, ROW, COL])
        dkind = rs.choice([ROW, COL])
        sld = (cols if skind == ROW else rows) + int(rs.choice([0, 0, 2, 4, 8, 3]))
        dld = (cols if dkind == ROW else rows) + int(rs.choice([0, 0, 8, 1]))
        soff, doff = int(rs.choice([0, 0, 1, 2, 8])), int(rs.choice([0, 0, 4]))
        lds = rs.choice([ROW, XOR])
        yield rows, cols, tr, tc, eb, threads, (skind, sld, soff), (dkind, dld, doff), lds


@pytest.mark.parametrize("case", list(_tiled_cases()))
def test_tiled_copy_plan_matches_oracle(case):
    rows, cols, tr, tc, eb, threads, s, d, lds = case
    base_addr = 1 << 20
    src_addr = base_addr + s[2] * eb
    dst_addr = (1 << 28) + d[2] * eb
    lds_side = Layout(lds, tc if lds == ROW else 0, 0)
    want_l = plan_tiles(rows, cols, tr, tc, 8 * eb, threads, Layout(s[0], s[1], src_addr // eb), lds_side)
    want_s = plan_tiles(rows, cols, tr, tc, 8 * eb, threads, Layout(d[0], d[1], dst_addr // eb), lds_side)
    dtype = {1: tg.TG_U8, 2: tg.TG_F16, 4: tg.TG_F32}[eb]
    opts = dict(tile_rows=tr, tile_cols=tc, threads=threads, lds_kind=KIND[lds])
    try:
        p = tg.tile_copy_plan(src_addr, dst_addr, (rows, cols), dtype, (KIND[s[0]], s[1]),
                              (KIND[d[0]], d[1]), opts)
        got_l = Plan(*[getattr(p.load, f) for f in ("outer", "threads", "vec", "vec_bits")])
        got_s = Plan(*[getattr(p.store, f) for f in ("outer", "threads", "vec", "vec_bits")])
        assert p.tiles == (rows // tr) * (cols // tc)
    except tg.TileError as e:
        got_l = got_s = Reject(CATEGORY.get(e.status, "other"), e.reason)
    assert same(got_l, want_l), (case, got_l, want_l)
    if not isinstance(got_l, Reject):
        assert same(got_s, want_s), (case, got_s, want_s)


def test_copy_plan_configs_and_rejections():
    # 32x32 f32 by one wavefront, row-major LDS
    p = tg.tile_copy_plan(1 << 20, 1 << 24, (32, 32), tg.TG_F32, None, None,
                          dict(tile_rows=32, tile_cols=32, threads=64, lds_kind=tg.TG_ROW_MAJOR))
    assert p.load.as_tuple() == (4, 64, 4, 128) and p.store.as_tuple() == (4, 64, 4, 128)
    # 128x64 f16, 256 threads, XOR LDS; defaults pick the same
    p = tg.tile_copy_plan(1 << 20, 1 << 24, (128, 64), tg.TG_F16)
    assert (p.tile_rows, p.tile_cols, p.lds_kind, p.tiles) == (128, 64, tg.TG_XOR_SWIZZLE, 1)
    assert p.load.as_tuple() == (4, 256, 8, 128)
    # the streaming copy: 16384^2 f16 in 128x64 tiles
    p = tg.tile_copy_plan(1 << 30, 1 << 31, (16384, 16384), tg.TG_F16)
    assert p.tiles == 32768 and p.load.as_tuple() == (4, 256, 8, 128) and p.lds_bytes == 16384
    # thread count must divide the tile: 64-element tile on 1024 threads
    with pytest.raises(tg.TileError) as e:
        tg.tile_copy_plan(1 << 20, 1 << 24, (1, 64), tg.TG_F16, None, None,
                          dict(tile_rows=1, tile_cols=64, threads=1024, lds_kind=tg.TG_ROW_MAJOR))
    assert e.value.status == tg.TG_E_THREADS
    # ragged tensor (not a whole number of tiles)
    with pytest.raises(tg.TileError) as e:
        tg.tile_copy_plan(1 << 20, 1 << 24, (100, 64), tg.TG_F16, None, None,
                          dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE))
    assert e.value.status == tg.TG_E_SHAPE
    # overlapping src/dst
    with pytest.raises(tg.TileError) as e:
        tg.tile_copy_plan(1 << 20, (1 << 20) + 64, (32, 32), tg.TG_F32)
    assert e.value.status == tg.TG_E_ALIAS
    # misaligned source narrows the load width, the store keeps 128 bits
    p = tg.tile_copy_plan((1 << 20) + 2, 1 << 24, (128, 64), tg.TG_F16)
    assert p.load.vec == 1 and p.store.vec == 8
    # empty tensor is a no-op plan
    p = tg.tile_copy_plan(None, None, (0, 64), tg.TG_F16)
    assert p.tiles == 0
    # bad dtype and layout
    for bad in (dict(dtype=99), dict(src=(7, 0))):
        with pytest.raises(tg.TileError):
            tg.tile_copy_plan(1 << 20, 1 << 24, (32, 32), bad.get("dtype", tg.TG_F32), bad.get("src"))


# ---------------------------------------------------------------- GEMM ----

A_ADDR, B_ADDR, C_ADDR, D_ADDR = 1 << 32, 1 << 33, 1 << 34, 1 << 35
ODT = {tg.TG_F16: "f16", tg.TG_BF16: "bf16"}


@pytest.mark.parametrize("M,N,K", [(16, 8, 16), (8, 8, 16), (16, 4, 16), (16, 8, 12), (32, 24, 40),
                                   (0, 8, 16), (16, 8, 0), (-16, 8, 8), (64, 64, 24), (512, 512, 256)])
@pytest.mark.parametrize("dtype", [tg.TG_F16, tg.TG_BF16, tg.TG_F32, tg.TG_I8])
@pytest.mark.parametrize("beta", [0.0, 1.0, 0.5, 2.0])
def test_gemm_validation_matches_oracle(M, N, K, dtype, beta):
    want_ok, want_cat = ogemm.accepts(M, N, K, ODT.get(dtype, "other"), ODT.get(dtype, "other"), beta=beta)
    try:
        tg.tile_gemm_plan(A_ADDR, B_ADDR, C_ADDR, D_ADDR, M, N, K, 0, 0, beta, dtype)
        got_ok, got_cat = True, None
    except tg.TileError as e:
        got_ok, got_cat = False, CATEGORY.get(e.status, "other")
    assert (got_ok, got_cat) == (want_ok, want_cat)


def test_gemm_rejections_need_no_gpu():
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm(A_ADDR, B_ADDR, C_ADDR, D_ADDR, 16, 8, 16, 0, 0, 0.5, tg.TG_F16)
    assert e.value.status == tg.TG_E_BETA
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm(A_ADDR, B_ADDR, None, D_ADDR, 16, 8, 16, 0, 0, 1.0, tg.TG_F16)
    assert e.value.status == tg.TG_E_NULL
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm(A_ADDR + 8, B_ADDR, None, D_ADDR, 16, 8, 16, 0, 0, 0.0, tg.TG_F16)
    assert e.value.status == tg.TG_E_ALIGN
    with pytest.raises(tg.TileError) as e:  # D overlaps A
        tg.tile_gemm(A_ADDR, B_ADDR, None, A_ADDR + 64, 16, 8, 16, 0, 0, 0.0, tg.TG_F16)
    assert e.value.status == tg.TG_E_ALIAS
    with pytest.raises(tg.TileError) as e:  # C partially overlaps D
        tg.tile_gemm(A_ADDR, B_ADDR, D_ADDR + 4, D_ADDR, 16, 8, 16, 0, 0, 1.0, tg.TG_F16)
    assert e.value.status == tg.TG_E_ALIAS
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm(A_ADDR, B_ADDR, None, D_ADDR, 16, 8, 16, 2, 0, 0.0, tg.TG_F16)
    assert e.value.status == tg.TG_E_ARG
    # C == D exactly is the allowed in-place form
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, D_ADDR, D_ADDR, 16, 8, 16, 0, 0, 1.0, tg.TG_F16)
    assert p.kernel == tg.TG_GEMM_ATOM


def test_binding_rejects_alpha():
    import torch
    a = torch.zeros(16, 16, dtype=torch.float16)
    with pytest.raises(tg.TileError):
        tg.gemm(a, a, alpha=2.0)


def test_gemm_kernel_choice():
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 16, 8, 16, 0, 0, 0.0, tg.TG_F16)
    assert (p.kernel, p.grid, p.threads) == (tg.TG_GEMM_ATOM, 1, 64)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, C_ADDR, D_ADDR, 512, 512, 256, 0, 1, 1.0, tg.TG_BF16)
    assert p.kernel == tg.TG_GEMM_TILED and p.grid >= 64 and not p.bounds_checked
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 8192, 8192, 8192, 0, 0, 0.0, tg.TG_BF16)
    assert (p.kernel, p.block_m, p.block_n, p.grid, p.bounds_checked) == (tg.TG_GEMM_TILED, 256, 256, 1024, 0)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 528, 520, 264, 1, 0, 0.0, tg.TG_F16)
    assert p.kernel == tg.TG_GEMM_TILED and p.bounds_checked
    # the direct-load kernel serves every shape with at least 256 blocks of 256x256, or else 128
    # of 128x128, ragged ones with range-checked operand loads and a masked epilogue; fewer
    # blocks take the VGPR-staged kernel on 64x64 tiles
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 8192, 8192, 8192, 0, 0, 0.0, tg.TG_BF16)
    assert (p.threads, p.bounds_checked, p.loader) == (512, 0, 1)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 8000, 8000, 8000, 0, 0, 0.0, tg.TG_BF16)
    assert (p.block_m, p.grid, p.threads, p.bounds_checked, p.loader) == (256, 1024, 512, 1, 1)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 16, 65544, 24, 0, 0, 0.0, tg.TG_F16)
    assert (p.block_m, p.grid, p.bounds_checked, p.loader) == (256, 257, 1, 1)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 2048, 2048, 2048, 0, 0, 0.0, tg.TG_F16)
    assert (p.block_m, p.grid, p.wave_m, p.wave_n, p.threads, p.loader) == (128, 256, 64, 32, 512, 1)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 1552, 2056, 200, 0, 0, 0.0, tg.TG_F16)
    assert (p.block_m, p.grid, p.bounds_checked, p.loader) == (128, 221, 1, 1)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 1024, 1024, 1024, 0, 0, 0.0, tg.TG_F16)
    assert (p.block_m, p.grid, p.loader) == (64, 256, 0)
    p = tg.tile_gemm_plan(None, None, None, D_ADDR, 16, 8, 0, 0, 0, 0.0, tg.TG_F16)
    assert p.kernel == tg.TG_GEMM_FILL
    # the direct kernel's 32-bit DMA offsets address whole 64-K stages of an M/N-major operand:
    # with M = 2^26 and K = 8 that operand is 1 GiB, but 64 k-rows of it are 8 GiB and the
    # offsets would wrap back into it, so it takes the 64-bit tiled kernel; whole stages of
    # exactly 2^32 bytes (M = 2^25) still do not wrap.  A K-major operand never addresses past
    # its own rows, so 2 GiB of it stays on the direct kernel whatever K is.
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 1 << 26, 8, 8, 1, 0, 0.0, tg.TG_BF16)
    assert (p.kernel, p.loader) == (tg.TG_GEMM_TILED, 0)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 16, 1 << 26, 8, 0, 0, 0.0, tg.TG_BF16)
    assert (p.kernel, p.loader) == (tg.TG_GEMM_TILED, 0)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, (1 << 25) + 16, 8, 8, 1, 0, 0.0, tg.TG_BF16)
    assert (p.kernel, p.loader) == (tg.TG_GEMM_TILED, 0)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 1 << 25, 8, 8, 1, 0, 0.0, tg.TG_BF16)
    assert (p.kernel, p.loader) == (tg.TG_GEMM_TILED, 1)
    p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, 1 << 26, 8, 8, 0, 0, 0.0, tg.TG_BF16)
    assert (p.kernel, p.loader) == (tg.TG_GEMM_TILED, 1)
    p = tg.tile_gemm_plan(None, None, None, None, 0, 8, 16, 0, 0, 0.0, tg.TG_F16)
    assert p.kernel == tg.TG_GEMM_NONE


# ------------------------------------------------------------ fp8 GEMM ----

ODT8 = {tg.TG_FP8_E4M3: "e4m3", tg.TG_FP8_E5M2: "e5m2", tg.TG_F16: "f16", tg.TG_BF16: "bf16"}


@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (8, 16, 128), (16, 8, 128), (16, 16, 64),
                                   (16, 16, 192), (0, 16, 128), (16, 16, 0), (-16, 16, 128),
                                   (272, 528, 384), (8192, 8192, 8192)])
@pytest.mark.parametrize("a_dt,b_dt", [(tg.TG_FP8_E4M3, tg.TG_FP8_E4M3), (tg.TG_FP8_E5M2, tg.TG_FP8_E4M3),
                                       (tg.TG_FP8_E4M3, tg.TG_F16), (tg.TG_BF16, tg.TG_FP8_E5M2),
                                       (tg.TG_I8, tg.TG_FP8_E4M3)])
@pytest.mark.parametrize("beta", [0.0, 1.0, 0.5])
def test_fp8_validation_matches_oracle(M, N, K, a_dt, b_dt, beta):
    want = ogemm.accepts_fp8(M, N, K, ODT8.get(a_dt, "other"), ODT8.get(b_dt, "other"), beta=beta)
    try:
        tg.tile_gemm_fp8_plan(A_ADDR, B_ADDR, C_ADDR, D_ADDR, M, N, K, 0, 1, beta, a_dt, b_dt)
        got = (True, None)
    except tg.TileError as e:
        got = (False, CATEGORY.get(e.status, "other"))
    assert got == want


def test_fp8_layouts_and_errors_need_no_gpu():
    e4 = tg.TG_FP8_E4M3
    # every stored orientation is served, with the same plan
    plans = set()
    for ta in (0, 1):
        for tb in (0, 1):
            p = tg.tile_gemm_fp8_plan(A_ADDR, B_ADDR, None, D_ADDR, 256, 512, 384, ta, tb, 0.0, e4, e4)
            plans.add((p.kernel, p.block_m, p.block_n, p.block_k, p.grid, p.bounds_checked, p.loader))
    assert plans == {(tg.TG_GEMM_TILED, 128, 128, 128, 8, 0, 1)}
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm_fp8(A_ADDR, B_ADDR, None, D_ADDR, 256, 256, 256, 0, 2, 0.0, e4, e4)
    assert e.value.status == tg.TG_E_ARG
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm_fp8(A_ADDR + 8, B_ADDR, None, D_ADDR, 256, 256, 256, 0, 1, 0.0, e4, e4)
    assert e.value.status == tg.TG_E_ALIGN
    with pytest.raises(tg.TileError) as e:   # D overlaps B (one-byte elements: N*K bytes)
        tg.tile_gemm_fp8(A_ADDR, B_ADDR, None, B_ADDR + 256 * 256 - 4, 256, 256, 256, 0, 1, 0.0, e4, e4)
    assert e.value.status == tg.TG_E_ALIAS
    # D just past the end of B (N*K bytes) does not overlap
    tg.tile_gemm_fp8_plan(A_ADDR, B_ADDR, None, B_ADDR + 256 * 256, 256, 256, 256, 0, 1, 0.0, e4, e4)
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm_fp8(A_ADDR, B_ADDR, None, D_ADDR, 256, 256, 256, 0, 1, 1.0, e4, e4)
    assert e.value.status == tg.TG_E_NULL
    with pytest.raises(tg.TileError) as e:   # an operand of 2 GiB
        tg.tile_gemm_fp8_plan(A_ADDR, B_ADDR, None, D_ADDR, 16384, 256, 131072, 0, 1, 0.0, e4, e4)
    assert e.value.status == tg.TG_E_SHAPE and "2 GiB" in e.value.reason


def test_fp8_kernel_choice():
    e4, e5 = tg.TG_FP8_E4M3, tg.TG_FP8_E5M2
    p = tg.tile_gemm_fp8_plan(A_ADDR, B_ADDR, None, D_ADDR, 8192, 8192, 8192, 0, 1, 0.0, e4, e4)
    assert (p.kernel, p.block_m, p.block_n, p.block_k, p.threads, p.grid, p.bounds_checked,
            p.loader) == (tg.TG_GEMM_TILED, 256, 256, 128, 512, 1024, 0, 1)
    # fewer than 256 blocks of 256x256: 128x128 blocks (3 x 5 of them here)
    p = tg.tile_gemm_fp8_plan(A_ADDR, B_ADDR, C_ADDR, D_ADDR, 272, 528, 384, 0, 1, 1.0, e5, e4)
    assert (p.kernel, p.block_m, p.grid, p.bounds_checked, p.loader) == (tg.TG_GEMM_TILED, 128, 15, 1, 1)
    p = tg.tile_gemm_fp8_plan(A_ADDR, B_ADDR, None, D_ADDR, 2048, 2048, 8192, 0, 1, 0.0, e4, e4)
    assert (p.block_m, p.wave_m, p.wave_n, p.threads, p.grid, p.bounds_checked, p.lds_bytes) == \
        (128, 64, 32, 512, 256, 0, 65536)
    p = tg.tile_gemm_fp8_plan(A_ADDR, B_ADDR, None, D_ADDR, 4096, 4096, 4096, 0, 1, 0.0, e4, e4)
    assert (p.block_m, p.grid) == (256, 256)
    # block-scaled fp8: the same block choice; its scale ring adds three groups of 2 x BS/16
    # blocks of 260 bytes
    p = tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, 1 << 36, 1 << 37, None, D_ADDR, 272, 528, 384, 0, 1, 0.0,
                             e5, e4)
    assert (p.block_m, p.grid, p.bounds_checked, p.lds_bytes) == (128, 15, 1, 4 * 128 * 128 + 3 * 2 * 260 * 8)
    p = tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, 1 << 36, 1 << 37, None, D_ADDR, 8192, 8192, 8192, 0, 1, 0.0,
                             e4, e4)
    assert (p.block_m, p.grid, p.bounds_checked, p.lds_bytes) == (256, 1024, 0, 4 * 256 * 128 + 3 * 2 * 260 * 16)
    p = tg.tile_gemm_fp8_plan(None, None, C_ADDR, D_ADDR, 16, 16, 0, 0, 1, 1.0, e4, e5)
    assert p.kernel == tg.TG_GEMM_FILL
    p = tg.tile_gemm_fp8_plan(None, None, None, None, 0, 16, 128, 0, 1, 0.0, e4, e4)
    assert p.kernel == tg.TG_GEMM_NONE


# ---------------------------------------------------- block-scaled fp8 ----

@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (8, 16, 128), (16, 16, 64), (0, 16, 128),
                                   (16, 16, 0), (272, 528, 384)])
@pytest.mark.parametrize("a_dt", [tg.TG_FP8_E4M3, tg.TG_FP8_E5M2, tg.TG_F16])
@pytest.mark.parametrize("beta", [0.0, 1.0, 2.0])
def test_mx_validation_matches_oracle(M, N, K, a_dt, beta):
    want = ogemm.accepts_fp8(M, N, K, ODT8.get(a_dt, "other"), "e4m3", beta=beta)
    SA_ADDR, SB_ADDR = 1 << 36, 1 << 37
    try:
        tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, SA_ADDR, SB_ADDR, C_ADDR, D_ADDR, M, N, K, 0, 1, beta,
                             a_dt, tg.TG_FP8_E4M3)
        got = (True, None)
    except tg.TileError as e:
        got = (False, CATEGORY.get(e.status, "other"))
    assert got == want


def test_mx_scale_arguments():
    e4 = tg.TG_FP8_E4M3
    SA_ADDR, SB_ADDR = 1 << 36, 1 << 37
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm_mx(A_ADDR, B_ADDR, None, SB_ADDR, None, D_ADDR, 256, 256, 256, 0, 1, 0.0, e4, e4)
    assert e.value.status == tg.TG_E_NULL
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm_mx(A_ADDR, B_ADDR, SA_ADDR + 2, SB_ADDR, None, D_ADDR, 256, 256, 256, 0, 1, 0.0,
                        e4, e4)
    assert e.value.status == tg.TG_E_ALIGN
    with pytest.raises(tg.TileError) as e:   # D overlaps SB ([N][K/32] bytes)
        tg.tile_gemm_mx(A_ADDR, B_ADDR, SA_ADDR, D_ADDR + 64, None, D_ADDR, 256, 256, 256, 0, 1, 0.0,
                        e4, e4)
    assert e.value.status == tg.TG_E_ALIAS
    # K == 0 reads no scales
    p = tg.tile_gemm_mx_plan(None, None, None, None, C_ADDR, D_ADDR, 32, 16, 0, 0, 1, 1.0, e4, e4)
    assert p.kernel == tg.TG_GEMM_FILL
    p = tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, SA_ADDR, SB_ADDR, None, D_ADDR, 8192, 8192, 8192, 1, 0,
                             0.0, e4, tg.TG_FP8_E5M2)
    assert (p.kernel, p.block_m, p.block_k, p.grid, p.loader) == (tg.TG_GEMM_TILED, 256, 128, 1024, 1)


# ------------------------------------------------- register GEMM atom choice ----

def _atom_name(code):
    return {tg.TG_MMA_32x32x16: "32x32x16", tg.TG_MMA_16x16x32: "16x16x32",
            tg.TG_MMA_32x32x8: "32x32x8", tg.TG_MMA_16x16x16: "16x16x16"}[code]


def test_gemm_atom_choice_matches_oracle():
    import itertools
    from oracle.fragment import select_gemm_atom
    for M, N, K, ta, tb, dt in itertools.product((16, 32, 48, 64, 96, 128, 256), (8, 16, 24, 32, 40, 64),
                                                 (8, 16, 24, 32, 40, 48, 64, 96, 200),
                                                 (0, 1), (0, 1), ("f16", "bf16")):
        code = tg.TG_F16 if dt == "f16" else tg.TG_BF16
        got = _atom_name(tg.tile_gemm_atom_select(M, N, K, code, ta, tb))
        assert got == select_gemm_atom(M, N, K, dt, bool(ta), bool(tb)), (M, N, K, ta, tb)
        if M * N <= 64 * 64:
            p = tg.tile_gemm_plan(A_ADDR, B_ADDR, None, D_ADDR, M, N, K, ta, tb, 0.0, code)
            assert p.kernel == tg.TG_GEMM_ATOM and _atom_name(p.atom) == got
            am = 32 if got.startswith("32") else 16
            assert (p.block_m, p.block_n, p.threads) == (am, am, 64)
            assert p.grid == -(-M // am) * -(-N // am)
            assert p.bounds_checked == int(M % am != 0 or N % am != 0)


def test_gemm_atom_select_rejections():
    for args, status in (((16, 8, 12, tg.TG_F16, 0, 0), tg.TG_E_SHAPE),
                         ((0, 8, 16, tg.TG_F16, 0, 0), tg.TG_E_SHAPE),
                         ((16, 8, 16, tg.TG_FP8_E4M3, 0, 0), tg.TG_E_DTYPE),
                         ((16, 8, 16, tg.TG_F16, 2, 0), tg.TG_E_ARG)):
        with pytest.raises(tg.TileError) as e:
            tg.tile_gemm_atom_select(*args)
        assert e.value.status == status
    # the page's atom and its K = 8 / 24 cases
    assert tg.tile_gemm_atom_select(16, 8, 16, tg.TG_F16, 0, 0) == tg.TG_MMA_16x16x16
    assert tg.tile_gemm_atom_select(16, 8, 8, tg.TG_F16, 0, 0) == tg.TG_MMA_32x32x8
    assert tg.tile_gemm_atom_select(32, 16, 24, tg.TG_BF16, 0, 1) == tg.TG_MMA_32x32x8


# ------------------------------------------ block-scaled 6- and 4-bit operands ----

def test_packed_mx_validation_matches_oracle():
    import itertools
    from oracle.gemm import accepts_mx
    name = {tg.TG_FP6_E2M3: "e2m3", tg.TG_FP6_E3M2: "e3m2", tg.TG_FP4_E2M1: "e2m1",
            tg.TG_FP8_E4M3: "e4m3", tg.TG_FP8_E5M2: "e5m2"}
    cat_of = {tg.TG_E_SHAPE: "shape", tg.TG_E_DTYPE: "dtype", tg.TG_E_LAYOUT: "layout",
              tg.TG_E_BETA: "beta"}
    for (M, N, K), af, bf, ta, tb, beta in itertools.product(
            [(32, 32, 128), (16, 48, 256), (40, 32, 128), (32, 32, 192), (0, 16, 128)],
            [tg.TG_FP6_E2M3, tg.TG_FP6_E3M2, tg.TG_FP4_E2M1, tg.TG_FP8_E4M3],
            [tg.TG_FP6_E3M2, tg.TG_FP4_E2M1, tg.TG_FP8_E5M2], (0, 1), (0, 1), (0.0, 1.0, 0.5)):
        if af == tg.TG_FP8_E4M3 and bf == tg.TG_FP8_E5M2:
            continue   # the fp8 pairs are the fp8 block-scaled path's own table
        ok, cat = accepts_mx(M, N, K, name[af], name[bf], bool(ta), bool(tb), beta=beta)
        try:
            tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, A_ADDR + (1 << 28), B_ADDR + (1 << 28),
                                 C_ADDR if beta else None, D_ADDR, M, N, K, ta, tb, beta, af, bf)
            got = (True, None)
        except tg.TileError as e:
            got = (False, cat_of.get(e.status, "other"))
        assert got == (ok, cat), (M, N, K, af, bf, ta, tb, beta, got)


def test_packed_mx_plan():
    p = tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, A_ADDR + (1 << 28), B_ADDR + (1 << 28), None, D_ADDR,
                             1040, 272, 640, 0, 1, 0.0, tg.TG_FP4_E2M1, tg.TG_FP6_E2M3)
    assert (p.kernel, p.block_m, p.block_n, p.block_k, p.threads, p.loader) == (tg.TG_GEMM_TILED, 128, 128, 128, 256, 0)
    assert (p.grid, p.bounds_checked) == (9 * 3, 1)
    assert p.lds_bytes == 2 * (128 * 80 + 128 * 104) + 2 * 256 * 4
    # 256 or more 256x256 blocks: 512 threads on 256x256 blocks
    p = tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, A_ADDR + (1 << 28), B_ADDR + (1 << 28), None, D_ADDR,
                             4096, 4112, 640, 0, 1, 0.0, tg.TG_FP6_E3M2, tg.TG_FP4_E2M1)
    assert (p.block_m, p.block_n, p.block_k, p.threads) == (256, 256, 128, 512)
    assert (p.grid, p.bounds_checked) == (16 * 17, 1)
    assert p.lds_bytes == 2 * (256 * 104 + 256 * 80) + 2 * 512 * 4
    p = tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, A_ADDR + (1 << 28), B_ADDR + (1 << 28), None, D_ADDR,
                             4096, 3840, 640, 0, 1, 0.0, tg.TG_FP4_E2M1, tg.TG_FP4_E2M1)
    assert (p.block_m, p.threads, p.grid, p.bounds_checked) == (128, 256, 32 * 30, 0)


@pytest.mark.parametrize("M,N,K,bs", [(4096, 4112, 1024, 256), (8192, 8192, 8192, 256),
                                      (1024, 1040, 512, 128), (144, 208, 256, 128)])
def test_packed_fp6_direct_plan(M, N, K, bs):
    # two 6-bit operands: the direct-load kernel, 128-K stages of 96-byte rows, block size as fp8
    for af, bf in ((tg.TG_FP6_E2M3, tg.TG_FP6_E2M3), (tg.TG_FP6_E3M2, tg.TG_FP6_E2M3)):
        p = tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, A_ADDR + (1 << 28), B_ADDR + (1 << 28), None,
                                 D_ADDR, M, N, K + 128, 0, 1, 0.0, af, bf)
        assert (p.kernel, p.block_m, p.block_k, p.threads, p.loader) == (tg.TG_GEMM_TILED, bs, 128, 512, 1)
        assert p.grid == ((M + bs - 1) // bs) * ((N + bs - 1) // bs)
        assert p.lds_bytes == 4 * bs * 128 + 3 * 2 * 260 * (bs // 16)
    # a 6-bit operand with an e2m1 one stays on the packed kernel
    q = tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, A_ADDR + (1 << 28), B_ADDR + (1 << 28), None, D_ADDR,
                             M, N, K, 0, 1, 0.0, tg.TG_FP6_E3M2, tg.TG_FP4_E2M1)
    assert (q.block_k, q.loader) == (128, 0)


@pytest.mark.parametrize("M,N,K,bs", [(4096, 4112, 1024, 256), (8192, 8192, 8192, 256),
                                      (1024, 1040, 512, 128), (144, 208, 256, 128)])
def test_packed_fp4_direct_plan(M, N, K, bs):
    # e2m1 x e2m1 with K % 256 == 0: the direct-load kernel, 256-K stages, block size as fp8
    p = tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, A_ADDR + (1 << 28), B_ADDR + (1 << 28), None, D_ADDR,
                             M, N, K, 0, 1, 0.0, tg.TG_FP4_E2M1, tg.TG_FP4_E2M1)
    assert (p.kernel, p.block_m, p.block_n, p.block_k, p.threads, p.loader) == (
        tg.TG_GEMM_TILED, bs, bs, 256, 512, 1)
    assert p.grid == ((M + bs - 1) // bs) * ((N + bs - 1) // bs)
    assert p.bounds_checked == int(M % bs != 0 or N % bs != 0)
    assert p.lds_bytes == 4 * bs * 128 + 3 * 2 * 260 * (bs // 16)
    # the same shape with K % 256 != 0, or a 6-bit operand, stays on the packed kernel
    for k, bf in ((K + 128, tg.TG_FP4_E2M1), (K, tg.TG_FP6_E2M3)):
        q = tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, A_ADDR + (1 << 28), B_ADDR + (1 << 28), None,
                                 D_ADDR, M, N, k, 0, 1, 0.0, tg.TG_FP4_E2M1, bf)
        assert (q.block_k, q.loader) == (128, 0)
