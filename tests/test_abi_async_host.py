"""Host-only checks of tile_copy_async (no GPU): its plan against the oracle's asynchronous
planner, the workgroup schedule, and every rejection."""

import numpy as np
import pytest

import tile_level_gemm_amd as tg
from oracle.layout import COL, ROW, XOR, Layout
from oracle.planner import Plan, Reject, plan_async

KIND = {ROW: tg.TG_ROW_MAJOR, COL: tg.TG_COL_MAJOR, XOR: tg.TG_XOR_SWIZZLE}
CATEGORY = {tg.TG_E_THREADS: "threads", tg.TG_E_LAYOUT: "layout", tg.TG_E_SHAPE: "shape",
            tg.TG_E_ALIGN: "align", tg.TG_E_ARG: "arg"}
DT = {1: tg.TG_U8, 2: tg.TG_F16, 4: tg.TG_F32}


def _cases():
    rs = np.random.default_rng(123)
    for _ in range(400):
        eb = int(rs.choice([1, 2, 4]))
        tr = int(rs.choice([4, 8, 16, 32, 64, 128]))
        tc = int(rs.choice([16, 32, 64, 128, 256]))
        rows, cols = tr * int(rs.integers(1, 4)), tc * int(rs.integers(1, 4))
        threads = int(rs.choice([32, 64, 128, 192, 256, 512, 1024]))
        dkind = rs.choice([ROW, ROW, ROW, COL])
        sld = cols + int(rs.choice([0, 0, 0, 2, 4, 8, 16, 3]))
        dld = (cols if dkind == ROW else rows) + int(rs.choice([0, 0, 8, 1, 32]))
        soff, doff = int(rs.choice([0, 0, 0, 1, 4, 8])), int(rs.choice([0, 0, 16, 2]))
        lds = rs.choice([ROW, XOR])
        depth = int(rs.choice([1, 2, 3, 4, 4, 0]))
        yield rows, cols, tr, tc, eb, threads, (sld, soff), (dkind, dld, doff), lds, depth


@pytest.mark.parametrize("case", list(_cases()))
def test_async_plan_matches_oracle(case):
    rows, cols, tr, tc, eb, threads, s, d, lds, depth = case
    src_addr = (1 << 20) + s[1] * eb
    dst_addr = (1 << 30) + d[2] * eb
    lds_side = Layout(lds, tc if lds == ROW else 0, 0)
    want = plan_async(rows, cols, tr, tc, 8 * eb, threads, Layout(ROW, s[0], src_addr // eb),
                      Layout(d[0], d[1], dst_addr // eb), lds_side, depth)
    opts = dict(tile_rows=tr, tile_cols=tc, threads=threads, lds_kind=KIND[lds], depth=depth)
    try:
        p = tg.tile_copy_async_plan(src_addr, dst_addr, (rows, cols), DT[eb], (tg.TG_ROW_MAJOR, s[0]),
                                    (KIND[d[0]], d[1]), opts)
        got = (Plan(*p.copy.load.as_tuple()), Plan(*p.copy.store.as_tuple()))
        assert p.depth == depth and p.copy.lds_bytes == depth * 16384
        tiles = (rows // tr) * (cols // tc)
        assert p.copy.tiles == tiles
        assert p.grid * p.tiles_per_workgroup >= tiles > (p.grid - 1) * p.tiles_per_workgroup
    except tg.TileError as e:
        got = Reject(CATEGORY.get(e.status, "other"), e.reason)
    if isinstance(want, Reject):
        assert isinstance(got, Reject) and got.category == want.category, (case, got, want)
    else:
        assert got == want, (case, got, want)


def test_the_streaming_configuration():
    opts = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE, depth=2)
    p = tg.tile_copy_async_plan(1 << 30, 1 << 31, (16384, 16384), tg.TG_F16, None, None, opts)
    assert p.copy.load.as_tuple() == (4, 256, 8, 128) == p.copy.store.as_tuple()
    assert (p.copy.tiles, p.tiles_per_workgroup, p.grid, p.copy.lds_bytes) == (32768, 4, 8192, 32768)


def test_width_narrows_to_32_bits_and_rejects_below():
    # 66-element f16 rows (132 bytes): 32-bit chunks only
    opts = dict(tile_rows=16, tile_cols=64, threads=64, lds_kind=tg.TG_ROW_MAJOR, depth=2)
    p = tg.tile_copy_async_plan(1 << 20, 1 << 30, (32, 64), tg.TG_F16, (tg.TG_ROW_MAJOR, 66), None, opts)
    assert p.copy.load.vec_bits == 32 and p.copy.load.outer == 8
    # 65-element rows: only 16-bit transfers would fit
    with pytest.raises(tg.TileError) as e:
        tg.tile_copy_async_plan(1 << 20, 1 << 30, (32, 64), tg.TG_F16, (tg.TG_ROW_MAJOR, 65), None, opts)
    assert e.value.status == tg.TG_E_ALIGN


@pytest.mark.parametrize("mutate,code", [
    (dict(opts=None), tg.TG_E_ARG),
    (dict(depth=0), tg.TG_E_ARG), (dict(depth=5), tg.TG_E_ARG), (dict(flags=1), tg.TG_E_ARG),
    (dict(tiles_per_workgroup=65), tg.TG_E_ARG), (dict(tiles_per_workgroup=-1), tg.TG_E_ARG),
    (dict(src_layout=(tg.TG_COL_MAJOR, 0)), tg.TG_E_LAYOUT),
    (dict(dst_layout=(tg.TG_COL_MAJOR, 0)), tg.TG_E_LAYOUT),
    (dict(threads=96), tg.TG_E_THREADS),
    (dict(threads=32), tg.TG_E_THREADS),
    (dict(tile_rows=256), tg.TG_E_SHAPE),                   # 32 KiB stage
    (dict(threads=1024, tile_rows=4), tg.TG_E_THREADS),      # 256 elements on 1024 threads
    (dict(shape=(100, 64)), tg.TG_E_SHAPE),
    (dict(src=None), tg.TG_E_NULL),
])
def test_rejections(mutate, code):
    args = dict(src=1 << 20, dst=1 << 30, shape=(256, 128), dtype=tg.TG_F16,
                src_layout=(tg.TG_ROW_MAJOR, 0), dst_layout=(tg.TG_ROW_MAJOR, 0))
    opts = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE, depth=2, flags=0,
                tiles_per_workgroup=0)
    for k in list(mutate):
        if k in opts:
            opts[k] = mutate.pop(k)
    args.update(mutate)
    o = args.pop("opts", opts) if "opts" in args else opts
    with pytest.raises(tg.TileError) as e:
        tg.tile_copy_async_plan(args["src"], args["dst"], args["shape"], args["dtype"],
                                args["src_layout"], args["dst_layout"], o)
    assert e.value.status == code
    # the copy itself refuses before launching anything
    with pytest.raises(tg.TileError) as e2:
        tg.tile_copy_async(args["src"], args["dst"], args["shape"], args["dtype"],
                           args["src_layout"], args["dst_layout"], o)
    assert e2.value.status == code


def test_explicit_tiles_per_workgroup():
    opts = dict(tile_rows=32, tile_cols=64, threads=128, depth=3, tiles_per_workgroup=9)
    p = tg.tile_copy_async_plan(1 << 20, 1 << 30, (32 * 29, 64), tg.TG_F16, None, None, opts)
    assert (p.tiles_per_workgroup, p.grid) == (9, 4)


def test_empty_tensor_is_a_no_op():
    opts = dict(tile_rows=128, tile_cols=64, threads=256, depth=3)
    tg.tile_copy_async(None, None, (0, 64), tg.TG_F16, None, None, opts)
    p = tg.tile_copy_async_plan(None, None, (0, 64), tg.TG_F16, None, None, opts)
    assert p.copy.tiles == 0 and p.depth == 3
