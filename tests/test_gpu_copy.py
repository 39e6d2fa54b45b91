"""GPU parity of tile_copy against the oracle: bit exact, guard bands intact."""

import numpy as np
import pytest
import torch

import synth
import tile_level_gemm_amd as tg
from oracle.copy import copy_ref
from oracle.layout import COL, ROW, XOR, Layout, extent
from tests.gpu_util import Guarded, say, upload_bits

pytestmark = pytest.mark.gpu

DT = {1: tg.TG_U8, 2: tg.TG_F16, 4: tg.TG_F32}
UINT = {1: np.uint8, 2: np.uint16, 4: np.uint32}
KIND = {ROW: tg.TG_ROW_MAJOR, COL: tg.TG_COL_MAJOR, XOR: tg.TG_XOR_SWIZZLE}


def run_copy(src_bits, rows, cols, eb, src_layout, dst_layout, opts=None, dtype=None, src_offset=0):
    """Copy through the library and through the oracle; returns (gpu image, oracle image, guards ok)."""
    n_dst = extent(dst_layout, rows, cols, eb)
    dst_init = synth.random_bits(1234, n_dst, eb)
    src_dev = upload_bits(np.concatenate([np.zeros(src_offset, UINT[eb]), src_bits]))
    dst = Guarded(n_dst * eb, fill=dst_init)
    sl = (KIND[src_layout.kind], src_layout.ld)
    dl = (KIND[dst_layout.kind], dst_layout.ld)
    src_ptr = src_dev.data_ptr() + src_offset * eb
    dtype = dtype or DT[eb]
    if opts is None:
        tg.tile_copy(src_ptr, dst.ptr, (rows, cols), dtype, sl, dl)
    else:
        tg.tile_copy_ex(src_ptr, dst.ptr, (rows, cols), dtype, sl, dl, opts)
    torch.cuda.synchronize()
    want = copy_ref(src_bits, dst_init, rows, cols, src_layout, dst_layout)
    return dst.host(UINT[eb]), want, dst.guards_intact()


def test_copy_32x32_f32_one_wavefront():
    say("copy 32x32 f32, 64 threads, row-major LDS")
    src = synth.copy32_input()
    got, want, guards = run_copy(src, 32, 32, 4, Layout(ROW), Layout(ROW),
                                 dict(tile_rows=32, tile_cols=32, threads=64, lds_kind=tg.TG_ROW_MAJOR))
    assert guards and np.array_equal(got, want)


def test_copy_128x64_f16_swizzled_block():
    say("copy 128x64 f16, 256 threads, XOR LDS")
    src = synth.copy128_input()
    opts = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE)
    got, want, guards = run_copy(src, 128, 64, 2, Layout(ROW), Layout(ROW), opts)
    assert guards and np.array_equal(got, want)


def test_copy_128x64_f16_lds_image_is_the_xor_layout():
    """Writing the tile out in LDS order exposes the swizzle: it must equal the oracle's xor image."""
    say("copy 128x64 f16 -> xor image")
    src = synth.copy128_input()
    opts = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE)
    got, want, guards = run_copy(src, 128, 64, 2, Layout(ROW), Layout(XOR), opts)
    assert guards and np.array_equal(got, want)
    assert not np.array_equal(got, src)


@pytest.mark.parametrize("eb,dtype", [(1, tg.TG_U8), (1, tg.TG_I8), (1, tg.TG_FP8_E4M3), (1, tg.TG_FP8_E5M2),
                                      (2, tg.TG_F16), (2, tg.TG_BF16), (4, tg.TG_F32)])
@pytest.mark.parametrize("threads", [32, 64, 128, 256])
def test_copy_dtypes_and_scopes(eb, dtype, threads):
    rows, cols = 64, 256 // eb
    say(f"copy dtype={dtype} threads={threads}")
    src = synth.random_bits(50 + eb + threads, rows * cols, eb)
    opts = dict(tile_rows=32, tile_cols=cols // 2, threads=threads, lds_kind=tg.TG_XOR_SWIZZLE)
    got, want, guards = run_copy(src, rows, cols, eb, Layout(ROW), Layout(ROW), opts, dtype=dtype)
    assert guards and np.array_equal(got, want)


@pytest.mark.parametrize("case", [
    # strided source, packed destination
    dict(rows=96, cols=40, eb=2, src=Layout(ROW, 56), dst=Layout(ROW), tile=(32, 40), threads=64, lds=ROW),
    # transposing copy: row-major -> column-major (width narrows to one element)
    dict(rows=64, cols=48, eb=4, src=Layout(ROW), dst=Layout(COL), tile=(16, 48), threads=64, lds=ROW),
    # column-major -> column-major with padding
    dict(rows=64, cols=32, eb=2, src=Layout(COL, 72), dst=Layout(COL, 64), tile=(64, 8), threads=64),
    # misaligned source pointer (odd element offset): load width narrows, result exact
    dict(rows=128, cols=64, eb=2, src=Layout(ROW), dst=Layout(ROW), tile=(128, 64), threads=256, off=3),
    # one-thread scope
    dict(rows=8, cols=16, eb=1, src=Layout(ROW), dst=Layout(ROW), tile=(8, 16), threads=1),
    # row stride 20 fp16 (narrows to 64-bit), 16-column tiles
    dict(rows=32, cols=16, eb=2, src=Layout(ROW, 20), dst=Layout(ROW), tile=(16, 16), threads=32),
    # non power-of-two tile width (division path), row-major LDS
    dict(rows=48, cols=24, eb=4, src=Layout(ROW), dst=Layout(ROW), tile=(12, 24), threads=32, lds=ROW),
    dict(rows=48, cols=24, eb=4, src=Layout(ROW), dst=Layout(ROW), tile=(12, 24), threads=36, lds=ROW),
])
def test_copy_layout_variants(case):
    rows, cols, eb = case["rows"], case["cols"], case["eb"]
    say(f"copy variant {case}")
    n_src = extent(case["src"], rows, cols, eb)
    src = synth.random_bits(60 + rows, n_src, eb)
    lds = KIND[case.get("lds", XOR)]
    opts = dict(tile_rows=case["tile"][0], tile_cols=case["tile"][1], threads=case["threads"], lds_kind=lds)
    got, want, guards = run_copy(src, rows, cols, eb, case["src"], case["dst"], opts,
                                 src_offset=case.get("off", 0))
    assert guards and np.array_equal(got, want)


def test_copy_every_f16_bit_pattern():
    say("copy all 65536 f16 patterns")
    src = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got, want, guards = run_copy(src, 256, 256, 2, Layout(ROW), Layout(ROW))
    assert guards and np.array_equal(got, want) and np.array_equal(got, src)


def test_copy_empty_is_noop():
    say("copy empty")
    dst = Guarded(64)
    tg.tile_copy(None, dst.ptr, (0, 32), tg.TG_F16)
    torch.cuda.synchronize()
    assert dst.guards_intact()


def test_copy_rejections_launch_nothing():
    say("copy rejections")
    src = upload_bits(synth.random_bits(3, 64 * 64, 2))
    dst = Guarded(64 * 64 * 2, fill=np.zeros(64 * 64, np.uint16))
    with pytest.raises(tg.TileError) as e:
        tg.tile_copy_ex(src, dst.ptr, (64, 64), tg.TG_F16, None, None,
                        dict(tile_rows=1, tile_cols=64, threads=1024, lds_kind=tg.TG_ROW_MAJOR))
    assert e.value.status == tg.TG_E_THREADS
    torch.cuda.synchronize()
    assert dst.guards_intact() and not dst.host(np.uint16).any()


def test_stream_copy_full_size():
    """16384 x 16384 f16 in 128x64 tiles, 256 threads, XOR LDS: the timed configuration."""
    rows = cols = 16384
    say("stream copy 16384^2 f16")
    src_bits = synth.stream_input(rows, cols)
    src = upload_bits(src_bits)
    dst = torch.empty_like(src)
    plan = tg.tile_copy_plan(src, dst, (rows, cols), tg.TG_F16)
    assert (plan.tile_rows, plan.tile_cols, plan.load.threads, plan.lds_kind) == (128, 64, 256, tg.TG_XOR_SWIZZLE)
    tg.tile_copy(src, dst, (rows, cols), tg.TG_F16)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint16)
    # oracle on a slab of rows (every tile column, four tile rows), identity on the rest
    slab = 512
    want = copy_ref(src_bits[:slab * cols], np.zeros(slab * cols, np.uint16), slab, cols, Layout(ROW), Layout(ROW))
    assert np.array_equal(got[:slab * cols], want)
    assert np.array_equal(got, src_bits)
