"""GPU parity of tile_copy_async against the oracle copy: bit exact, guard bands intact, gaps
of ld untouched, at every depth, both transfer widths, both LDS layouts and ragged
per-workgroup tile counts; the one-tile LDS image equals the oracle's XOR image."""

import numpy as np
import pytest
import torch

import synth
import tile_level_gemm_amd as tg
from oracle.copy import copy_ref
from oracle.layout import ROW, XOR, Layout, extent
from tests.gpu_util import Guarded, say, upload_bits

pytestmark = pytest.mark.gpu

DT = {1: tg.TG_U8, 2: tg.TG_F16, 4: tg.TG_F32}
UINT = {1: np.uint8, 2: np.uint16, 4: np.uint32}
LDS = {ROW: tg.TG_ROW_MAJOR, XOR: tg.TG_XOR_SWIZZLE}


def run_async(rows, cols, eb, opts, sld=0, dld=0, soff=0, doff=0, dst_kind=ROW, seed=3):
    src_layout = Layout(ROW, sld, 0)
    dst_layout = Layout(dst_kind, dld, 0)
    n_src = extent(src_layout, rows, cols, eb)
    n_dst = extent(dst_layout, rows, cols, eb)
    src_bits = synth.random_bits(seed, n_src, eb)
    dst_init = synth.random_bits(seed + 1, n_dst + doff, eb)
    src = upload_bits(np.concatenate([np.zeros(soff, UINT[eb]), src_bits]))
    dst = Guarded((n_dst + doff) * eb, fill=dst_init)
    say(f"copy_async {rows}x{cols} eb={eb} {opts} sld={sld} dld={dld} soff={soff} doff={doff} "
        f"dst={dst_kind}")
    tg.tile_copy_async(src.data_ptr() + soff * eb, dst.ptr + doff * eb, (rows, cols), DT[eb],
                       (tg.TG_ROW_MAJOR, sld), (LDS[dst_kind] if dst_kind == XOR else tg.TG_ROW_MAJOR, dld),
                       opts)
    torch.cuda.synchronize()
    want = copy_ref(src_bits, dst_init[doff:], rows, cols, src_layout, dst_layout)
    got = dst.host(UINT[eb])
    return np.array_equal(got[:doff], dst_init[:doff]) and np.array_equal(got[doff:], want), \
        dst.guards_intact()


@pytest.mark.parametrize("depth", [1, 2, 3, 4])
@pytest.mark.parametrize("lds", [ROW, XOR])
def test_several_tiles_every_depth(depth, lds):
    # 29 tiles: per-workgroup counts that are not multiples of the depth
    opts = dict(tile_rows=32, tile_cols=64, threads=128, lds_kind=LDS[lds], depth=depth,
                tiles_per_workgroup=9)
    ok, guards = run_async(32 * 29, 64, 2, opts)
    assert ok and guards


@pytest.mark.parametrize("depth", [1, 2, 4])
def test_the_streaming_tile_many_tiles(depth):
    # 128x64 fp16 tiles on 256 threads (4 rounds of 128 bits), 9 x 7 tiles, padded rows
    opts = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE, depth=depth,
                tiles_per_workgroup=16)
    ok, guards = run_async(128 * 9, 64 * 7, 2, opts, sld=64 * 7 + 8, dld=64 * 7 + 24)
    assert ok and guards


@pytest.mark.parametrize("eb,tr,tc,threads", [(1, 64, 128, 64), (4, 32, 32, 128), (4, 16, 128, 512),
                                              (2, 8, 64, 64), (1, 128, 128, 1024)])
@pytest.mark.parametrize("depth", [2, 3])
def test_element_sizes_and_rounds(eb, tr, tc, threads, depth):
    opts = dict(tile_rows=tr, tile_cols=tc, threads=threads, lds_kind=tg.TG_XOR_SWIZZLE, depth=depth,
                tiles_per_workgroup=4)
    ok, guards = run_async(tr * 5, tc * 3, eb, opts, seed=eb * 10 + depth)
    assert ok and guards


@pytest.mark.parametrize("depth", [1, 4])
def test_32_bit_transfers(depth):
    # 260-byte source rows (ld 130 fp16) and bases 4 and 12 bytes off: 32-bit transfers
    opts = dict(tile_rows=16, tile_cols=64, threads=64, lds_kind=tg.TG_ROW_MAJOR, depth=depth,
                tiles_per_workgroup=5)
    p = tg.tile_copy_async_plan((1 << 20) + 4, (1 << 30) + 12, (16 * 7, 64 * 2), tg.TG_F16,
                                (tg.TG_ROW_MAJOR, 130), None, opts)
    assert p.copy.load.vec_bits == 32 and p.tiles_per_workgroup == 5
    ok, guards = run_async(16 * 7, 64 * 2, 2, opts, sld=130, soff=2, doff=6)
    assert ok and guards


def test_one_tile_lds_image_is_the_xor_layout():
    # the destination is the tile written in LDS order: the swizzled placement the lanes' slots
    # produced must be exactly the oracle's XOR layout
    opts = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE, depth=2)
    ok, guards = run_async(128, 64, 2, opts, dst_kind=XOR)
    assert ok and guards


def test_empty_tensor():
    say("copy_async empty")
    tg.tile_copy_async(None, None, (0, 64), tg.TG_F16, None, None,
                       dict(tile_rows=32, tile_cols=64, threads=64, depth=2))
    torch.cuda.synchronize()


def test_full_size_stream_bit_exact():
    rows = cols = 16384
    src_bits = synth.stream_input(rows, cols)
    src = upload_bits(src_bits)
    dst = torch.empty_like(src)
    opts = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE, depth=2)
    say("copy_async 16384^2 f16 depth 2")
    tg.tile_copy_async(src, dst, (rows, cols), tg.TG_F16, None, None, opts)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
