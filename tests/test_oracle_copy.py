"""Pins of the copy and layout oracle (CPU only)."""

import numpy as np
import pytest

import synth
from oracle.copy import copy_ref
from oracle.layout import COL, ROW, XOR, Layout, offsets, xor_offset

TILES = [(128, 64, 2), (32, 32, 4), (64, 128, 1), (16, 128, 2), (8, 32, 4), (4, 8, 2), (24, 128, 1)]


@pytest.mark.parametrize("rows,cols,eb", TILES)
def test_xor_layout_is_a_bijection_with_whole_chunks(rows, cols, eb):
    off = offsets(Layout(XOR), rows, cols, eb)
    assert sorted(off.ravel().tolist()) == list(range(rows * cols))
    ce = 16 // eb
    # every 16-byte chunk of a row lands as one contiguous, chunk-aligned run
    for r in range(rows):
        for c0 in range(0, cols, ce):
            run = off[r, c0:c0 + ce]
            assert run[0] % ce == 0
            assert np.array_equal(run, run[0] + np.arange(ce))
        # rows are not mixed: row r stays inside its own row of the tile
        assert off[r].min() >= r * cols and off[r].max() < (r + 1) * cols


@pytest.mark.parametrize("rows,cols,eb", TILES)
def test_xor_layout_is_an_involution(rows, cols, eb):
    ce = 16 // eb
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    off = xor_offset(r, c, cols, eb)
    pr, pc = off // cols, off % cols
    assert np.array_equal(xor_offset(pr, pc, cols, eb), r * cols + c)
    assert np.all(pr == r)


def test_xor_matches_byte_address_form_for_128_byte_rows():
    """128-byte rows: phys = x ^ ((x & 0x380) >> 3) on the byte offset x (the
    swizzle family of [TCGEN05-CP] 调度算法 step 2 with 16-byte atoms, 8-row period)."""
    for eb, cols in ((2, 64), (4, 32), (1, 128)):
        rows = 64
        off = offsets(Layout(XOR), rows, cols, eb)
        x = (np.arange(rows)[:, None] * cols + np.arange(cols)[None, :]) * eb
        phys = x ^ ((x & 0x380) >> 3)
        assert np.array_equal(off * eb, phys)


def test_copy_identity_and_untouched_bits():
    src = synth.random_bits(3, 40 * 24, 2)
    dst = synth.random_bits(4, 50 * 24, 2)
    out = copy_ref(src, dst, 40, 24, Layout(ROW), Layout(ROW, base=5 * 24))
    assert np.array_equal(out[5 * 24:45 * 24], src)
    assert np.array_equal(out[:5 * 24], dst[:5 * 24]) and np.array_equal(out[45 * 24:], dst[45 * 24:])


def test_copy_row_to_col_is_transpose():
    rows, cols = 24, 40
    src = synth.random_bits(5, rows * cols, 4)
    dst = np.zeros(rows * cols, dtype=np.uint32)
    out = copy_ref(src, dst, rows, cols, Layout(ROW), Layout(COL))
    assert np.array_equal(out.reshape(cols, rows), src.reshape(rows, cols).T)


def test_copy_strided_row_major_is_slice():
    rows, cols, ld = 16, 24, 40
    src = synth.random_bits(6, rows * ld, 1)
    dst = np.zeros(rows * cols, dtype=np.uint8)
    out = copy_ref(src, dst, rows, cols, Layout(ROW, ld=ld), Layout(ROW))
    assert np.array_equal(out.reshape(rows, cols), src.reshape(rows, ld)[:, :cols])


@pytest.mark.parametrize("rows,cols,eb", TILES)
def test_copy_through_xor_round_trips(rows, cols, eb):
    src = synth.random_bits(7, rows * cols, eb)
    mid = copy_ref(src, np.zeros_like(src), rows, cols, Layout(ROW), Layout(XOR))
    back = copy_ref(mid, np.zeros_like(src), rows, cols, Layout(XOR), Layout(ROW))
    assert np.array_equal(back, src)
    if rows >= 2 and cols * eb >= 32:
        assert not np.array_equal(mid, src)   # the swizzle really permutes


def test_copy_keeps_nan_payloads_and_negative_zero():
    src = np.array([0x7E01, 0xFC00, 0x8000, 0x0001, 0x7C01, 0xFFFF, 0x0000, 0x3C00], dtype=np.uint16)
    out = copy_ref(src, np.zeros(8, np.uint16), 1, 8, Layout(ROW), Layout(ROW))
    assert np.array_equal(out, src)


def test_copy_empty_is_noop():
    dst = synth.random_bits(8, 16, 2)
    assert np.array_equal(copy_ref(np.zeros(0, np.uint16), dst, 0, 8, Layout(ROW), Layout(ROW)), dst)
