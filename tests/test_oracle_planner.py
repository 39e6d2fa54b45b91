"""Pins of the vec_auto partition planner oracle (CPU only)."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle.layout import COL, ROW, XOR, Layout, offsets
from oracle.planner import Plan, Reject, chunk_coords, fused_order, plan_region, plan_tiles

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def lay(d):
    return Layout(d["kind"], d.get("ld", 0), d.get("base", 0))


def test_worked_example_32x32_f32_one_warp():
    g = load("planner_worked_example.json")
    p = plan_region(g["rows"], g["cols"], g["elem_bits"], g["threads"], lay(g["src"]), lay(g["dst"]))
    e = g["expect"]
    assert p == Plan(e["outer"], e["threads"], e["vec"], e["vec_bits"])
    # fused index of round f, thread t is f*128 + t*4 (row-major over the 32x32 tile)
    for f in range(p.outer):
        for t in range(p.threads):
            (r, c) = chunk_coords(p, 32, 32, ROW, f, t)[0]
            assert r * 32 + c == f * 128 + t * 4


def test_dtype_rounds_table():
    g = load("planner_dtype_rounds.json")
    for case in g["cases"]:
        p = plan_region(g["rows"], g["cols"], case["elem_bits"], g["threads"], Layout(ROW), Layout(ROW))
        assert (p.vec, p.outer, p.vec_bits) == (case["vec"], case["outer"], 128), case


def test_rejections_and_narrowing():
    g = load("planner_rejections_and_narrowing.json")
    for case in g["reject"]:
        p = plan_region(case["rows"], case["cols"], case["elem_bits"], case["threads"], Layout(ROW), Layout(ROW))
        assert isinstance(p, Reject) and p.category == case["category"], case
    for case in g["narrow"]:
        p = plan_region(case["rows"], case["cols"], case["elem_bits"], case["threads"],
                        lay(case["src"]), lay(case["dst"]))
        assert (p.vec, p.vec_bits, p.outer) == (case["vec"], case["vec_bits"], case["outer"]), case


def test_swizzled_side_caps_vector_at_one_chunk():
    # u8 tile of 32x128 with 128 threads: 128 bits = 16 elements fill one chunk exactly.
    p = plan_region(32, 128, 8, 128, Layout(ROW), Layout(XOR))
    assert p.vec == 16 and p.outer == 2
    # a row that is not a power-of-two count of 16-byte chunks cannot be xor
    p = plan_region(16, 24, 16, 64, Layout(ROW), Layout(XOR))
    assert isinstance(p, Reject) and p.category == "layout"


def _check_plan_brute_force(rows, cols, eb, threads, drive, other, plan):
    """Every chunk is contiguous and vec-aligned on both sides, and chunks tile the region."""
    order = fused_order(drive)
    offs = [offsets(s, rows, cols, eb) for s in (drive, other)]
    seen = np.zeros((rows, cols), dtype=np.int32)
    for f in range(plan.outer):
        for t in range(plan.threads):
            coords = chunk_coords(plan, rows, cols, order, f, t)
            for off in offs:
                run = np.array([off[r, c] for r, c in coords])
                if not (np.array_equal(run, run[0] + np.arange(plan.vec)) and run[0] % plan.vec == 0):
                    return False
                if other.kind == XOR and off is offs[1]:
                    if (run[0] * eb) // 16 != ((run[-1] * eb) // 16):
                        return False
            for r, c in coords:
                seen[r, c] += 1
    return bool(np.all(seen == 1))


def _cases():
    rs = np.random.default_rng(1234)
    shapes = [(8, 16), (16, 16), (4, 24), (32, 32), (16, 8), (6, 40), (1, 64), (8, 64)]
    for (rows, cols), eb, threads in itertools.product(shapes, (1, 2, 4), (1, 4, 8, 32, 64)):
        if (rows * cols) % threads:
            continue
        kind = rs.choice([ROW, ROW, COL])
        full_ld = (cols if kind == ROW else rows) + int(rs.choice([0, 0, 1, 2, 4, 8, 16]))
        base = int(rs.choice([0, 0, 1, 2, 4, 8, 16, 3]))
        drive = Layout(kind, full_ld, base)
        other = Layout(rs.choice([ROW, ROW, XOR, COL]))
        yield rows, cols, eb, threads, drive, other


@pytest.mark.parametrize("case", list(_cases()))
def test_plan_is_valid_and_widest(case):
    rows, cols, eb, threads, drive, other = case
    p = plan_region(rows, cols, 8 * eb, threads, drive, other)
    if isinstance(p, Reject):
        # only a non power-of-two xor row may be rejected here
        assert other.kind == XOR and p.category == "layout"
        return
    assert p.outer * p.threads * p.vec == rows * cols
    assert _check_plan_brute_force(rows, cols, eb, threads, drive, other, p)
    # the next wider width (if it is a candidate) must be invalid
    wider = p.vec * 2
    if wider * eb * 8 <= 128 and (rows * cols // threads) % wider == 0:
        q = Plan(rows * cols // (threads * wider), threads, wider, wider * eb * 8)
        assert not _check_plan_brute_force(rows, cols, eb, threads, drive, other, q)


def test_tiled_plan_is_min_over_tiles():
    # tiles of a tensor whose row length breaks 16-byte alignment of the second tile row
    p = plan_tiles(8, 72, 4, 8, 16, 4, Layout(ROW), Layout(ROW))
    assert p.vec == 8      # ld 72: every tile base (multiples of 8 and of 4*72) stays aligned
    p = plan_tiles(8, 68, 4, 4, 16, 2, Layout(ROW), Layout(ROW))
    assert p.vec == 4      # ld 68 admits 4, not 8
    p = plan_tiles(8, 64, 4, 16, 16, 8, Layout(ROW, base=2), Layout(ROW))
    assert p.vec == 2
    assert isinstance(plan_tiles(8, 60, 4, 16, 16, 64, Layout(ROW), Layout(ROW)), Reject)
    assert plan_tiles(0, 64, 4, 16, 16, 64, Layout(ROW), Layout(ROW)).outer == 0


# ---- the asynchronous copy's plan (oracle.planner.plan_async), hand-derived ---------------------

def test_plan_async_hand_derived():
    from oracle.planner import Plan, Reject, plan_async
    from oracle.layout import Layout
    lds = Layout("xor", 0, 0)
    # 128x64 fp16 tiles, 256 threads: 16 KiB per tile = 256 threads x 16 B x 4 rounds
    p = plan_async(16384, 16384, 128, 64, 16, 256, Layout("row"), Layout("row"), lds, 2)
    assert p == (Plan(4, 256, 8, 128), Plan(4, 256, 8, 128))
    # 132-byte source rows (ld 66 fp16): the copy's width is 32 bits -> 32-bit transfers, 8 rounds
    # for a 16 x 64 tile on 64 threads (2 KiB = 64 x 4 B x 8)
    rl = Layout("row", 0, 0)
    p = plan_async(32, 64, 16, 64, 16, 64, Layout("row", 66), Layout("row"), rl, 1)
    assert p == (Plan(8, 64, 2, 32), Plan(8, 64, 2, 32))
    # 136-byte rows allow 64-bit copies, but there is no 64-bit direct load: 32-bit
    p = plan_async(32, 64, 16, 64, 16, 64, Layout("row", 68), Layout("row"), rl, 1)
    assert p[0].vec_bits == 32
    # 130-byte rows: 16-bit only -> rejected
    assert plan_async(32, 64, 16, 64, 16, 64, Layout("row", 65), Layout("row"), rl, 1).category == "align"
    # a 32 KiB stage, 96 threads, depth 5, a column-major source: rejected
    assert plan_async(256, 64, 256, 64, 16, 256, Layout("row"), Layout("row"), rl, 2).category == "shape"
    assert plan_async(128, 64, 128, 64, 16, 96, Layout("row"), Layout("row"), rl, 2).category == "threads"
    assert plan_async(128, 64, 128, 64, 16, 256, Layout("row"), Layout("row"), rl, 5).category == "arg"
    assert plan_async(128, 64, 128, 64, 16, 256, Layout("col"), Layout("row"), rl, 2).category == "layout"
    # 16 rounds per thread (16 KiB on 64 threads at 128 bits) is outside 1, 2, 4, 8
    assert plan_async(128, 64, 128, 64, 16, 64, Layout("row"), Layout("row"), lds, 2).category == "threads"
