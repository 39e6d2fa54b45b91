"""vec_auto copy partition planner (oracle; test infrastructure).

Restates [VEC-AUTO]:

* 接受什么输入 (the gate, _divides_thread_cnt): the thread count must be positive
  and must divide the element count of the region; otherwise the copy is
  rejected rather than masked by a slow scalar path.
* 算法核心 step 1: the region is split into a three-level iteration
  [outer, threads, vec]; the global side fixes the canonical (stride-descending)
  order, the vec iteration is its contiguous innermost part and each thread owns
  consecutive fused-index slots.  The generated IR of the demo shows the fused
  index of round f, thread t as f·(threads·vec) + t·vec (生成的 TIRx IR).
* step 2: vector widths of 128, 64, 32, 16 and 8 bits are tried widest first; a
  width is taken when every transfer moves one aligned vector on both sides.  The
  page states this as (a) the contiguous tail divides by the width and (b) every
  non-vector stride on both sides, the thread iteration included, and both base
  offsets are multiples of it.  The oracle does not restate that rule: it lists
  the element offsets of every transfer on both sides and checks the plain
  property the rule stands for (_width_ok): the offsets are consecutive and the
  first is a multiple of the width.
* 输入如何改变算法 / swizzled shared 布局: with a swizzled shared side the vector
  may not leave one 16-byte swizzle chunk (checked transfer by transfer as well).
* 对齐约束的兜底: misaligned strides or a region starting at an odd column narrow
  the width, down to one element.

Readings (the page is silent):

* widths narrower than the element, or not a multiple of it, are skipped;
* the width must also divide elements/threads, so that elements = outer·threads·vec;
* "misaligned" is measured in elements from the side's base: base offset (pointer
  address / element size plus region offset) and leading dimension; an element
  offset of a side therefore counts from that side's base.

Pinned by tests/test_oracle_planner.py: the page's worked example (32 threads,
32x32 float32 -> vec 4 = 128 bits, outer 8, fused index f·128 + t·4), the
per-dtype rounds of the same tile, the 64-elements-on-1024-threads rejection,
and the two narrowing examples (fp16 row stride 20; a region starting at
column 3); plus a re-derivation, thread by thread and round by round, that every
planned chunk is contiguous and aligned on both sides and that the next wider width
is not.
"""

import numpy as np

from .layout import ROW, COL, XOR, CHUNK_BYTES, offsets, xor_defined

WIDTHS_BITS = (128, 64, 32, 16, 8)


class Plan:
    def __init__(self, outer, threads, vec, vec_bits):
        self.outer, self.threads, self.vec, self.vec_bits = outer, threads, vec, vec_bits

    def __repr__(self):
        return f"Plan(outer={self.outer}, threads={self.threads}, vec={self.vec}, bits={self.vec_bits})"

    def __eq__(self, other):
        return isinstance(other, Plan) and (self.outer, self.threads, self.vec, self.vec_bits) == (
            other.outer, other.threads, other.vec, other.vec_bits)


class Reject:
    """category is "threads" (count <= 0 or not dividing the elements) or "layout"."""

    def __init__(self, category, reason):
        self.category, self.reason = category, reason

    def __repr__(self):
        return f"Reject({self.category!r}: {self.reason})"


def fused_order(drive):
    """Canonical order of the driving (global) side: "row" or "col"."""
    return COL if drive.kind == COL else ROW


def _transfers(side, rows, cols, order, v, elem_bytes):
    """Element offsets on `side` of every v-element transfer: an (n / v, v) array.

    Transfer k covers the fused positions [k·v, k·v + v) of the region in `order`
    (算法核心 step 1: the vec iteration is the innermost, contiguous part of the fused
    index); position x is (outer, inner) = divmod(x, inner extent).
    """
    off = offsets(side, rows, cols, elem_bytes)          # [r, c]
    fused = off.reshape(-1) if order == ROW else off.T.reshape(-1)
    return fused.reshape(-1, v)


def _width_ok(side, rows, cols, order, v, elem_bytes):
    """Does every transfer of v elements land as one aligned vector on this side?

    The plain definition of 算法核心 step 2 and 对齐约束的兜底, checked transfer by
    transfer: the v offsets are consecutive, the first is a multiple of v (an element
    offset counts from the side's base, so the base enters here), and on a swizzled
    side the transfer's bytes stay inside one 16-byte swizzle chunk
    (输入如何改变算法).
    """
    t = _transfers(side, rows, cols, order, v, elem_bytes)
    if not (t == t[:, :1] + np.arange(v, dtype=np.int64)).all():
        return False
    if (t[:, 0] % v).any():
        return False
    if side.kind == XOR:
        first = (t[:, 0] * elem_bytes) // CHUNK_BYTES
        last = ((t[:, -1] + 1) * elem_bytes - 1) // CHUNK_BYTES
        if (first != last).any():
            return False
    return True


def plan_region(rows, cols, elem_bits, threads, drive, other):
    """Partition one rows x cols region copied between `drive` (global side) and `other`."""
    if threads <= 0:
        return Reject("threads", "thread count must be positive")
    n = rows * cols
    if n % threads:
        return Reject("threads", f"{n} elements do not divide over {threads} threads")
    eb = elem_bits // 8
    for side in (drive, other):
        if side.kind == XOR and not xor_defined(cols, eb):
            return Reject("layout", "xor layout needs rows of a power-of-two count of 16-byte chunks")
        if side.kind == XOR and side.ld not in (0, cols):
            return Reject("layout", "the xor layout is a packed tile")
    order = fused_order(drive)
    if n == 0:
        return Plan(0, threads, 1, elem_bits)
    for bits in WIDTHS_BITS:
        if bits < elem_bits or bits % elem_bits:
            continue
        v = bits // elem_bits
        if (n // threads) % v:
            continue
        if all(_width_ok(s, rows, cols, order, v, eb) for s in (drive, other)):
            return Plan(n // (threads * v), threads, v, bits)
    return Reject("layout", "no vector width keeps every transfer contiguous")


def chunk_coords(plan, rows, cols, order, f, t):
    """Logical (r, c) pairs of the elements thread t moves in round f (fused order)."""
    inner = cols if order == ROW else rows
    x0 = f * plan.threads * plan.vec + t * plan.vec
    out = []
    for j in range(plan.vec):
        o, i = divmod(x0 + j, inner)
        out.append((o, i) if order == ROW else (i, o))
    return out


def plan_tiles(rows, cols, tile_rows, tile_cols, elem_bits, threads, tensor_side, lds_side):
    """Plan of a rows x cols tensor copied tile by tile: every tile must accept the vector.

    Brute force over every tile: the tensor side of tile (i, j) is the tensor
    layout with its base moved to (i·tile_rows, j·tile_cols).  The chosen width
    is the widest that every tile accepts (acceptance is closed under halving,
    so this is the minimum of the per-tile widths).
    """
    from .layout import Layout
    if threads <= 0:
        return Reject("threads", "thread count must be positive")
    if rows == 0 or cols == 0:
        return Plan(0, threads, 1, elem_bits)
    if tile_rows <= 0 or tile_cols <= 0 or rows % tile_rows or cols % tile_cols:
        return Reject("layout", "tensor is not a whole number of tiles")
    full_ld = tensor_side.ld or (rows if tensor_side.kind == COL else cols)
    best = None
    for i in range(rows // tile_rows):
        for j in range(cols // tile_cols):
            r0, c0 = i * tile_rows, j * tile_cols
            if tensor_side.kind == ROW:
                view = Layout(ROW, full_ld, tensor_side.base + r0 * full_ld + c0)
            else:
                view = Layout(COL, full_ld, tensor_side.base + c0 * full_ld + r0)
            p = plan_region(tile_rows, tile_cols, elem_bits, threads, view, lds_side)
            if isinstance(p, Reject):
                return p
            if best is None or p.vec < best.vec:
                best = p
    return best


# ---- the asynchronous copy ([TCGEN05-CP] 一个算子、六个变体, 与其他异步变体的协作关系) ----------
#
# Readings (the pages describe the variant family, not these limits):
# * the issue-only global -> LDS transfer has the widths of the hardware's direct loads to LDS:
#   128 and 32 bits are used (there is no 64-bit one); both directions move the same width, the
#   widest of those two that the copy's own widest-first width (step 2) allows in each direction;
# * a wave issues together, so the thread count is a multiple of 64;
# * one LDS stage holds one tile of at most 16 KiB, and 1 .. 4 stages are in flight;
# * the source is row-major; the destination row-major or the one-tile LDS image;
# * a thread runs 1, 2, 4 or 8 rounds per tile.
ASYNC_WIDTHS_BITS = (128, 32)
ASYNC_STAGE_BYTES = 16384


def plan_async(rows, cols, tile_rows, tile_cols, elem_bits, threads, src_side, dst_side, lds_side,
               depth):
    """(load plan, store plan) of the asynchronous tile copy, or a Reject.

    Reject categories: "arg" (depth), "layout", "threads", "shape", "align", and those of
    plan_tiles."""
    if depth not in (1, 2, 3, 4):
        return Reject("arg", "depth must be 1 .. 4")
    if src_side.kind != ROW:
        return Reject("layout", "the source must be row-major")
    if dst_side.kind not in (ROW, XOR):
        return Reject("layout", "the destination must be row-major or the LDS image")
    tile_bits = tile_rows * tile_cols * elem_bits
    if tile_rows > 0 and tile_cols > 0 and tile_bits > 8 * ASYNC_STAGE_BYTES:
        return Reject("shape", "a stage holds at most 16 KiB")
    load = plan_tiles(rows, cols, tile_rows, tile_cols, elem_bits, threads, src_side, lds_side)
    if isinstance(load, Reject):
        return load
    store = plan_tiles(rows, cols, tile_rows, tile_cols, elem_bits, threads, dst_side, lds_side)
    if isinstance(store, Reject):
        return store
    if rows == 0 or cols == 0:
        return load, store
    if threads % 64:
        return Reject("threads", "whole waves only")
    allowed = min(load.vec_bits, store.vec_bits)
    widths = [w for w in ASYNC_WIDTHS_BITS if w <= allowed]
    if not widths:
        return Reject("align", "neither 128- nor 32-bit transfers fit the rows")
    w = widths[0]
    rounds = tile_bits // (threads * w)
    if rounds not in (1, 2, 4, 8):
        return Reject("threads", "1, 2, 4 or 8 rounds per thread")
    p = Plan(rounds, threads, w // elem_bits, w)
    return p, p
