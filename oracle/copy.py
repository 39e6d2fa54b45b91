"""Tile copy oracle: an element-by-element bit copy between two layouts (test infrastructure).

[VEC-AUTO], opening section: copy is a synchronous element copy src -> dst; the
gate requires equal dtype and equal extents on both sides, so the copy never
converts a value.  The expected destination image is rebuilt from the
destination layout alone and compared bit for bit, the method of [TCGEN05-CP]
测试矩阵 (its round-trip checks rebuild the expected value on the host from the
destination layout and compare bitwise).

The oracle works on raw unsigned integer views (uint8 / uint16 / uint32), never
on floats, so NaN payloads, -0 and subnormals survive.

Pinned by tests/test_oracle_copy.py: identity for equal layouts, a row-major ->
column-major copy equals the array transpose, a copy into "xor" and back is the
identity, untouched destination elements keep their old bits.
"""

import numpy as np

from .layout import offsets

UINT_OF_BYTES = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def copy_ref(src_mem, dst_mem, rows, cols, src_layout, dst_layout):
    """Return a new destination image with dst[off_dst(r,c)] = src[off_src(r,c)] for all (r, c).

    src_mem and dst_mem are 1-D arrays of the same unsigned integer dtype (the
    element bits).  Elements of dst_mem that no (r, c) maps to keep their bits.
    """
    src_mem = np.asarray(src_mem)
    dst_mem = np.asarray(dst_mem)
    if src_mem.dtype != dst_mem.dtype or src_mem.dtype.kind != "u":
        raise ValueError("oracle: copy operands must share one unsigned element type")
    eb = src_mem.dtype.itemsize
    out = dst_mem.copy()
    if rows == 0 or cols == 0:
        return out
    so = offsets(src_layout, rows, cols, eb)
    do = offsets(dst_layout, rows, cols, eb)
    if np.unique(do).size != do.size:
        raise ValueError("oracle: destination layout maps two elements to one offset")
    out[do.ravel()] = src_mem[so.ravel()]
    return out
