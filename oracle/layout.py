"""Element offsets of the layouts a tile copy moves between (oracle; test infrastructure).

A layout maps a logical (row, col) of a rows x cols region to an element offset
in a flat buffer:

* "row":  base + row·ld + col   (ld defaults to cols)
* "col":  base + col·ld + row   (ld defaults to rows)
* "xor":  the XOR-swizzled tile layout.  The tile is row-major and packed; each
  row is cut into 16-byte chunks and the chunk index is XOR-ed with the low bits
  of the row index:  phys_chunk = chunk XOR (row mod P), P = min(8, chunks/row).

The "xor" layout is our reading of the swizzle family of [TCGEN05-CP], 调度算法
step 2 (the hardware form that XORs the masked high address bits, shifted down by
the atom length, into the low bits), specialised to 16-byte atoms: for a tile
whose rows are 128 bytes, phys = x XOR ((x AND 0x380) >> 3) on the byte offset x,
i.e. chunk bits 4..6 XOR row bits 7..9, a period of 8 rows = 1 KiB.  [VEC-AUTO]
"swizzled shared 布局" fixes that the low bits inside one chunk are never
swizzled, so a vector transfer must stay inside one chunk.  For other row widths
the same chunk-XOR-row rule is applied with P = min(8, chunks per row); the row
must be a whole power-of-two number of 16-byte chunks.

Pinned by tests/test_oracle_copy.py: brute-force bijection of "xor" over tiles,
involution, chunk contiguity, and agreement with the byte-address form above for
128-byte rows.
"""

import numpy as np

ROW, COL, XOR = "row", "col", "xor"
CHUNK_BYTES = 16


class Layout:
    """kind in {"row", "col", "xor"}; ld in elements (0 = packed); base = element offset."""

    def __init__(self, kind=ROW, ld=0, base=0):
        if kind not in (ROW, COL, XOR):
            raise ValueError(f"oracle: unknown layout kind {kind!r}")
        self.kind, self.ld, self.base = kind, int(ld), int(base)

    def __repr__(self):
        return f"Layout({self.kind!r}, ld={self.ld}, base={self.base})"

    def eff_ld(self, rows, cols):
        if self.ld:
            return self.ld
        return rows if self.kind == COL else cols


def xor_defined(cols, elem_bytes):
    """True when a rows x cols tile of elem_bytes elements admits the "xor" layout."""
    row_bytes = cols * elem_bytes
    if row_bytes % CHUNK_BYTES:
        return False
    chunks = row_bytes // CHUNK_BYTES
    return chunks > 0 and (chunks & (chunks - 1)) == 0


def xor_offset(r, c, cols, elem_bytes):
    """Element offset of logical (r, c) in the XOR-swizzled packed tile."""
    ce = CHUNK_BYTES // elem_bytes           # elements per 16-byte chunk
    chunks = cols // ce
    period = min(8, chunks)
    r = np.asarray(r, dtype=np.int64)
    c = np.asarray(c, dtype=np.int64)
    phys_chunk = (c // ce) ^ (r % period)
    return r * cols + phys_chunk * ce + c % ce


def offsets(layout, rows, cols, elem_bytes):
    """(rows, cols) int64 array of element offsets for every logical (r, c)."""
    r = np.arange(rows, dtype=np.int64)[:, None]
    c = np.arange(cols, dtype=np.int64)[None, :]
    ld = layout.eff_ld(rows, cols)
    if layout.kind == ROW:
        off = r * ld + c
    elif layout.kind == COL:
        off = c * ld + r
    else:
        if layout.ld not in (0, cols):
            raise ValueError("oracle: the xor layout is packed (ld == cols)")
        if not xor_defined(cols, elem_bytes):
            raise ValueError("oracle: xor layout needs rows of a power-of-two count of 16-byte chunks")
        off = xor_offset(r, c, cols, elem_bytes)
    return layout.base + off


def extent(layout, rows, cols, elem_bytes):
    """Number of elements a buffer needs to hold the region (max offset + 1)."""
    if rows == 0 or cols == 0:
        return layout.base
    return int(offsets(layout, rows, cols, elem_bytes).max()) + 1
