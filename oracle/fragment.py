"""Register-side copies: matrix <-> MFMA fragment registers (oracle; test infrastructure).

[VEC-AUTO] (opening section and closing reading list): the copy primitive moves data between
global, shared and register (local) storage; vec_auto's second path is the register path,
whose partition is induced by the register layout's thread axis, and the ldstmatrix variant
moves warp-collective matrix fragments.  On gfx950 the register layouts that matter are
the matrix cores' operand and accumulator fragments.  A fragment kind is a tile of
rows x cols and a map (lane, register element) -> (row, col) of the tile; a matrix of whole
tiles is copied tile by tile (row-major tile order), and a tile's register image is
[64 lanes][E elements], each lane's elements contiguous as they sit in its VGPRs.

Readings:
* Kinds and maps (wave64, e is the register element index):
    a16_32x32x16  32 x 16   16-bit  e < 8   (l % 32, 8 (l / 32) + e)
    b16_32x32x16  16 x 32   16-bit  e < 8   (8 (l / 32) + e, l % 32)
    a16_16x16x32  16 x 32   16-bit  e < 8   (l % 16, 8 (l / 16) + e)
    b16_16x16x32  32 x 16   16-bit  e < 8   (8 (l / 16) + e, l % 16)
    a8_32x32x64   32 x 64   8-bit   e < 32  (l % 32, 32 (e / 16) + 16 (l / 32) + e % 16)
    b8_32x32x64   64 x 32   8-bit   e < 32  (32 (e / 16) + 16 (l / 32) + e % 16, l % 32)
    a16_32x32x8   32 x 8    16-bit  e < 4   (l % 32, 4 (l / 32) + e)
    b16_32x32x8   8 x 32    16-bit  e < 4   (4 (l / 32) + e, l % 32)
    a16_16x16x16  16 x 16   16-bit  e < 4   (l % 16, 4 (l / 16) + e)
    b16_16x16x16  16 x 16   16-bit  e < 4   (4 (l / 16) + e, l % 16)
    c32_32x32     32 x 32   32-bit  e < 16  (8 (e / 4) + 4 (l / 32) + e % 4, l % 32)
    c32_16x16     16 x 16   32-bit  e < 4   (4 (l / 16) + e, l % 16)
  (the A / B maps pair A row m with B column n over the same K per register element, as the
  MFMA sums; the 8-bit K order follows the unit's 32-K blocks).
* The register path's vector width: the widest v in {128, 64, 32, 16, 8} bits (v elements a
  power of two dividing E) such that every aligned run of v consecutive register elements of
  every lane of every tile is contiguous in memory and starts on a v-element boundary of the
  absolute address — the page's width rule with the register layout as the driving side.
* Atom selection: the widest shape (most multiply-adds per instruction) whose atom divides
  (M, N, K), tried in a fixed candidate order (select_mma).

* The register-level product ([SYNC-GEMM] 一 and 四: A / B fragments and the C / D
  accumulator live in registers, the caller loads the fragments first, and each output tile
  accumulates one matrix instruction per K atom in place): frag_mma_ref unpacks the images to
  matrices, forms D = A·B (+ C) in float64 from the decoded operands, and packs D with the
  accumulator map.

Pinned by tests/test_oracle_fragment.py: each map is a bijection onto its tile; the A and B
maps of each matrix-instruction shape pair the same K in the same (lane half, element) slot,
so the lane-by-lane sum over those slots equals the matrix product (checked against matmul
and against Fraction brute force); the accumulator maps against the quad and column
structure of the result registers; the width rule against brute force over addresses and
hand-derived cases; load / store round trips and untouched elements outside the matrix.
"""

import numpy as np

from .gemm import logical_operands
from .layout import COL, ROW, Layout

# kind -> (tile rows, tile cols, element bits, elements per lane)
KINDS = {
    "a16_32x32x16": (32, 16, 16, 8),
    "b16_32x32x16": (16, 32, 16, 8),
    "a16_16x16x32": (16, 32, 16, 8),
    "b16_16x16x32": (32, 16, 16, 8),
    "a8_32x32x64": (32, 64, 8, 32),
    "b8_32x32x64": (64, 32, 8, 32),
    "a16_32x32x8": (32, 8, 16, 4),
    "b16_32x32x8": (8, 32, 16, 4),
    "a16_16x16x16": (16, 16, 16, 4),
    "b16_16x16x16": (16, 16, 16, 4),
    "c32_32x32": (32, 32, 32, 16),
    "c32_16x16": (16, 16, 32, 4),
}

LANES = 64


def coords(kind):
    """(rows, cols) int arrays [64, E]: the tile coordinate of lane l's register element e."""
    tr, tc, _, E = KINDS[kind]
    l = np.arange(LANES)[:, None]
    e = np.arange(E)[None, :]
    if kind == "a16_32x32x16":
        r, c = l % 32 + 0 * e, 8 * (l // 32) + e
    elif kind == "b16_32x32x16":
        r, c = 8 * (l // 32) + e, l % 32 + 0 * e
    elif kind == "a16_16x16x32":
        r, c = l % 16 + 0 * e, 8 * (l // 16) + e
    elif kind == "b16_16x16x32":
        r, c = 8 * (l // 16) + e, l % 16 + 0 * e
    elif kind == "a8_32x32x64":
        r, c = l % 32 + 0 * e, 32 * (e // 16) + 16 * (l // 32) + e % 16
    elif kind == "b8_32x32x64":
        r, c = 32 * (e // 16) + 16 * (l // 32) + e % 16, l % 32 + 0 * e
    elif kind == "a16_32x32x8":
        r, c = l % 32 + 0 * e, 4 * (l // 32) + e
    elif kind == "b16_32x32x8":
        r, c = 4 * (l // 32) + e, l % 32 + 0 * e
    elif kind == "a16_16x16x16":
        r, c = l % 16 + 0 * e, 4 * (l // 16) + e
    elif kind == "b16_16x16x16":
        r, c = 4 * (l // 16) + e, l % 16 + 0 * e
    elif kind == "c32_32x32":
        r, c = 8 * (e // 4) + 4 * (l // 32) + e % 4, l % 32 + 0 * e
    elif kind == "c32_16x16":
        r, c = 4 * (l // 16) + e, l % 16 + 0 * e
    else:
        raise ValueError(f"oracle: unknown fragment kind {kind!r}")
    return np.broadcast_to(r, (LANES, E)).copy(), np.broadcast_to(c, (LANES, E)).copy()


def tiles(kind, rows, cols):
    """Tile origins (row-major tile order) of a rows x cols matrix of whole tiles."""
    tr, tc, _, _ = KINDS[kind]
    if rows % tr or cols % tc:
        raise ValueError("oracle: the matrix is not a whole number of fragment tiles")
    return [(i * tr, j * tc) for i in range(rows // tr) for j in range(cols // tc)]


def element_offsets(kind, rows, cols, layout):
    """[tiles, 64, E] element offsets (from the matrix base) of every register element."""
    r, c = coords(kind)
    ld = layout.eff_ld(rows, cols)
    out = []
    for (r0, c0) in tiles(kind, rows, cols):
        rr, cc = r + r0, c + c0
        if layout.kind == ROW:
            out.append(rr * ld + cc + layout.base)
        elif layout.kind == COL:
            out.append(cc * ld + rr + layout.base)
        else:
            raise ValueError("oracle: register copies take row- or column-major memory")
    return np.asarray(out, dtype=np.int64).reshape(-1, LANES, KINDS[kind][3])


def frag_load(mem, rows, cols, layout, kind):
    """Register image [tiles, 64, E] of a matrix held in `mem` (a flat array of bit patterns)."""
    return np.asarray(mem)[element_offsets(kind, rows, cols, layout)]


def frag_store(image, mem, rows, cols, layout, kind):
    """Write a register image back into `mem` (a copy is returned; other elements kept)."""
    out = np.array(mem, copy=True)
    off = element_offsets(kind, rows, cols, layout)
    out[off.reshape(-1)] = np.asarray(image).reshape(-1)
    return out


def reg_vec(kind, rows, cols, layout, base_addr=0):
    """Vector width (elements) of the register path, by the widest-first rule.

    base_addr: byte address of the matrix base (element 0), for the alignment test."""
    _, _, bits, E = KINDS[kind]
    eb = bits // 8
    off = element_offsets(kind, rows, cols, layout) if rows and cols else None
    for vbits in (128, 64, 32, 16, 8):
        if vbits < bits or vbits % bits:
            continue
        v = vbits // bits
        if E % v:
            continue
        if off is None:
            return v
        runs = off.reshape(off.shape[0], LANES, E // v, v)
        contiguous = np.all(np.diff(runs, axis=3) == 1)
        aligned = np.all(((base_addr + runs[..., 0] * eb) % (v * eb)) == 0)
        if contiguous and aligned:
            return v
    return 1


# matrix-instruction shape -> (A kind, B kind, accumulator kind, (M, N, K) of one atom)
SHAPES = {
    "32x32x16": ("a16_32x32x16", "b16_32x32x16", "c32_32x32", (32, 32, 16)),
    "16x16x32": ("a16_16x16x32", "b16_16x16x32", "c32_16x16", (16, 16, 32)),
    "32x32x64_f8": ("a8_32x32x64", "b8_32x32x64", "c32_32x32", (32, 32, 64)),
    "32x32x8": ("a16_32x32x8", "b16_32x32x8", "c32_32x32", (32, 32, 8)),
    "16x16x16": ("a16_16x16x16", "b16_16x16x16", "c32_16x16", (16, 16, 16)),
}

# Widest first ([TCGEN05-CP] 形状选择: candidates are tried from the widest atom down and the
# first that fits wins; [SYNC-GEMM] 二: the k16 atom when K allows it, else k8).  "Widest" is
# the multiply-adds one instruction performs; at equal width the longer K comes first (fewer
# accumulator passes over the same output).  The 8-bit formats have the one shape.
CANDIDATES_16 = ("32x32x16", "16x16x32", "32x32x8", "16x16x16")
CANDIDATES_8 = ("32x32x64_f8",)


def select_mma(M, N, K, a_fmt, b_fmt):
    """The widest shape whose atom divides (M, N, K) exactly, or None."""
    fp8 = a_fmt in ("e4m3", "e5m2")
    for shape in (CANDIDATES_8 if fp8 else CANDIDATES_16):
        if accepts_mma(M, N, K, shape, a_fmt, b_fmt, 0.0)[0]:
            return shape
    return None


def gemm_atom_loads(shape, trans_a, trans_b):
    """Global load instructions one lane issues per atom step for its A and B fragments.

    A lane's fragment is a run of K values of one row of A (one column of B).  Stored
    K-contiguous (A with trans_a false, B with trans_b true) the run is one vector load; stored
    M- or N-contiguous the run crosses memory lines, one load per element."""
    run = KINDS[SHAPES[shape][0]][3]          # K elements per lane
    a = 1 if not trans_a else run
    b = 1 if trans_b else run
    return a + b


def select_gemm_atom(M, N, K, fmt, trans_a, trans_b):
    """The matrix instruction of the register-level GEMM for a whole problem, or None.

    Readings of [TCGEN05-CP] 形状选择 (candidates from the widest atom down, each tested against
    the operands' layouts) and [SYNC-GEMM] 二 (the k16 atom when K allows it, else k8):
      * an atom is admissible when its K depth divides K: the K of an atom is never padded;
      * M and N are padded up to the atom (no matrix instruction has an 8-wide N; padded rows
        and columns are zero and never stored);
      * the admissible atom with the least padded work (multiply-adds after padding) wins;
      * ties go to the fewest global load instructions per multiply-add for the operands'
        stored layouts (gemm_atom_loads), then to the earlier candidate (the wider atom).
    For these four candidates a wider atom never needs more loads per multiply-add, so the
    layout term never reverses the order that width gives (tests pin this).
    """
    if fmt not in ("f16", "bf16") or min(M, N, K) <= 0:
        return None
    best, best_key = None, None
    for order, shape in enumerate(CANDIDATES_16):
        am, an, ak = SHAPES[shape][3]
        if K % ak:
            continue
        work = (-(-M // am) * am) * (-(-N // an) * an) * K
        loads_per_mac = gemm_atom_loads(shape, trans_a, trans_b) / (am * an * ak)
        key = (work, loads_per_mac, order)
        if best_key is None or key < best_key:
            best, best_key = shape, key
    return best


def unpack(image, rows, cols, kind, dtype):
    """The packed row-major rows x cols matrix a register image holds."""
    mem = np.zeros(rows * cols, dtype=dtype)
    return frag_store(image, mem, rows, cols, Layout(ROW), kind).reshape(rows, cols)


def accepts_mma(M, N, K, shape, a_fmt, b_fmt, beta):
    """Acceptance of the register-level product: whole atoms, one operand format pair the
    instruction takes, beta 0 or 1 (alpha is 1).  Returns (ok, category)."""
    if shape not in SHAPES:
        return False, "shape"
    am, an, ak = SHAPES[shape][3]
    if min(M, N, K) < 0 or M % am or N % an or K % ak:
        return False, "extent"
    fmts = ("e4m3", "e5m2") if shape.endswith("_f8") else ("f16", "bf16")
    if a_fmt not in fmts or b_fmt not in fmts or (not shape.endswith("_f8") and a_fmt != b_fmt):
        return False, "dtype"
    if beta not in (0.0, 1.0):
        return False, "beta"
    return True, "ok"


def frag_mma_ref(a_img, b_img, c_img, M, N, K, shape, beta, a_fmt, b_fmt):
    """D image and bound image of D = A·B (+ C when beta == 1) over register images.

    a_img: A [M, K] in the shape's A map (bit patterns), b_img: B [K, N] in its B map,
    c_img: C [M, N] in the accumulator map (float32; not read when beta == 0).
    Returns (d_img, bound_img): float64 images in the accumulator map, the bound being
    sum_k |A_ik B_kj| per output."""
    ok, why = accepts_mma(M, N, K, shape, a_fmt, b_fmt, beta)
    if not ok:
        raise ValueError(f"oracle: call rejected ({why})")
    ka, kb, kc, _ = SHAPES[shape]
    if not (M and N):
        e = KINDS[kc][3]
        return np.zeros((0, LANES, e)), np.zeros((0, LANES, e))
    bits = np.uint8 if shape.endswith("_f8") else np.uint16
    a_bits = unpack(a_img, M, K, ka, bits) if K else np.zeros((M, 0), bits)
    b_bits = unpack(b_img, K, N, kb, bits) if K else np.zeros((0, N), bits)
    a, b = logical_operands(a_bits, b_bits, M, N, K, 0, 0, a_fmt, b_fmt)
    d = np.matmul(a, b) if K else np.zeros((M, N))
    bound = np.matmul(np.abs(a), np.abs(b)) if K else np.zeros((M, N))
    if beta == 1.0:
        d = d + unpack(c_img, M, N, kc, np.float32).astype(np.float64)
    flat = Layout(ROW)
    return frag_load(d.reshape(-1), M, N, flat, kc), frag_load(bound.reshape(-1), M, N, flat, kc)
