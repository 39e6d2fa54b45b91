"""Pins of oracle/fragment.py: the register fragment maps, the register-path width rule and
the register-level product, each against something other than the oracle's own formulas."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import fragment as fr
from oracle.layout import Layout
from oracle.numerics import decode
from synth import fp8_bits

KINDS = list(fr.KINDS)


def lane_groups(shape):
    """(R, H): result rows / columns per lane group and the number of lane groups."""
    m = fr.SHAPES[shape][3][0]
    return m, fr.LANES // m


def lane_product(a_img, b_img, shape):
    """One atom as the matrix unit describes its operand registers: lane l of A supplies row
    l % R, lane l of B column l % R, and for each lane group h and register element e the
    two lanes of group h hold the same K, so D[m][n] sums A[m + R h][e] · B[n + R h][e]."""
    R, H = lane_groups(shape)
    d = np.zeros((R, R))
    for m in range(R):
        for n in range(R):
            d[m, n] = sum(float(a_img[m + R * h, e]) * float(b_img[n + R * h, e])
                          for h in range(H) for e in range(a_img.shape[1]))
    return d


@pytest.mark.parametrize("kind", KINDS)
def test_map_is_a_bijection_onto_the_tile(kind):
    tr, tc, _, e = fr.KINDS[kind]
    r, c = fr.coords(kind)
    assert r.shape == c.shape == (64, e)
    assert 64 * e == tr * tc
    seen = np.zeros((tr, tc), int)
    np.add.at(seen, (r, c), 1)
    assert (seen == 1).all()


@pytest.mark.parametrize("kind", KINDS)
def test_each_lane_holds_one_run_per_register_group(kind):
    # Every lane's registers are runs of 16 bytes (8 for the K = 8 / 16 atoms, whose lanes hold
    # four 16-bit values) along one axis of the tile: the span the vector width rule can reach.
    tr, tc, bits, e = fr.KINDS[kind]
    run = min(128 // bits, e)
    r, c = fr.coords(kind)
    for lane in range(64):
        for g in range(e // run):
            rr, cc = r[lane, g * run:(g + 1) * run], c[lane, g * run:(g + 1) * run]
            along_cols = (rr == rr[0]).all() and (np.diff(cc) == 1).all()
            along_rows = (cc == cc[0]).all() and (np.diff(rr) == 1).all()
            assert along_cols != along_rows
            start = cc[0] if along_cols else rr[0]
            assert start % run == 0


@pytest.mark.parametrize("shape", list(fr.SHAPES))
def test_operand_maps_pair_k_as_the_product_needs(shape):
    # A random integer atom: the lane-by-lane sum over the paired register slots must give
    # A·B exactly.  A transposed map, a wrong K order on one side or a dropped half fails.
    ka, kb, _, (M, N, K) = fr.SHAPES[shape]
    rng = np.random.default_rng(7)
    a = rng.integers(-9, 10, size=(M, K)).astype(np.int64)
    b = rng.integers(-9, 10, size=(K, N)).astype(np.int64)
    a_img = fr.frag_load(a.reshape(-1), M, K, Layout("row"), ka)[0]
    b_img = fr.frag_load(b.reshape(-1), K, N, Layout("row"), kb)[0]
    assert np.array_equal(lane_product(a_img, b_img, shape), (a @ b).astype(float))


@pytest.mark.parametrize("kind,R", [("c32_32x32", 32), ("c32_16x16", 16)])
def test_accumulator_map_has_the_result_register_structure(kind, R):
    # The result registers: lane l holds column l % R (the lanes that supply B's column);
    # rows come in blocks of four consecutive rows, the lane groups take turns block by
    # block, and rows ascend with the register index.  Those three facts determine the map.
    r, c = fr.coords(kind)
    H = 64 // R
    for lane in range(64):
        assert (c[lane] == lane % R).all()
        rows = r[lane]
        assert (np.diff(rows) > 0).all()
        assert ((rows // 4) % H == lane // R).all()


def _fraction_dot(a, b):
    return [[sum((Fraction(float(a[i, k])) * Fraction(float(b[k, j])) for k in range(a.shape[1])),
                 Fraction(0)) for j in range(b.shape[1])] for i in range(a.shape[0])]


@pytest.mark.parametrize("shape,fmt", [("32x32x16", "f16"), ("16x16x32", "bf16"),
                                       ("32x32x64_f8", "e4m3"), ("32x32x64_f8", "e5m2")])
def test_frag_mma_ref_against_fraction_brute_force(shape, fmt):
    ka, kb, kc, (am, an, ak) = fr.SHAPES[shape]
    M, N, K = am, 2 * an, 2 * ak
    rng = np.random.default_rng(11)
    if shape.endswith("_f8"):
        a_bits = fp8_bits(rng.uniform(-4, 4, M * K), fmt)
        b_bits = fp8_bits(rng.uniform(-4, 4, K * N), fmt)
    else:
        import torch
        tdt = torch.float16 if fmt == "f16" else torch.bfloat16
        a_bits = torch.tensor(rng.uniform(-2, 2, M * K)).to(tdt).view(torch.int16).numpy().view(np.uint16)
        b_bits = torch.tensor(rng.uniform(-2, 2, K * N)).to(tdt).view(torch.int16).numpy().view(np.uint16)
    c = rng.uniform(-1, 1, M * N).astype(np.float32)
    a_img = fr.frag_load(a_bits, M, K, Layout("row"), ka)
    b_img = fr.frag_load(b_bits, K, N, Layout("row"), kb)
    c_img = fr.frag_load(c, M, N, Layout("row"), kc)
    a = decode(a_bits, fmt).reshape(M, K)
    b = decode(b_bits, fmt).reshape(K, N)
    exact = _fraction_dot(a, b)
    for beta in (0.0, 1.0):
        d_img, bound_img = fr.frag_mma_ref(a_img, b_img, c_img, M, N, K, shape, beta, fmt, fmt)
        d = fr.unpack(d_img, M, N, kc, np.float64)
        bound = fr.unpack(bound_img, M, N, kc, np.float64)
        for i in range(M):
            for j in range(N):
                want = exact[i][j] + (Fraction(float(c[i * N + j])) if beta else 0)
                assert abs(Fraction(float(d[i, j])) - want) <= Fraction(1, 2**40) * (1 + abs(want))
                assert bound[i, j] == pytest.approx(float(np.abs(a[i]) @ np.abs(b[:, j])))


def test_frag_mma_ref_beta0_ignores_c():
    ka, kb, kc, _ = fr.SHAPES["32x32x16"]
    a_bits = np.full(32 * 16, 0x3C00, np.uint16)     # 1.0 in f16
    b_bits = np.full(16 * 32, 0x4000, np.uint16)     # 2.0
    a_img = fr.frag_load(a_bits, 32, 16, Layout("row"), ka)
    b_img = fr.frag_load(b_bits, 16, 32, Layout("row"), kb)
    c_img = np.full((1, 64, 16), np.nan, np.float32)
    d_img, _ = fr.frag_mma_ref(a_img, b_img, c_img, 32, 32, 16, "32x32x16", 0.0, "f16", "f16")
    assert (d_img == 32.0).all()
    d1, _ = fr.frag_mma_ref(a_img, b_img, np.ones((1, 64, 16), np.float32), 32, 32, 16,
                            "32x32x16", 1.0, "f16", "f16")
    assert (d1 == 33.0).all()


def test_frag_mma_ref_empty_and_k0():
    kc = fr.SHAPES["16x16x32"][2]
    d, b = fr.frag_mma_ref(None, None, None, 0, 16, 32, "16x16x32", 0.0, "f16", "f16")
    assert d.shape == (0, 64, 4)
    c = np.arange(16 * 16, dtype=np.float32)
    c_img = fr.frag_load(c, 16, 16, Layout("row"), kc)
    d, b = fr.frag_mma_ref(None, None, c_img, 16, 16, 0, "16x16x32", 1.0, "bf16", "bf16")
    assert np.array_equal(fr.unpack(d, 16, 16, kc, np.float64).reshape(-1), c)
    assert (b == 0).all()


def test_select_mma_widest_first():
    assert fr.select_mma(64, 64, 64, "f16", "f16") == "32x32x16"
    assert fr.select_mma(16, 16, 64, "bf16", "bf16") == "16x16x32"     # M, N only 16-divisible
    assert fr.select_mma(32, 64, 24, "f16", "f16") == "32x32x8"         # K % 16 == 8: the k8 atom
    assert fr.select_mma(48, 16, 16, "f16", "f16") == "16x16x16"
    assert fr.select_mma(16, 8, 16, "f16", "f16") is None                # N = 8 fits no atom
    assert fr.select_mma(32, 32, 8, "f16", "bf16") is None               # mixed 16-bit formats
    assert fr.select_mma(32, 32, 128, "e4m3", "e5m2") == "32x32x64_f8"
    assert fr.select_mma(32, 32, 32, "e4m3", "e4m3") is None


def test_candidates_are_ordered_by_width_and_the_first_fit_wins():
    macs = [int(np.prod(fr.SHAPES[s][3])) for s in fr.CANDIDATES_16]
    assert macs == sorted(macs, reverse=True)
    for M in (16, 32, 48, 64):
        for N in (16, 32, 48):
            for K in (8, 16, 24, 32, 48, 64):
                got = fr.select_mma(M, N, K, "f16", "f16")
                fits = [s for s in fr.CANDIDATES_16
                        if all(x % a == 0 for x, a in zip((M, N, K), fr.SHAPES[s][3]))]
                assert got == (fits[0] if fits else None)


@pytest.mark.parametrize("args,why", [
    ((16, 32, 16, "32x32x16", "f16", "f16", 0.0), "extent"),
    ((32, 32, 8, "32x32x16", "f16", "f16", 0.0), "extent"),
    ((32, 32, 32, "32x32x64_f8", "e4m3", "e4m3", 0.0), "extent"),
    ((32, 32, 16, "32x32x16", "f16", "bf16", 0.0), "dtype"),
    ((32, 32, 16, "32x32x16", "e4m3", "e4m3", 0.0), "dtype"),
    ((32, 32, 64, "32x32x64_f8", "f16", "f16", 0.0), "dtype"),
    ((16, 16, 32, "16x16x32", "f16", "f16", 0.5), "beta"),
    ((16, 16, 32, "8x8x8", "f16", "f16", 0.0), "shape"),
])
def test_accepts_mma_rejections(args, why):
    assert fr.accepts_mma(*args) == (False, why)
    assert fr.accepts_mma(32, 32, 64, "32x32x64_f8", "e5m2", "e4m3", 1.0) == (True, "ok")


# ---- the register path's vector width ---------------------------------------------------------

@pytest.mark.parametrize("kind,rows,cols,layout,base,want", [
    ("a16_32x32x16", 64, 32, Layout("row"), 0, 8),          # 16 contiguous bytes per lane
    ("a16_32x32x16", 64, 32, Layout("col"), 0, 1),          # the run crosses memory lines
    ("a16_32x32x16", 64, 32, Layout("row", ld=36), 0, 4),   # 72-byte lines: 8-byte aligned
    ("a16_32x32x16", 64, 32, Layout("row", ld=34), 0, 2),   # 68-byte lines: 4-byte aligned
    ("a16_32x32x16", 64, 32, Layout("row", ld=33), 0, 1),   # 66-byte lines
    ("a16_32x32x16", 64, 32, Layout("row"), 2, 1),          # base off by one element
    ("a16_32x32x16", 64, 32, Layout("row"), 8, 4),          # base 8-byte aligned only
    ("b16_32x32x16", 32, 64, Layout("col"), 0, 8),
    ("b16_32x32x16", 32, 64, Layout("row"), 0, 1),
    ("a16_16x16x32", 32, 64, Layout("row"), 0, 8),
    ("b16_16x16x32", 64, 32, Layout("col", ld=68), 0, 4),  # 136-byte lines: 8-byte aligned
    ("b16_16x16x32", 64, 32, Layout("col", ld=66), 0, 2),  # 132-byte lines: 4-byte aligned
    ("a8_32x32x64", 32, 128, Layout("row"), 0, 16),
    ("a8_32x32x64", 32, 128, Layout("row", ld=136), 0, 8),
    ("a8_32x32x64", 32, 128, Layout("col"), 0, 1),
    ("b8_32x32x64", 64, 64, Layout("col"), 0, 16),
    ("b8_32x32x64", 64, 64, Layout("col"), 4, 4),
    ("c32_32x32", 64, 64, Layout("col"), 0, 4),
    ("c32_32x32", 64, 64, Layout("row"), 0, 1),
    ("c32_32x32", 64, 64, Layout("col", ld=66), 0, 2),
    ("c32_16x16", 32, 32, Layout("col", ld=33), 0, 1),
])
def test_reg_vec_hand_derived(kind, rows, cols, layout, base, want):
    assert fr.reg_vec(kind, rows, cols, layout, base_addr=base) == want


def _brute_vec(kind, rows, cols, layout, base):
    # Independent of element_offsets: a memory filled with its own byte addresses, read
    # back through the register map, and each candidate width tested on the addresses.
    tr, tc, bits, e = fr.KINDS[kind]
    eb = bits // 8
    ld = layout.eff_ld(rows, cols)
    addr = {}
    for i in range(rows):
        for j in range(cols):
            off = i * ld + j if layout.kind == "row" else j * ld + i
            addr[(i, j)] = base + eb * off
    r, c = fr.coords(kind)
    for vb in (16, 8, 4, 2, 1):
        if vb < eb or (vb // eb) > e:       # a transfer never spans more than a lane's registers
            continue
        v = vb // eb
        ok = True
        for ti in range(rows // tr):
            for tj in range(cols // tc):
                for lane in range(64):
                    for s in range(0, e, v):
                        a = [addr[(ti * tr + r[lane, s + u], tj * tc + c[lane, s + u])] for u in range(v)]
                        ok &= a[0] % vb == 0 and all(a[u] == a[0] + u * eb for u in range(v))
        if ok:
            return v
    raise AssertionError("no width")


@pytest.mark.parametrize("kind", KINDS)
def test_reg_vec_against_brute_force_addresses(kind):
    tr, tc, bits, _ = fr.KINDS[kind]
    eb = bits // 8
    rng = np.random.default_rng(5)
    for _ in range(6):
        rows, cols = tr * int(rng.integers(1, 3)), tc * int(rng.integers(1, 3))
        lk = "row" if rng.integers(2) else "col"
        minld = cols if lk == "row" else rows
        ld = minld + int(rng.integers(0, 9))
        base = eb * int(rng.integers(0, 9))
        lay = Layout(lk, ld=ld)
        assert fr.reg_vec(kind, rows, cols, lay, base) == _brute_vec(kind, rows, cols, lay, base)


# ---- load / store ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("lk", ["row", "col"])
def test_load_then_store_round_trip_keeps_padding(kind, lk):
    tr, tc, _, e = fr.KINDS[kind]
    rows, cols = 2 * tr, 3 * tc
    ld = (cols if lk == "row" else rows) + 5
    lay = Layout(lk, ld=ld)
    size = ld * ((rows if lk == "row" else cols) - 1) + (cols if lk == "row" else rows)
    mem = np.arange(size, dtype=np.int64) * 7 + 3
    img = fr.frag_load(mem, rows, cols, lay, kind)
    assert img.shape == (6, 64, e)
    # tile order is row-major over tiles; within a tile the map decides
    r, c = fr.coords(kind)
    t = 1 * 3 + 2                                          # tile (1, 2)
    i, j = tr + r, 2 * tc + c
    want = mem[i * ld + j] if lk == "row" else mem[j * ld + i]
    assert np.array_equal(img[t], want)
    blank = np.full(size, -1, np.int64)
    back = fr.frag_store(img, blank, rows, cols, lay, kind)
    touched = back != -1
    assert np.array_equal(back[touched], mem[touched])
    assert touched.sum() == rows * cols                   # padding left alone


def test_tiles_reject_ragged_matrices():
    with pytest.raises(ValueError):
        fr.tiles("a16_32x32x16", 48, 16)
    with pytest.raises(ValueError):
        fr.frag_load(np.zeros(64 * 8), 32, 8, Layout("row"), "a16_32x32x16")


# ---- planted mistakes: each must trip one of the pins above ------------------------------------

def _mutant(kind, how):
    good = fr.coords

    def coords(k):
        r, c = good(k)
        if k != kind:
            return r, c
        lane = np.arange(64)[:, None] + 0 * r
        e = np.arange(r.shape[1])[None, :] + 0 * r
        if how == "k_reversed":              # one operand's K runs backwards inside a lane
            return (r, c.max() - c) if kind.startswith("a") else (r.max() - r, c)
        if how == "halves_swapped":          # lane halves hold the other half's K
            return (r, (c + r.shape[1]) % (c.max() + 1)) if kind.startswith("a") else \
                ((r + r.shape[1]) % (r.max() + 1), c)
        if how == "transposed":              # rows and columns exchanged (square tiles only)
            return c, r
        if how == "block_order":             # fp8: 32-K blocks not interleaved by lane half
            return (r, 16 * (e // 16) * 0 + 32 * (lane // 32) + e) if kind.startswith("a") else \
                (32 * (lane // 32) + e, c)
        if how == "rows_by_lane_half":       # accumulator: halves hold rows 0-15 / 16-31
            return 16 * (lane // 32) + e, c
        raise AssertionError(how)
    return coords


def _pins_fail(monkeypatch, kind, how):
    monkeypatch.setattr(fr, "coords", _mutant(kind, how))
    checks = []
    for shape, (ka, kb, kc, _) in fr.SHAPES.items():
        if kind in (ka, kb):
            checks.append(lambda s=shape: test_operand_maps_pair_k_as_the_product_needs(s))
    if kind.startswith("c"):
        checks.append(lambda: test_accumulator_map_has_the_result_register_structure(
            kind, 32 if kind == "c32_32x32" else 16))
    checks.append(lambda: test_map_is_a_bijection_onto_the_tile(kind))
    failed = 0
    for check in checks:
        try:
            check()
        except (AssertionError, IndexError):
            failed += 1
    return failed


@pytest.mark.parametrize("kind,how", [
    ("a16_32x32x16", "k_reversed"), ("b16_16x16x32", "k_reversed"), ("b8_32x32x64", "k_reversed"),
    ("a16_16x16x32", "halves_swapped"), ("b16_32x32x16", "halves_swapped"),
    ("c32_32x32", "transposed"), ("c32_16x16", "transposed"),
    ("a16_32x32x8", "k_reversed"), ("b16_16x16x16", "halves_swapped"),
    ("a8_32x32x64", "block_order"), ("b8_32x32x64", "block_order"),
    ("c32_32x32", "rows_by_lane_half"),
])
def test_planted_map_mistakes_are_caught(monkeypatch, kind, how):
    assert _pins_fail(monkeypatch, kind, how) >= 1


# ---- the register-level GEMM's atom choice (select_gemm_atom) ------------------------------

def test_gemm_atom_page_cases():
    from oracle.fragment import select_gemm_atom as sel
    # the 16x8x16 atom of the page: N pads to 16 and the 16x16x16 atom does no other padding
    assert sel(16, 8, 16, "f16", False, False) == "16x16x16"
    # K = 8 and K = 24 ([SYNC-GEMM] test coverage): only the 8-deep atom takes K whole
    assert sel(16, 8, 8, "f16", False, False) == "32x32x8"
    assert sel(32, 16, 24, "bf16", False, True) == "32x32x8"
    # K = 32 on a 16x16 output: the 16x16x32 atom (one load per operand per 8192 MACs) beats
    # 16x16x16 at the same work
    assert sel(16, 16, 32, "f16", False, False) == "16x16x32"
    # whole 32x32 tiles: every atom does the same work; 32x32x16 has the fewest loads per MAC
    assert sel(64, 64, 64, "bf16", False, True) == "32x32x16"
    # stored transposed, a lane's K run is one load per element: the 8-deep 32x32 atom issues
    # as many loads per MAC as 32x32x16 and the wider one wins the tie
    assert sel(64, 64, 64, "bf16", True, False) == "32x32x16"
    assert sel(16, 16, 0, "f16", False, False) is None
    assert sel(16, 16, 16, "e4m3", False, False) is None


def test_gemm_atom_brute_force_minimum():
    # brute force over small problems: the chosen atom takes K whole, does the least padded work
    # of all atoms that take K whole, and no cheaper-to-load atom does the same work
    from itertools import product
    from oracle.fragment import CANDIDATES_16, SHAPES, gemm_atom_loads, select_gemm_atom as sel
    for M, N, K, ta, tb in product((16, 32, 48, 64), (8, 16, 24, 40, 64), (8, 16, 24, 32, 48, 64),
                                   (False, True), (False, True)):
        got = sel(M, N, K, "f16", ta, tb)
        am, an, ak = SHAPES[got][3]
        assert K % ak == 0
        work = lambda s: (-(-M // SHAPES[s][3][0]) * SHAPES[s][3][0]) * \
            (-(-N // SHAPES[s][3][1]) * SHAPES[s][3][1]) * K
        lpm = lambda s: gemm_atom_loads(s, ta, tb) / np.prod(SHAPES[s][3])
        ok = [s for s in CANDIDATES_16 if K % SHAPES[s][3][2] == 0]
        assert work(got) == min(work(s) for s in ok), (M, N, K, got)
        assert all(lpm(got) <= lpm(s) for s in ok if work(s) == work(got)), (M, N, K, ta, tb, got)


def test_gemm_atom_load_counts():
    from oracle.fragment import gemm_atom_loads
    # K-major A and B: one vector load each, whatever the atom
    assert gemm_atom_loads("32x32x16", False, True) == 2
    assert gemm_atom_loads("16x16x16", False, True) == 2
    # A stored [K, M]: its 8 (or 4) K values per lane are 8 (4) loads; B [K, N] likewise
    assert gemm_atom_loads("16x16x32", True, True) == 9
    assert gemm_atom_loads("32x32x8", True, False) == 8


def test_gemm_atom_layout_term_never_reverses_width():
    # For the four 16-bit shapes a wider atom never issues more loads per multiply-add, in any
    # stored orientation: the layout term only separates ties that width already orders, so the
    # choice is the same for all four (transA, transB).  (The term is kept because it is the
    # page's criterion; this pin records that it does not bite for these candidates.)
    from itertools import product
    from oracle.fragment import CANDIDATES_16, SHAPES, gemm_atom_loads, select_gemm_atom as sel
    for ta, tb in product((False, True), (False, True)):
        lpm = [gemm_atom_loads(s, ta, tb) / np.prod(SHAPES[s][3]) for s in CANDIDATES_16]
        macs = [np.prod(SHAPES[s][3]) for s in CANDIDATES_16]
        for i in range(4):
            for j in range(4):
                if macs[i] > macs[j]:
                    assert lpm[i] <= lpm[j]
    for M, N, K in product((16, 32, 48, 64), (8, 16, 24, 40, 64), (8, 16, 24, 32, 48, 64)):
        assert len({sel(M, N, K, "bf16", ta, tb) for ta in (False, True) for tb in (False, True)}) == 1
