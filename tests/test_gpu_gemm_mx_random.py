"""Seeded random block-scaled GEMM problems with 6- and 4-bit operands ([SYNC-GEMM] 七: fp4
operands with SFA / SFB block scales) across every kernel the planner can choose for them —
the direct-load kernel for e2m1 x e2m1 (K % 256 == 0) and for 6-bit pairs, the packed kernel
for the rest, 128- and 256-wide blocks, whole and ragged — each checked element by element
against the oracle with the fp8 bar."""

import numpy as np
import pytest

import synth
import tile_level_gemm_amd as tg
from tests.gpu_util import say
from tests.test_gpu_gemm_mx_small import FMT, full_check

A_ADDR, B_ADDR, D_ADDR = 0x100000, 0x40000000, 0xC0000000

# size classes: (M units of 16, N units of 16, K units of 128) ranges
CLASSES = [((1, 16), (1, 16), (1, 8)),          # a few 128-wide blocks
           ((32, 96), (32, 96), (1, 6)),        # many 128-wide blocks
           ((256, 272), (256, 272), (1, 3))]    # 256-wide blocks
N_CASES = 24
TYPES = ["e2m1", "e2m3", "e3m2"]


def cases():
    g = synth.rng(20261203)
    out = []
    for i in range(N_CASES):
        (m0, m1), (n0, n1), (k0, k1) = CLASSES[i % len(CLASSES)]
        M = 16 * int(g.integers(m0, m1 + 1))
        N = 16 * int(g.integers(n0, n1 + 1))
        K = 128 * int(g.integers(k0, k1 + 1))
        af, bf = TYPES[int(g.integers(0, 3))], TYPES[int(g.integers(0, 3))]
        if i % 4 == 0:
            af = bf = "e2m1"      # keep the e2m1 pair frequent: its route depends on K
            if i % 8 == 0:
                K = 256 * ((K + 255) // 256)
        beta = float(g.integers(0, 2))
        dist = "codes" if g.integers(0, 2) else "normal"
        out.append((M, N, K, af, bf, beta, dist, 300 + i))
    return out


CASES = cases()


def plan_of(M, N, K, af, bf, beta):
    return tg.tile_gemm_mx_plan(A_ADDR, B_ADDR, A_ADDR + (1 << 28), B_ADDR + (1 << 28),
                                0x80000000 if beta else None, D_ADDR, M, N, K, 0, 1, beta,
                                FMT[af], FMT[bf])


def test_random_cases_cover_every_kernel_path():
    # host only: the planner's choices over the cases include each configuration
    seen = set()
    for M, N, K, af, bf, beta, _, _ in CASES:
        p = plan_of(M, N, K, af, bf, beta)
        seen.add((p.block_m, p.block_k, p.loader, p.bounds_checked))
    want = {(128, 256, 1, 1), (256, 256, 1, 1),      # e2m1 x e2m1, direct
            (128, 128, 1, 1), (256, 128, 1, 1),      # 6-bit pairs, direct
            (128, 128, 0, 1), (256, 128, 0, 1)}      # packed kernel
    assert want <= seen, sorted(seen)


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K,af,bf,beta,dist,seed", CASES)
def test_random_problem(M, N, K, af, bf, beta, dist, seed):
    p = plan_of(M, N, K, af, bf, beta)
    say(f"gemm_mx random {M}x{N}x{K} {af} x {bf} beta={beta} {dist} (block {p.block_m}, "
        f"loader {p.loader}, block_k {p.block_k})")
    full_check(M, N, K, af, bf, beta, seed, dist=dist)
