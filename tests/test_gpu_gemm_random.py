"""Seeded random GEMM problems across every kernel the planner can choose (register atom,
VGPR-staged 64/128/256 tiles, direct-load 128 and 256 blocks, whole and ragged, every
stage-count shape and partial last stages), each checked element by element against the
oracle: |D - D_ref| <= 1e-4·sum|a·b| + 1e-6."""

import numpy as np
import pytest

import synth
import tile_level_gemm_amd as tg
from tests.gpu_util import say
from tests.test_gpu_gemm import FMT, full_check

# size classes: (M units of 16, N units of 8, K units of 8) ranges
CLASSES = [((1, 8), (1, 16), (1, 8)),          # a few atoms
           ((4, 40), (8, 80), (1, 40)),        # small tiled
           ((64, 160), (128, 320), (1, 64)),   # 128-wide blocks
           ((250, 270), (500, 540), (1, 48))]  # 256-wide blocks
N_CASES = 48


def cases():
    g = synth.rng(20261202)
    out = []
    for i in range(N_CASES):
        (m0, m1), (n0, n1), (k0, k1) = CLASSES[i % len(CLASSES)]
        M = 16 * int(g.integers(m0, m1 + 1))
        N = 8 * int(g.integers(n0, n1 + 1))
        K = 8 * int(g.integers(k0, k1 + 1))
        ta, tb = bool(g.integers(0, 2)), bool(g.integers(0, 2))
        beta = float(g.integers(0, 2))
        fmt = "f16" if g.integers(0, 2) else "bf16"
        out.append((M, N, K, ta, tb, beta, fmt, 100 + i))
    return out


CASES = cases()


def plan_of(M, N, K, ta, tb, beta, fmt):
    return tg.tile_gemm_plan(0x100000, 0x40000000, 0x80000000 if beta else None, 0xC0000000,
                             M, N, K, int(ta), int(tb), beta, FMT[fmt])


def test_random_cases_cover_every_kernel_path():
    # host only: the planner's choices over the cases include each kernel configuration
    seen = set()
    for M, N, K, ta, tb, beta, fmt, _ in CASES:
        p = plan_of(M, N, K, ta, tb, beta, fmt)
        seen.add((p.kernel, p.block_m, p.loader, p.bounds_checked))
    want = {(tg.TG_GEMM_ATOM, 16, 0, 0), (tg.TG_GEMM_ATOM, 16, 0, 1),
            (tg.TG_GEMM_TILED, 64, 0, 1), (tg.TG_GEMM_TILED, 128, 1, 1),
            (tg.TG_GEMM_TILED, 256, 1, 1)}
    assert want <= seen, sorted(seen)


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K,ta,tb,beta,fmt,seed", CASES)
def test_random_problem(M, N, K, ta, tb, beta, fmt, seed):
    p = plan_of(M, N, K, ta, tb, beta, fmt)
    say(f"gemm random {M}x{N}x{K} {fmt} transA={ta} transB={tb} beta={beta} "
        f"(kernel {p.kernel}, block {p.block_m}, loader {p.loader}, bounds {p.bounds_checked})")
    full_check(M, N, K, fmt, ta, tb, beta, (seed, seed + 1000, seed + 2000))
