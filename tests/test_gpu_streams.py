"""The library on caller streams and inside a captured HIP graph.

Every entry point launches on the stream it is given, allocates nothing and never
synchronises, so a caller may run it on any stream or record it into a graph.  These tests
check that results are the same bits on a side stream, and that a captured graph recomputes
from the current contents of its inputs on every replay, with eager work in between."""

import numpy as np
import pytest
import torch

import synth
import tile_level_gemm_amd as tg
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _up8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(DEV)


def _gemm_inputs(M, N, K, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    A = (torch.randn(M, K, device=DEV, generator=g) / K ** 0.5).to(dtype)
    B = (torch.randn(K, N, device=DEV, generator=g) / K ** 0.5).to(dtype)
    C = torch.rand(M, N, device=DEV, generator=g)
    return A, B, C


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 512), (4096, 4096, 256), (528, 520, 264)])
def test_side_stream_same_bits(M, N, K):
    say(f"streams: gemm {M}x{N}x{K} bf16 on a side stream")
    A, B, C = _gemm_inputs(M, N, K, torch.bfloat16, 1)
    D0 = torch.empty(M, N, device=DEV)
    D1 = torch.empty(M, N, device=DEV)
    tg.tile_gemm(A, B, C, D0, M, N, K, 0, 0, 1.0, tg.TG_BF16)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tg.tile_gemm(A, B, C, D1, M, N, K, 0, 0, 1.0, tg.TG_BF16)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(D0, D1)


def test_graph_replays_recompute():
    M = N = 2048
    K = 1024
    say(f"streams: graph of gemm {M}x{N}x{K} bf16 + fp8 gemm + tile copy, replayed 3 times")
    A, B, C = _gemm_inputs(M, N, K, torch.bfloat16, 2)
    A_alt, _, _ = _gemm_inputs(M, N, K, torch.bfloat16, 3)
    A_orig = A.clone()
    A8 = torch.randn(M, K, device=DEV).to(torch.float8_e4m3fn)
    B8 = torch.randn(N, K, device=DEV).to(torch.float8_e4m3fn)
    src = torch.randint(-30000, 30000, (4096 * 4096,), dtype=torch.int16, device=DEV)
    src_orig = src.clone()
    src_alt = torch.randint(-30000, 30000, (4096 * 4096,), dtype=torch.int16, device=DEV)
    D = torch.empty(M, N, device=DEV)
    D8 = torch.empty(M, N, device=DEV)
    dst = torch.empty_like(src)
    e4 = tg.TG_FP8_E4M3
    copy_opts = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE)

    def work():
        tg.tile_gemm(A, B, C, D, M, N, K, 0, 0, 1.0, tg.TG_BF16)
        tg.tile_gemm_fp8(A8, B8, None, D8, M, N, K, 0, 1, 0.0, e4, e4)
        tg.tile_copy_ex(src, dst, (4096, 4096), tg.TG_F16, None, None, copy_opts)

    # eager results for both contents of A
    work()
    torch.cuda.synchronize()
    want_d, want_d8 = D.clone(), D8.clone()
    want_alt = torch.empty_like(D)
    tg.tile_gemm(A_alt, B, C, want_alt, M, N, K, 0, 0, 1.0, tg.TG_BF16)
    torch.cuda.synchronize()
    assert torch.equal(dst, src) and not torch.equal(want_alt, want_d)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between replays: new input contents, outputs cleared
        alt = rep == 1
        A.copy_(A_alt if alt else A_orig)
        src.copy_(src_alt if alt else src_orig)
        D.fill_(float("nan"))
        D8.fill_(float("nan"))
        dst.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(D, want_alt if alt else want_d), rep
        assert torch.equal(D8, want_d8), rep
        assert torch.equal(dst, src), rep


def test_graph_replays_block_scaled_and_atom_paths():
    # one captured graph over the 6/4-bit kernels (e2m1 and 6-bit pairs on the direct-load
    # kernel, an e2m1 x e2m3 pair on the packed kernel) and the register atom kernel; every
    # replay, with eager work between them, must give the eager results
    say("streams: graph of block-scaled e2m1 / e2m3 / mixed gemms + a 16x8x16 atom, replayed 3 times")
    M, N, K = 512, 384, 1024
    runs = []
    for (af, bf, code_a, code_b, seed) in (("e2m1", "e2m1", tg.TG_FP4_E2M1, tg.TG_FP4_E2M1, 91),
                                           ("e2m3", "e3m2", tg.TG_FP6_E2M3, tg.TG_FP6_E3M2, 94),
                                           ("e2m1", "e2m3", tg.TG_FP4_E2M1, tg.TG_FP6_E2M3, 97)):
        pa, pb, _, _, sa, sb, _ = synth.gemm_mx_small_inputs(M, N, K, af, bf, 0.0,
                                                             (seed, seed + 1, seed + 2), dist="normal")
        runs.append((_up8(pa), _up8(pb), _up8(sa), _up8(sb), torch.empty(M, N, device=DEV), code_a,
                     code_b))
    Aa = torch.randn(16, 16, device=DEV).to(torch.float16)
    Ba = torch.randn(16, 8, device=DEV).to(torch.float16)
    Da = torch.empty(16, 8, device=DEV)

    def work():
        for A, B, SA, SB, D, ca, cb in runs:
            tg.tile_gemm_mx(A, B, SA, SB, None, D, M, N, K, 0, 1, 0.0, ca, cb)
        tg.tile_gemm(Aa, Ba, None, Da, 16, 8, 16, 0, 0, 0.0, tg.TG_F16)

    work()
    torch.cuda.synchronize()
    want = [r[4].clone() for r in runs] + [Da.clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        for r in runs:
            r[4].fill_(float("nan"))
        Da.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [r[4] for r in runs] + [Da]
        for g_, w_ in zip(got, want):
            assert torch.equal(g_, w_), rep
