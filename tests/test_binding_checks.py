"""The binding refuses tensors the library would read or write out of bounds (CPU only).

The library sees addresses only, so the binding checks every tensor argument before the
call: it must be on a GPU, on one GPU per call, of the element size the format implies and
at least as long as the sizes imply.  Here the library is replaced by a recorder, and
`_on_gpu` by a predicate that accepts host tensors, so the checks run without a GPU.
"""

import pytest
import torch

import tile_level_gemm_amd as tg


class Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        if name == "tile_last_error":
            return lambda: b""

        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    monkeypatch.setattr(tg, "_lib", r)
    monkeypatch.setattr(tg, "_on_gpu", lambda t: t.device.type in ("cpu", "meta"))
    return r


def t(n, dtype=torch.int16, device="cpu"):
    return torch.zeros(n, dtype=dtype, device=device)


def test_host_tensor_is_refused_before_the_library():
    # no stub: a host tensor must never reach the library
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm(t(16 * 16), t(16 * 8), None, t(16 * 8, torch.float32), 16, 8, 16, 0, 0, 0.0,
                     tg.TG_F16)
    assert e.value.status == tg.TG_E_ARG and "not on a GPU" in e.value.reason


def test_valid_gemm_reaches_the_library(rec):
    tg.tile_gemm(t(16 * 16), t(16 * 8), None, t(16 * 8, torch.float32), 16, 8, 16, 0, 0, 0.0,
                 tg.TG_F16)
    assert rec.calls == ["tile_gemm"]


@pytest.mark.parametrize("which,status", [
    ("A short", tg.TG_E_SHAPE), ("B short", tg.TG_E_SHAPE), ("D short", tg.TG_E_SHAPE),
    ("C short", tg.TG_E_SHAPE), ("A bytes", tg.TG_E_DTYPE), ("D bytes", tg.TG_E_DTYPE),
    ("devices", tg.TG_E_ARG)])
def test_gemm_tensor_mismatch_is_refused(rec, which, status):
    M, N, K = 32, 16, 64
    A, B, C, D = t(M * K), t(K * N), t(M * N, torch.float32), t(M * N, torch.float32)
    if which == "A short":
        A = t(M * K - 1)
    elif which == "B short":
        B = t(K * N - 8)
    elif which == "D short":
        D = t(M * N - 1, torch.float32)
    elif which == "C short":
        C = t(M * N - 4, torch.float32)
    elif which == "A bytes":
        A = t(M * K, torch.float32)
    elif which == "D bytes":
        D = t(M * N * 2, torch.int16)
    elif which == "devices":
        B = t(K * N, device="meta")
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm(A, B, C, D, M, N, K, 0, 0, 1.0, tg.TG_BF16)
    assert e.value.status == status
    assert rec.calls == []


def test_c_is_not_measured_when_beta_is_zero(rec):
    M, N, K = 32, 16, 64
    tg.tile_gemm(t(M * K), t(K * N), t(1, torch.float32), t(M * N, torch.float32), M, N, K, 0, 0,
                 0.0, tg.TG_BF16)
    assert rec.calls == ["tile_gemm"]


def test_gemm_helper_checks_k_and_output_shapes(rec):
    A = torch.zeros(32, 64, dtype=torch.bfloat16)
    with pytest.raises(tg.TileError) as e:
        tg.gemm(A, torch.zeros(48, 16, dtype=torch.bfloat16))
    assert e.value.status == tg.TG_E_SHAPE and "K" in e.value.reason
    with pytest.raises(tg.TileError) as e:
        tg.gemm(A, torch.zeros(16, 48, dtype=torch.bfloat16), trans_b=True)
    assert e.value.status == tg.TG_E_SHAPE
    B = torch.zeros(64, 16, dtype=torch.bfloat16)
    with pytest.raises(tg.TileError):
        tg.gemm(A, B, C=torch.zeros(16, 32), beta=1.0)
    with pytest.raises(tg.TileError):
        tg.gemm(A, B, out=torch.zeros(32, 16, dtype=torch.float16))
    assert rec.calls == []
    tg.gemm(A, B, out=torch.zeros(32, 16))
    assert rec.calls == ["tile_gemm"]


def test_fp8_and_block_scaled_sizes(rec):
    M, N, K = 32, 32, 128
    A, B, D = t(M * K, torch.uint8), t(K * N, torch.uint8), t(M * N, torch.float32)
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm_fp8(t(M * K), B, None, D, M, N, K, 0, 0, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3)
    assert e.value.status == tg.TG_E_DTYPE
    tg.tile_gemm_fp8(A, B, None, D, M, N, K, 0, 0, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3)
    SA, SB = t(M * K // 32, torch.uint8), t(N * K // 32, torch.uint8)
    with pytest.raises(tg.TileError) as e:
        tg.tile_gemm_mx(A, B, SA[:-1], SB, None, D, M, N, K, 0, 0, 0.0, tg.TG_FP8_E4M3,
                        tg.TG_FP8_E4M3)
    assert e.value.status == tg.TG_E_SHAPE
    tg.tile_gemm_mx(A, B, SA, SB, None, D, M, N, K, 0, 0, 0.0, tg.TG_FP8_E4M3, tg.TG_FP8_E4M3)
    assert rec.calls == ["tile_gemm_fp8", "tile_gemm_mx"]


def test_copy_extents_follow_the_layouts(rec):
    # 8 x 16 fp16 read with row stride 24: the last row ends at 7*24 + 16 = 184 elements
    src, dst = t(184), t(128)
    tg.tile_copy(src, dst, (8, 16), tg.TG_F16, (tg.TG_ROW_MAJOR, 24), None)
    with pytest.raises(tg.TileError) as e:
        tg.tile_copy(t(183), dst, (8, 16), tg.TG_F16, (tg.TG_ROW_MAJOR, 24), None)
    assert e.value.status == tg.TG_E_SHAPE
    # column-major 8 x 16 with ld 10: (16-1)*10 + 8 = 158
    tg.tile_copy_ex(t(158), dst, (8, 16), tg.TG_F16, (tg.TG_COL_MAJOR, 10), None,
                    dict(tile_rows=8, tile_cols=16, threads=64))
    with pytest.raises(tg.TileError):
        tg.tile_copy_ex(t(157), dst, (8, 16), tg.TG_F16, (tg.TG_COL_MAJOR, 10), None,
                        dict(tile_rows=8, tile_cols=16, threads=64))
    with pytest.raises(tg.TileError) as e:
        tg.tile_copy(t(128, torch.float32), dst, (8, 16), tg.TG_F16)
    assert e.value.status == tg.TG_E_DTYPE
    assert rec.calls == ["tile_copy", "tile_copy_ex"]


def test_fragment_calls_check_image_and_matrix(rec):
    shape = (32, 16)
    mem, img = t(32 * 16), t(32 * 16)
    tg.tile_frag_load(mem, img, shape, tg.TG_F16, None, tg.TG_FRAG_A16_32x32x16)
    with pytest.raises(tg.TileError):
        tg.tile_frag_load(mem, t(32 * 16 - 1), shape, tg.TG_F16, None, tg.TG_FRAG_A16_32x32x16)
    with pytest.raises(tg.TileError):
        tg.tile_frag_store(img, t(100), shape, tg.TG_F16, None, tg.TG_FRAG_A16_32x32x16)
    with pytest.raises(tg.TileError):
        tg.tile_frag_mma(t(32 * 16), t(16 * 32), None, t(32 * 32 - 1, torch.float32), 32, 32, 16,
                         0.0, tg.TG_F16, tg.TG_F16, tg.TG_MMA_32x32x16)
    assert rec.calls == ["tile_frag_load"]
