"""Python binding of libtilegemm.so (argument marshalling only).

Every function of include/tilegemm.h is exposed under the same name and takes the
same arguments; device buffers may be given as torch tensors or raw addresses.
All compute runs in the library's HIP kernels; PyTorch only provides device
memory and the current stream.  There is no fallback: if the library is not built
every call raises.

`torch` is imported before the library is loaded so that the library binds to the
HIP runtime torch already loaded (one runtime per process).

Tensor arguments are checked here before the library is called, because the library
only sees addresses: every tensor must live on a GPU, all tensors of one call on the same
GPU, with the element size the call's format implies and at least the bytes its sizes
imply (a shorter buffer would be read or written past its end).  A failed check raises
TileError and launches nothing.  Integer addresses are passed through unchecked: a caller
who passes raw addresses vouches for them.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtilegemm.so")

# enums of include/tilegemm.h
TG_F16, TG_BF16, TG_F32, TG_U8, TG_I8, TG_FP8_E4M3, TG_FP8_E5M2 = 1, 2, 3, 4, 5, 6, 7
TG_FP6_E2M3, TG_FP6_E3M2, TG_FP4_E2M1 = 8, 9, 10   # packed K-contiguous rows (tile_gemm_mx)
TG_OK, TG_E_NULL, TG_E_SHAPE, TG_E_DTYPE, TG_E_BETA, TG_E_ALIAS = 0, -1, -2, -3, -4, -5
TG_E_ALIGN, TG_E_THREADS, TG_E_LAYOUT, TG_E_HIP, TG_E_ARG = -6, -7, -8, -9, -10
TG_ROW_MAJOR, TG_COL_MAJOR, TG_XOR_SWIZZLE = 0, 1, 2
TG_GEMM_NONE, TG_GEMM_ATOM, TG_GEMM_TILED, TG_GEMM_FILL = 0, 1, 2, 3
(TG_FRAG_A16_32x32x16, TG_FRAG_B16_32x32x16, TG_FRAG_A16_16x16x32, TG_FRAG_B16_16x16x32,
 TG_FRAG_A8_32x32x64, TG_FRAG_B8_32x32x64, TG_FRAG_C32_32x32, TG_FRAG_C32_16x16,
 TG_FRAG_A16_32x32x8, TG_FRAG_B16_32x32x8, TG_FRAG_A16_16x16x16, TG_FRAG_B16_16x16x16) = range(1, 13)
TG_FRAG_AUTO, TG_FRAG_DIRECT, TG_FRAG_LDS = 0, 1, 2
TG_MMA_32x32x16, TG_MMA_16x16x32, TG_MMA_32x32x64_F8, TG_MMA_32x32x8, TG_MMA_16x16x16 = 1, 2, 3, 4, 5

STATUS_NAMES = {0: "TG_OK", -1: "TG_E_NULL", -2: "TG_E_SHAPE", -3: "TG_E_DTYPE", -4: "TG_E_BETA",
                -5: "TG_E_ALIAS", -6: "TG_E_ALIGN", -7: "TG_E_THREADS", -8: "TG_E_LAYOUT",
                -9: "TG_E_HIP", -10: "TG_E_ARG"}

TORCH_DTYPES = {torch.float16: TG_F16, torch.bfloat16: TG_BF16, torch.float32: TG_F32,
                torch.uint8: TG_U8, torch.int8: TG_I8}
for _name, _code in (("float8_e4m3fn", TG_FP8_E4M3), ("float8_e5m2", TG_FP8_E5M2)):
    if hasattr(torch, _name):
        TORCH_DTYPES[getattr(torch, _name)] = _code


class Layout(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("reserved", ctypes.c_int32), ("ld", ctypes.c_int64)]


class CopyOpts(ctypes.Structure):
    _fields_ = [("tile_rows", ctypes.c_int32), ("tile_cols", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("lds_kind", ctypes.c_int32), ("flags", ctypes.c_int32)]


class CopyPhase(ctypes.Structure):
    _fields_ = [("outer", ctypes.c_int32), ("threads", ctypes.c_int32), ("vec", ctypes.c_int32),
                ("vec_bits", ctypes.c_int32)]

    def as_tuple(self):
        return (self.outer, self.threads, self.vec, self.vec_bits)


class CopyPlan(ctypes.Structure):
    _fields_ = [("load", CopyPhase), ("store", CopyPhase), ("tile_rows", ctypes.c_int32),
                ("tile_cols", ctypes.c_int32), ("lds_kind", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("tiles", ctypes.c_int64)]


class AsyncOpts(ctypes.Structure):
    _fields_ = [("tile_rows", ctypes.c_int32), ("tile_cols", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("lds_kind", ctypes.c_int32), ("depth", ctypes.c_int32),
                ("tiles_per_workgroup", ctypes.c_int32), ("flags", ctypes.c_int32)]


class AsyncPlan(ctypes.Structure):
    _fields_ = [("copy", CopyPlan), ("depth", ctypes.c_int32),
                ("tiles_per_workgroup", ctypes.c_int32), ("grid", ctypes.c_int64)]


class GemmPlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("wave_m", ctypes.c_int32), ("wave_n", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("bounds_checked", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("grid", ctypes.c_int64), ("loader", ctypes.c_int32),
                ("atom", ctypes.c_int32)]


class FragPlan(ctypes.Structure):
    _fields_ = [("route", ctypes.c_int32), ("vec", ctypes.c_int32), ("vec_bits", ctypes.c_int32),
                ("transposed", ctypes.c_int32), ("tile_rows", ctypes.c_int32),
                ("tile_cols", ctypes.c_int32), ("elems", ctypes.c_int32),
                ("elem_bits", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("tiles", ctypes.c_int64), ("grid", ctypes.c_int64)]


class TileError(RuntimeError):
    """A non-TG_OK status; .status holds the code, str() the library's reason."""

    def __init__(self, status, reason):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {reason}")
        self.status = status
        self.reason = reason


_lib = None

_I64, _INT, _VP, _F = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
_SIGS = {
    "tile_gemm": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _F, _INT, _VP]),
    "tile_gemm_plan": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _F, _INT,
                              ctypes.POINTER(GemmPlan)]),
    "tile_gemm_fp8": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _F, _INT, _INT,
                             _VP]),
    "tile_gemm_fp8_plan": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _F, _INT,
                                  _INT, ctypes.POINTER(GemmPlan)]),
    "tile_gemm_mx": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _F, _INT,
                            _INT, _VP]),
    "tile_gemm_mx_plan": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _F,
                                 _INT, _INT, ctypes.POINTER(GemmPlan)]),
    "tile_copy": (_INT, [_VP, _VP, ctypes.POINTER(_I64), _INT, ctypes.POINTER(Layout),
                         ctypes.POINTER(Layout), _VP]),
    "tile_copy_ex": (_INT, [_VP, _VP, ctypes.POINTER(_I64), _INT, ctypes.POINTER(Layout),
                            ctypes.POINTER(Layout), ctypes.POINTER(CopyOpts), _VP]),
    "tile_copy_plan": (_INT, [_VP, _VP, ctypes.POINTER(_I64), _INT, ctypes.POINTER(Layout),
                              ctypes.POINTER(Layout), ctypes.POINTER(CopyOpts),
                              ctypes.POINTER(CopyPlan)]),
    "tile_copy_partition": (_INT, [_I64, _I64, _INT, _INT, ctypes.POINTER(Layout), _I64,
                                   ctypes.POINTER(Layout), _I64, ctypes.POINTER(CopyPhase)]),
    "tile_frag_load": (_INT, [_VP, _VP, ctypes.POINTER(_I64), _INT, ctypes.POINTER(Layout), _INT,
                              _INT, _VP]),
    "tile_frag_store": (_INT, [_VP, _VP, ctypes.POINTER(_I64), _INT, ctypes.POINTER(Layout), _INT,
                               _INT, _VP]),
    "tile_frag_plan": (_INT, [_INT, _VP, _VP, ctypes.POINTER(_I64), _INT, ctypes.POINTER(Layout),
                              _INT, _INT, ctypes.POINTER(FragPlan)]),
    "tile_frag_mma": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _F, _INT, _INT, _INT, _VP]),
    "tile_mma_select": (_INT, [_I64, _I64, _I64, _INT, _INT, ctypes.POINTER(ctypes.c_int)]),
    "tile_gemm_atom_select": (_INT, [_I64, _I64, _I64, _INT, _INT, _INT, ctypes.POINTER(ctypes.c_int)]),
    "tile_copy_async": (_INT, [_VP, _VP, ctypes.POINTER(_I64), _INT, ctypes.POINTER(Layout),
                               ctypes.POINTER(Layout), ctypes.POINTER(AsyncOpts), _VP]),
    "tile_copy_async_plan": (_INT, [_VP, _VP, ctypes.POINTER(_I64), _INT, ctypes.POINTER(Layout),
                                    ctypes.POINTER(Layout), ctypes.POINTER(AsyncOpts),
                                    ctypes.POINTER(AsyncPlan)]),
    "tile_last_error": (ctypes.c_char_p, []),
    "tile_abi_version": (_INT, []),
}


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m tile_level_gemm_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def tile_last_error():
    return lib().tile_last_error().decode()


def tile_abi_version():
    return lib().tile_abi_version()


def _check(status):
    if status != TG_OK:
        raise TileError(status, tile_last_error())


def _addr(x):
    """Device address of a tensor (or an int address, or None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        if x.numel() and not x.is_contiguous():
            raise ValueError("tensors passed to the library must be contiguous")
        return x.data_ptr() if x.numel() else (x.data_ptr() or None)
    raise TypeError(f"expected a tensor, an int address or None, got {type(x)}")


ELEM_BYTES = {TG_F16: 2, TG_BF16: 2, TG_F32: 4, TG_U8: 1, TG_I8: 1, TG_FP8_E4M3: 1, TG_FP8_E5M2: 1}
PACKED_BITS = {TG_FP6_E2M3: 6, TG_FP6_E3M2: 6, TG_FP4_E2M1: 4}


def _on_gpu(t):
    """True for a tensor in GPU memory (the library dereferences device addresses only)."""
    return t.is_cuda


def _checked(*args):
    """Validate the tensor arguments of one call: (name, value, element bytes or None, bytes).

    value None or an int address is not checked.  A tensor must be on a GPU, on the same GPU
    as the call's other tensors, have the given element size and hold at least `bytes`."""
    dev = None
    for name, x, esize, nbytes in args:
        if not isinstance(x, torch.Tensor):
            continue
        if not _on_gpu(x):
            raise TileError(TG_E_ARG, f"{name} is on {x.device}, not on a GPU")
        if dev is None:
            dev = x.device
        elif x.device != dev:
            raise TileError(TG_E_ARG, f"{name} is on {x.device}, the call's other tensors on {dev}")
        if esize is not None and x.element_size() != esize:
            raise TileError(TG_E_DTYPE, f"{name} has {x.element_size()}-byte elements, the call "
                                        f"expects {esize}-byte elements")
        have = x.numel() * x.element_size()
        if have < nbytes:
            raise TileError(TG_E_SHAPE, f"{name} holds {have} bytes, the sizes need {nbytes}")


def _extent(shape, layout, esize):
    """Bytes a layout of `shape` spans from its first element: the largest offset + 1."""
    rows, cols = int(shape[0]), int(shape[1])
    if rows <= 0 or cols <= 0:
        return 0
    lay = _layout(layout)
    if lay.kind == TG_XOR_SWIZZLE:
        return rows * cols * esize
    if lay.kind == TG_COL_MAJOR:
        ld = lay.ld or rows
        return ((cols - 1) * ld + rows) * esize
    ld = lay.ld or cols
    return ((rows - 1) * ld + cols) * esize


def _gemm_tensors(A, B, C, D, M, N, K, beta, ea, eb):
    """ea, eb: operand element bytes (None for a format the library will reject)."""
    m, n, k = max(int(M), 0), max(int(N), 0), max(int(K), 0)
    _checked(("A", A, ea, m * k * (ea or 1)), ("B", B, eb, k * n * (eb or 1)),
             ("C", C, 4, m * n * 4 if float(beta) == 1.0 else 0), ("D", D, 4, m * n * 4))


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _layout(x):
    if x is None:
        return Layout(TG_ROW_MAJOR, 0, 0)
    if isinstance(x, Layout):
        return x
    kind, ld = (x, 0) if isinstance(x, int) else x
    return Layout(kind, 0, ld)


def _shape(shape):
    return (ctypes.c_int64 * 2)(int(shape[0]), int(shape[1]))


# ------------------------------------------------------------------ GEMM ----

def tile_gemm(A, B, C, D, M, N, K, transA, transB, beta, dtype, stream=None):
    """D = A·B + beta·C through the library (see include/tilegemm.h)."""
    e = ELEM_BYTES.get(int(dtype))
    _gemm_tensors(A, B, C, D, M, N, K, beta, e, e)
    _check(lib().tile_gemm(_addr(A), _addr(B), _addr(C), _addr(D), M, N, K, int(transA),
                           int(transB), float(beta), int(dtype), _stream(stream)))


def tile_gemm_plan(A, B, C, D, M, N, K, transA, transB, beta, dtype):
    out = GemmPlan()
    _check(lib().tile_gemm_plan(_addr(A), _addr(B), _addr(C), _addr(D), M, N, K, int(transA),
                                int(transB), float(beta), int(dtype), ctypes.byref(out)))
    return out


def gemm(A, B, C=None, beta=0.0, trans_a=False, trans_b=False, alpha=1.0, out=None, stream=None):
    """Tensor convenience: returns D (fp32) = A·B (+C).  alpha must be 1 (the primitive has none)."""
    if alpha != 1.0:
        raise TileError(TG_E_ARG, "alpha must be 1.0")
    if A.dtype != B.dtype or A.dtype not in (torch.float16, torch.bfloat16):
        raise TileError(TG_E_DTYPE, "A and B must both be float16 or both bfloat16")
    if A.dim() != 2 or B.dim() != 2:
        raise TileError(TG_E_SHAPE, "A and B must be matrices")
    M = A.shape[1] if trans_a else A.shape[0]
    K = A.shape[0] if trans_a else A.shape[1]
    N = B.shape[0] if trans_b else B.shape[1]
    kb = B.shape[1] if trans_b else B.shape[0]
    if kb != K:
        raise TileError(TG_E_SHAPE, f"A has K = {K}, B has K = {kb}")
    for name, t in (("C", C), ("out", out)):
        if t is not None and (tuple(t.shape) != (M, N) or t.dtype != torch.float32):
            raise TileError(TG_E_SHAPE, f"{name} must be a ({M}, {N}) float32 tensor, got "
                                        f"{tuple(t.shape)} {t.dtype}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    tile_gemm(A, B, C, out, M, N, K, trans_a, trans_b, beta, TORCH_DTYPES[A.dtype], stream)
    return out


def tile_gemm_fp8(A, B, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype, stream=None):
    """D = A·B + beta·C with fp8 operands through the library (see include/tilegemm.h)."""
    _gemm_tensors(A, B, C, D, M, N, K, beta, 1, 1)
    _check(lib().tile_gemm_fp8(_addr(A), _addr(B), _addr(C), _addr(D), M, N, K, int(transA),
                               int(transB), float(beta), int(a_dtype), int(b_dtype),
                               _stream(stream)))


def tile_gemm_fp8_plan(A, B, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype):
    out = GemmPlan()
    _check(lib().tile_gemm_fp8_plan(_addr(A), _addr(B), _addr(C), _addr(D), M, N, K, int(transA),
                                    int(transB), float(beta), int(a_dtype), int(b_dtype),
                                    ctypes.byref(out)))
    return out


def tile_gemm_mx(A, B, SA, SB, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype,
                 stream=None):
    """Block-scaled GEMM (fp8, or packed 6- / 4-bit rows) through the library (see
    include/tilegemm.h)."""
    m, n, k = max(int(M), 0), max(int(N), 0), max(int(K), 0)
    if int(a_dtype) in PACKED_BITS or int(b_dtype) in PACKED_BITS:
        # byte tensors holding packed rows of K codes
        _checked(("A", A, 1, m * k * PACKED_BITS.get(int(a_dtype), 8) // 8),
                 ("B", B, 1, n * k * PACKED_BITS.get(int(b_dtype), 8) // 8),
                 ("C", C, 4, m * n * 4 if float(beta) == 1.0 else 0), ("D", D, 4, m * n * 4))
    else:
        _gemm_tensors(A, B, C, D, M, N, K, beta, 1, 1)
    kb = k // 32
    _checked(("A", A, None, 0), ("SA", SA, 1, max(int(M), 0) * kb),
             ("SB", SB, 1, max(int(N), 0) * kb), ("D", D, None, 0))
    _check(lib().tile_gemm_mx(_addr(A), _addr(B), _addr(SA), _addr(SB), _addr(C), _addr(D), M, N,
                              K, int(transA), int(transB), float(beta), int(a_dtype),
                              int(b_dtype), _stream(stream)))


def tile_gemm_mx_plan(A, B, SA, SB, C, D, M, N, K, transA, transB, beta, a_dtype, b_dtype):
    out = GemmPlan()
    _check(lib().tile_gemm_mx_plan(_addr(A), _addr(B), _addr(SA), _addr(SB), _addr(C), _addr(D),
                                   M, N, K, int(transA), int(transB), float(beta), int(a_dtype),
                                   int(b_dtype), ctypes.byref(out)))
    return out


# ------------------------------------------------------------------ copy ----

def _opts(opts):
    if opts is None or isinstance(opts, CopyOpts):
        return opts
    return CopyOpts(int(opts.get("tile_rows", 0)), int(opts.get("tile_cols", 0)),
                    int(opts.get("threads", 0)), int(opts.get("lds_kind", TG_XOR_SWIZZLE)),
                    int(opts.get("flags", 0)))


def _copy_tensors(src, dst, shape, dtype, src_layout, dst_layout):
    e = ELEM_BYTES.get(int(dtype))
    _checked(("src", src, e, _extent(shape, src_layout, e or 1)),
             ("dst", dst, e, _extent(shape, dst_layout, e or 1)))


def tile_copy(src, dst, shape, dtype, src_layout=None, dst_layout=None, stream=None):
    sl, dl = _layout(src_layout), _layout(dst_layout)
    _copy_tensors(src, dst, shape, dtype, src_layout, dst_layout)
    _check(lib().tile_copy(_addr(src), _addr(dst), _shape(shape), int(dtype), ctypes.byref(sl),
                           ctypes.byref(dl), _stream(stream)))


def tile_copy_ex(src, dst, shape, dtype, src_layout, dst_layout, opts, stream=None):
    sl, dl, o = _layout(src_layout), _layout(dst_layout), _opts(opts)
    _copy_tensors(src, dst, shape, dtype, src_layout, dst_layout)
    _check(lib().tile_copy_ex(_addr(src), _addr(dst), _shape(shape), int(dtype), ctypes.byref(sl),
                              ctypes.byref(dl), ctypes.byref(o) if o is not None else None,
                              _stream(stream)))


def tile_copy_plan(src, dst, shape, dtype, src_layout=None, dst_layout=None, opts=None):
    sl, dl, o = _layout(src_layout), _layout(dst_layout), _opts(opts)
    out = CopyPlan()
    _check(lib().tile_copy_plan(_addr(src), _addr(dst), _shape(shape), int(dtype), ctypes.byref(sl),
                                ctypes.byref(dl), ctypes.byref(o) if o is not None else None,
                                ctypes.byref(out)))
    return out


def _async_opts(opts):
    if opts is None or isinstance(opts, AsyncOpts):
        return opts
    return AsyncOpts(int(opts["tile_rows"]), int(opts["tile_cols"]), int(opts["threads"]),
                     int(opts.get("lds_kind", TG_XOR_SWIZZLE)), int(opts.get("depth", 2)),
                     int(opts.get("tiles_per_workgroup", 0)), int(opts.get("flags", 0)))


def tile_copy_async(src, dst, shape, dtype, src_layout, dst_layout, opts, stream=None):
    """Copy with issue-only global -> LDS transfers, `depth` tiles in flight per workgroup."""
    sl, dl, o = _layout(src_layout), _layout(dst_layout), _async_opts(opts)
    _copy_tensors(src, dst, shape, dtype, src_layout, dst_layout)
    _check(lib().tile_copy_async(_addr(src), _addr(dst), _shape(shape), int(dtype), ctypes.byref(sl),
                                 ctypes.byref(dl), ctypes.byref(o) if o is not None else None,
                                 _stream(stream)))


def tile_copy_async_plan(src, dst, shape, dtype, src_layout, dst_layout, opts):
    sl, dl, o = _layout(src_layout), _layout(dst_layout), _async_opts(opts)
    out = AsyncPlan()
    _check(lib().tile_copy_async_plan(_addr(src), _addr(dst), _shape(shape), int(dtype),
                                      ctypes.byref(sl), ctypes.byref(dl),
                                      ctypes.byref(o) if o is not None else None, ctypes.byref(out)))
    return out


def tile_copy_partition(rows, cols, elem_bits, threads, drive, drive_base, other, other_base):
    d, o = _layout(drive), _layout(other)
    out = CopyPhase()
    _check(lib().tile_copy_partition(rows, cols, elem_bits, threads, ctypes.byref(d), drive_base,
                                     ctypes.byref(o), other_base, ctypes.byref(out)))
    return out


# ------------------------------------------------------------- fragments ----

def tile_frag_load(src, image, shape, dtype, src_layout, kind, route=TG_FRAG_AUTO, stream=None):
    """Matrix -> register image of fragment `kind` (see include/tilegemm.h)."""
    lay = _layout(src_layout)
    e = ELEM_BYTES.get(int(dtype))
    n = max(int(shape[0]), 0) * max(int(shape[1]), 0)
    _checked(("src", src, e, _extent(shape, src_layout, e or 1)), ("image", image, None, n * (e or 1)))
    _check(lib().tile_frag_load(_addr(src), _addr(image), _shape(shape), int(dtype),
                                ctypes.byref(lay), int(kind), int(route), _stream(stream)))


def tile_frag_store(image, dst, shape, dtype, dst_layout, kind, route=TG_FRAG_AUTO, stream=None):
    """Register image of fragment `kind` -> matrix."""
    lay = _layout(dst_layout)
    e = ELEM_BYTES.get(int(dtype))
    n = max(int(shape[0]), 0) * max(int(shape[1]), 0)
    _checked(("image", image, None, n * (e or 1)), ("dst", dst, e, _extent(shape, dst_layout, e or 1)))
    _check(lib().tile_frag_store(_addr(image), _addr(dst), _shape(shape), int(dtype),
                                 ctypes.byref(lay), int(kind), int(route), _stream(stream)))


def tile_frag_plan(store, mem, image, shape, dtype, layout, kind, route=TG_FRAG_AUTO):
    lay = _layout(layout)
    out = FragPlan()
    _check(lib().tile_frag_plan(int(store), _addr(mem), _addr(image), _shape(shape), int(dtype),
                                ctypes.byref(lay), int(kind), int(route), ctypes.byref(out)))
    return out


def tile_frag_mma(a_image, b_image, c_image, d_image, M, N, K, beta, a_dtype, b_dtype, shape,
                  stream=None):
    """D = A·B (+ C) over register images of the shape's kinds."""
    ea, eb = ELEM_BYTES.get(int(a_dtype), 1), ELEM_BYTES.get(int(b_dtype), 1)
    m, n, k = max(int(M), 0), max(int(N), 0), max(int(K), 0)
    _checked(("a_image", a_image, None, m * k * ea), ("b_image", b_image, None, k * n * eb),
             ("c_image", c_image, None, m * n * 4 if float(beta) == 1.0 else 0),
             ("d_image", d_image, None, m * n * 4))
    _check(lib().tile_frag_mma(_addr(a_image), _addr(b_image), _addr(c_image), _addr(d_image), M,
                               N, K, float(beta), int(a_dtype), int(b_dtype), int(shape),
                               _stream(stream)))


def tile_mma_select(M, N, K, a_dtype, b_dtype):
    """The widest matrix-instruction shape whose atom divides (M, N, K) (a TG_MMA_* code)."""
    out = ctypes.c_int(0)
    _check(lib().tile_mma_select(M, N, K, int(a_dtype), int(b_dtype), ctypes.byref(out)))
    return out.value


def tile_gemm_atom_select(M, N, K, dtype, transA, transB):
    """The matrix instruction tile_gemm's register kernel runs for a problem (a TG_MMA_* code)."""
    out = ctypes.c_int(0)
    _check(lib().tile_gemm_atom_select(M, N, K, int(dtype), int(transA), int(transB), ctypes.byref(out)))
    return out.value
