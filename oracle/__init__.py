"""CPU oracle for the tile GEMM and the tile copy.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code, table or constant
generator with the HIP library under ``tile_level_gemm_amd/``; the two meet
only through the seeded input generators in ``synth/``, which hold none of the
arithmetic below.

The oracle is written from these pages (cited by title and section):

[SYNC-GEMM]  "TVM TIRx 同步 GEMM 深度解析：warp 级 mma.sync 的寄存器碎片排布与
             完整下放链路" (trdm.cn/news/580350).  Sections are the article's own
             numbered headings 一 … 八 and its closing test-coverage part.
[VEC-AUTO]   "TVM TIRx CUDA 向量化内存拷贝实战：vec_auto 变体的 global↔shared 实现
             路径（gmem_smem）深度解析" (0539edu.com/news/4886382).
[TCGEN05-CP] "TVM Blackwell tcgen05.cp 全解析：shared→tmem 异步拷贝的形状选择、
             矩阵描述符与调度算法" (pnsm.cn/news/1939927).

Modules:
  numerics  exact decoding of fp16 / bf16 / fp8 (e4m3, e5m2) / e8m0 bit patterns, and of the
            6- and 4-bit element types (e2m3, e3m2, e2m1) and their packed rows, to float64
  gemm      D = A·B (+C) in float64 (16-bit operands, the fp8 operands of the asynchronous
            GEMM's precision family, block-scaled fp8 and 6/4-bit operands), the acceptance
            tables, the error bound and the fp8 comparison bar
  fragment  the matrix instructions' register maps, register images, the register-level
            product over them, and the atom selection rules
  layout    logical (row, col) -> element offset for row-major, column-major and
            the XOR-swizzled tile layout
  copy      element-by-element copy between two layouts (bit patterns)
  planner   the [outer, threads, vec] partition and the widest-aligned vector
            width rule of the vec_auto copy

Every function that has no pin of its own says "parity unpinned" in its
docstring; at present every function is pinned by tests/test_oracle_*.py.
"""

from . import numerics, gemm, layout, copy, planner, fragment  # noqa: F401
