"""Benchmark of the hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * tile GEMM  D = A·B, M = N = K = 8192, bf16 A/B normal(0,1)/sqrt(K), fp32 D, beta = 0
  * streaming tile copy of 2^28 fp16 values viewed as 16384 x 16384, 128x64 tiles staged
    through XOR-swizzled LDS by 256-thread workgroups, out of place.
Inputs are resident in HBM before the timed region.  Each kernel is bracketed by HIP
events on the stream it is launched on (torch's current stream, which the binding
passes to the library); `value` is the GEMM's TFLOP/s over the timed steps, the copy's
GB/s is reported beside it.  The fp16 transA beta=1 variant of the same GEMM is timed
after the steps and reported as an extra field, and so is the fp8 (e4m3 x e4m3, A [M,K], B [N,K])
GEMM of the same size against the dense fp8 peak, the block-scaled fp8 GEMM, and two register
fragment copies: the 16384 x 16384 fp16 matrix stored column-major loaded into 32x32x16 A
fragments (runs across memory lines: transposing LDS reads), and 8192 x 16384 fp32 32x32
accumulator fragments stored to a row-major matrix, both against the HBM peak; the
asynchronous copy (4 tiles in flight) of the same 16384 x 16384 tensor; and the register-level
product at 4096^3 with each matrix-instruction shape that divides it; and the GEMM at other
sizes (8000^3 bf16, 2048^3 bf16 and e4m3).  A CPU baseline times the oracle on bounded samples
of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 60] [--no-cpu-baseline]

Warm-up: the part needs about 60 ms of sustained load before its clocks settle (measured:
with 10 warm-up steps the bf16 GEMM averaged 1363-1369 TFLOP/s and the fp8 one 2432-2444,
with 60 steps 1409-1411 and 2744-2756), so the default is 60 steps, and each leg timed after
the steps gets at least 60 untimed launches of its own kernel.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2516.6   # dense fp16/bf16: 256 CU x 2.4 GHz x 4096 flop/clk/CU
LEG_WARMUP = 60               # untimed launches before each leg timed after the steps
PEAK_FP8_TFLOPS = 5033.2    # dense fp8: twice the fp16/bf16 rate
PEAK_FP4_TFLOPS = 10100.0   # dense fp6 and fp4 (MI355X published)
PEAK_HBM_GBS = 8000.0       # HBM3E
M = N = K = 8192
ROWS = COLS = 16384
METRIC = "GEMM TFLOP/s + % MFMA peak (bf16 8192³); tile-copy GB/s + % HBM peak"


KERNEL_SOURCES = {
    "gemm": ("gemm_direct.hip", "gemm_direct_launch.h", "direct_gemm.h", "gemm_kernels.hip", "lds_layout.h",
             "tg_internal.h"),
    "fp8": ("gemm_fp8.hip", "gemm_fp8_launch.h", "direct_gemm.h", "tg_internal.h"),
    "mx": ("gemm_mx_kk.hip", "gemm_fp8_launch.h", "direct_gemm.h", "tg_internal.h"),
    "copy": ("copy_kernels.hip", "lds_layout.h", "tg_internal.h"),
    "packed": ("gemm_mx_packed.hip", "tg_internal.h"),
    "fp4": ("gemm_mx_fp4.hip", "direct_gemm.h", "tg_internal.h"),
    "fp6": ("gemm_mx_fp6.hip", "direct_gemm.h", "tg_internal.h"),
    "frag": ("frag_kernels.hip", "tg_internal.h"),
    "async": ("async_copy.hip", "lds_layout.h", "tg_internal.h"),
}


def kernel_sources_sha(which):
    """Hash of the sources a kernel is built from (counters go stale when it changes)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tile_level_gemm_amd", "csrc")
    for name in KERNEL_SOURCES[which]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    # profiles/traffic.json: {kernel: {"sources": "gemm"|"copy", "sources_sha": ..., "bytes_per_launch": ...}}
    """HBM bytes per launch from the committed rocprofv3 counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(kernel)
    if not rec or rec.get("sources_sha") != kernel_sources_sha(rec.get("sources", "")):
        return None
    return rec.get("bytes_per_launch")


TRAFFIC_KERNELS = {
    # traffic.json key: (kernel-name substring in the rocprofv3 csv, sources, algorithmic bytes)
    "gemm_direct_256x256_bf16_nn": ("gemm_direct<false, true, 2, 2, 4, false, 0>", "gemm",
                                    2 * M * K * 2 + M * N * 4),
    "gemm_direct_256x256_f16_transA_beta1": ("gemm_direct<true, true, 1, 2, 4, false, 0>", "gemm",
                                             2 * M * K * 2 + 2 * M * N * 4),
    "gemm_fp8_256x256_e4m3_tn": ("gemm_direct<false, false, 16, 2, 4, false, 0>", "fp8",
                                 2 * M * K + M * N * 4),
    "gemm_mx_256x256_e4m3_tn": ("gemm_direct<false, false, 32, 2, 4, false, 0>", "mx",
                                2 * M * K + 2 * M * (K // 32) + M * N * 4),
    "gemm_mx_256x256_e2m1_tn": ("gemm_direct<false, false, 64, 2, 4, false, 0>", "fp4",
                                2 * M * K // 2 + 2 * M * (K // 32) + M * N * 4),
    "gemm_mx_256x256_e2m3_tn": ("gemm_direct<false, false, 96, 2, 4, false, 0>", "fp6",
                                2 * M * K * 6 // 8 + 2 * M * (K // 32) + M * N * 4),
    "gemm_mx_256x256_e2m1xe2m3_tn": ("gemm_mx_packed<4, 2, false, 256>", "packed",
                                     M * K // 2 + M * K * 6 // 8 + 2 * M * (K // 32) + M * N * 4),
    "tile_copy_16384x16384_f16": ("tile_copy_rows<16, 4, 4, 128>", "copy", 2 * ROWS * COLS * 2),
    "frag_load_a16_32x32x16_col_16384x16384": ("frag_lds<1, false, true>", "frag",
                                               2 * ROWS * COLS * 2),
    "frag_store_c32_32x32_row_8192x16384": ("frag_lds<7, true, true>", "frag",
                                            2 * (ROWS // 2) * COLS * 4),
    "tile_copy_async_16384x16384_f16_depth4": ("tile_copy_async_kernel<16, 4, 4>", "async",
                                               2 * ROWS * COLS * 2),
}


def summarize_counters(fetch_dir, write_dir, out_path):
    """Write profiles/traffic.json from two rocprofv3 --pmc runs of `bench.py --calib-copy`.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by the factors that make the
    calibration copy (torch copy_ of the 512 MiB copy source: grid 131072 x 512) read and
    write exactly 512 MiB; bytes_per_launch = scaled fetch + scaled write, averaged.
    """
    import csv

    def load(d, counter):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        return [r for r in rows if r["Counter_Name"] == counter]

    known = ROWS * COLS * 2
    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")

    def calib(rows):
        cands = [float(r["Counter_Value"]) for r in rows
                 if "copyBuffer" in r["Kernel_Name"] and r["Grid_Size"] == "131072"]
        return max(cands)

    ff = known / 1024.0 / calib(fetch)
    wf = known / 1024.0 / calib(write)
    out = {"_calibration": {"kernel": "__amd_rocclr_copyBuffer, 512 MiB device-to-device",
                            "fetch_factor": ff, "write_factor": wf,
                            "FETCH_SIZE_KiB": calib(fetch), "WRITE_SIZE_KiB": calib(write),
                            "commands": [f"rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- "
                                         "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --calib-copy"
                                         for c in ("FETCH_SIZE", "WRITE_SIZE")]}}
    for key, (sub, src, algo) in TRAFFIC_KERNELS.items():
        fv = [float(r["Counter_Value"]) for r in fetch if sub in r["Kernel_Name"]]
        wv = [float(r["Counter_Value"]) for r in write if sub in r["Kernel_Name"]]
        if not fv or not wv:
            continue
        f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
        out[key] = {"kernel": sub, "sources": src, "sources_sha": kernel_sources_sha(src),
                    "FETCH_SIZE_KiB": f_kib, "WRITE_SIZE_KiB": w_kib,
                    "bytes_per_launch": round((f_kib * ff + w_kib * wf) * 1024),
                    "algorithmic_bytes": algo}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def _stats(ms):
    """avg / median / min of a list of milliseconds."""
    a = np.asarray(ms, dtype=np.float64)
    return {"avg_ms": round(float(a.mean()), 5), "median_ms": round(float(np.median(a)), 5),
            "min_ms": round(float(a.min()), 5)}


def cpu_baseline(gemm_inputs, copy_src, c3_inputs, budget_s=12.0):
    """Time the oracle as it stands on bounded samples of the same workload (host cores)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import gemm as og
    from oracle.copy import copy_ref
    from oracle.layout import Layout
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = os.cpu_count() or 1
    a_bits, b_bits, _ = gemm_inputs
    # GEMM: oracle.gemm.gemm_ref (float64 matmul) on a slab of rows of A
    rows = 64
    while True:
        t0 = time.perf_counter()
        og.gemm_ref(a_bits[:rows], b_bits, None, rows, N, K, False, False, 0.0, "bf16")
        dt = time.perf_counter() - t0
        if dt > budget_s / 4 or rows >= M:
            break
        rows = min(M, rows * max(2, int(budget_s / 4 / max(dt, 1e-3))))
        rows -= rows % 16
    # when the whole GEMM takes less than that, repeat it until about half the budget is spent
    reps, total = 1, dt
    while rows >= M and total < budget_s / 2:
        t0 = time.perf_counter()
        og.gemm_ref(a_bits, b_bits, None, M, N, K, False, False, 0.0, "bf16")
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    gemm_tflops = 2.0 * rows * N * K / dt / 1e12
    # copy: oracle.copy.copy_ref on a slab of rows of the 16384 x 16384 f16 tensor, grown until
    # one call takes about an eighth of the budget (one thread)
    slab = 256
    while True:
        src = copy_src[:slab * COLS]
        t0 = time.perf_counter()
        copy_ref(src, np.zeros_like(src), slab, COLS, Layout("row"), Layout("row"))
        cdt = time.perf_counter() - t0
        if cdt > budget_s / 8 or slab >= ROWS:
            break
        slab = min(ROWS, slab * max(2, int(budget_s / 4 / max(cdt, 1e-3))))
    copy_gbs = 2.0 * src.nbytes / cdt / 1e9
    # the same oracle on every affinity core: a thread pool over row blocks of the whole tensor
    ncore = len(os.sched_getaffinity(0))
    blk = -(-ROWS // ncore)

    def part(i):
        r0, r1 = i * blk, min(ROWS, (i + 1) * blk)
        piece = copy_src[r0 * COLS:r1 * COLS]
        copy_ref(piece, np.zeros_like(piece), r1 - r0, COLS, Layout("row"), Layout("row"))

    with ThreadPoolExecutor(ncore) as ex:
        t0 = time.perf_counter()
        list(ex.map(part, range(-(-ROWS // blk))))
        pdt = time.perf_counter() - t0
    copy_all_gbs = 2.0 * copy_src.nbytes / pdt / 1e9
    # the 512x512x256 bf16 transB beta=1 GEMM, whole, as the oracle computes it
    a3, b3, c3 = c3_inputs
    t0 = time.perf_counter()
    n3 = 0
    while True:
        og.gemm_ref(a3, b3, c3, 512, 512, 256, False, True, 1.0, "bf16")
        n3 += 1
        c3dt = (time.perf_counter() - t0) / n3
        if time.perf_counter() - t0 > 1.0:
            break
    return {
        "value": round(gemm_tflops, 6), "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
        "sample": (f"gemm: oracle.gemm.gemm_ref (float64 matmul after exact bf16 decode) on rows "
                   f"0..{rows} of the 8192^3 bf16 GEMM, {reps} call(s), {dt:.2f} s each; copy: "
                   f"oracle.copy.copy_ref on {slab} of 16384 rows ({cdt:.2f} s, single thread) = "
                   f"{copy_gbs:.3f} GB/s, and on all 16384 rows split over {ncore} threads "
                   f"({pdt:.2f} s) = {copy_all_gbs:.3f} GB/s; 512x512x256 bf16 transB beta=1 "
                   f"whole: {c3dt * 1e3:.1f} ms per call"),
        "copy_value": round(copy_gbs, 4), "copy_unit": "GB/s", "copy_cores": 1,
        "copy_all_cores": {"value": round(copy_all_gbs, 4), "unit": "GB/s", "cores": ncore},
        "gemm_512x512x256": {"ms": round(c3dt * 1e3, 3), "cores": int(blas_threads)},
        "host_cpus": os.cpu_count(), "affinity_cpus": ncore,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="before warmup, run one plain device-to-device copy of the 512 MiB copy "
                         "source (torch copy_) as the known-size kernel that scales HBM counters")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc csv directories and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        res = summarize_counters(*args.summarize_counters, os.path.join(ROOT, "profiles", "traffic.json"))
        print(json.dumps(res, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the tile GEMM and tile copy "
              "run on a single MI355X and this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import tile_level_gemm_amd as tg
    from oracle import fragment as ofr
    from oracle import gemm as og
    from oracle.copy import copy_ref
    from oracle.layout import Layout as OLayout

    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    def up8(bits):
        return torch.from_numpy(np.ascontiguousarray(bits)).to(dev)

    # ---- 1. every input, generated on the host and uploaded before any timing -----------------
    print("bench: generating inputs", file=sys.stderr, flush=True)
    gin = synth.gemm8k_bf16_inputs()
    A, B = up(gin[0]), up(gin[1])
    D = torch.empty((M, N), dtype=torch.float32, device=dev)
    copy_src_bits = synth.stream_input(ROWS, COLS)
    S = up(copy_src_bits)
    T = torch.empty_like(S)
    atoms_in = {beta: synth.atom_inputs(beta) for beta in (0.0, 1.0)}
    src32, src128 = synth.copy32_input(), synth.copy128_input()
    c3 = synth.gemm512_inputs()
    hin = synth.gemm8k_f16_inputs()
    fin = synth.gemm8k_fp8_inputs()
    g = synth.rng(64)
    sa = g.integers(117, 138, size=(M, K // 32)).astype(np.uint8)
    sb = g.integers(117, 138, size=(N, K // 32)).astype(np.uint8)
    # 6- and 4-bit legs: e2m1 and e2m3 pairs (direct-load kernel), e2m1 x e2m3 (packed kernel)
    small_pairs = {"e2m1": ("e2m1", "e2m1", (65, 66, 67)), "e2m3": ("e2m3", "e2m3", (68, 69, 70)),
                   "e2m1xe2m3": ("e2m1", "e2m3", (71, 72, 73))}
    small_in = {f: synth.gemm_mx_small_inputs(M, N, K, af, bf, 0.0, seeds, dist="normal")
                for f, (af, bf, seeds) in small_pairs.items()}
    cr, cc = ROWS // 2, COLS
    acc_bits = synth.uniform(43, cr * cc).view(np.uint32)
    other_in = {}
    for tag, (m_, n_, k_), kind, sd in (("bf16_8000", (8000, 8000, 8000), "bf16", (91, 92)),
                                        ("bf16_2048", (2048, 2048, 2048), "bf16", (93, 94)),
                                        ("fp8_2048", (2048, 2048, 2048), "fp8", (95, 96))):
        if kind == "bf16":
            sc = float(1.0 / np.sqrt(k_))
            ab, bb, _ = synth.gemm_inputs(m_, n_, k_, "bf16", False, False, 0.0, (sd[0], sd[1], 0),
                                          a_scale=sc, b_scale=sc)
        else:
            ab, bb, _ = synth.gemm_fp8_inputs(m_, n_, k_, "e4m3", "e4m3", False, True, 0.0,
                                              (sd[0], sd[1], 0))
        other_in[tag] = ((m_, n_, k_), kind, sd, ab, bb)
    torch.cuda.synchronize()
    if args.calib_copy:
        T.copy_(S)
        torch.cuda.synchronize()
    flops = 2.0 * M * N * K
    reps = max(3, args.steps // 2)
    leg_warmup = max(args.warmup, LEG_WARMUP)
    e4 = tg.TG_FP8_E4M3

    def per_launch(call, n=reps, warm=leg_warmup):
        """`warm` untimed launches, then n launches each between its own pair of events."""
        for _ in range(warm):
            call()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for ev in evs:
            ev[0].record()
            call()
            ev[1].record()
        torch.cuda.synchronize()
        return [ev[0].elapsed_time(ev[1]) for ev in evs]

    def batched(call, groups=7, per_group=None, warm=leg_warmup):
        """Launches back to back: `groups` batches of `per_group` launches, each batch between one
        pair of events; returns the per-launch ms of each batch (small kernels take about as long
        as a launch from Python, and events around each launch would time the gaps too)."""
        per_group = per_group or reps
        for _ in range(warm):
            call()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(groups)]
        for ev in evs:
            ev[0].record()
            for _ in range(per_group):
                call()
            ev[1].record()
        torch.cuda.synchronize()
        return [ev[0].elapsed_time(ev[1]) / per_group for ev in evs]

    def graphed(call, n=100, groups=5):
        """Per-launch ms inside a HIP graph of `n` launches (captured on a side stream), replayed
        `groups` times between events: the kernels without the per-call host cost.  None when
        the capture fails (the figure is then reported as null; nothing else depends on it)."""
        try:
            return _graphed(call, n, groups)
        except RuntimeError as e:
            print(f"bench: graph timing skipped ({e})", file=sys.stderr, flush=True)
            torch.cuda.synchronize()
            return None

    def _graphed(call, n, groups):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(n):
                    call()
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(groups)]
        for ev in evs:
            ev[0].record()
            graph.replay()
            ev[1].record()
        torch.cuda.synchronize()
        return [ev[0].elapsed_time(ev[1]) / n for ev in evs]

    def _gus(gms):
        return round(float(np.median(gms)) * 1e3, 3) if gms else None

    # ---- 2. the other legs, back to back on the GPU, each into buffers of its own ------------
    t_gpu = time.perf_counter()
    print("bench: small configurations", file=sys.stderr, flush=True)
    small, small_out = {}, {}
    for beta, (a, b, c) in atoms_in.items():
        Aa, Ba = up(a), up(b)
        Ca = torch.from_numpy(c).to(dev) if beta else None
        Da = torch.empty((16, 8), dtype=torch.float32, device=dev)
        atom = lambda: tg.tile_gemm(Aa, Ba, Ca, Da, 16, 8, 16, 0, 0, beta, tg.TG_F16)  # noqa: E731
        ms = batched(atom, per_group=200)
        gms = graphed(atom)
        small[f"atom_16x8x16_f16_beta{int(beta)}"] = {"us": round(float(np.median(ms)) * 1e3, 3),
                                                        **_stats(ms),
                                                        "graph_us": _gus(gms)}
        small_out[beta] = Da
    s32 = torch.from_numpy(src32.view(np.int32)).to(dev)
    d32 = torch.empty_like(s32)
    o32 = dict(tile_rows=32, tile_cols=32, threads=64, lds_kind=tg.TG_ROW_MAJOR)
    c32 = lambda: tg.tile_copy_ex(s32, d32, (32, 32), tg.TG_F32, None, None, o32)  # noqa: E731
    ms, gms = batched(c32, per_group=200), graphed(c32)
    small["copy_32x32_f32_wave64"] = {"us": round(float(np.median(ms)) * 1e3, 3), **_stats(ms),
                                      "graph_us": _gus(gms)}
    s128 = up(src128)
    d128 = torch.empty_like(s128)
    x128 = torch.empty_like(s128)
    o128 = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE)
    c128 = lambda: tg.tile_copy_ex(s128, d128, (128, 64), tg.TG_F16, None, None, o128)  # noqa: E731
    ms, gms = batched(c128, per_group=200), graphed(c128)
    small["copy_128x64_f16_xor_256t"] = {"us": round(float(np.median(ms)) * 1e3, 3), **_stats(ms),
                                         "graph_us": _gus(gms)}
    # the LDS image of the tile (a global destination in the XOR layout), checked later
    tg.tile_copy_ex(s128, x128, (128, 64), tg.TG_F16, None, (tg.TG_XOR_SWIZZLE, 0), o128)
    A3, B3, C3 = up(c3[0]), up(c3[1]), torch.from_numpy(c3[2]).to(dev)
    D3 = torch.empty((512, 512), dtype=torch.float32, device=dev)
    g3 = lambda: tg.tile_gemm(A3, B3, C3, D3, 512, 512, 256, 0, 1, 1.0, tg.TG_BF16)  # noqa: E731
    ms, gms = batched(g3, per_group=100), graphed(g3)
    t3 = float(np.median(ms)) * 1e-3
    tg3 = float(np.median(gms)) * 1e-3 if gms else None
    fl3, by3 = 2.0 * 512 * 512 * 256, 2 * 512 * 256 * 2 + 2 * 512 * 512 * 4
    t_roof = max(fl3 / (PEAK_MFMA_TFLOPS * 1e12), by3 / (PEAK_HBM_GBS * 1e9))
    small["gemm_512x512x256_bf16_transB_beta1"] = {
        "us": round(t3 * 1e6, 3), **_stats(ms), "TFLOP/s": round(fl3 / t3 / 1e12, 3),
        "graph_us": round(tg3 * 1e6, 3) if tg3 else None,
        "graph_TFLOP/s": round(fl3 / tg3 / 1e12, 3) if tg3 else None,
        "roofline": {"bound": "hbm (the larger of the MFMA and HBM times)",
                     "time_at_roofline_us": round(t_roof * 1e6, 4), "frac": round(t_roof / t3, 4),
                     "graph_frac": round(t_roof / tg3, 4) if tg3 else None, "compulsory_bytes": by3}}

    print("bench: fp16 transA beta=1 gemm", file=sys.stderr, flush=True)
    Ah, Bh = up(hin[0]), up(hin[1])
    Ch = torch.from_numpy(hin[2]).to(dev)
    Dh = torch.empty((M, N), dtype=torch.float32, device=dev)
    h_ms = per_launch(lambda: tg.tile_gemm(Ah, Bh, Ch, Dh, M, N, K, 1, 0, 1.0, tg.TG_F16))
    del Ah, Bh, Ch

    print("bench: fp8 and block-scaled fp8 gemm", file=sys.stderr, flush=True)
    A8, B8 = up8(fin[0]), up8(fin[1])
    D8 = torch.empty((M, N), dtype=torch.float32, device=dev)
    f8_list = per_launch(lambda: tg.tile_gemm_fp8(A8, B8, None, D8, M, N, K, 0, 1, 0.0, e4, e4))
    SA, SB = up8(sa), up8(sb)
    Dm = torch.empty((M, N), dtype=torch.float32, device=dev)
    mx_list = per_launch(lambda: tg.tile_gemm_mx(A8, B8, SA, SB, None, Dm, M, N, K, 0, 1, 0.0, e4, e4))
    del A8, B8, SA, SB

    print("bench: 6- and 4-bit block-scaled gemm", file=sys.stderr, flush=True)
    small_code = {"e2m1": tg.TG_FP4_E2M1, "e2m3": tg.TG_FP6_E2M3}
    small_run = {}
    for f, (pa_, pb_, _, _, sa_, sb_, _) in small_in.items():
        Ap, Bp, SAp, SBp = up8(pa_), up8(pb_), up8(sa_), up8(sb_)
        Dp = torch.empty((M, N), dtype=torch.float32, device=dev)
        ca_, cb_ = small_code[small_pairs[f][0]], small_code[small_pairs[f][1]]
        lst = per_launch(lambda: tg.tile_gemm_mx(Ap, Bp, SAp, SBp, None, Dp, M, N, K, 0, 1, 0.0, ca_, cb_))
        small_run[f] = (lst, Dp)
        del Ap, Bp, SAp, SBp

    print("bench: fragment copies and the asynchronous copy", file=sys.stderr, flush=True)
    img = torch.empty_like(S)
    fl_list = per_launch(lambda: tg.tile_frag_load(S, img, (ROWS, COLS), tg.TG_F16, (tg.TG_COL_MAJOR, 0),
                                                   tg.TG_FRAG_A16_32x32x16))
    acc = torch.from_numpy(acc_bits.view(np.int32)).to(dev)
    mat = torch.empty_like(acc)
    fs_list = per_launch(lambda: tg.tile_frag_store(acc, mat, (cr, cc), tg.TG_F32, (tg.TG_ROW_MAJOR, 0),
                                                    tg.TG_FRAG_C32_32x32))
    T2 = torch.zeros_like(S)
    aopts = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE, depth=4)
    ac_list = per_launch(lambda: tg.tile_copy_async(S, T2, (ROWS, COLS), tg.TG_F16, None, None, aopts))

    # widest-first atom selection: the register-level product at 4096^3 f16 with each atom that
    # divides it; tile_mma_select names the first of them
    print("bench: register-level product per atom", file=sys.stderr, flush=True)
    n4 = 4096
    sel = tg.tile_mma_select(n4, n4, n4, tg.TG_F16, tg.TG_F16)
    img_a = torch.empty(n4 * n4, dtype=torch.int16, device=dev).random_(0, 14000)   # finite f16
    img_b = torch.empty_like(img_a).random_(0, 14000)
    img_d = torch.empty(n4 * n4, dtype=torch.float32, device=dev)
    atoms = {}
    atom_codes = (("32x32x16", tg.TG_MMA_32x32x16), ("16x16x32", tg.TG_MMA_16x16x32),
                  ("32x32x8", tg.TG_MMA_32x32x8), ("16x16x16", tg.TG_MMA_16x16x16))
    for name, code in atom_codes:
        lst = per_launch(lambda: tg.tile_frag_mma(img_a, img_b, None, img_d, n4, n4, n4, 0.0,
                                                  tg.TG_F16, tg.TG_F16, code))
        ms_ = float(np.mean(lst))
        atoms[name] = {**_stats(lst), "TFLOP/s": round(2.0 * n4 ** 3 / (ms_ * 1e-3) / 1e12, 3)}
    del img_a, img_b, img_d

    # the block-size choice on problems other than the headline: ragged 8000^3 and mid-size
    # 2048^3 (128x128 blocks), bf16 and fp8
    print("bench: other sizes", file=sys.stderr, flush=True)
    other_run = {}
    for tag, ((m_, n_, k_), kind, sd, ab, bb) in other_in.items():
        Dx = torch.empty((m_, n_), dtype=torch.float32, device=dev)
        if kind == "bf16":
            Ax, Bx = up(ab), up(bb)
            plan = tg.tile_gemm_plan(Ax, Bx, None, Dx, m_, n_, k_, 0, 0, 0.0, tg.TG_BF16)
            call = lambda: tg.tile_gemm(Ax, Bx, None, Dx, m_, n_, k_, 0, 0, 0.0, tg.TG_BF16)  # noqa: E731
        else:
            Ax, Bx = up8(ab), up8(bb)
            plan = tg.tile_gemm_fp8_plan(Ax, Bx, None, Dx, m_, n_, k_, 0, 1, 0.0, e4, e4)
            call = lambda: tg.tile_gemm_fp8(Ax, Bx, None, Dx, m_, n_, k_, 0, 1, 0.0, e4, e4)  # noqa: E731
        other_run[tag] = (batched(call, groups=5), plan.block_m, Dx)
        del Ax, Bx

    # context, not this library: the vendor GEMM (torch.mm -> hipBLASLt) on the headline's
    # operands, bf16 in, fp32 out, timed the same way; its result is compared with ours after
    # the timed steps
    print("bench: library GEMM (context)", file=sys.stderr, flush=True)
    lib_ctx = {}
    Ab, Bb = A.view(torch.bfloat16), B.view(torch.bfloat16)
    try:
        Dl = torch.mm(Ab, Bb, out_dtype=torch.float32)
        lib_out = "fp32"
    except (RuntimeError, TypeError):
        Dl = torch.mm(Ab, Bb)
        lib_out = "bf16"
    lib_ms = per_launch(lambda: torch.mm(Ab, Bb, out_dtype=torch.float32) if lib_out == "fp32"
                        else torch.mm(Ab, Bb))
    lib_ctx = {"lst": lib_ms, "out": lib_out, "D": Dl}
    gpu_legs_s = time.perf_counter() - t_gpu

    # ---- 3. the headline steps: W warm-up steps, then K timed steps -------------------------
    def step(ev=None):
        if ev is not None:
            ev[0].record()
        tg.tile_gemm(A, B, None, D, M, N, K, 0, 0, 0.0, tg.TG_BF16)
        if ev is not None:
            ev[1].record()
        tg.tile_copy(S, T, (ROWS, COLS), tg.TG_F16)
        if ev is not None:
            ev[2].record()

    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print("bench: timed steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gemm_ms = [e[0].elapsed_time(e[1]) for e in events]
    copy_ms = [e[1].elapsed_time(e[2]) for e in events]
    g_avg = float(np.mean(gemm_ms))
    c_avg = float(np.mean(copy_ms))
    tflops = flops / (g_avg * 1e-3) / 1e12
    copy_bytes = 2.0 * ROWS * COLS * 2
    gbs = copy_bytes / (c_avg * 1e-3) / 1e9

    # the same copy back to back (no GEMM between launches): the copy on its own
    bb_list = batched(lambda: tg.tile_copy(S, T, (ROWS, COLS), tg.TG_F16), groups=5,
                      per_group=max(5, args.steps // 2), warm=1)
    bb_ms = float(np.mean(bb_list))
    bb_gbs = copy_bytes / (bb_ms * 1e-3) / 1e9
    # context: the runtime's own device-to-device copy of the same 512 MiB, back to back
    # (into a buffer of its own: T is checked against S below)
    T3 = torch.empty_like(S)
    rt_list = batched(lambda: T3.copy_(S), groups=5, per_group=max(5, args.steps // 2), warm=1)
    rt_gbs = copy_bytes / (float(np.mean(rt_list)) * 1e-3) / 1e9
    del T3

    def hbm_leg(lst, nbytes, traffic_key, parity, workload):
        ms = float(np.mean(lst))
        gb = nbytes / (ms * 1e-3) / 1e9
        return {"value": round(gb, 2), "unit": "GB/s", **_stats(lst), "workload": workload,
                "roofline": {"bound": "hbm", "achieved": round(gb, 2), "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": round(gb / PEAK_HBM_GBS, 4),
                             "traffic": traffic_for(traffic_key)},
                "parity": parity}

    def mfma_leg(lst, peak, traffic_key, parity, workload):
        tf = flops / (float(np.mean(lst)) * 1e-3) / 1e12
        return {"value": round(tf, 3), "unit": "TFLOP/s", **_stats(lst), "workload": workload,
                "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": peak, "unit": "TFLOP/s",
                             "frac": round(tf / peak, 4), "traffic": traffic_for(traffic_key)},
                "parity": parity}

    # ---- 4. parity of every leg against the oracle (host) ------------------------------------
    print("bench: parity checks (oracle)", file=sys.stderr, flush=True)
    rows, cols = synth.sample_points(M, N, 53, count=256)
    ref, bound = og.gemm_ref_at(gin[0], gin[1], None, M, N, K, False, False, 0.0, "bf16", rows, cols)
    g_ok, g_worst = og.check(D.cpu().numpy()[rows, cols], ref, bound)
    c_ok = bool(torch.equal(S, T))
    lib_diff = round(float((lib_ctx["D"].float() - D).abs().max()), 6)
    del lib_ctx["D"]
    for beta, (a, b, c) in atoms_in.items():
        ok, worst = og.check(small_out[beta].cpu().numpy(),
                             og.gemm_ref(a, b, c, 16, 8, 16, False, False, beta, "f16"),
                             og.abs_bound(a, b, 16, 8, 16, False, False, "f16"))
        small[f"atom_16x8x16_f16_beta{int(beta)}"]["parity"] = {"ok": bool(ok),
                                                                  "worst_err_over_tol": round(worst, 5)}
    small["copy_32x32_f32_wave64"]["parity"] = {
        "bit_exact": bool(np.array_equal(d32.cpu().numpy().view(np.uint32), src32))}
    want = copy_ref(src128, np.zeros_like(src128), 128, 64, OLayout("row"), OLayout("xor"))
    small["copy_128x64_f16_xor_256t"]["parity"] = {
        "bit_exact": bool(np.array_equal(d128.cpu().numpy().view(np.uint16), src128)),
        "lds_image_is_xor_layout": bool(np.array_equal(x128.cpu().numpy().view(np.uint16), want))}
    ok, worst = og.check(D3.cpu().numpy(), og.gemm_ref(c3[0], c3[1], c3[2], 512, 512, 256, False, True,
                                                        1.0, "bf16"),
                         og.abs_bound(c3[0], c3[1], 512, 512, 256, False, True, "bf16"))
    small["gemm_512x512x256_bf16_transB_beta1"]["parity"] = {"ok": bool(ok),
                                                             "worst_err_over_tol": round(worst, 5)}
    hr, hc = synth.sample_points(M, N, 57, count=256)
    refh, boundh = og.gemm_ref_at(hin[0], hin[1], hin[2], M, N, K, True, False, 1.0, "f16", hr, hc)
    h_ok, h_worst = og.check(Dh.cpu().numpy()[hr, hc], refh, boundh)
    ref8, bound8 = og.gemm_fp8_ref_at(fin[0], fin[1], None, M, N, K, False, True, 0.0, "e4m3",
                                      "e4m3", rows, cols)
    got8 = D8.cpu().numpy()[rows, cols]
    f8_ok, f8_worst = og.check_fp8(got8, ref8, bound8, fin[0], fin[1], M, N, K, False, True, "e4m3",
                                   "e4m3", rows, cols)
    f8_plain = og.check(got8, ref8, bound8)[1]
    refm, boundm = og.gemm_mx_ref_at(fin[0], fin[1], sa, sb, None, M, N, K, False, True, 0.0, "e4m3",
                                     "e4m3", rows, cols)
    gotm = Dm.cpu().numpy()[rows, cols]
    mx_ok, mx_worst = og.check_fp8(gotm, refm, boundm, fin[0], fin[1], M, N, K, False, True, "e4m3",
                                   "e4m3", rows, cols, sa_bits=sa, sb_bits=sb)
    mx_plain = og.check(gotm, refm, boundm)[1]
    small_legs = {}
    for f, (lst, Dp) in small_run.items():
        pa_, pb_, _, _, sa_, sb_, _ = small_in[f]
        af_, bf_ = small_pairs[f][0], small_pairs[f][1]
        refp, boundp = og.gemm_mx_ref_at(pa_, pb_, sa_, sb_, None, M, N, K, False, True, 0.0, af_, bf_,
                                         rows, cols)
        gotp = Dp.cpu().numpy()[rows, cols]
        p_ok, p_worst = og.check_fp8(gotp, refp, boundp, pa_, pb_, M, N, K, False, True, af_, bf_,
                                     rows, cols, sa_bits=sa_, sb_bits=sb_)
        small_legs[f"gemm_mx_{f}_tn"] = mfma_leg(
            lst, PEAK_FP4_TFLOPS, f"gemm_mx_256x256_{f}_tn",
            {"sampled_ok": bool(p_ok), "worst_err_over_tol": round(p_worst, 5),
             "worst_err_over_16bit_tol": round(og.check(gotp, refp, boundp)[1], 5)},
            f"tile_gemm_mx 8192x8192x8192, A {af_} [M,K] and B {bf_} [N,K] packed rows, N(0,1) rounded "
            f"to the format, E8M0 scales per 32 K in 2^-10..2^10, fp32 D, beta=0"
            + (" (packed kernel)" if af_ != bf_ else " (direct-load kernel)"))
    gi = synth.rng(79)
    fl_ok = True
    imgv = img.view(-1, 64, 8)
    for _ in range(64):
        ti, tj = int(gi.integers(ROWS // 32)), int(gi.integers(COLS // 16))
        want = ofr.frag_load(copy_src_bits, 32, 16, OLayout("col", ld=ROWS, base=tj * 16 * ROWS + ti * 32),
                             "a16_32x32x16")[0]
        fl_ok &= bool(np.array_equal(imgv[ti * (COLS // 16) + tj].cpu().numpy().view(np.uint16), want))
    r_, c_ = ofr.coords("c32_32x32")
    host = mat.view(cr, cc)
    accv = acc_bits.reshape(-1, 64, 16)
    fs_ok = True
    for _ in range(64):
        ti, tj = int(gi.integers(cr // 32)), int(gi.integers(cc // 32))
        got = host[ti * 32:(ti + 1) * 32, tj * 32:(tj + 1) * 32].cpu().numpy().view(np.uint32)
        fs_ok &= bool(np.array_equal(got[r_, c_], accv[ti * (cc // 32) + tj]))
    ac_ok = bool(torch.equal(S, T2))
    sizes = {}
    for tag, ((m_, n_, k_), kind, sd, ab, bb) in other_in.items():
        ms_list, block, Dx = other_run[tag]
        ms_ = float(np.mean(ms_list))
        rs, cs = synth.sample_points(m_, n_, sd[0] + 100, count=256, tile=(block, block))
        got = Dx.cpu().numpy()[rs, cs]
        if kind == "bf16":
            ref_, bnd_ = og.gemm_ref_at(ab, bb, None, m_, n_, k_, False, False, 0.0, "bf16", rs, cs)
            ok_, worst_ = og.check(got, ref_, bnd_)
        else:
            ref_, bnd_ = og.gemm_fp8_ref_at(ab, bb, None, m_, n_, k_, False, True, 0.0, "e4m3", "e4m3",
                                            rs, cs)
            ok_, worst_ = og.check_fp8(got, ref_, bnd_, ab, bb, m_, n_, k_, False, True, "e4m3", "e4m3",
                                       rs, cs)
        sizes[tag] = {"shape": [m_, n_, k_], "block": block, **_stats(ms_list),
                      "TFLOP/s": round(2.0 * m_ * n_ * k_ / (ms_ * 1e-3) / 1e12, 3),
                      "parity": {"sampled_ok": bool(ok_), "worst_err_over_tol": round(float(worst_), 5)}}

    base = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        base = cpu_baseline(gin, copy_src_bits, c3)

    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("tile GEMM 8192x8192x8192 bf16 A,B normal(0,1)/sqrt(K), fp32 D, beta=0 + "
                         "streaming tile copy 2^28 fp16 (16384x16384, 128x64 tiles, 256 threads, "
                         "XOR-swizzled LDS)"),
            "M": M, "N": N, "K": K, "copy_rows": ROWS, "copy_cols": COLS,
        },
        "roofline": {
            "bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_MFMA_TFLOPS, 4), "traffic": traffic_for("gemm_direct_256x256_bf16_nn"),
            "kernel": "gemm_direct<A K-major, B N-major, bf16, 2x4 waves> 256x256x64", **_stats(gemm_ms),
        },
        "timing_note": (f"the legs below ran on the GPU first, back to back ({gpu_legs_s:.1f} s; their "
                        "oracle checks ran after the timed steps), then the warm-up steps and the "
                        "timed steps; HIP events on the launch stream"),
        "copy": {
            "value": round(gbs, 2), "unit": "GB/s", **_stats(copy_ms),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_for("tile_copy_16384x16384_f16")},
            "back_to_back": {"value": round(bb_gbs, 2), "unit": "GB/s", **_stats(bb_list),
                             "frac": round(bb_gbs / PEAK_HBM_GBS, 4),
                             "note": "the same copy launched back to back after the timed steps "
                                     "(5 batches); value above is each step's copy, right after its GEMM"},
            "runtime_copy": {"value": round(rt_gbs, 2), "unit": "GB/s", **_stats(rt_list),
                             "frac": round(rt_gbs / PEAK_HBM_GBS, 4),
                             "note": "context, not this library: torch copy_ (the HIP runtime's "
                                     "device-to-device copy kernel) of the same 512 MiB, back to back"},
        },
        "library_gemm_context": {
            "value": round(flops / (float(np.mean(lib_ctx["lst"])) * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            **_stats(lib_ctx["lst"]),
            "frac": round(flops / (float(np.mean(lib_ctx["lst"])) * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
            "max_abs_diff_vs_tile_gemm": lib_diff,
            "note": f"context, not this library: torch.mm (hipBLASLt) on the same 8192^3 bf16 operands, "
                    f"{lib_ctx['out']} out, per-launch HIP events"},
        "small_configs": small,
        "gemm_f16_transA_beta1": mfma_leg(
            h_ms, PEAK_MFMA_TFLOPS, "gemm_direct_256x256_f16_transA_beta1",
            {"sampled_ok": bool(h_ok), "worst_err_over_tol": round(h_worst, 5)},
            "tile_gemm 8192^3 fp16, A stored [K,M] N(0,1)/sqrt(K), B [K,N], C U[-1,1], beta=1, fp32 D"),
        "gemm_fp8_e4m3_tn": mfma_leg(
            f8_list, PEAK_FP8_TFLOPS, "gemm_fp8_256x256_e4m3_tn",
            {"sampled_ok": bool(f8_ok), "worst_err_over_tol": round(f8_worst, 5),
             "worst_err_over_16bit_tol": round(f8_plain, 5)},
            "tile_gemm_fp8 8192x8192x8192, A e4m3 [M,K] N(0,1), B e4m3 [N,K] N(0,1), fp32 D, beta=0"),
        "gemm_mx_e4m3_tn": mfma_leg(
            mx_list, PEAK_FP8_TFLOPS, "gemm_mx_256x256_e4m3_tn",
            {"sampled_ok": bool(mx_ok), "worst_err_over_tol": round(mx_worst, 5),
             "worst_err_over_16bit_tol": round(mx_plain, 5)},
            "tile_gemm_mx 8192x8192x8192, A e4m3 [M,K], B e4m3 [N,K], E8M0 scales per 32 K in "
            "2^-10..2^10, fp32 D, beta=0"),
        **small_legs,
        "frag_load_a16_32x32x16_col": hbm_leg(
            fl_list, 2.0 * ROWS * COLS * 2, "frag_load_a16_32x32x16_col_16384x16384",
            {"sampled_tiles_bit_exact": fl_ok, "tiles_checked": 64},
            "tile_frag_load: 16384x16384 fp16 U[-1,1] stored column-major -> 32x32x16 A fragments "
            "(runs across memory lines, LDS route with ds_read_b64_tr_b16)"),
        "frag_store_c32_32x32_row": hbm_leg(
            fs_list, 2.0 * cr * cc * 4, "frag_store_c32_32x32_row_8192x16384",
            {"sampled_tiles_bit_exact": fs_ok, "tiles_checked": 64},
            "tile_frag_store: 8192x16384 fp32 32x32 accumulator fragments -> row-major matrix (runs "
            "across memory lines, LDS route)"),
        "copy_async_depth4": hbm_leg(
            ac_list, 2.0 * ROWS * COLS * 2, "tile_copy_async_16384x16384_f16_depth4", {"bit_exact": ac_ok},
            "tile_copy_async: 16384x16384 fp16, 128x64 tiles, 256 threads, XOR LDS, 4 tiles in flight "
            "per workgroup (buffer_load ... lds issue, vmcnt wait for the oldest)"),
        "mma_atoms_4096": {
            "workload": "tile_frag_mma 4096x4096x4096 f16 register images (one wave per output tile, "
                        "operands streamed from the images); each atom that divides the shape",
            "selected": {code: name for name, code in atom_codes}[sel],
            "atoms": atoms,
        },
        "gemm_other_sizes": {
            "workload": "tile_gemm / tile_gemm_fp8 beyond the headline: 8000^3 bf16 (ragged 256x256 "
                        "blocks, 125 K stages) and 2048^3 bf16 / e4m3 (128x128 blocks); A [M,K], "
                        "B [K,N] (bf16) or [N,K] (fp8), beta 0; launches back to back, 5 batches",
            "sizes": sizes,
        },
        "parity": {"gemm_sampled_ok": bool(g_ok), "gemm_worst_err_over_tol": round(g_worst, 5),
                   "copy_bit_exact": c_ok},
        "cpu_baseline": base,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
