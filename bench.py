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
    "gemm_fp8_256x256_e4m3_tn": ("gemm_direct<false, false, 16, 2, 4, false, 0>", "fp8",
                                 2 * M * K + M * N * 4),
    "gemm_mx_256x256_e4m3_tn": ("gemm_direct<false, false, 32, 2, 4, false, 0>", "mx",
                                2 * M * K + 2 * M * (K // 32) + M * N * 4),
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


def cpu_baseline(gemm_inputs, copy_src, budget_s=12.0):
    """Time the oracle as it stands on bounded samples of the same workload (host cores)."""
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
    # one call takes about a quarter of the budget
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
    return {
        "value": round(gemm_tflops, 6), "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
        "sample": (f"gemm: oracle.gemm.gemm_ref (float64 matmul after exact bf16 decode) on rows "
                   f"0..{rows} of the 8192^3 bf16 GEMM, {reps} call(s), {dt:.2f} s each; copy: "
                   f"oracle.copy.copy_ref on {slab} of 16384 rows ({cdt:.2f} s, single thread) = "
                   f"{copy_gbs:.3f} GB/s"),
        "copy_value": round(copy_gbs, 4), "copy_unit": "GB/s", "copy_cores": 1,
        "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
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
              "run on a single MI355X and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import tile_level_gemm_amd as tg

    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    print("bench: generating inputs", file=sys.stderr, flush=True)
    gin = synth.gemm8k_bf16_inputs()
    A, B = up(gin[0]), up(gin[1])
    D = torch.empty((M, N), dtype=torch.float32, device=dev)
    copy_src_bits = synth.stream_input(ROWS, COLS)
    S = up(copy_src_bits)
    T = torch.empty_like(S)
    torch.cuda.synchronize()
    if args.calib_copy:
        T.copy_(S)
        torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        tg.tile_gemm(A, B, None, D, M, N, K, 0, 0, 0.0, tg.TG_BF16)
        if ev is not None:
            ev[1].record()
        tg.tile_copy(S, T, (ROWS, COLS), tg.TG_F16)
        if ev is not None:
            ev[2].record()

    # the legs timed after the steps: at least LEG_WARMUP untimed launches each
    leg_warmup = max(args.warmup, LEG_WARMUP)
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
    flops = 2.0 * M * N * K
    tflops = flops / (g_avg * 1e-3) / 1e12
    copy_bytes = 2.0 * ROWS * COLS * 2
    gbs = copy_bytes / (c_avg * 1e-3) / 1e9

    # parity spot check of the timed outputs (sampled GEMM outputs, full copy identity)
    from oracle import gemm as og
    rows, cols = synth.sample_points(M, N, 53, count=256)
    ref, bound = og.gemm_ref_at(gin[0], gin[1], None, M, N, K, False, False, 0.0, "bf16", rows, cols)
    g_ok, g_worst = og.check(D.cpu().numpy()[rows, cols], ref, bound)
    c_ok = bool(torch.equal(S, T))

    # the same copy back to back (no GEMM between launches): the copy on its own
    bb_reps = max(5, args.steps // 2)
    bev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    tg.tile_copy(S, T, (ROWS, COLS), tg.TG_F16)
    torch.cuda.synchronize()
    bev[0].record()
    for _ in range(bb_reps):
        tg.tile_copy(S, T, (ROWS, COLS), tg.TG_F16)
    bev[1].record()
    torch.cuda.synchronize()
    bb_ms = bev[0].elapsed_time(bev[1]) / bb_reps
    bb_gbs = copy_bytes / (bb_ms * 1e-3) / 1e9

    # fp16 transA beta=1 variant of the same GEMM
    hin = synth.gemm8k_f16_inputs()
    Ah, Bh = up(hin[0]), up(hin[1])
    Ch = torch.from_numpy(hin[2]).to(dev)
    for _ in range(leg_warmup):
        tg.tile_gemm(Ah, Bh, Ch, D, M, N, K, 1, 0, 1.0, tg.TG_F16)
    hev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    hev[0].record()
    reps = max(3, args.steps // 2)
    for _ in range(reps):
        tg.tile_gemm(Ah, Bh, Ch, D, M, N, K, 1, 0, 1.0, tg.TG_F16)
    hev[1].record()
    torch.cuda.synchronize()
    h_ms = hev[0].elapsed_time(hev[1]) / reps
    del Ah, Bh, Ch

    # fp8 e4m3 x e4m3 GEMM of the same size, K-contiguous A [M,K] and B [N,K]
    print("bench: fp8 gemm", file=sys.stderr, flush=True)
    fin = synth.gemm8k_fp8_inputs()
    A8 = torch.from_numpy(np.ascontiguousarray(fin[0])).to(dev)
    B8 = torch.from_numpy(np.ascontiguousarray(fin[1])).to(dev)
    e4 = tg.TG_FP8_E4M3
    for _ in range(leg_warmup):
        tg.tile_gemm_fp8(A8, B8, None, D, M, N, K, 0, 1, 0.0, e4, e4)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    torch.cuda.synchronize()
    for ev in fev:
        ev[0].record()
        tg.tile_gemm_fp8(A8, B8, None, D, M, N, K, 0, 1, 0.0, e4, e4)
        ev[1].record()
    torch.cuda.synchronize()
    f8_ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in fev]))
    f8_tflops = flops / (f8_ms * 1e-3) / 1e12
    ref8, bound8 = og.gemm_fp8_ref_at(fin[0], fin[1], None, M, N, K, False, True, 0.0, "e4m3",
                                      "e4m3", rows, cols)
    f8_ok, f8_worst = og.check_fp8(D.cpu().numpy()[rows, cols], ref8, bound8, fin[0], fin[1], M, N,
                                   K, False, True, "e4m3", "e4m3", rows, cols)

    # block-scaled (MX) e4m3 GEMM: E8M0 scales per 32 K, 2^-10 .. 2^10
    print("bench: mx gemm", file=sys.stderr, flush=True)
    g = synth.rng(64)
    sa = g.integers(117, 138, size=(M, K // 32)).astype(np.uint8)
    sb = g.integers(117, 138, size=(N, K // 32)).astype(np.uint8)
    SA = torch.from_numpy(sa).to(dev)
    SB = torch.from_numpy(sb).to(dev)
    for _ in range(leg_warmup):
        tg.tile_gemm_mx(A8, B8, SA, SB, None, D, M, N, K, 0, 1, 0.0, e4, e4)
    mev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    torch.cuda.synchronize()
    for ev in mev:
        ev[0].record()
        tg.tile_gemm_mx(A8, B8, SA, SB, None, D, M, N, K, 0, 1, 0.0, e4, e4)
        ev[1].record()
    torch.cuda.synchronize()
    mx_ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in mev]))
    mx_tflops = flops / (mx_ms * 1e-3) / 1e12
    refm, boundm = og.gemm_mx_ref_at(fin[0], fin[1], sa, sb, None, M, N, K, False, True, 0.0, "e4m3",
                                     "e4m3", rows, cols)
    mx_ok, mx_worst = og.check_fp8(D.cpu().numpy()[rows, cols], refm, boundm, fin[0], fin[1], M, N, K,
                                   False, True, "e4m3", "e4m3", rows, cols, sa_bits=sa, sb_bits=sb)
    del A8, B8, SA, SB

    # register fragment copies (tile_frag_load / tile_frag_store, LDS route)
    print("bench: fragment copies", file=sys.stderr, flush=True)
    from oracle import fragment as ofr
    from oracle.layout import Layout as OLayout
    img = torch.empty_like(S)
    col = (tg.TG_COL_MAJOR, 0)
    frag = {}

    def time_call(call, nbytes):
        for _ in range(leg_warmup):
            call()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        torch.cuda.synchronize()
        for ev in evs:
            ev[0].record()
            call()
            ev[1].record()
        torch.cuda.synchronize()
        ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in evs]))
        gb = nbytes / (ms * 1e-3) / 1e9
        return ms, gb

    fl_ms, fl_gbs = time_call(lambda: tg.tile_frag_load(S, img, (ROWS, COLS), tg.TG_F16, col,
                                                        tg.TG_FRAG_A16_32x32x16), 2.0 * ROWS * COLS * 2)
    gi = synth.rng(79)
    fl_ok = True
    imgv = img.view(-1, 64, 8)
    for _ in range(64):
        ti, tj = int(gi.integers(ROWS // 32)), int(gi.integers(COLS // 16))
        want = ofr.frag_load(copy_src_bits, 32, 16, OLayout("col", ld=ROWS, base=tj * 16 * ROWS + ti * 32),
                             "a16_32x32x16")[0]
        fl_ok &= bool(np.array_equal(imgv[ti * (COLS // 16) + tj].cpu().numpy().view(np.uint16), want))
    frag["frag_load_a16_32x32x16_col"] = {
        "value": round(fl_gbs, 2), "unit": "GB/s", "avg_ms": round(fl_ms, 5),
        "workload": "tile_frag_load: 16384x16384 fp16 U[-1,1] stored column-major -> 32x32x16 A "
                    "fragments (runs across memory lines, LDS route with ds_read_b64_tr_b16)",
        "roofline": {"bound": "hbm", "achieved": round(fl_gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(fl_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for("frag_load_a16_32x32x16_col_16384x16384")},
        "parity": {"sampled_tiles_bit_exact": fl_ok, "tiles_checked": 64},
    }
    cr, cc = ROWS // 2, COLS
    acc_bits = synth.uniform(43, cr * cc).view(np.uint32)
    acc = torch.from_numpy(acc_bits.view(np.int32)).to(dev)
    mat = torch.empty_like(acc)
    fs_ms, fs_gbs = time_call(lambda: tg.tile_frag_store(acc, mat, (cr, cc), tg.TG_F32,
                                                         (tg.TG_ROW_MAJOR, 0), tg.TG_FRAG_C32_32x32),
                              2.0 * cr * cc * 4)
    r_, c_ = ofr.coords("c32_32x32")
    host = mat.view(cr, cc)
    accv = acc_bits.reshape(-1, 64, 16)
    fs_ok = True
    for _ in range(64):
        ti, tj = int(gi.integers(cr // 32)), int(gi.integers(cc // 32))
        got = host[ti * 32:(ti + 1) * 32, tj * 32:(tj + 1) * 32].cpu().numpy().view(np.uint32)
        fs_ok &= bool(np.array_equal(got[r_, c_], accv[ti * (cc // 32) + tj]))
    frag["frag_store_c32_32x32_row"] = {
        "value": round(fs_gbs, 2), "unit": "GB/s", "avg_ms": round(fs_ms, 5),
        "workload": "tile_frag_store: 8192x16384 fp32 32x32 accumulator fragments -> row-major "
                    "matrix (runs across memory lines, LDS route)",
        "roofline": {"bound": "hbm", "achieved": round(fs_gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(fs_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for("frag_store_c32_32x32_row_8192x16384")},
        "parity": {"sampled_tiles_bit_exact": fs_ok, "tiles_checked": 64},
    }
    del img, acc, mat

    # asynchronous tile copy: issue-only global -> LDS transfers, 4 tiles in flight per workgroup
    print("bench: async copy", file=sys.stderr, flush=True)
    aopts = dict(tile_rows=128, tile_cols=64, threads=256, lds_kind=tg.TG_XOR_SWIZZLE, depth=4)
    T.zero_()
    ac_ms, ac_gbs = time_call(lambda: tg.tile_copy_async(S, T, (ROWS, COLS), tg.TG_F16, None, None,
                                                         aopts), 2.0 * ROWS * COLS * 2)
    frag["copy_async_depth4"] = {
        "value": round(ac_gbs, 2), "unit": "GB/s", "avg_ms": round(ac_ms, 5),
        "workload": "tile_copy_async: 16384x16384 fp16, 128x64 tiles, 256 threads, XOR LDS, 4 tiles "
                    "in flight per workgroup (buffer_load ... lds issue, vmcnt wait for the oldest)",
        "roofline": {"bound": "hbm", "achieved": round(ac_gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(ac_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for("tile_copy_async_16384x16384_f16_depth4")},
        "parity": {"bit_exact": bool(torch.equal(S, T))},
    }

    # widest-first atom selection: the register-level product at 4096^3 f16 with each atom that
    # divides it; tile_mma_select names the first of them
    print("bench: register-level product per atom", file=sys.stderr, flush=True)
    n4 = 4096
    sel = tg.tile_mma_select(n4, n4, n4, tg.TG_F16, tg.TG_F16)
    img_a = torch.empty(n4 * n4, dtype=torch.int16, device=dev).random_(0, 14000)   # finite f16
    img_b = torch.empty_like(img_a).random_(0, 14000)
    img_d = torch.empty(n4 * n4, dtype=torch.float32, device=dev)
    atoms = {}
    for name, code in (("32x32x16", tg.TG_MMA_32x32x16), ("16x16x32", tg.TG_MMA_16x16x32),
                       ("32x32x8", tg.TG_MMA_32x32x8), ("16x16x16", tg.TG_MMA_16x16x16)):
        ms_, _ = time_call(lambda: tg.tile_frag_mma(img_a, img_b, None, img_d, n4, n4, n4, 0.0,
                                                    tg.TG_F16, tg.TG_F16, code), 1.0)
        atoms[name] = {"avg_ms": round(ms_, 5),
                       "TFLOP/s": round(2.0 * n4 ** 3 / (ms_ * 1e-3) / 1e12, 3)}
    frag["mma_atoms_4096"] = {
        "workload": "tile_frag_mma 4096x4096x4096 f16 register images (one wave per output tile, "
                    "operands streamed from the images); each atom that divides the shape",
        "selected": {v: k for k, v in {"32x32x16": tg.TG_MMA_32x32x16, "16x16x32": tg.TG_MMA_16x16x32,
                                       "32x32x8": tg.TG_MMA_32x32x8,
                                       "16x16x16": tg.TG_MMA_16x16x16}.items()}[sel],
        "atoms": atoms,
    }
    del img_a, img_b, img_d

    # the block-size choice on problems other than the headline: ragged 8000^3 and mid-size
    # 2048^3 (128x128 blocks), bf16 and fp8, each with sampled outputs against the oracle
    print("bench: other sizes", file=sys.stderr, flush=True)
    sizes = {}
    for tag, (m_, n_, k_), kind in (("bf16_8000", (8000, 8000, 8000), "bf16"),
                                    ("bf16_2048", (2048, 2048, 2048), "bf16"),
                                    ("fp8_2048", (2048, 2048, 2048), "fp8")):
        sd = {"bf16_8000": (91, 92), "bf16_2048": (93, 94), "fp8_2048": (95, 96)}[tag]
        if kind == "bf16":
            sc = float(1.0 / np.sqrt(k_))
            ab, bb, _ = synth.gemm_inputs(m_, n_, k_, "bf16", False, False, 0.0, (sd[0], sd[1], 0),
                                          a_scale=sc, b_scale=sc)
        else:
            ab, bb, _ = synth.gemm_fp8_inputs(m_, n_, k_, "e4m3", "e4m3", False, True, 0.0,
                                              (sd[0], sd[1], 0))
        Ax, Bx = up(ab), up(bb)
        Dx = torch.empty((m_, n_), dtype=torch.float32, device=dev)
        if kind == "bf16":
            plan = tg.tile_gemm_plan(Ax, Bx, None, Dx, m_, n_, k_, 0, 0, 0.0, tg.TG_BF16)
            call = lambda: tg.tile_gemm(Ax, Bx, None, Dx, m_, n_, k_, 0, 0, 0.0, tg.TG_BF16)  # noqa: E731
        else:
            plan = tg.tile_gemm_fp8_plan(Ax, Bx, None, Dx, m_, n_, k_, 0, 1, 0.0, e4, e4)
            call = lambda: tg.tile_gemm_fp8(Ax, Bx, None, Dx, m_, n_, k_, 0, 1, 0.0, e4, e4)  # noqa: E731
        # launched back to back between one pair of events: at 2048^3 a kernel takes about as
        # long as a launch from Python, and events around each launch would time the gaps too
        for _ in range(leg_warmup):
            call()
        bev2 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        bev2[0].record()
        for _ in range(reps):
            call()
        bev2[1].record()
        torch.cuda.synchronize()
        ms_ = bev2[0].elapsed_time(bev2[1]) / reps
        rs, cs = synth.sample_points(m_, n_, sd[0] + 100, count=256, tile=(plan.block_m, plan.block_n))
        got = Dx.cpu().numpy()[rs, cs]
        if kind == "bf16":
            ref_, bnd_ = og.gemm_ref_at(ab, bb, None, m_, n_, k_, False, False, 0.0, "bf16", rs, cs)
            ok_, worst_ = og.check(got, ref_, bnd_)
        else:
            ref_, bnd_ = og.gemm_fp8_ref_at(ab, bb, None, m_, n_, k_, False, True, 0.0, "e4m3", "e4m3",
                                            rs, cs)
            ok_, worst_ = og.check_fp8(got, ref_, bnd_, ab, bb, m_, n_, k_, False, True, "e4m3", "e4m3",
                                       rs, cs)
        sizes[tag] = {"shape": [m_, n_, k_], "block": plan.block_m, "avg_ms": round(ms_, 5),
                      "TFLOP/s": round(2.0 * m_ * n_ * k_ / (ms_ * 1e-3) / 1e12, 3),
                      "parity": {"sampled_ok": bool(ok_), "worst_err_over_tol": round(float(worst_), 5)}}
        del Ax, Bx, Dx
    frag["gemm_other_sizes"] = {
        "workload": "tile_gemm / tile_gemm_fp8 beyond the headline: 8000^3 bf16 (ragged 256x256 "
                    "blocks, 125 K stages) and 2048^3 bf16 / e4m3 (128x128 blocks); A [M,K], "
                    "B [K,N] (bf16) or [N,K] (fp8), beta 0; launches back to back, averaged",
        "sizes": sizes,
    }

    base = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        base = cpu_baseline(gin, copy_src_bits)

    gemm_traffic = traffic_for("gemm_direct_256x256_bf16_nn")
    copy_traffic = traffic_for("tile_copy_16384x16384_f16")
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
            "frac": round(tflops / PEAK_MFMA_TFLOPS, 4), "traffic": gemm_traffic,
            "kernel": "gemm_direct<A K-major, B N-major, bf16, 2x4 waves> 256x256x64", "avg_ms": round(g_avg, 5),
        },
        "copy": {
            "value": round(gbs, 2), "unit": "GB/s", "avg_ms": round(c_avg, 5),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": copy_traffic},
            "back_to_back": {"value": round(bb_gbs, 2), "unit": "GB/s", "avg_ms": round(bb_ms, 5),
                             "frac": round(bb_gbs / PEAK_HBM_GBS, 4),
                             "note": "the same copy launched back to back after the timed steps; "
                                     "value above is each step's copy, right after its GEMM"},
        },
        "gemm_f16_transA_beta1": {"value": round(flops / (h_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
                                   "avg_ms": round(h_ms, 5),
                                   "frac": round(flops / (h_ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4)},
        "gemm_fp8_e4m3_tn": {
            "value": round(f8_tflops, 3), "unit": "TFLOP/s", "avg_ms": round(f8_ms, 5),
            "workload": "tile_gemm_fp8 8192x8192x8192, A e4m3 [M,K] N(0,1), B e4m3 [N,K] N(0,1), "
                        "fp32 D, beta=0",
            "roofline": {"bound": "mfma", "achieved": round(f8_tflops, 3), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(f8_tflops / PEAK_FP8_TFLOPS, 4),
                         "traffic": traffic_for("gemm_fp8_256x256_e4m3_tn")},
            "parity": {"sampled_ok": bool(f8_ok), "worst_err_over_tol": round(f8_worst, 5)},
        },
        "gemm_mx_e4m3_tn": {
            "value": round(mx_tflops, 3), "unit": "TFLOP/s", "avg_ms": round(mx_ms, 5),
            "workload": "tile_gemm_mx 8192x8192x8192, A e4m3 [M,K], B e4m3 [N,K], E8M0 scales per "
                        "32 K in 2^-10..2^10, fp32 D, beta=0",
            "roofline": {"bound": "mfma", "achieved": round(mx_tflops, 3), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(mx_tflops / PEAK_FP8_TFLOPS, 4),
                         "traffic": traffic_for("gemm_mx_256x256_e4m3_tn")},
            "parity": {"sampled_ok": bool(mx_ok), "worst_err_over_tol": round(mx_worst, 5)},
        },
        **frag,
        "parity": {"gemm_sampled_ok": bool(g_ok), "gemm_worst_err_over_tol": round(g_worst, 5),
                   "copy_bit_exact": c_ok},
        "cpu_baseline": base,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
