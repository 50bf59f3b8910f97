"""Benchmark of the hot path on one MI355X: multi-destination all-gather + fused GEMM + all-gather.

One step = one complete logical all-gather job on one GPU:
  * all-gather: every one of the W=8 logical ranks calls ag_all_gather on its
    1024 x 4096 fp16 input (tile 8x256, 128 programs), so every heap region
    ends up with the 8192 x 4096 gathered tensor;
  * fused: every one of the 8 logical ranks calls ag_gemm_all_gather with
    A_g 16384 x 8192 and the shared B 8192 x 3584 (fp16, fp32 accumulate),
    so every region ends up with the 131072 x 3584 gathered C (the fused
    workload whose MFMA-utilisation target is stated; --fused-m 1024 selects
    the M_local = 1024 variant).
Inputs are seeded synthetic tensors already resident in HBM.

Printed: one JSON line.  value = all-gather HBM GB/s over the whole job
((1+W)*M_local*N*e bytes per call, W calls per step); the fused path's
TFLOP/s is reported in the "fused" object, each with its roofline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "all-gather achieved HBM GB/s (+% peak); fused GEMM+AG TFLOP/s (+% MFMA peak)"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0

# all-gather workload: W=8 logical ranks, 1024 x 4096 fp16 per rank, tile 8x256; of the program
# counts the workload is defined for (64/128/256, all three timed in "context"), 128
AG_W, AG_M, AG_N, AG_DTYPE, AG_TILE, AG_PROGRAMS = 8, 1024, 4096, "f16", (8, 256), 128
# fused workload: W=8, M_local 16384, K 8192, N 3584, fp16
FU_W, FU_N, FU_K, FU_DTYPE = 8, 3584, 8192, "f16"
FU_M = 16384


def _src_hash(name: str) -> str:
    with open(os.path.join(ROOT, "gemm_all_gather_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(summary: str, source: str, per_launch_alg: float):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None.

    The summary records the source hash of the kernel file it was taken on;
    a changed kernel makes the recorded counters stale (None).
    """
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != _src_hash(source):
        return None
    return float(m_bytes.group(1))


def _cpu_baseline_copy(seconds: float):
    """The oracle's all-gather of the same workload on the host cores (a bounded sample)."""
    import numpy as np
    from gemm_all_gather_amd import inputs as gen
    import oracle

    e = 2
    blk = AG_M * AG_N * e
    S = AG_W * blk
    ins = [gen.uniform_pm1((AG_M, AG_N), AG_DTYPE, 1, j) for j in range(AG_W)]
    slab = np.zeros(AG_W * S, dtype=np.uint8)
    oracle.all_gather_oracle(slab, S, ins, 0, 1, 0)        # warm-up
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.all_gather_oracle(slab, S, ins, 0, 1, 0)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    job_bytes = AG_W * (1 + AG_W) * blk
    return {"value": job_bytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} whole all-gather jobs (W=8, {AG_M}x{AG_N} fp16 per rank, full 8-region heap "
                      f"copy included) in {reps * dt:.1f} s with numpy on 1 host thread"}


def _cpu_baseline_fused(seconds: float):
    """The oracle's fused GEMM + all-gather for a bounded sample of output rows of one rank's call."""
    import numpy as np
    from gemm_all_gather_amd import inputs as gen
    import oracle

    threads = len(os.sched_getaffinity(0))
    rows = 64
    a = gen.normal_scaled((rows, FU_K), FU_DTYPE, FU_K ** -0.5, 2, 0)
    b = gen.normal_scaled((FU_N, FU_K), FU_DTYPE, FU_K ** -0.5, 3)
    oracle.gemm_oracle(a[:8], b, FU_DTYPE, "nk")             # warm-up
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.gemm_oracle(a, b, FU_DTYPE, "nk")
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    flops = 2.0 * rows * FU_N * FU_K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x {rows} output rows of one rank's {FU_M}x{FU_N}x{FU_K} fp16 product "
                      f"(float64 numpy matmul + rounding), {reps * dt:.1f} s; BLAS may use up to {threads} threads"}


def _context(args, stream, timed, views, ins, geom):
    """Context measurements beside the headline (each job = the 8 ranks' calls, timed like it).

    * the all-gather workload at the three program counts it is defined for;
    * destination groups 1/2/4 and the partitioned schedule (all-gather variants);
    * the all-to-all on the same heap: W=8, 8 chunks of 1024x4096 fp16 per rank, tile and partitioned
      schedules;
    * the all-gather at 16384x8192 per rank in fp16, bf16 and fp32 (2.4 / 2.4 / 4.8 GB per call);
    * the edge shapes: 1000x4100 fp16 (8-byte vectors, partial last column tile) at W=8, and the
      strided group of ranks 1, 3, 5, 7 (W=4) at 1000x4100 and 16384x8192.
    """
    import torch
    from gemm_all_gather_amd import binding as ag

    steps = max(10, args.steps // 4)
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup = steps, max(2, args.warmup // 2)
    blk = AG_M * AG_N * 2
    per_call = (1 + AG_W) * blk

    def gbs(ms, bytes_per_call):
        return round(AG_W * bytes_per_call / (ms / 1e3) / 1e9, 1)

    ctx = {"steps": steps}
    res = {}
    for P in (64, 128, 256):
        ms, _ = timed_sub(sub, timed, lambda P=P: [ag.all_gather(views[j], AG_W, 0, 1, ins[j], 0, AG_M, AG_N, AG_DTYPE,
                                                                  *AG_TILE, P, stream) for j in range(AG_W)])
        res[str(P)] = gbs(ms, per_call)
    ctx["all_gather_GBs_by_programs"] = res
    res = {}
    for G in (1, 2, 4):
        ms, _ = timed_sub(sub, timed, lambda G=G: [ag.all_gather_ex(views[j], AG_W, 0, 1, ins[j], 0, AG_M, AG_N,
                                                                     AG_DTYPE, *AG_TILE, AG_PROGRAMS, G, 0, stream)
                                                   for j in range(AG_W)])
        res[str(G)] = gbs(ms, per_call)
    ctx["all_gather_GBs_by_dest_group"] = res
    res = {}
    for P in (64, 128, 256):
        ms, _ = timed_sub(sub, timed, lambda P=P: [ag.all_gather_ex(views[j], AG_W, 0, 1, ins[j], 0, AG_M, AG_N,
                                                                     AG_DTYPE, *AG_TILE, P, 0, "partitioned", stream)
                                                   for j in range(AG_W)])
        # HBM bytes of the schedule: every destination reads the tile itself
        res[str(P)] = gbs(ms, 2 * AG_W * blk)
    ctx["partitioned_GBs_by_programs"] = res

    # all-to-all: each rank sends 8 chunks of 1024x4096 fp16 (64 MiB per rank); 8x512 tiles, two 16-byte
    # vectors per thread (measured 5.3 TB/s against 5.0 for 8x256 at 256 programs)
    A2A_TILE = (8, 512)
    mc = AG_M
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    a2a_in = [torch.randint(-32768, 32767, (AG_W * mc * AG_N,), generator=g, dtype=torch.int16, device="cuda")
              for _ in range(AG_W)]
    a2a_plan = ag.plan_all_to_all(geom, AG_W, 0, 1, a2a_in[0], 0, mc, AG_N, AG_DTYPE, *A2A_TILE, 256)
    ms, _ = timed_sub(sub, timed, lambda: [ag.all_to_all(views[j], AG_W, 0, 1, a2a_in[j], 0, mc, AG_N, AG_DTYPE,
                                                         *A2A_TILE, 256, stream) for j in range(AG_W)])
    a2a_bytes = a2a_plan.bytes_read + a2a_plan.bytes_written
    launch_s = ms / 1e3 / AG_W
    ctx["all_to_all"] = {
        "workload": f"all-to-all W={AG_W}, {AG_W} chunks of {mc}x{AG_N} fp16 per rank, tile {A2A_TILE[0]}x{A2A_TILE[1]}, "
                    f"{a2a_plan.n_programs} programs (8 calls per job)",
        "value": round(AG_W * a2a_bytes / (ms / 1e3) / 1e9, 1), "unit": "GB/s",
        "roofline": {"bound": "hbm", "achieved": round(a2a_bytes / launch_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(a2a_bytes / launch_s / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": _traffic(f"ag_a2a_kernel_w{AG_W}_{mc}x{AG_N}_f16_pmc.md", "ag_copy.hip", a2a_bytes),
                     "alg_bytes_per_launch": a2a_bytes, "avg_launch_us": round(launch_s * 1e6, 3)},
    }
    # the partitioned schedule of the same exchange (program p copies one chunk to destination p mod W)
    ms, _ = timed_sub(sub, timed, lambda: [ag.all_to_all_ex(views[j], AG_W, 0, 1, a2a_in[j], 0, mc, AG_N, AG_DTYPE,
                                                            16, 512, 256, schedule="partitioned", stream=stream)
                                           for j in range(AG_W)])
    ctx["all_to_all"]["partitioned_16x512_256_programs_GBs"] = round(AG_W * a2a_bytes / (ms / 1e3) / 1e9, 1)
    del a2a_in

    sub3 = argparse.Namespace(**vars(sub))
    sub3.steps, sub3.warmup = 5, 1

    def gather_rate(M3, N3, dtype, W3, start, stride, programs, seed):
        """GB/s of one group's all-gather job ((1+W)*M*N*e per call) on a fresh 8-region heap."""
        e3 = 4 if dtype == "f32" else 2
        blk3 = M3 * N3 * e3
        S3 = ((8 * blk3) // (2 << 20) + 1) * (2 << 20)
        slab3 = torch.empty(8 * S3, dtype=torch.uint8, device="cuda")
        heap3 = ag.Heap.wrap(slab3, 8, S3)
        views3 = [heap3.view(r) for r in range(8)]
        members = [start + i * stride for i in range(W3)]
        g.manual_seed(seed)
        in3 = [torch.randint(-32768, 32767, (blk3 // 2,), generator=g, dtype=torch.int16, device="cuda")
               for _ in members]
        ms, _ = timed_sub(sub3, timed, lambda: [ag.all_gather(views3[r], W3, start, stride, in3[i], 0, M3, N3,
                                                              dtype, 0, 0, programs, stream)
                                                for i, r in enumerate(members)])
        for v in views3:
            v.destroy()
        heap3.destroy()
        del slab3, in3
        torch.cuda.empty_cache()
        return round(W3 * (1 + W3) * blk3 / (ms / 1e3) / 1e9, 1)

    # the all-gather at 16384 x 8192 per rank (2.4 GB per call in 16 bits), three element types
    ctx["all_gather_16384x8192_256_programs_GBs_by_dtype"] = {
        dt: gather_rate(16384, 8192, dt, AG_W, 0, 1, 256, 6) for dt in ("f16", "bf16", "f32")}
    # the edge shapes: rows of 4100 elements (8-byte vectors, partial last column tile); the strided
    # group of ranks 1, 3, 5, 7 (W=4) at both sizes
    ctx["all_gather_edges_GBs"] = {
        "1000x4100_f16_W8": gather_rate(1000, 4100, "f16", AG_W, 0, 1, 256, 7),
        "1000x4100_f16_W4_group_1_2": gather_rate(1000, 4100, "f16", 4, 1, 2, 256, 8),
        "16384x8192_f16_W4_group_1_2": gather_rate(16384, 8192, "f16", 4, 1, 2, 256, 9),
    }
    return ctx


def _context_fused(args, stream, timed, views, fu_off):
    """The fused workload at M_local 1024 (fp16), at M_local 16384 in bf16, and at M_local 16384 in fp16 with B
    stored N-contiguous (a row-major K x N matrix), W=8, timed like the headline."""
    import numpy as np
    import torch
    from gemm_all_gather_amd import binding as ag
    from gemm_all_gather_amd import inputs as gen

    res = {}
    region = views[0].geometry().bytes_per_rank
    for name, M, dtype, layout in (("M1024_f16", 1024, "f16", "k"), ("M16384_bf16", 16384, "bf16", "k"),
                                   ("M16384_f16_B_row_major_KxN", 16384, "f16", "n")):
        sub = argparse.Namespace(**vars(args))
        if M * FU_N * FU_K < (1 << 36):
            # short calls (~75 us): the headline's warm-up steps, so the clocks settle after the workloads
            # before (2 steps, about 1 ms, measured 88-93 us per call against 74.6 with 50)
            sub.steps, sub.warmup = max(20, args.steps // 5), args.warmup
        else:
            sub.steps, sub.warmup = max(5, args.steps // 10), 2
        own = None
        if M != FU_M:
            # a heap of its own, regions sized for this workload's gathered output, as for the
            # all-gather workloads (the region stride moves the store rate)
            S = -(-(FU_W * M * FU_N * 2) // (2 << 20)) * (2 << 20)
            own_slab = torch.zeros(FU_W * S, dtype=torch.uint8, device="cuda")
            own = ag.Heap.wrap(own_slab, FU_W, S)
            vws, off = [own.view(r) for r in range(FU_W)], 0
        else:
            vws, off = views, fu_off
        if off + FU_W * M * FU_N * 2 > (region if own is None else S):
            continue
        fa = [torch.from_numpy(gen.normal_scaled((M, FU_K), dtype, FU_K ** -0.5, 12, j).view(np.uint8)
                               .reshape(-1).copy()).cuda() for j in range(FU_W)]
        b_nk = gen.normal_scaled((FU_N, FU_K), dtype, FU_K ** -0.5, 13)
        b_host = b_nk if layout == "k" else np.ascontiguousarray(b_nk.T)
        ldb = FU_K if layout == "k" else FU_N
        fb = torch.from_numpy(b_host.view(np.uint8).reshape(-1).copy()).cuda()
        ms, _ = timed(lambda: [ag.gemm_all_gather_ex(vws[j], FU_W, 0, 1, fa[j], FU_K, fb, ldb, off, M, FU_N,
                                                     FU_K, dtype, 0, 0, 0, 0, b_layout=layout, stream=stream)
                               for j in range(FU_W)], sub)
        flops = 2.0 * M * FU_N * FU_K
        tf = FU_W * flops / (ms / 1e3) / 1e12
        res[name] = {"TFLOPs": round(tf, 1), "frac_of_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                     "us_per_call": round(ms * 1e3 / FU_W, 1)}
        del fa, fb
        if own is not None:
            torch.cuda.synchronize()
            for v in vws:
                v.destroy()
            own.destroy()
            del own_slab
        torch.cuda.empty_cache()
    return res


def _calibration(stream):
    """Plain device copy and fill of 2 GiB: what the part reaches on a pure stream (context only)."""
    import torch
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    out = {}
    for name, fn, nbytes in (("copy_2GiB_GBs", lambda: dst.copy_(src), 2 * n), ("fill_2GiB_GBs", lambda: dst.fill_(3), n)):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        ts.sort()
        out[name] = round(nbytes / ts[len(ts) // 2] / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return out


def timed_sub(sub, timed, job):
    return timed(job, sub)


def main() -> int:
    global FU_M
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused-m", type=int, default=FU_M, help="M_local of the fused workload (16384 or 1024)")
    ap.add_argument("--only", choices=["all", "copy", "fused"], default="all",
                    help="restrict the timed step to one kernel (profiling runs)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context measurements (program counts, destination groups, partitioned "
                         "schedule, all-to-all, 16384x8192 all-gather in three types, edge shapes, the fused "
                         "workload at M_local 1024 and in bf16, plain copy/fill calibration)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB "
                         "(reference for HBM byte counters)")
    args = ap.parse_args()
    FU_M = args.fused_m
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the W logical ranks are regions of one GPU's HBM; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from gemm_all_gather_amd import binding as ag
    from gemm_all_gather_amd import inputs as gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ag.lib()
    dev_props = torch.cuda.get_device_properties(0)
    stream = torch.cuda.current_stream()

    # ---------------- all-gather setup
    e = 2
    blk = AG_M * AG_N * e
    # each workload has a heap of its own, every region sized for its gathered output (2 MiB multiples)
    S = -(-(AG_W * blk) // (2 << 20)) * (2 << 20)
    slab = torch.empty(AG_W * S, dtype=torch.uint8, device="cuda")
    slab.zero_()
    heap = ag.Heap.wrap(slab, AG_W, S)
    views = [heap.view(r) for r in range(AG_W)]
    ins = [torch.from_numpy(gen.uniform_pm1((AG_M, AG_N), AG_DTYPE, 1, j).view(np.uint8).reshape(-1).copy()).cuda()
           for j in range(AG_W)]
    geom = views[0].geometry()
    ag_plan = ag.plan_all_gather(geom, AG_W, 0, 1, ins[0], 0, AG_M, AG_N, AG_DTYPE, *AG_TILE, AG_PROGRAMS)

    def copy_job():
        if args.only == "fused":
            return
        for j in range(AG_W):
            ag.all_gather(views[j], AG_W, 0, 1, ins[j], 0, AG_M, AG_N, AG_DTYPE, AG_TILE[0], AG_TILE[1],
                          AG_PROGRAMS, stream)

    # ---------------- fused setup
    fused_ok = args.only != "copy"
    fa = [torch.from_numpy(gen.normal_scaled((FU_M, FU_K), FU_DTYPE, FU_K ** -0.5, 2, j).view(np.uint8)
                           .reshape(-1).copy()).cuda() for j in range(FU_W)]
    fb = torch.from_numpy(gen.normal_scaled((FU_N, FU_K), FU_DTYPE, FU_K ** -0.5, 3).view(np.uint8)
                          .reshape(-1).copy()).cuda()
    fblk = FU_M * FU_N * 2
    SF = -(-(FU_W * fblk) // (2 << 20)) * (2 << 20)
    fslab = torch.empty(FU_W * SF, dtype=torch.uint8, device="cuda")
    fslab.zero_()
    fheap = ag.Heap.wrap(fslab, FU_W, SF)
    fviews = [fheap.view(r) for r in range(FU_W)]
    fu_off = 0

    def fused_job():
        if args.only == "copy":
            return
        for j in range(FU_W):
            ag.gemm_all_gather(fviews[j], FU_W, 0, 1, fa[j], FU_K, fb, FU_K, fu_off, FU_M, FU_N, FU_K, FU_DTYPE,
                               0, 0, 0, 0, stream)

    fu_plan = ag.plan_gemm_all_gather(fviews[0].geometry(), FU_W, 0, 1, fa[0], FU_K, fb, FU_K, fu_off, FU_M, FU_N,
                                      FU_K, FU_DTYPE)

    # ---------------- warm-up and timed regions: the all-gather job K times, then the fused job K
    # times, each region bracketed by device synchronisation; a step is one of each
    spread = {}

    # K steps between one pair of HIP events, bracketed by device synchronisation.  (An event pair
    # around every step measured ~2% slower on the all-gather job: the kernel after each event
    # record starts later.)  With blocks > 0, that many further runs of up to 20 steps, each with
    # its own event pair, give the spread of the per-step time.
    def timed(job, a=args, blocks=0):
        for _ in range(a.warmup):
            job()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(a.steps):
            job()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per_step = start.elapsed_time(end) / a.steps
        if blocks:
            nb = min(20, a.steps)
            runs = []
            for _ in range(blocks):
                s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s0.record(stream)
                for _ in range(nb):
                    job()
                s1.record(stream)
                torch.cuda.synchronize()
                runs.append(s0.elapsed_time(s1) / nb)
            runs.sort()
            spread[id(job)] = {"blocks": blocks, "steps_per_block": nb, "step_ms_median": round(runs[len(runs) // 2], 5),
                               "step_ms_min": round(runs[0], 5), "step_ms_max": round(runs[-1], 5)}
        return per_step, wall

    copy_ms, wall_copy = timed(copy_job, blocks=3) if args.only != "fused" else (0.0, 0.0)
    fused_ms, wall_fused = timed(fused_job, blocks=3) if (fused_ok and args.only != "copy") else (0.0, 0.0)
    step_ms = copy_ms + fused_ms
    wall = wall_copy + wall_fused
    if args.calib_copy_mib > 0:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- rates and rooflines
    per_call_bytes = ag_plan.bytes_read + ag_plan.bytes_written          # (1+W) * M_local * N * e
    copy_launch_s = max(copy_ms, 1e-9) / 1e3 / AG_W     # profiling runs with --only fused time no copy
    copy_gbs = AG_W * per_call_bytes / (max(copy_ms, 1e-9) / 1e3) / 1e9
    traffic = _traffic(f"ag_copy_kernel_w8_{AG_M}x{AG_N}_f16_pmc.md", "ag_copy.hip", per_call_bytes)
    out = {
        "metric": METRIC,
        "value": round(copy_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"all-gather W={AG_W} logical ranks, {AG_M}x{AG_N} fp16 per rank, tile "
                        f"{AG_TILE[0]}x{AG_TILE[1]}, {AG_PROGRAMS} programs (8 calls per step)"
                        + (f" + fused GEMM+all-gather W={FU_W}, M_local={FU_M} K={FU_K} N={FU_N} fp16 "
                           f"(8 calls per step)" if fused_ok else ""),
            "parallelism": "one GPU; W logical ranks are heap regions",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(per_call_bytes / copy_launch_s / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(per_call_bytes / copy_launch_s / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": f"ag_copy_kernel<VEC={ag_plan.vec_bytes},W={AG_W},VPT={ag_plan.vectors_per_thread}>",
            "alg_bytes_per_launch": per_call_bytes,
            "avg_launch_us": round(copy_launch_s * 1e6, 3),
        },
        "spread": spread.get(id(copy_job)),
        "device": {"name": dev_props.name, "cus": dev_props.multi_processor_count},
        "plan_all_gather": {k: ag_plan.as_dict()[k] for k in ("vec_bytes", "n_programs", "threads", "total_tiles",
                                                              "vectors_per_thread")},
        "wall_s_timed": round(wall, 4),
    }
    if fused_ok:
        flops = fu_plan.flops
        fu_launch_s = max(fused_ms, 1e-9) / 1e3 / FU_W
        fu_tflops = FU_W * flops / (max(fused_ms, 1e-9) / 1e3) / 1e12
        out["fused"] = {
            "metric": "fused GEMM+all-gather TFLOP/s",
            "value": round(fu_tflops, 2),
            "unit": "TFLOP/s",
            "ms_per_job": round(fused_ms, 5),
            "roofline": {
                "bound": "mfma",
                "achieved": round(flops / fu_launch_s / 1e12, 2),
                "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(flops / fu_launch_s / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": _traffic(f"ag_gemm_kernel_w8_{FU_M}x{FU_N}x{FU_K}_f16_pmc.md", "ag_gemm.hip", 0.0),
                "kernel": f"ag_gemm_kernel<f16,W={FU_W},{fu_plan.tile_m}x{fu_plan.tile_n}>",
                "alg_flops_per_launch": flops,
                "avg_launch_us": round(fu_launch_s * 1e6, 3),
            },
            "plan": {k: fu_plan.as_dict()[k] for k in ("tile_m", "tile_n", "tile_k", "n_programs", "threads",
                                                       "total_tiles")},
            "spread": spread.get(id(fused_job)),
        }
    out["copy_ms_per_job"] = round(copy_ms, 5)
    if not args.no_context and args.only == "all":
        out["context"] = _context(args, stream, timed, views, ins, geom)
        out["context"]["fused"] = _context_fused(args, stream, timed, fviews, fu_off)
        out["context"]["calibration"] = _calibration(stream)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline_copy(args.cpu_seconds)
        if fused_ok:
            out["fused"]["cpu_baseline"] = _cpu_baseline_fused(args.cpu_seconds)
    print(json.dumps(out), flush=True)
    for v in views + fviews:
        v.destroy()
    heap.destroy()
    fheap.destroy()
    return 0


if __name__ == "__main__":
    sys.exit(main())
