"""Benchmark of the hot path on one MI355X: multi-destination all-gather + fused GEMM + all-gather.

One step = one complete logical all-gather job and one fused job on one GPU:
  * all-gather: every one of the W=8 logical ranks calls ag_all_gather on its
    16384 x 8192 fp16 input (uniform[-1,1), tile 8x256, 256 programs), so every
    heap region ends up with the 131072 x 8192 gathered tensor (2.4 GB of HBM
    traffic per call, far beyond the last-level cache);
  * fused: every one of the 8 logical ranks calls ag_gemm_all_gather with
    A_g 16384 x 8192 and the shared B 8192 x 3584 (fp16 ~ N(0,1)/sqrt(K), fp32
    accumulate), so every region ends up with the 131072 x 3584 gathered C
    (--fused-m 1024 selects the M_local = 1024 variant).
Inputs are seeded synthetic tensors already resident in HBM.

Printed: one JSON line.  value = all-gather HBM GB/s over the whole job
((1+W)*M_local*N*e bytes per call, W calls per step); the fused path's
TFLOP/s is reported in the "fused" object, each with its roofline.  The
"context" object holds the other program counts and element types of the
16384 x 8192 all-gather, the 1024 x 4096 all-gather (75 MB per call, partly
held by the last-level cache), the variants, the all-to-all, edge shapes,
the other fused workloads and a plain copy/fill calibration.
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

# all-gather workload: W=8 logical ranks, 16384 x 8192 fp16 per rank, tile 8x256, 256 programs (the CU
# count; 64 and 128, and bf16 and fp32, are timed in "context")
AG_W, AG_M, AG_N, AG_DTYPE, AG_TILE, AG_PROGRAMS = 8, 16384, 8192, "f16", (8, 256), 256
# the smaller all-gather workload (context): 1024 x 4096 fp16 per rank, 75 MB per call
SM_M, SM_N, SM_PROGRAMS = 1024, 4096, 128
# fused workload: W=8, M_local 16384, K 8192, N 3584, fp16
FU_W, FU_N, FU_K, FU_DTYPE = 8, 3584, 8192, "f16"
FU_M = 16384


def _code_text(src: str) -> str:
    """C++ source with its comments removed and whitespace collapsed: what the compiler sees of it.

    String and character literals are kept as written (a // inside one is not a comment).
    """
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def _src_hash(name: str) -> str:
    """Hash of a kernel source's code (comments and layout excluded): a counter summary recorded on one
    version of the code stays valid across comment edits and goes stale with any change to the code."""
    with open(os.path.join(ROOT, "gemm_all_gather_amd", "csrc", name), encoding="utf-8") as f:
        return hashlib.sha256(_code_text(f.read()).encode()).hexdigest()[:16]


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


def _host_threads() -> int:
    """Host threads for the CPU baseline: the process's cores, at most the OpenMP thread count set for it."""
    cores = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", cores))
    except ValueError:
        cap = cores
    return max(1, min(cores, cap))


def _cpu_baseline_copy(seconds: float, host_input):
    """The oracle's store of one rank's input into the W member regions, on the host cores (bounded sample).

    One call's work: the 16384 x 8192 fp16 input (the same bytes as rank 0's device input) written at the
    rank's row block of W preallocated host regions (each sized for the gathered output), with the oracle's
    multi-destination store (oracle.store_to_members); the rows are split among the threads, each thread
    storing its rows to all W regions.
    """
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle

    threads = _host_threads()
    data = np.ascontiguousarray(host_input).view(np.uint8).reshape(-1)
    blk = data.size
    regions = [np.empty(AG_W * blk, dtype=np.uint8) for _ in range(AG_W)]
    g = 0                                              # the calling rank's group index
    bounds = [blk * t // threads // 4096 * 4096 for t in range(threads)] + [blk]
    pool = ThreadPoolExecutor(max_workers=threads)

    def call():
        futs = [pool.submit(oracle.store_to_members, regions, g * blk + bounds[t], data[bounds[t]:bounds[t + 1]])
                for t in range(threads)]
        for f in futs:
            f.result()

    call()                                             # warm-up: first touch of the regions
    reps, t0 = 0, time.perf_counter()
    while True:
        call()
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    pool.shutdown()
    del regions
    call_bytes = (1 + AG_W) * blk
    return {"value": call_bytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} calls of one rank's all-gather (W={AG_W}, its {AG_M}x{AG_N} fp16 input stored at its "
                      f"row block of {AG_W} preallocated host regions by oracle.store_to_members, rows split over "
                      f"{threads} threads) in {reps * dt:.1f} s; GB/s = (1+W)*M_local*N*e per call"}


def _cpu_baseline_fused(seconds: float):
    """The oracle's fused GEMM + all-gather for a bounded sample of output rows of one rank's call."""
    import numpy as np
    from gemm_all_gather_amd import inputs as gen
    import oracle

    threads = _host_threads()
    rows = 64
    a = gen.normal_scaled((rows, FU_K), FU_DTYPE, FU_K ** -0.5, 2, 0)
    b = gen.normal_scaled((FU_N, FU_K), FU_DTYPE, FU_K ** -0.5, 3)
    regions = [np.empty(rows * FU_N * 2, dtype=np.uint8) for _ in range(FU_W)]

    def call():
        c = oracle.gemm_oracle(a, b, FU_DTYPE, "nk")
        oracle.store_to_members(regions, 0, c.view(np.uint8).reshape(-1))

    call()                                             # warm-up
    reps, t0 = 0, time.perf_counter()
    while True:
        call()
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    flops = 2.0 * rows * FU_N * FU_K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x {rows} output rows of one rank's {FU_M}x{FU_N}x{FU_K} fp16 product (float64 numpy "
                      f"matmul, rounding, stores to {FU_W} host regions), {reps * dt:.1f} s; BLAS threads up to "
                      f"{threads}"}


def _device_uniform(n_elems: int, dtype: str, seed: int):
    """Seeded uniform[-1,1) values drawn on the device (float32 2u - 1, rounded to the storage type), as bytes."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    x = torch.rand(n_elems, generator=g, dtype=torch.float32, device="cuda") * 2.0 - 1.0
    return x.to(tdt).view(torch.uint8)


def _device_normal(n_elems: int, dtype: str, scale: float, seed: int):
    """Seeded N(0,1)*scale values drawn on the device in float32, rounded to the storage type, as bytes."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    x = torch.randn(n_elems, generator=g, dtype=torch.float32, device="cuda") * scale
    return x.to(tdt).view(torch.uint8)


class _Workload:
    """An 8-region heap sized for one all-gather shape, with every member's device input."""

    def __init__(self, M, N, dtype, W=AG_W, start=0, stride=1, seed=1, n_regions=8, out_bytes=None):
        import torch
        from gemm_all_gather_amd import binding as ag
        self.M, self.N, self.dtype, self.W, self.start, self.stride = M, N, dtype, W, start, stride
        self.e = 4 if dtype == "f32" else 2
        self.blk = M * N * self.e
        # every region sized for the gathered output, laid out as ag_heap_create lays out its regions
        out_bytes = W * self.blk if out_bytes is None else out_bytes
        self.S = ag.heap_region_bytes(out_bytes)
        self.slab = torch.empty(n_regions * self.S, dtype=torch.uint8, device="cuda")
        self.slab.zero_()
        self.heap = ag.Heap.wrap(self.slab, n_regions, self.S)
        self.members = [start + i * stride for i in range(W)]
        self.views = {r: self.heap.view(r) for r in self.members}
        self.ins = [_device_uniform(M * N, dtype, seed * 100 + i) for i in range(W)]
        self.geom = self.views[start].geometry()

    def job(self, ag, stream, tile=(0, 0), programs=0, dest_group=0, schedule="tiles", tile_order="auto"):
        """All W members' calls, in group order."""
        def run():
            for i, r in enumerate(self.members):
                if tile_order != "auto":
                    ag.all_gather_ex(self.views[r], self.W, self.start, self.stride, self.ins[i], 0, self.M, self.N,
                                     self.dtype, tile[0], tile[1], programs, dest_group, schedule, stream,
                                     tile_order=tile_order)
                elif dest_group == 0 and schedule == "tiles":
                    ag.all_gather(self.views[r], self.W, self.start, self.stride, self.ins[i], 0, self.M, self.N,
                                  self.dtype, tile[0], tile[1], programs, stream)
                else:
                    ag.all_gather_ex(self.views[r], self.W, self.start, self.stride, self.ins[i], 0, self.M, self.N,
                                     self.dtype, tile[0], tile[1], programs, dest_group, schedule, stream)
        return run

    def plan(self, ag, tile=(0, 0), programs=0, tile_order="auto"):
        return ag.plan_all_gather_ex(self.geom, self.W, self.start, self.stride, self.ins[0], 0, self.M, self.N,
                                     self.dtype, tile[0], tile[1], programs, tile_order=tile_order)

    def close(self):
        import torch
        torch.cuda.synchronize()
        for v in self.views.values():
            v.destroy()
        self.heap.destroy()
        del self.slab, self.ins
        torch.cuda.empty_cache()


def _context(args, stream, timed, head):
    """Context measurements beside the headline (each job = the group members' calls, timed like it).

    * the 16384x8192 all-gather at 64/128/256 programs (and 192) in fp16, bf16 and fp32, in the library's
      tile order (tickets at this size) and in the fixed grid-stride order;
    * its variants: destination groups 1/2/4 and the partitioned schedule at 64/128/256 programs;
    * the 1024x4096 all-gather at 64/128/256 programs (75 MB per call: partly held by the last-level
      cache, so its rate exceeds what HBM sustains for the larger shape);
    * the all-to-all: W=8, 8 chunks of 1024x4096 fp16 per rank, tile and partitioned schedules, and 8 chunks
      of 2048x8192 in both tile orders at 256 / 128 / 64 programs;
    * the edge shapes: 1000x4100 fp16 (partial last column tile) at W=8, and the strided group of ranks
      1, 3, 5, 7 (W=4) at 1000x4100 and 16384x8192.
    """
    import torch
    from gemm_all_gather_amd import binding as ag

    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup = max(20, args.steps // 5), max(10, args.warmup // 5)
    ctx = {"steps": sub.steps, "warmup": sub.warmup}

    def rate(wl, **kw):
        ms, _ = timed(wl.job(ag, stream, **kw), sub)
        return round(wl.W * (1 + wl.W) * wl.blk / (ms / 1e3) / 1e9, 1), ms

    # the 16384 x 8192 all-gather: three program counts, three element types (fp16 is the headline heap)
    big = {}
    for dt in ("f16", "bf16", "f32"):
        wl = head if dt == "f16" else _Workload(AG_M, AG_N, dt, seed=6)
        big[dt] = {}
        for P in (64, 128, 192, 256):   # the workload's 64/128/256 programs, and 192 between them
            gb, ms = rate(wl, tile=AG_TILE, programs=P)
            p = wl.plan(ag, AG_TILE, P)
            entry = {"GBs": gb, "frac": round(gb / HBM_PEAK_GBS, 4), "us_per_call": round(ms * 1e3 / wl.W, 2),
                     "tile_order": {1: "stride", 2: "tickets"}[p.tile_order], "tiles_per_ticket": p.tiles_per_ticket,
                     "threads": p.threads, "vectors_per_thread": p.vectors_per_thread}
            if p.tile_order == ag.AG_ORDER_TICKETS:
                # the same call with the fixed grid-stride tile order
                gs, mss = rate(wl, tile=AG_TILE, programs=P, tile_order="stride")
                entry["grid_stride_order"] = {"GBs": gs, "frac": round(gs / HBM_PEAK_GBS, 4),
                                              "us_per_call": round(mss * 1e3 / wl.W, 2),
                                              "threads": wl.plan(ag, AG_TILE, P, "stride").threads}
            big[dt][str(P)] = entry
        if wl is not head:
            wl.close()
    ctx["all_gather_16384x8192"] = big
    # its variants on the headline heap: destination groups at 256 programs, the partitioned schedule
    # (every destination reads the tile itself: 2*W*M*N*e HBM bytes per call)
    ctx["all_gather_16384x8192_f16_by_dest_group"] = {str(G): rate(head, tile=AG_TILE, programs=AG_PROGRAMS,
                                                                   dest_group=G)[0] for G in (1, 2, 4)}
    part = {}
    for P in (64, 128, 256):
        ms, _ = timed(head.job(ag, stream, tile=AG_TILE, programs=P, schedule="partitioned"), sub)
        part[str(P)] = round(head.W * 2 * head.W * head.blk / (ms / 1e3) / 1e9, 1)
    ctx["all_gather_16384x8192_f16_partitioned_GBs_by_programs"] = part

    # the 1024 x 4096 all-gather (75 MB per call)
    small = _Workload(SM_M, SM_N, "f16", seed=2)
    sm = {str(P): rate(small, tile=AG_TILE, programs=P)[0] for P in (64, 128, 256)}
    ctx["all_gather_1024x4096_f16_cache_assisted_GBs_by_programs"] = sm
    small.close()

    ctx["all_to_all"] = _all_to_all(sub, stream, timed)

    # the edge shapes: rows of 4100 elements (partial last column tile); the strided group of ranks
    # 1, 3, 5, 7 (W=4) at both sizes
    edges = {}
    for name, M, N, W, start, stride, seed in (("1000x4100_f16_W8", 1000, 4100, AG_W, 0, 1, 7),
                                               ("1000x4100_f16_W4_group_1_2", 1000, 4100, 4, 1, 2, 8),
                                               ("16384x8192_f16_W4_group_1_2", 16384, 8192, 4, 1, 2, 9)):
        wl = _Workload(M, N, "f16", W=W, start=start, stride=stride, seed=seed)
        edges[name] = rate(wl, programs=256)[0]
        wl.close()
    ctx["all_gather_edges_GBs"] = edges
    return ctx


def _all_to_all(sub, stream, timed):
    """The all-to-all on its own heap: W=8, 8 chunks of 1024x4096 fp16 per rank, tile and partitioned schedules;
    then 8 chunks of 2048x8192 per rank in both tile orders."""
    from gemm_all_gather_amd import binding as ag

    # all-to-all: each rank sends 8 chunks of 1024x4096 fp16 (64 MiB per rank); 8x512 tiles, two 16-byte
    # vectors per thread (22.9 us per call against 28.5 for 8x256 and 23.0-24.6 for larger tiles at 256
    # programs)
    A2A_TILE = (8, 512)
    mc, n = SM_M, SM_N
    # inputs of W chunks; regions sized for the exchanged output (W chunks of M_chunk x N)
    a2a = _Workload(AG_W * mc, n, "f16", seed=5, out_bytes=AG_W * mc * n * 2)
    a2a_in = a2a.ins
    a2a_plan = ag.plan_all_to_all(a2a.geom, AG_W, 0, 1, a2a_in[0], 0, mc, n, "f16", *A2A_TILE, 256)
    views = a2a.views
    ms, _ = timed(lambda: [ag.all_to_all(views[j], AG_W, 0, 1, a2a_in[j], 0, mc, n, "f16", *A2A_TILE, 256, stream)
                           for j in range(AG_W)], sub)
    a2a_bytes = a2a_plan.bytes_read + a2a_plan.bytes_written
    launch_s = ms / 1e3 / AG_W
    res = {
        "workload": f"all-to-all W={AG_W}, {AG_W} chunks of {mc}x{n} fp16 per rank, tile {A2A_TILE[0]}x{A2A_TILE[1]}, "
                    f"{a2a_plan.n_programs} programs (8 calls per job)",
        "value": round(AG_W * a2a_bytes / (ms / 1e3) / 1e9, 1), "unit": "GB/s",
        "roofline": {"bound": "hbm", "achieved": round(a2a_bytes / launch_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(a2a_bytes / launch_s / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": _traffic(f"ag_a2a_kernel_w{AG_W}_{mc}x{n}_f16_pmc.md", "ag_copy.hip", a2a_bytes),
                     "alg_bytes_per_launch": a2a_bytes, "avg_launch_us": round(launch_s * 1e6, 3)},
    }
    # the partitioned schedule of the same exchange (program p copies one chunk to destination p mod W)
    ms, _ = timed(lambda: [ag.all_to_all_ex(views[j], AG_W, 0, 1, a2a_in[j], 0, mc, n, "f16", 16, 512, 256,
                                            schedule="partitioned", stream=stream) for j in range(AG_W)], sub)
    res["partitioned_16x512_256_programs_GBs"] = round(AG_W * a2a_bytes / (ms / 1e3) / 1e9, 1)
    a2a.close()

    # a long exchange: 8 chunks of 2048x8192 fp16 per rank (256 MiB), 8x512 tiles, in the library's tile
    # order and in the other one, at 256 / 128 / 64 programs
    bm, bn = 2048, 8192
    big = _Workload(AG_W * bm, bn, "f16", seed=6, out_bytes=AG_W * bm * bn * 2)
    big_bytes = 2 * AG_W * bm * bn * 2
    out = {}
    for P in (256, 128, 64):
        auto = ag.plan_all_to_all(big.geom, AG_W, 0, 1, big.ins[0], 0, bm, bn, "f16", *A2A_TILE, P)
        row = {}
        for order in ("stride", "tickets"):
            ms, _ = timed(lambda: [ag.all_to_all_ex(big.views[j], AG_W, 0, 1, big.ins[j], 0, bm, bn, "f16", *A2A_TILE, P,
                                                    stream=stream, tile_order=order) for j in range(AG_W)], sub)
            row[order] = {"GBs": round(AG_W * big_bytes / (ms / 1e3) / 1e9, 1),
                          "us_per_call": round(ms * 1e3 / AG_W, 2)}
        row["library_order"] = "tickets" if auto.tile_order == ag.AG_ORDER_TICKETS else "stride"
        out[str(P)] = row
    res[f"{bm}x{bn}_8x512_by_programs"] = out
    big.close()
    return res


def _context_fused(args, stream, timed, views, fu_off):
    """The fused workload at M_local 1024 and 4096 (fp16; with 16384, the pages' three fused rows), at M_local
    16384 in bf16, at M_local 16384 in fp16 with the pages' 256x256 output tile, and at M_local 16384 in fp16
    with B stored N-contiguous (a row-major K x N matrix), W=8, timed like the headline."""
    import torch
    from gemm_all_gather_amd import binding as ag

    res = {}
    region = views[0].geometry().bytes_per_rank
    for name, M, dtype, layout, tile in (("M1024_f16", 1024, "f16", "k", (0, 0, 0)),
                                         ("M4096_f16", 4096, "f16", "k", (0, 0, 0)),
                                         ("M16384_bf16", 16384, "bf16", "k", (0, 0, 0)),
                                         ("M16384_f16_tile_256x256x64", 16384, "f16", "k", (256, 256, 64)),
                                         ("M16384_f16_B_row_major_KxN", 16384, "f16", "n", (0, 0, 0))):
        sub = argparse.Namespace(**vars(args))
        if M * FU_N * FU_K < (1 << 38):
            # short calls (75-220 us): the headline's warm-up steps, so the clocks settle after the workloads
            # before (2 steps, about 1 ms, measured 88-93 us per call against 74.6 with 50 at M_local 1024)
            sub.steps, sub.warmup = max(20, args.steps // 5), args.warmup
        else:
            sub.steps, sub.warmup = max(5, args.steps // 10), 2
        own = None
        if M != FU_M:
            # a heap of its own, regions sized for this workload's gathered output, as for the
            # all-gather workloads (the region stride moves the store rate)
            S = ag.heap_region_bytes(FU_W * M * FU_N * 2)
            own_slab = torch.zeros(FU_W * S, dtype=torch.uint8, device="cuda")
            own = ag.Heap.wrap(own_slab, FU_W, S)
            vws, off = [own.view(r) for r in range(FU_W)], 0
        else:
            vws, off = views, fu_off
        if off + FU_W * M * FU_N * 2 > (region if own is None else S):
            continue
        fa = [_device_normal(M * FU_K, dtype, FU_K ** -0.5, 1200 + j) for j in range(FU_W)]
        fb = _device_normal(FU_N * FU_K, dtype, FU_K ** -0.5, 1300)    # the N x K (or K x N) B: same count
        ldb = FU_K if layout == "k" else FU_N
        ms, _ = timed(lambda: [ag.gemm_all_gather_ex(vws[j], FU_W, 0, 1, fa[j], FU_K, fb, ldb, off, M, FU_N,
                                                     FU_K, dtype, *tile, 0, b_layout=layout, stream=stream)
                               for j in range(FU_W)], sub)
        flops = 2.0 * M * FU_N * FU_K
        tf = FU_W * flops / (ms / 1e3) / 1e12
        res[name] = {"TFLOPs": round(tf, 1), "frac_of_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                     "us_per_call": round(ms * 1e3 / FU_W, 1), "warmup": sub.warmup, "steps": sub.steps}
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


def main() -> int:
    global FU_M
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused-m", type=int, default=FU_M, help="M_local of the fused workload (16384, 4096 or 1024)")
    ap.add_argument("--only", choices=["all", "copy", "fused", "a2a"], default="all",
                    help="restrict the timed step to one kernel (profiling runs); a2a times the all-to-all "
                         "context workload alone")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context measurements (program counts and element types, variants, the "
                         "1024x4096 all-gather, all-to-all, edge shapes, the other fused workloads, plain "
                         "copy/fill calibration)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB "
                         "(reference for HBM byte counters)")
    args = ap.parse_args()
    FU_M = args.fused_m
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the W logical ranks are regions of one GPU's HBM; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import torch
    from gemm_all_gather_amd import binding as ag

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ag.lib()
    dev_props = torch.cuda.get_device_properties(0)
    stream = torch.cuda.current_stream()

    if args.only == "a2a":   # profiling run of the all-to-all workload alone
        def timed_a2a(job, a):
            for _ in range(a.warmup):
                job()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(a.steps):
                job()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / a.steps, 0.0
        res = _all_to_all(args, stream, timed_a2a)
        if args.calib_copy_mib > 0:
            src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"metric": "all-to-all HBM GB/s", "value": res["value"], "unit": "GB/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "all_to_all": res}), flush=True)
        return 0

    # ---------------- all-gather setup: 16384 x 8192 fp16 per rank, 8 regions of 2 GiB
    head = _Workload(AG_M, AG_N, AG_DTYPE, seed=1) if args.only != "fused" else None
    ag_plan = head.plan(ag, AG_TILE, AG_PROGRAMS) if head is not None else None
    copy_job = head.job(ag, stream, tile=AG_TILE, programs=AG_PROGRAMS) if head is not None else None

    # ---------------- fused setup
    fused_ok = args.only != "copy"
    if fused_ok:
        fa = [_device_normal(FU_M * FU_K, FU_DTYPE, FU_K ** -0.5, 200 + j) for j in range(FU_W)]
        fb = _device_normal(FU_N * FU_K, FU_DTYPE, FU_K ** -0.5, 300)
        fblk = FU_M * FU_N * 2
        SF = ag.heap_region_bytes(FU_W * fblk)
        fslab = torch.empty(FU_W * SF, dtype=torch.uint8, device="cuda")
        fslab.zero_()
        fheap = ag.Heap.wrap(fslab, FU_W, SF)
        fviews = [fheap.view(r) for r in range(FU_W)]
        fu_off = 0

        def fused_job():
            for j in range(FU_W):
                ag.gemm_all_gather(fviews[j], FU_W, 0, 1, fa[j], FU_K, fb, FU_K, fu_off, FU_M, FU_N, FU_K, FU_DTYPE,
                                   0, 0, 0, 0, stream)

        fu_plan = ag.plan_gemm_all_gather(fviews[0].geometry(), FU_W, 0, 1, fa[0], FU_K, fb, FU_K, fu_off, FU_M,
                                          FU_N, FU_K, FU_DTYPE)

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

    copy_ms, wall_copy = timed(copy_job, blocks=3) if head is not None else (0.0, 0.0)
    fused_ms, wall_fused = timed(fused_job, blocks=3) if fused_ok else (0.0, 0.0)
    step_ms = copy_ms + fused_ms
    wall = wall_copy + wall_fused
    if args.calib_copy_mib > 0:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- rates and rooflines
    out = {
        "metric": METRIC,
        "value": None,
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
            "workload": (f"all-gather W={AG_W} logical ranks, {AG_M}x{AG_N} fp16 per rank, tile "
                         f"{AG_TILE[0]}x{AG_TILE[1]}, {AG_PROGRAMS} programs (8 calls per step)"
                         if head is not None else "")
                        + (f" + fused GEMM+all-gather W={FU_W}, M_local={FU_M} K={FU_K} N={FU_N} fp16 "
                           f"(8 calls per step)" if fused_ok else ""),
            "parallelism": "one GPU; W logical ranks are heap regions",
        },
        "device": {"name": dev_props.name, "cus": dev_props.multi_processor_count},
        "wall_s_timed": round(wall, 4),
    }
    if head is not None:
        per_call_bytes = ag_plan.bytes_read + ag_plan.bytes_written          # (1+W) * M_local * N * e
        copy_launch_s = copy_ms / 1e3 / AG_W
        copy_gbs = AG_W * per_call_bytes / (copy_ms / 1e3) / 1e9
        out["value"] = round(copy_gbs, 2)
        out["roofline"] = {
            "bound": "hbm",
            "achieved": round(per_call_bytes / copy_launch_s / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(per_call_bytes / copy_launch_s / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": _traffic(f"{'ag_copy_ticket_kernel' if ag_plan.tile_order == ag.AG_ORDER_TICKETS else 'ag_copy_kernel'}"
                                f"_w8_{AG_M}x{AG_N}_f16_pmc.md", "ag_copy.hip", per_call_bytes),
            "kernel": (f"ag_copy_ticket_kernel<VEC={ag_plan.vec_bytes},W={AG_W},VPT={ag_plan.vectors_per_thread},"
                       f"G={ag_plan.tiles_per_ticket}>" if ag_plan.tile_order == ag.AG_ORDER_TICKETS else
                       f"ag_copy_kernel<VEC={ag_plan.vec_bytes},W={AG_W},VPT={ag_plan.vectors_per_thread}>"),
            "alg_bytes_per_launch": per_call_bytes,
            "avg_launch_us": round(copy_launch_s * 1e6, 3),
        }
        out["spread"] = spread.get(id(copy_job))
        out["plan_all_gather"] = {k: ag_plan.as_dict()[k] for k in ("vec_bytes", "n_programs", "threads",
                                                                    "total_tiles", "vectors_per_thread",
                                                                    "tile_order", "tiles_per_ticket")}
        out["copy_ms_per_job"] = round(copy_ms, 5)
    if fused_ok:
        flops = fu_plan.flops
        fu_launch_s = fused_ms / 1e3 / FU_W
        fu_tflops = FU_W * flops / (fused_ms / 1e3) / 1e12
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
            # the minimum HBM bytes of a call (A and B read once, the W output copies written) over its time
            "alg_bytes_per_launch": fu_plan.bytes_read + fu_plan.bytes_written,
            "achieved_alg_GBs": round((fu_plan.bytes_read + fu_plan.bytes_written) / fu_launch_s / 1e9, 1),
            "plan": {k: fu_plan.as_dict()[k] for k in ("tile_m", "tile_n", "tile_k", "n_programs", "threads",
                                                       "total_tiles")},
            "spread": spread.get(id(fused_job)),
        }
    if not args.no_context and args.only == "all":
        out["context"] = _context(args, stream, timed, head)
        out["context"]["fused"] = _context_fused(args, stream, timed, fviews, fu_off)
        out["context"]["calibration"] = _calibration(stream)

    if not args.no_cpu_baseline:
        if head is not None:
            host_in = head.ins[0].cpu().numpy()
            out["cpu_baseline"] = _cpu_baseline_copy(args.cpu_seconds, host_in)
            del host_in
        if fused_ok:
            out["fused"]["cpu_baseline"] = _cpu_baseline_fused(args.cpu_seconds)
    print(json.dumps(out), flush=True)
    if head is not None:
        head.close()
    if fused_ok:
        for v in fviews:
            v.destroy()
        fheap.destroy()
    return 0


if __name__ == "__main__":
    sys.exit(main())
