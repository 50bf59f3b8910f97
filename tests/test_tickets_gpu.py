"""Parity of the all-gather in ticket order (AG_ORDER_TICKETS) with the CPU oracle.

The tile order changes which program copies which tile and when, never the
result: every case compares the whole heap with the oracle byte for byte
(outputs, guards, regions outside the group).  The per-rank tile counters must
be back at zero after every call (the last program to finish resets them).
"""

import itertools

import numpy as np
import pytest
import torch

from gemm_all_gather_amd import binding as ag
from gemm_all_gather_amd import inputs as gen
from oracle import all_gather_oracle, all_to_all_oracle
from tests.gpu_util import TorchHeap, log, require_gpu, to_device

pytestmark = pytest.mark.gpu

E = {"f16": 2, "bf16": 2, "f32": 4}


def _counters(th: TorchHeap) -> np.ndarray:
    """The heap's per-rank tile counters (two words in a 64-byte block per rank, after the base table)."""
    info = th.heap.info()
    n = info["n_ranks"]
    start = info["base_table"] + -(-8 * n // 256) * 256

    class _C:
        __cuda_array_interface__ = {"shape": (n * 16,), "typestr": "<u4", "data": (start, False), "version": 3,
                                    "strides": None}

    torch.cuda.synchronize()
    return torch.as_tensor(_C(), device="cuda").cpu().numpy().reshape(n, 16)[:, :2]


def _run(th, dev, W, start, stride, off, M, N, dtype, tile, programs, order="tickets", stream=None):
    for j in range(W):
        ag.all_gather_ex(th.view(start + j * stride), W, start, stride, dev[j], off, M, N, dtype, tile[0], tile[1],
                         programs, tile_order=order, stream=stream)


def _check(th, before, ins, S, start, stride, off):
    got = th.host()
    want = all_gather_oracle(before, S, ins, start, stride, off)
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        raise AssertionError(f"{bad.size} bytes differ; first at region {bad[0] // S} offset {bad[0] % S}")
    assert not _counters(th).any(), "a tile counter was left non-zero"
    return got


_CASES = []
_rng = np.random.default_rng(31)
for W, (start, stride), M, N in itertools.product([1, 2, 3, 5, 8], [(0, 1), (1, 2), (3, 1)], [1, 7, 64, 300, 1000],
                                                  [256, 264, 520, 4104]):
    if start + (W - 1) * stride >= 8:
        continue
    _CASES.append((W, start, stride, M, N))
_CASES = [c for c in _CASES if _rng.random() < 0.4]


@pytest.mark.parametrize("W,start,stride,M,N", _CASES)
def test_ticket_order_sweep(W, start, stride, M, N):
    require_gpu()
    rng = np.random.default_rng([W, start, stride, M, N, 5])
    dtype = ["f16", "bf16", "f32"][int(rng.integers(0, 3))]
    e = E[dtype]
    # one or two 16-byte vectors per thread and tile
    tiles = [(8, 256), (4, 512), (16, 128), (1, 2048), (8, 512), (16, 256)] if e == 2 else \
        [(8, 256), (4, 256), (2, 512), (1, 1024)]
    tile = tiles[int(rng.integers(0, len(tiles)))]
    programs = [1, 3, 7, 64, 256, 10_000][int(rng.integers(0, 6))]
    off = 16 * int(rng.integers(0, 8))
    S = ((off + W * M * N * e + 300) // 256 + 1) * 256
    log(f"tickets W={W} group=({start},{stride}) M={M} N={N} {dtype} tile={tile} programs={programs} off={off}")
    th = TorchHeap(8, S)
    try:
        ins = [gen.uniform_pm1((M, N), dtype, W * 100 + M, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        p = ag.plan_all_gather_ex(th.view(start).geometry(), W, start, stride, dev[0], off, M, N, dtype, *tile,
                                  programs, tile_order="tickets")
        assert p.tile_order == ag.AG_ORDER_TICKETS and p.tiles_per_ticket in (2, 3, 4, 8, 16)
        before = th.host()
        _run(th, dev, W, start, stride, off, M, N, dtype, tile, programs)
        _check(th, before, ins, S, start, stride, off)
    finally:
        th.close()


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_ticket_order_every_world_on_every_cu(W, dtype):
    """A program per CU, 8x256 tiles: each W takes the tiles per ticket of its 96 KiB floor (3 to 16 with one
    16-byte vector per thread, 2 to 8 with two) and the schedule that takes tickets after the stores."""
    require_gpu()
    e = E[dtype]
    # 25 tile columns (the last one partial) and enough tiles that every program takes tickets: 3200 tiles
    # up to W=4 (16 or 8 per ticket), 1600 from W=5 (at most 4 per ticket)
    M, N = (1024 if W <= 4 else 512), 6152
    start, stride = (0, 1) if W > 4 else (1, 2) if W > 1 else (1, 1)
    S = ((W * M * N * e + 4096) // 256 + 1) * 256
    th = TorchHeap(8, S)
    try:
        ins = [gen.uniform_pm1((M, N), dtype, 70 + W, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        cus = th.view(start).geometry().num_cus
        p = ag.plan_all_gather_ex(th.view(start).geometry(), W, start, stride, dev[0], 0, M, N, dtype, 8, 256, cus,
                                  tile_order="tickets")
        tile_bytes = 8 * 256 * e
        assert p.tile_order == ag.AG_ORDER_TICKETS
        assert p.tiles_per_ticket * tile_bytes * (1 + W) >= 96 << 10 or p.tiles_per_ticket == (16 if e == 2 else 8)
        assert p.n_programs >= 3 * cus // 4 and p.ticket_wait == 1
        log(f"tickets on every CU: W={W} {dtype} G={p.tiles_per_ticket} wait={p.ticket_wait} "
            f"programs={p.n_programs}")
        before = th.host()
        _run(th, dev, W, start, stride, 0, M, N, dtype, (8, 256), cus)
        _check(th, before, ins, S, start, stride, 0)
    finally:
        th.close()


_A2A_CASES = []
_rng2 = np.random.default_rng(37)
for W, (start, stride), M, N in itertools.product([1, 2, 3, 5, 8], [(0, 1), (1, 2), (3, 1)], [1, 7, 64, 300],
                                                  [256, 264, 520, 4104]):
    if start + (W - 1) * stride >= 8:
        continue
    _A2A_CASES.append((W, start, stride, M, N))
_A2A_CASES = [c for c in _A2A_CASES if _rng2.random() < 0.35]


def _a2a_tickets(W, start, stride, M, N, dtype, tile, programs, off, seed):
    e = E[dtype]
    S = ((off + W * M * N * e + 300) // 256 + 1) * 256
    th = TorchHeap(8, S)
    try:
        ins = [gen.random_bit_patterns((W * M, N), e, seed, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        p = ag.plan_all_to_all_ex(th.view(start).geometry(), W, start, stride, dev[0], off, M, N, dtype, *tile,
                                  programs, tile_order="tickets")
        assert p.tile_order == ag.AG_ORDER_TICKETS and p.tiles_per_ticket in (8, 16)
        log(f"all-to-all tickets W={W} group=({start},{stride}) M_chunk={M} N={N} {dtype} tile={tile} "
            f"programs={programs} off={off} G={p.tiles_per_ticket} wait={p.ticket_wait} grid={p.n_programs}")
        before = th.host()
        for j in range(W):
            ag.all_to_all_ex(th.view(start + j * stride), W, start, stride, dev[j], off, M, N, dtype, *tile, programs,
                             tile_order="tickets")
        got = th.host()
        want = all_to_all_oracle(before, S, ins, start, stride, off)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            raise AssertionError(f"{bad.size} bytes differ; first at region {bad[0] // S} offset {bad[0] % S}")
        assert not _counters(th).any(), "a tile counter was left non-zero"
        return p
    finally:
        th.close()


@pytest.mark.parametrize("W,start,stride,M,N", _A2A_CASES)
def test_all_to_all_ticket_order_sweep(W, start, stride, M, N):
    """The all-to-all in ticket order: W chunk copies as one tile sequence, G tiles per ticket."""
    require_gpu()
    rng = np.random.default_rng([W, start, stride, M, N, 9])
    dtype = ["f16", "bf16", "f32"][int(rng.integers(0, 3))]
    tiles = [(8, 256), (4, 512), (16, 128), (8, 512), (16, 256)] if E[dtype] == 2 else [(8, 256), (4, 256), (2, 512)]
    tile = tiles[int(rng.integers(0, len(tiles)))]
    programs = [1, 3, 7, 64, 256, 10_000][int(rng.integers(0, 6))]
    off = 16 * int(rng.integers(0, 8))
    _a2a_tickets(W, start, stride, M, N, dtype, tile, programs, off, seed=W * 100 + M)


@pytest.mark.parametrize("W", [2, 5, 8])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_all_to_all_ticket_order_on_every_cu(W, dtype):
    """A program per CU and at least 3400 tiles in the sequence: every program takes tickets, after the
    stores of the batch before (16 tiles of 8x256 fp16 or 8 of fp32 per ticket), with ragged columns."""
    require_gpu()
    M, N = 8 * -(-200 // W), 4104
    p = _a2a_tickets(W, 0 if W > 2 else 1, 1 if W > 2 else 2, M, N, dtype, (8, 256), 0, 0, seed=W + 40)
    assert p.n_programs >= 192 and p.ticket_wait == 1


def test_ticket_order_repeated_calls_and_counter_reset():
    """The same call again and again, then other ranks and shapes: the counters are zero between calls."""
    require_gpu()
    W, M, N, dtype = 8, 777, 1024, "bf16"
    S = ((W * M * N * 2 + 4096) // 256 + 1) * 256
    th = TorchHeap(8, S)
    try:
        ins = [gen.uniform_pm1((M, N), dtype, 61, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        before = th.host()
        for programs in (5, 5, 5, 256, 64, 1, 300):
            log(f"tickets repeated: programs={programs}")
            for j in (3, 3, 0, 7, 1, 2, 4, 5, 6):
                ag.all_gather_ex(th.view(j), W, 0, 1, dev[j], 0, M, N, dtype, 8, 256, programs, tile_order="tickets")
            assert not _counters(th).any()
        _check(th, before, ins, S, 0, 1, 0)
    finally:
        th.close()


def test_ticket_order_concurrent_ranks_on_streams():
    """Different ranks' calls on four streams at once (each rank has its own counter)."""
    require_gpu()
    W, M, N, dtype = 8, 2048, 2048, "f16"
    S = ((W * M * N * 2 + 4096) // 256 + 1) * 256
    th = TorchHeap(8, S)
    try:
        ins = [gen.uniform_pm1((M, N), dtype, 62, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        before = th.host()
        streams = [torch.cuda.Stream() for _ in range(4)]
        torch.cuda.synchronize()
        log("tickets on four streams")
        for j in range(W):
            ag.all_gather_ex(th.view(j), W, 0, 1, dev[j], 0, M, N, dtype, 8, 256, 64, tile_order="tickets",
                             stream=streams[j % 4])
        torch.cuda.synchronize()
        _check(th, before, ins, S, 0, 1, 0)
    finally:
        th.close()


def test_ticket_order_in_place_and_random_bit_patterns():
    require_gpu()
    W, M, N = 4, 300, 776
    S = ((W * M * N * 4 + 1024) // 256 + 1) * 256
    th = TorchHeap(4, S)
    try:
        before = th.fill_random(63)
        ins = [gen.random_bit_patterns((M, N), 4, 64, j) for j in range(W)]
        blk = M * N * 4
        # rank j's input already sits in its own slot of its own region (in place)
        for j in range(W):
            th.region(j)[j * blk:(j + 1) * blk].copy_(torch.from_numpy(ins[j].view(np.uint8).reshape(-1)))
        torch.cuda.synchronize()
        before = th.host()
        log("tickets in place, fp32 bit patterns")
        for j in range(W):
            ag.all_gather_ex(th.view(j), W, 0, 1, th.heap.rank_ptr(j, j * blk), 0, M, N, "f32", 8, 256, 16,
                             tile_order="tickets")
        _check(th, before, ins, S, 0, 1, 0)
    finally:
        th.close()


@pytest.mark.parametrize("dtype,programs", [("f16", 256), ("bf16", 300), ("f32", 256), ("f16", 128), ("f32", 96),
                                            ("f32", 64), ("f16", 192)])
def test_ticket_order_with_and_without_the_wait_after_each_ticket(dtype, programs):
    """Wide launches take each ticket after the stores of the batch before it (plan.ticket_wait), narrower
    ones before; same bytes either way."""
    require_gpu()
    W, M, N = 4, 2048, 2048
    e = E[dtype]
    S = ((W * M * N * e + 4096) // 256 + 1) * 256
    th = TorchHeap(8, S)
    try:
        ins = [gen.uniform_pm1((M, N), dtype, 65, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        p = ag.plan_all_gather_ex(th.view(2).geometry(), W, 2, 1, dev[0], 256, M, N, dtype, 8, 256, programs,
                                  tile_order="tickets")
        cus = th.view(2).geometry().num_cus
        assert p.ticket_wait == (1 if 4 * min(programs, -(-p.total_tiles // p.tiles_per_ticket)) * p.vectors_per_thread
                                 >= 3 * cus else 0)
        log(f"tickets {dtype} W={W} {M}x{N} programs={programs}: wait={p.ticket_wait} G={p.tiles_per_ticket}")
        before = th.host()
        _run(th, dev, W, 2, 1, 256, M, N, dtype, (8, 256), programs)
        _check(th, before, ins, S, 2, 1, 256)
    finally:
        th.close()


def test_stale_counter_from_overlapping_calls_and_its_clearing():
    """A counter left non-zero (what calls of one rank overlapping in time can leave, planted here from the
    host) makes that rank's next ticket-order call skip tiles; ag_heap_clear_tickets restores it.  Every
    kernel still ends normally: tickets past the last tile only end a program's loop."""
    require_gpu()
    W, M, N, dtype = 2, 512, 4096, "f16"
    S = ((W * M * N * 2 + 4096) // 256 + 1) * 256
    th = TorchHeap(2, S)
    try:
        ins = [gen.uniform_pm1((M, N), dtype, 66, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        info = th.heap.info()
        start = info["base_table"] + -(-8 * info["n_ranks"] // 256) * 256

        class _C:
            __cuda_array_interface__ = {"shape": (info["n_ranks"] * 16,), "typestr": "<u4", "data": (start, False),
                                        "version": 3, "strides": None}

        counters = torch.as_tensor(_C(), device="cuda")
        counters[0] = 100000          # rank 0's ticket counter, past every ticket of the call
        counters[1] = 7               # and its finished-programs count
        torch.cuda.synchronize()
        before = th.host()
        log("tickets: stale counter planted on rank 0")
        _run(th, dev, W, 0, 1, 0, M, N, dtype, (8, 256), 4)
        got = th.host()
        want = all_gather_oracle(before, S, ins, 0, 1, 0)
        blk = M * N * 2
        # rank 0's rows were not stored anywhere; rank 1's were
        for r in range(W):
            assert np.array_equal(got[r * S:r * S + blk], before[r * S:r * S + blk]), "stale counter still copied"
            assert np.array_equal(got[r * S + blk:r * S + 2 * blk], want[r * S + blk:r * S + 2 * blk])
        th.heap.clear_tickets()
        assert not _counters(th).any()
        th.fill(gen.SENTINEL16)
        torch.cuda.synchronize()
        before = th.host()
        log("tickets: after ag_heap_clear_tickets")
        _run(th, dev, W, 0, 1, 0, M, N, dtype, (8, 256), 4)
        _check(th, before, ins, S, 0, 1, 0)
    finally:
        th.close()
