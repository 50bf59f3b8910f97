"""The launching entry points under HIP graph capture, replayed.

A serving loop captures its calls once and replays the graph.  Every call here
only launches kernels on the stream it is given (no allocation, no memset, no
copy), and the ticket order's counters are back at zero when each launch ends,
so a captured call must give the oracle's result on every replay.  Each graph
is replayed several times; between replays the program's own eager work
refills the heap and changes the inputs in place, with synchronisations, and
the whole heap is compared with the CPU oracle after every replay.
"""

import numpy as np
import pytest
import torch

from gemm_all_gather_amd import binding as ag
from gemm_all_gather_amd import inputs as gen
from oracle import all_gather_oracle, all_to_all_oracle, gemm_all_gather_oracle
from tests.gpu_util import TorchHeap, log, require_gpu, to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(calls):
    """A graph of calls(stream) captured on a side stream (after one eager warm-up run there)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return g


def _check(got, want, what):
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        raise AssertionError(f"{what}: {bad.size} bytes differ, first at byte {bad[0]}")


def _replays(th, dev, make_inputs, graph, oracle, what):
    for rep in range(REPLAYS):
        ins = make_inputs(rep)
        th.fill(gen.SENTINEL16)                              # eager work between replays
        for d, x in zip(dev, ins):
            d.copy_(torch.from_numpy(np.ascontiguousarray(x).view(np.uint8).reshape(-1)))
        torch.cuda.synchronize()
        before = th.host()
        log(f"{what}: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        _check(th.host(), oracle(before, ins), f"{what}, replay {rep}")


@pytest.mark.parametrize("noalloc", [False, True])
def test_all_gather_in_ticket_order_replayed(noalloc):
    require_gpu()
    W, M, N, off, programs = 4, 2048, 4096, 512, 64
    S = ((W * M * N * 2 + off + 4096) // 256 + 1) * 256
    th = TorchHeap(4, S)
    try:
        dev = [to_device(gen.uniform_pm1((M, N), "f16", 80, j)) for j in range(W)]
        p = ag.plan_all_gather(th.view(0).geometry(), W, 0, 1, dev[0], off, M, N, "f16", 8, 256, programs)
        assert p.tile_order == ag.AG_ORDER_TICKETS               # the counter is part of every replay
        call = ag.all_gather_noalloc if noalloc else ag.all_gather

        def calls(stream):
            for j in range(W):
                call(th.view(j), W, 0, 1, dev[j], off, M, N, "f16", 8, 256, programs, stream=stream)

        g = _capture(calls)
        _replays(th, dev, lambda rep: [gen.uniform_pm1((M, N), "f16", 81 + rep, j) for j in range(W)], g,
                 lambda before, ins: all_gather_oracle(before, S, ins, 0, 1, off),
                 f"all_gather{'_noalloc' if noalloc else ''} graph")
    finally:
        th.close()


@pytest.mark.parametrize("order", ["stride", "tickets"])
def test_all_to_all_replayed(order):
    require_gpu()
    W, Mc, N = 4, 64, 1024
    S = ((W * Mc * N * 2 + 4096) // 256 + 1) * 256
    th = TorchHeap(4, S)
    try:
        dev = [to_device(gen.random_bit_patterns((W * Mc, N), 2, 90, j)) for j in range(W)]
        p = ag.plan_all_to_all_ex(th.view(0).geometry(), W, 0, 1, dev[0], 0, Mc, N, "f16", 0, 0, 0, tile_order=order)
        assert p.tile_order == (ag.AG_ORDER_TICKETS if order == "tickets" else ag.AG_ORDER_STRIDE)

        def calls(stream):
            for j in range(W):
                ag.all_to_all_ex(th.view(j), W, 0, 1, dev[j], 0, Mc, N, "f16", 0, 0, 0, stream=stream, tile_order=order)

        g = _capture(calls)
        _replays(th, dev, lambda rep: [gen.random_bit_patterns((W * Mc, N), 2, 91 + rep, j) for j in range(W)], g,
                 lambda before, ins: all_to_all_oracle(before, S, ins, 0, 1, 0), f"all_to_all graph ({order})")
    finally:
        th.close()


def test_fused_gemm_all_gather_replayed():
    """Integer operands (every partial sum exact in fp32): bit-exact on every replay."""
    require_gpu()
    W, M, N, K = 4, 300, 264, 128
    S = ((W * M * N * 2 + 4096) // 256 + 1) * 256
    th = TorchHeap(4, S)
    try:
        b = [gen.small_integers((N, K), "f16", -3, 3, 92, j) for j in range(W)]
        b_dev = [to_device(x) for x in b]
        a_dev = [to_device(gen.small_integers((M, K), "f16", -3, 3, 93, j)) for j in range(W)]

        def calls(stream):
            for j in range(W):
                ag.gemm_all_gather(th.view(j), W, 0, 1, a_dev[j], K, b_dev[j], K, 0, M, N, K, "f16", 0, 0, 0, 0,
                                   stream=stream)

        g = _capture(calls)
        _replays(th, a_dev, lambda rep: [gen.small_integers((M, K), "f16", -3, 3, 94 + rep, j) for j in range(W)], g,
                 lambda before, a: gemm_all_gather_oracle(before, S, a, b, "f16", 0, 1, 0), "fused graph")
    finally:
        th.close()
