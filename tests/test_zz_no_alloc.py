"""ag_all_gather_noalloc (the allocation-free entry point) against ag_all_gather_ex, through the C ABI.

Two calls in a row, the second with a smaller input, each in the ticket order
(the path whose tile counter lives in the library's fixed device array) and in
the library's own choice of order; the whole heap must match the allocating
entry point's byte for byte, and the oracle's.
"""

import numpy as np
import pytest

from gemm_all_gather_amd import binding as ag
from gemm_all_gather_amd import inputs as gen
from oracle import all_gather_oracle
from tests.gpu_util import TorchHeap, log, require_gpu, to_device

pytestmark = pytest.mark.gpu


def _gather(fn, th, dev, W, M, N, dtype, order, programs):
    for j in range(W):
        fn(th.view(j), W, 0, 1, dev[j], 4096, M, N, dtype, 8, 256, programs, tile_order=order)


@pytest.mark.parametrize("order", ["tickets", "auto"])
def test_noalloc_matches_the_allocating_entry_point(order):
    require_gpu()
    W = 8
    # the second call's input is smaller than the first's
    for M, N, dtype, programs in [(2048, 4096, "f16", 256), (333, 1032, "bf16", 64)]:
        log(f"noalloc vs ag_all_gather_ex: W={W} {M}x{N} {dtype} programs={programs} order={order}")
        S = ((4096 + W * M * N * 2 + 4096) // 256 + 1) * 256
        ins = [gen.uniform_pm1((M, N), dtype, 71, M, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        ref, got = TorchHeap(8, S), TorchHeap(8, S)
        try:
            before = ref.host()
            assert np.array_equal(before, got.host())
            _gather(ag.all_gather_ex, ref, dev, W, M, N, dtype, order, programs)
            _gather(ag.all_gather_noalloc, got, dev, W, M, N, dtype, order, programs)
            a, b = ref.host(), got.host()
            assert np.array_equal(a, b), "the allocation-free entry point differs from ag_all_gather_ex"
            assert np.array_equal(b, all_gather_oracle(before, S, ins, 0, 1, 4096))
        finally:
            ref.close()
            got.close()


def test_noalloc_rejects_heaps_beyond_its_counters():
    require_gpu()
    n = ag.AG_NOALLOC_MAX_RANKS + 1
    th = TorchHeap(n, 1 << 16)
    try:
        x = to_device(gen.uniform_pm1((8, 256), "f16", 72))
        with pytest.raises(ag.AgError) as ei:
            ag.all_gather_noalloc(th.view(n - 1), 1, n - 1, 1, x, 0, 8, 256, "f16")
        assert ei.value.status == ag.AG_ERR_UNSUPPORTED and str(ag.AG_NOALLOC_MAX_RANKS) in ei.value.message
        assert np.all(th.host().view(np.uint16) == gen.SENTINEL16)          # nothing launched
    finally:
        th.close()
