"""Parity at the group sizes the other sweeps leave out (W = 5, 6 and 7), and
the fused kernel on small persistent grids.

The kernels unroll the destination loop for every W in 1..8; these cases run
the plain all-gather, the all-to-all and the fused GEMM + all-gather at the
three odd-sized groups, contiguous and offset, each against the oracle over
the whole heap (bit-exact; the fused cases use small-integer operands, whose
products and sums are exact).  The last test gives the fused kernel 1 to 24
programs for a ragged 600 x 464 output, so every program walks many tiles.
"""

import numpy as np
import pytest

from gemm_all_gather_amd import inputs as gen
from oracle import gemm_all_gather_oracle
from tests.gpu_util import TorchHeap, log, require_gpu, to_device
from tests.test_copy_gpu import _case
from tests.test_fused_gpu import _region_size, _run_fused
from tests.test_variants_gpu import _a2a, _size

pytestmark = pytest.mark.gpu

# (W, rank_start, rank_stride) inside 8 regions
GROUPS = [(5, 0, 1), (5, 3, 1), (6, 1, 1), (6, 2, 1), (7, 0, 1), (7, 1, 1)]


@pytest.mark.parametrize("W,start,stride", GROUPS)
@pytest.mark.parametrize("M,N,dtype,tile,programs,off", [
    (13, 257, "f16", (8, 256), 3, 6),          # 2-byte vectors, partial tiles
    (64, 520, "bf16", (4, 64), 64, 6),
    (9, 300, "f32", (8, 256), 10_000, 12),
    (40, 264, "f16", (8, 256), 16, 0),         # 16-byte vectors, ragged last column tile
    (33, 1024, "bf16", (8, 512), 7, 4096),     # 16-byte vectors, two per thread
])
def test_all_gather_odd_worlds(W, start, stride, M, N, dtype, tile, programs, off):
    e = 4 if dtype == "f32" else 2
    S = ((off + W * M * N * e + 300) // 256 + 1) * 256
    _case(8, S, W, start, stride, M, N, dtype, off, tile, programs, seed=W * 100 + start)


@pytest.mark.parametrize("W,start,stride", GROUPS)
def test_all_to_all_odd_worlds(W, start, stride):
    M, N = 7, 264
    _a2a(8, _size(W, M, N, 2, 64), W, start, stride, M, N, "f16", 64, (8, 256), 5, seed=W + start)


@pytest.mark.parametrize("W,start,stride", [(5, 0, 1), (6, 2, 1), (7, 1, 1)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fused_odd_worlds_bit_exact(W, start, stride, dtype):
    require_gpu()
    M, N, K = 300, 232, 192
    tile = (0, 0, 0)
    lo, hi = (-3, 3) if dtype == "f16" else (-2, 2)
    off = 1024
    log(f"fused int M={M} N={N} K={K} {dtype} W={W} group=({start},{stride}) off={off}")
    a = [gen.small_integers((M, K), dtype, lo, hi, 5, W, j) for j in range(W)]
    b = [gen.small_integers((N, K), dtype, lo, hi, 6, W, j) for j in range(W)]
    S = _region_size(W, M, N, off)
    th = TorchHeap(8, S)
    try:
        before = th.host()
        _run_fused(th, [to_device(x) for x in a], [to_device(x) for x in b], W, start, stride, off, M, N, K,
                   dtype, tile)
        got = th.host()
        want = gemm_all_gather_oracle(before, S, a, b, dtype, start, stride, off)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            raise AssertionError(f"{bad.size} bytes differ, first at region {bad[0] // S} offset {bad[0] % S}")
    finally:
        th.close()


@pytest.mark.parametrize("programs", [1, 3, 8, 24])
@pytest.mark.parametrize("tile", [(256, 224, 64), (256, 256, 64), (128, 128, 64)])
def test_fused_few_programs_many_tiles_bit_exact(programs, tile):
    """Small persistent grids: every program walks many tiles (ragged in M and N), with and without the
    XCD renumbering of the tile order (program counts that are, or are not, multiples of 8)."""
    require_gpu()
    M, N, K, dtype = 600, 464, 256, "f16"
    W, start, stride = 4, 1, 2
    off = 4096
    log(f"fused int M={M} N={N} K={K} tile={tile} programs={programs} W={W} group=({start},{stride})")
    a = [gen.small_integers((M, K), dtype, -3, 3, 7, programs, j) for j in range(W)]
    b = [gen.small_integers((N, K), dtype, -3, 3, 8, programs, j) for j in range(W)]
    S = _region_size(W, M, N, off)
    th = TorchHeap(8, S)
    try:
        before = th.host()
        _run_fused(th, [to_device(x) for x in a], [to_device(x) for x in b], W, start, stride, off, M, N, K,
                   dtype, tile, programs)
        got = th.host()
        want = gemm_all_gather_oracle(before, S, a, b, dtype, start, stride, off)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            raise AssertionError(f"{bad.size} bytes differ, first at region {bad[0] // S} offset {bad[0] % S}")
    finally:
        th.close()
