"""Parity of the fused GEMM + all-gather with B stored N-contiguous (a row-major
K x N matrix, ag_gemm_all_gather_ex with AG_B_N_CONTIGUOUS) against the oracle.

* small-integer operands: exact products and sums, so the whole heap must
  match the oracle bit for bit (the oracle takes B in its K x N form);
* random operands: the N-contiguous kernel must reproduce the K-contiguous
  kernel's output bit for bit (both accumulate every entry over k in the same
  order), and stay within the tolerance of the float64 product;
* the benchmark's full size: sampled entries against the oracle, every
  member region identical, guards untouched.
"""

import numpy as np
import pytest
import torch

from gemm_all_gather_amd import binding as ag
from gemm_all_gather_amd import inputs as gen
from oracle import gemm_all_gather_oracle
from tests.fused_check import check_entries, tile_samples
from tests.gpu_util import TorchHeap, log, require_gpu, to_device
from tests.test_fused_gpu import _full_size_heap, _region_size

pytestmark = pytest.mark.gpu

TILES_N = [(256, 224, 64), (128, 128, 64), (0, 0, 0)]


def _kn(b_nk: np.ndarray, ldb: int) -> np.ndarray:
    """N x K bit patterns -> a K x ldb row-major array holding B^T; columns past N are padding."""
    n, k = b_nk.shape
    out = np.full((k, ldb), 0x3C00, dtype=np.uint16)
    out[:, :n] = b_nk.T
    return np.ascontiguousarray(out)


def _run(th, a_dev, b_dev, W, start, stride, off, M, N, K, ldb, dtype, tile, layout, programs=0):
    for j in range(W):
        ag.gemm_all_gather_ex(th.view(start + j * stride), W, start, stride, a_dev[j], K, b_dev[j], ldb, off, M, N,
                              K, dtype, tile[0], tile[1], tile[2], programs, b_layout=layout)


CASES = []
for M, N, K in [(1, 8, 64), (37, 136, 128), (256, 224, 64), (300, 520, 192), (129, 232, 448), (512, 256, 128)]:
    for tile in TILES_N:
        CASES.append((M, N, K, tile))


@pytest.mark.parametrize("M,N,K,tile", CASES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_n_contiguous_integer_operands_bit_exact(M, N, K, tile, dtype):
    require_gpu()
    rng = np.random.default_rng([M, N, K, tile[0], tile[1], 7])
    W, start, stride = [(1, 0, 1), (2, 1, 1), (4, 0, 2), (8, 0, 1), (3, 2, 2)][int(rng.integers(0, 5))]
    ldb = N + 8 * int(rng.integers(0, 3))
    lo, hi = (-3, 3) if dtype == "f16" else (-2, 2)
    off = 512 * int(rng.integers(0, 4))
    log(f"fused N-contiguous B int M={M} N={N} K={K} ldb={ldb} tile={tile} {dtype} W={W} group=({start},{stride})")
    a = [gen.small_integers((M, K), dtype, lo, hi, 11, M, N, K, j) for j in range(W)]
    b = [gen.small_integers((N, K), dtype, lo, hi, 12, M, N, K, j) for j in range(W)]
    S = _region_size(W, M, N, off)
    th = TorchHeap(8, S)
    try:
        before = th.host()
        _run(th, [to_device(x) for x in a], [to_device(_kn(x, ldb)) for x in b], W, start, stride, off, M, N, K,
             ldb, dtype, tile, "n")
        got = th.host()
        want = gemm_all_gather_oracle(before, S, a, [np.ascontiguousarray(x.T) for x in b], dtype, start, stride,
                                      off, b_layout="kn")
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            raise AssertionError(f"{bad.size} bytes differ, first at region {bad[0] // S} offset {bad[0] % S}")
    finally:
        th.close()


@pytest.mark.parametrize("tile", [(256, 224, 64), (128, 128, 64)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_n_contiguous_matches_k_contiguous_and_tolerance(tile, dtype):
    require_gpu()
    M, N, K, W = 600, 464, 1024, 4
    off = 4096
    log(f"fused layouts M={M} N={N} K={K} tile={tile} {dtype} W={W}")
    a = [gen.normal_scaled((M, K), dtype, 1.0, 13, j) for j in range(W)]
    b = [gen.normal_scaled((N, K), dtype, K ** -0.5, 14, j) for j in range(W)]
    S = _region_size(W, M, N, off)
    outs = []
    for layout in ("k", "n"):
        th = TorchHeap(8, S)
        try:
            b_dev = [to_device(x) for x in b] if layout == "k" else [to_device(_kn(x, N)) for x in b]
            ldb = K if layout == "k" else N
            _run(th, [to_device(x) for x in a], b_dev, W, 0, 1, off, M, N, K, ldb, dtype, tile, layout)
            outs.append(th.host())
        finally:
            th.close()
    # each layout within the tolerance of the oracle's float64 product (every member, a lattice of entries) ...
    rows = np.arange(0, M, 7)
    cols = np.arange(0, N, 5)
    rr, cc = (x.ravel() for x in np.meshgrid(rows, cols, indexing="ij"))
    for layout, out in zip(("k", "n"), outs):
        blk = out[off:off + W * M * N * 2].view(np.uint16).reshape(W * M, N)
        for j in range(W):
            # unit-variance C: bf16's own rounding exceeds the 2e-2 absolute bar, the fp32 bound still holds
            check_entries(blk[j * M + rr, cc], a[j], b[j], dtype, rr, cc,
                          max_abs=None if dtype == "bf16" else 2e-2, what=f"{layout} rank {j}")
    # ... and the two layouts bit-identical over the whole heap
    assert np.array_equal(outs[0], outs[1]), "the two B layouts give different bits"


def test_n_contiguous_full_size_m16384_fp16():
    """The four corners and one interior entry of every output tile of every rank, B N-contiguous."""
    require_gpu()
    M, N, K, W, dtype = 16384, 3584, 8192, 8, "f16"
    log(f"full-size fused, B N-contiguous, W=8 M_local={M} N={N} K={K} {dtype}: generating inputs")
    a = [gen.normal_scaled((M, K), dtype, K ** -0.5, 42, j) for j in range(W)]
    b_nk = gen.normal_scaled((N, K), dtype, K ** -0.5, 42, 99)
    b_kn = np.ascontiguousarray(b_nk.T)
    a_dev = [to_device(x) for x in a]
    b_dev = to_device(b_kn)
    blk = M * N * 2
    guard = 1 << 20
    S = W * blk + 2 * guard
    th = TorchHeap(W, S)
    try:
        p = ag.plan_gemm_all_gather_ex(th.view(0).geometry(), W, 0, 1, a_dev[0], K, b_dev, N, guard, M, N, K, dtype,
                                       0, 0, 0, 0, b_layout="n")
        log(f"  running ({p.tile_m}x{p.tile_n} tiles)")
        _run(th, a_dev, [b_dev] * W, W, 0, 1, guard, M, N, K, N, dtype, (0, 0, 0), "n")
        torch.cuda.synchronize()
        ref_region = _full_size_heap(th, W, blk, guard)
        out = ref_region.cpu().numpy().view(np.uint16).reshape(W * M, N)
        rng = np.random.default_rng(42)
        for j in range(W):
            rows, cols = tile_samples(M, N, p.tile_m, p.tile_n, rng)
            check_entries(out[j * M + rows, cols], a[j], b_kn, dtype, rows, cols, b_layout="kn", what=f"rank {j}")
    finally:
        th.close()
