"""Parity of the HIP fused GEMM + all-gather (through the C ABI) with the CPU oracle.

* small-integer operands: every partial sum is exact in fp32 and C is exact
  in the 16-bit output type, so the GPU must match the oracle bit for bit
  over the whole heap (outputs, guards, non-member regions);
* random operands: within the stated tolerance (max |err| <= 2e-2 and
  normwise relative error <= 1e-2) and inside a rigorous per-element bound
  for fp32 accumulation followed by one rounding;
* full-size workloads: sampled entries computed one by one by the oracle,
  plus invariants (every member region identical, guards untouched).
"""

import numpy as np
import pytest
import torch

from gemm_all_gather_amd import binding as ag
from gemm_all_gather_amd import inputs as gen
from oracle import gemm_all_gather_oracle, decode_bits
from tests.fused_check import MAX_ABS, check_entries, check_full, tile_samples
from tests.gpu_util import TorchHeap, log, require_gpu, to_device

pytestmark = pytest.mark.gpu

TILES = [(256, 256, 64), (256, 224, 64), (128, 128, 64), (0, 0, 0)]


def _run_fused(th, a_dev, b_dev, W, start, stride, off, M, N, K, dtype, tile, programs=0, stream=None):
    for j in range(W):
        r = start + j * stride
        ag.gemm_all_gather(th.view(r), W, start, stride, a_dev[j], K, b_dev[j], K, off, M, N, K, dtype,
                           tile[0], tile[1], tile[2], programs, stream)


def _region_size(W, M, N, off):
    return ((off + W * M * N * 2 + 4096) // 256 + 1) * 256


CASES = []
for M, N, K in [(1, 8, 64), (37, 136, 128), (256, 224, 64), (300, 520, 192), (129, 232, 448), (512, 256, 128)]:
    for tile in TILES:
        CASES.append((M, N, K, tile))


@pytest.mark.parametrize("M,N,K,tile", CASES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_integer_operands_bit_exact(M, N, K, tile, dtype):
    require_gpu()
    rng = np.random.default_rng([M, N, K, tile[0], tile[1]])
    W, start, stride = [(1, 0, 1), (2, 1, 1), (4, 0, 2), (8, 0, 1), (3, 2, 2)][int(rng.integers(0, 5))]
    lo, hi = (-3, 3) if dtype == "f16" else (-2, 2)
    off = 512 * int(rng.integers(0, 4))
    log(f"fused int M={M} N={N} K={K} tile={tile} {dtype} W={W} group=({start},{stride}) off={off}")
    a = [gen.small_integers((M, K), dtype, lo, hi, 1, M, N, K, j) for j in range(W)]
    b = [gen.small_integers((N, K), dtype, lo, hi, 2, M, N, K, j) for j in range(W)]
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


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("scale_a", ["scaled", "unit"])
def test_random_operands_within_tolerance(dtype, tile, scale_a):
    require_gpu()
    M, N, K, W = 300, 520, 1024, 2
    log(f"fused random {dtype} tile={tile} A={scale_a}")
    sa = K ** -0.5 if scale_a == "scaled" else 1.0       # N(0,1)/sqrt(K) on both, or unit-variance C
    a = [gen.normal_scaled((M, K), dtype, sa, 3, j) for j in range(W)]
    b = [gen.normal_scaled((N, K), dtype, K ** -0.5, 4, j) for j in range(W)]
    S = _region_size(W, M, N, 0)
    th = TorchHeap(2, S)
    try:
        _run_fused(th, [to_device(x) for x in a], [to_device(x) for x in b], W, 0, 1, 0, M, N, K, dtype, tile)
        host = th.host()
        blk = M * N * 2
        for r in range(W):
            for j in range(W):
                out = host[r * S + j * blk:r * S + (j + 1) * blk].view(np.uint16).reshape(M, N)
                # with unit-variance C, bf16's own rounding (half an ulp is 2^-8 |C|) exceeds 2e-2 once |C| > 5
                check_full(out, a[j], b[j], dtype,
                           max_abs=None if (scale_a == "unit" and dtype == "bf16") else MAX_ABS,
                           what=f"region {r} rank {j}")
                if scale_a == "unit":
                    assert np.abs(decode_bits(out, dtype)).max() > 0.5     # non-trivial output
    finally:
        th.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_identity_b_returns_a(dtype):
    require_gpu()
    M, K = 200, 256
    log(f"fused B=I {dtype}")
    a = [gen.uniform_pm1((M, K), dtype, 5)]
    eye = np.eye(K, dtype=np.float32)
    b = [gen._encode_f32(eye, dtype)]
    S = _region_size(1, M, K, 0)
    th = TorchHeap(1, S)
    try:
        _run_fused(th, [to_device(a[0])], [to_device(b[0])], 1, 0, 1, 0, M, K, K, dtype, (0, 0, 0))
        out = th.host()[:M * K * 2].view(np.uint16).reshape(M, K)
        assert np.array_equal(out, a[0])
    finally:
        th.close()


def test_fused_equals_gemm_then_all_gather():
    require_gpu()
    M, N, K, W, dtype = 260, 360, 512, 4, "f16"
    log("fused vs W=1 GEMM + all-gather")
    a = [gen.normal_scaled((M, K), dtype, K ** -0.5, 6, j) for j in range(W)]
    b = gen.normal_scaled((N, K), dtype, K ** -0.5, 7)
    a_dev = [to_device(x) for x in a]
    b_dev = to_device(b)
    S = _region_size(W, M, N, 0)
    fused = TorchHeap(W, S)
    split = TorchHeap(W, S)
    scratch = TorchHeap(W, ((M * N * 2) // 256 + 1) * 256)
    try:
        _run_fused(fused, a_dev, [b_dev] * W, W, 0, 1, 0, M, N, K, dtype, (0, 0, 0))
        cs = []
        for j in range(W):   # C_j alone in region j of a scratch heap, then gathered by the copy kernel
            ag.gemm_all_gather(scratch.view(j), 1, j, 1, a_dev[j], K, b_dev, K, 0, M, N, K, dtype)
            cs.append(scratch.heap.rank_ptr(j, 0))
        torch.cuda.synchronize()
        for j in range(W):
            ag.all_gather(split.view(j), W, 0, 1, cs[j], 0, M, N, dtype)
        assert np.array_equal(fused.host(), split.host())
    finally:
        fused.close()
        split.close()
        scratch.close()


def test_fused_validation_on_launching_entry_point():
    require_gpu()
    log("fused validation")
    th = TorchHeap(2, 1 << 20)
    try:
        a = to_device(gen.uniform_pm1((64, 128), "f16", 8))
        b = to_device(gen.uniform_pm1((64, 128), "f16", 9))
        base = dict(W=2, rank_start=0, rank_stride=1, A=a, lda=128, B=b, ldb=128, out_offset=0, M_local=64, N=64,
                    K=128, dtype="f16")
        for over, status in [(dict(dtype="f32"), ag.AG_ERR_UNSUPPORTED), (dict(K=100), ag.AG_ERR_UNSUPPORTED),
                             (dict(lda=64), ag.AG_ERR_INVALID_ARG), (dict(out_offset=8), ag.AG_ERR_UNSUPPORTED),
                             (dict(A=0), ag.AG_ERR_INVALID_ARG), (dict(W=9), ag.AG_ERR_UNSUPPORTED)]:
            with pytest.raises(ag.AgError) as ei:
                ag.gemm_all_gather(th.view(0), **dict(base, **over))
            assert ei.value.status == status
        torch.cuda.synchronize()
        assert np.all(th.host().view(np.uint16) == gen.SENTINEL16)
        ag.gemm_all_gather(th.view(1), **dict(base, M_local=0))       # no-op
        torch.cuda.synchronize()
        assert np.all(th.host().view(np.uint16) == gen.SENTINEL16)
    finally:
        th.close()


# ---------------------------------------------------------------------------
# many tiles per program over full groups of the grouped tile order, bit-exact
# ---------------------------------------------------------------------------

# (tile, programs): 256x224 gives 10 x 3 tiles at M=2400, N=464 (8 tile rows of the grouped order, then a
# ragged group of 2), 128x128 gives 19 x 4 (8 + 8 + 3), 256x256 gives 10 x 2; the program counts give each
# program 4 to 10 tiles, with and without the XCD renumbering (counts that are multiples of 8), and one tile
# per program at 256
MANY_TILES = [((256, 224, 64), 6), ((256, 224, 64), 8), ((128, 128, 64), 8), ((128, 128, 64), 16),
              ((128, 128, 64), 19), ((256, 256, 64), 5), ((256, 224, 64), 256), ((0, 0, 0), 0)]


@pytest.mark.parametrize("tile,programs", MANY_TILES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_integer_operands_many_tiles_per_program_bit_exact(tile, programs, dtype):
    require_gpu()
    M, N, K, W = 2400, 464, 128, 8
    lo, hi = (-3, 3) if dtype == "f16" else (-2, 2)     # every partial sum an integer below 2^24
    off = 1024
    log(f"fused int many tiles M={M} N={N} K={K} tile={tile} programs={programs} {dtype} W={W}")
    a = [gen.small_integers((M, K), dtype, lo, hi, 21, j) for j in range(W)]
    b = [gen.small_integers((N, K), dtype, lo, hi, 22, j) for j in range(W)]
    S = _region_size(W, M, N, off)
    th = TorchHeap(8, S)
    try:
        if tile != (0, 0, 0):
            p = ag.plan_gemm_all_gather(th.view(0).geometry(), W, 0, 1, 1 << 40, K, 1 << 41, K, off, M, N, K, dtype,
                                        tile[0], tile[1], tile[2], programs)
            assert p.tiles_m >= 9                                   # full 8-row groups plus a ragged one
            if programs < 256:
                assert -(-p.total_tiles // p.n_programs) >= 4            # the busiest program walks >= 4 tiles
        before = th.host()
        _run_fused(th, [to_device(x) for x in a], [to_device(x) for x in b], W, 0, 1, off, M, N, K, dtype, tile,
                   programs)
        got = th.host()
        want = gemm_all_gather_oracle(before, S, a, b, dtype, 0, 1, off)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            raise AssertionError(f"{bad.size} bytes differ, first at region {bad[0] // S} offset {bad[0] % S}")
    finally:
        th.close()


# ---------------------------------------------------------------------------
# full-size workloads (the benchmark's launch configuration: tiles and programs chosen by the library,
# and the 256x256 tile of the pages' fused kernel)
# ---------------------------------------------------------------------------

def _full_size_heap(th, W, blk, guard):
    """Every member region identical, guards untouched, no output word left at the fill pattern, all finite."""
    sentinel = torch.tensor([int(np.uint16(gen.SENTINEL16).view(np.int16))], device="cuda", dtype=torch.int16)
    ref_region = th.region(0)[guard:guard + W * blk]
    for r in range(W):
        reg = th.region(r)
        assert torch.equal(reg[guard:guard + W * blk], ref_region), f"region {r} differs from region 0"
        assert torch.all(reg[:guard].view(torch.int16) == sentinel), f"guard before region {r}'s output"
        assert torch.all(reg[guard + W * blk:].view(torch.int16) == sentinel), f"guard after region {r}'s output"
    words = ref_region.view(torch.int16)
    assert not torch.any(words == sentinel), "an output word still holds the fill pattern (unwritten entry)"
    return ref_region


_INPUTS = {}


def _inputs(M, N, K, dtype, seed, W=8):
    """Seeded operands, cached across the full-size cases of one shape (N(0,1)/sqrt(K) on A and B)."""
    key = (M, N, K, dtype, seed)
    if key not in _INPUTS:
        _INPUTS.clear()
        a = [gen.normal_scaled((M, K), dtype, K ** -0.5, seed, j) for j in range(W)]
        b = gen.normal_scaled((N, K), dtype, K ** -0.5, seed, 99)
        _INPUTS[key] = (a, b)
    return _INPUTS[key]


def test_full_size_m1024_fp16_every_element():
    """M_local 1024 (fused context workload): every element of every rank's C_j against the oracle."""
    require_gpu()
    M, N, K, W, dtype = 1024, 3584, 8192, 8, "f16"
    log(f"full-size fused W=8 M_local={M} N={N} K={K} {dtype}: generating inputs")
    a, b = _inputs(M, N, K, dtype, 40)
    a_dev = [to_device(x) for x in a]
    b_dev = to_device(b)
    blk = M * N * 2
    guard = 1 << 20
    S = W * blk + 2 * guard
    th = TorchHeap(W, S)
    try:
        log("  running")
        _run_fused(th, a_dev, [b_dev] * W, W, 0, 1, guard, M, N, K, dtype, (0, 0, 0))
        torch.cuda.synchronize()
        ref_region = _full_size_heap(th, W, blk, guard)
        out = ref_region.cpu().numpy().view(np.uint16).reshape(W * M, N)
        log("  comparing every element with the oracle")
        worst = 0.0
        for j in range(W):
            err, rel = check_full(out[j * M:(j + 1) * M], a[j], b, dtype, what=f"rank {j}")
            worst = max(worst, err)
        log(f"  max abs error {worst:.3e}")
    finally:
        th.close()


@pytest.mark.parametrize("tile", [(0, 0, 0), (256, 256, 64)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_full_size_m16384(dtype, tile):
    """M_local 16384: the four corners and one interior entry of every output tile of every rank."""
    _full_size_sampled(16384, dtype, tile, 41)


def test_full_size_m4096_fp16():
    """M_local 4096 (the pages' middle fused row: 256 tiles of 256x224, one per CU), sampled per tile."""
    _full_size_sampled(4096, "f16", (0, 0, 0), 42)


def _full_size_sampled(M, dtype, tile, seed):
    require_gpu()
    N, K, W = 3584, 8192, 8
    log(f"full-size fused W=8 M_local={M} N={N} K={K} {dtype} tile={tile}: generating inputs")
    a, b = _inputs(M, N, K, dtype, seed)
    a_dev = [to_device(x) for x in a]
    b_dev = to_device(b)
    blk = M * N * 2
    guard = 1 << 20
    S = W * blk + 2 * guard
    th = TorchHeap(W, S)
    try:
        p = ag.plan_gemm_all_gather(th.view(0).geometry(), W, 0, 1, a_dev[0], K, b_dev, K, guard, M, N, K, dtype,
                                    *tile, 0)
        log(f"  running ({p.tile_m}x{p.tile_n} tiles, {p.n_programs} programs)")
        _run_fused(th, a_dev, [b_dev] * W, W, 0, 1, guard, M, N, K, dtype, tile)
        torch.cuda.synchronize()
        ref_region = _full_size_heap(th, W, blk, guard)
        out = ref_region.cpu().numpy().view(np.uint16).reshape(W * M, N)
        rng = np.random.default_rng([seed, p.tile_m, p.tile_n])
        worst = 0.0
        for j in range(W):
            rows, cols = tile_samples(M, N, p.tile_m, p.tile_n, rng)
            err, _ = check_entries(out[j * M + rows, cols], a[j], b, dtype, rows, cols, what=f"rank {j}")
            worst = max(worst, err)
        log(f"  {rows.size} entries per rank, max abs error {worst:.3e}")
    finally:
        th.close()
        del a_dev, b_dev
        torch.cuda.empty_cache()
