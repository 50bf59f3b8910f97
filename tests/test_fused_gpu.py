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
from oracle import (gemm_all_gather_oracle, gemm_oracle, gemm_oracle_entries, all_gather_oracle,
                    decode_bits, group_members)
from tests.gpu_util import TorchHeap, log, require_gpu, to_device

pytestmark = pytest.mark.gpu

TILES = [(256, 256, 64), (256, 224, 64), (128, 128, 64), (0, 0, 0)]
MAX_ABS = 2e-2
MAX_REL = 1e-2


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


def _check_tolerance(got_bits, a_bits, b_bits, dtype, exact=None, max_abs=MAX_ABS):
    """Tolerance and rigorous fp32-accumulation bound against the float64 product.

    max_abs=None skips the absolute bar: with unit-variance C, bf16's own
    rounding (half an ulp is 2^-8 |C|) exceeds 2e-2 once |C| > 5.
    """
    A = decode_bits(a_bits, dtype)
    B = decode_bits(b_bits, dtype)
    if exact is None:
        exact = A @ B.T
    got = decode_bits(got_bits, dtype)
    K = A.shape[1]
    err = np.abs(got - exact)
    assert np.all(np.isfinite(got))
    if max_abs is not None:
        assert err.max() <= max_abs, f"max abs error {err.max()}"
    rel = np.linalg.norm(got - exact) / max(np.linalg.norm(exact), 1e-300)
    assert rel <= MAX_REL, f"relative error {rel}"
    # |fl32(sum) - exact| <= K u32 sum|a||b|; the final rounding adds at most one ulp of the output type
    ulp = (2.0 ** -10 if dtype == "f16" else 2.0 ** -7) * np.maximum(np.abs(exact), 2.0 ** -14)
    bound = ulp + 2 * K * 2.0 ** -24 * (np.abs(A) @ np.abs(B).T)
    assert np.all(err <= bound), f"{np.count_nonzero(err > bound)} entries outside the fp32 bound"
    return err.max(), rel


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
                _check_tolerance(out, a[j], b[j], dtype,
                                 max_abs=None if (scale_a == "unit" and dtype == "bf16") else MAX_ABS)
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
# full-size workloads (the benchmark's launch configuration: tiles and programs chosen by the library)
# ---------------------------------------------------------------------------

def _full_size(M, N, K, dtype, seed, samples=1500):
    require_gpu()
    W = 8
    log(f"full-size fused W=8 M_local={M} N={N} K={K} {dtype}: generating inputs")
    a = [gen.normal_scaled((M, K), dtype, K ** -0.5, seed, j) for j in range(W)]
    b = gen.normal_scaled((N, K), dtype, K ** -0.5, seed, 99)
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
        sentinel = torch.tensor([int(np.uint16(gen.SENTINEL16).view(np.int16))], device="cuda", dtype=torch.int16)
        ref_region = th.region(0)[guard:guard + W * blk]
        for r in range(W):
            reg = th.region(r)
            assert torch.equal(reg[guard:guard + W * blk], ref_region), f"region {r} differs from region 0"
            assert torch.all(reg[:guard].view(torch.int16) == sentinel)
            assert torch.all(reg[guard + W * blk:].view(torch.int16) == sentinel)
        out = ref_region.cpu().numpy().view(np.uint16).reshape(W * M, N)
        rng = np.random.default_rng(seed)
        worst = 0.0
        for j in range(W):
            rows = rng.integers(0, M, samples)
            cols = rng.integers(0, N, samples)
            rows[:4] = [0, M - 1, 0, M - 1]
            cols[:4] = [0, N - 1, N - 1, 0]
            want = gemm_oracle_entries(a[j], b, dtype, rows, cols, "nk")
            got = out[j * M + rows, cols]
            A = decode_bits(a[j][rows], dtype)
            Bc = decode_bits(b[cols], dtype)
            exact = np.einsum("ik,ik->i", A, Bc)
            g = decode_bits(got, dtype)
            err = np.abs(g - exact)
            worst = max(worst, err.max())
            assert err.max() <= MAX_ABS
            ulp = (2.0 ** -10 if dtype == "f16" else 2.0 ** -7) * np.maximum(np.abs(exact), 2.0 ** -14)
            bound = ulp + 2 * K * 2.0 ** -24 * np.einsum("ik,ik->i", np.abs(A), np.abs(Bc))
            assert np.all(err <= bound)
            # the oracle's rounded value and the GPU's differ by at most one output ulp
            assert np.all(np.abs(decode_bits(want, dtype) - g) <= ulp + bound)
        log(f"  max abs error over samples {worst:.3e}")
    finally:
        th.close()


def test_full_size_m1024_fp16():
    _full_size(1024, 3584, 8192, "f16", 40)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_full_size_m16384(dtype):
    _full_size(16384, 3584, 8192, dtype, 41)
