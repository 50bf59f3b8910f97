"""CPU checks of the fused-GEMM tolerance helpers used by the GPU parity tests.

A float32-accumulated product rounded once to the 16-bit type (computed here by
torch on the CPU) must pass; outputs with a planted mistake must fail; the
tile sampler must reach every tile of the grid.
"""

import numpy as np
import pytest
import torch

from gemm_all_gather_amd import inputs as gen
from oracle import decode_bits, round_f64_to_bf16_bits, round_f64_to_f16_bits
from tests.fused_check import check_entries, check_full, tile_samples


def _fp32_product(a, b, dtype):
    c32 = torch.from_numpy(decode_bits(a, dtype).astype(np.float32)) @ \
        torch.from_numpy(decode_bits(b, dtype).astype(np.float32)).T
    c = c32.numpy().astype(np.float64)
    return round_f64_to_f16_bits(c) if dtype == "f16" else round_f64_to_bf16_bits(c)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp32_accumulation_passes_and_planted_mistakes_fail(dtype):
    M, N, K = 96, 80, 1024
    a = gen.normal_scaled((M, K), dtype, K ** -0.5, 31)
    b = gen.normal_scaled((N, K), dtype, K ** -0.5, 32)
    got = _fp32_product(a, b, dtype)
    check_full(got, a, b, dtype)
    rows, cols = tile_samples(M, N, 32, 32, np.random.default_rng(0))
    check_entries(got[rows, cols], a, b, dtype, rows, cols)
    big = np.unravel_index(np.argmax(np.abs(decode_bits(got, dtype))), got.shape)
    for mistake in ("sign", "exponent", "fill", "transposed"):
        bad = got.copy()
        if mistake == "sign":
            bad[big] ^= 0x8000
        elif mistake == "exponent":
            bad[big] ^= 0x0400 if dtype == "f16" else 0x0080
        elif mistake == "fill":
            bad[big] = gen.SENTINEL16                  # an entry the kernel never wrote
        else:
            bad[:32, :32] = bad[:32, :32].T.copy()     # a tile stored transposed
        with pytest.raises(AssertionError):
            check_full(bad, a, b, dtype)


def test_tile_samples_reach_every_tile_and_its_corners():
    M, N, tm, tn = 1000, 700, 256, 224
    rows, cols = tile_samples(M, N, tm, tn, np.random.default_rng(1))
    tiles = {(r // tm, c // tn) for r, c in zip(rows, cols)}
    assert tiles == {(i, j) for i in range(-(-M // tm)) for j in range(-(-N // tn))}
    pts = set(zip(rows.tolist(), cols.tolist()))
    assert {(0, 0), (M - 1, N - 1), (0, N - 1), (M - 1, 0), (255, 223), (256, 224), (999, 672)} <= pts
    assert rows.max() < M and cols.max() < N
