"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and encodes them in the storage types;
it holds none of the all-gather's or the GEMM's arithmetic.  Both the oracle
and the HIP path receive exactly the arrays produced here.

Shapes and distributions follow the workloads on the iris all-gather pages:
per-rank inputs uniform on [-1, 1) for the copy path (ROCm/iris #594,
"Reviewer performance evaluation": random inputs, M x N in fp16/bf16/fp32),
N(0, 1)/sqrt(K) operands for the fused matmul (ROCm/iris #626, "Benchmark":
fp16, N=3584, K=8192).  16-bit values are returned as their uint16 bit
patterns; fp32 as float32.
"""

from __future__ import annotations

import numpy as np

# fp16 quiet NaN used to pre-fill heaps so that any stray write is visible
SENTINEL16 = 0x7E00


def rng_for(*key: int) -> np.random.Generator:
    """Generator seeded by an integer key, e.g. (config_id, rank)."""
    return np.random.default_rng([int(k) for k in key])


def _encode_f32(values_f32: np.ndarray, dtype: str) -> np.ndarray:
    values_f32 = np.asarray(values_f32, dtype=np.float32)
    if dtype == "f32":
        return values_f32
    if dtype == "f16":
        return values_f32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch  # CPU cast only: float32 -> bfloat16, round to nearest even
        t = torch.from_numpy(np.ascontiguousarray(values_f32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown dtype {dtype!r}")


def uniform_pm1(shape, dtype: str, *key: int) -> np.ndarray:
    """Uniform on [-1, 1): float32 2u - 1, then rounded to the storage type."""
    u = rng_for(*key).random(shape, dtype=np.float32)
    return _encode_f32(2.0 * u - 1.0, dtype)


def normal_scaled(shape, dtype: str, scale: float, *key: int) -> np.ndarray:
    """N(0, 1) * scale drawn in float32, rounded to the storage type."""
    x = rng_for(*key).standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return _encode_f32(x, dtype)


def small_integers(shape, dtype: str, lo: int, hi: int, *key: int) -> np.ndarray:
    """Integers uniform on [lo, hi], exactly representable in every storage type."""
    x = rng_for(*key).integers(lo, hi + 1, size=shape).astype(np.float32)
    return _encode_f32(x, dtype)


def random_bit_patterns(shape, elem_bytes: int, *key: int) -> np.ndarray:
    """Arbitrary bit patterns (NaN payloads, -0, subnormals, infinities included)."""
    dt = {2: np.uint16, 4: np.uint32}[elem_bytes]
    info = np.iinfo(dt)
    return rng_for(*key).integers(0, int(info.max) + 1, size=shape, dtype=dt)


def sentinel_slab(total_bytes: int, pattern16: int = SENTINEL16) -> np.ndarray:
    """Host bytes of a heap pre-filled with a repeated 16-bit pattern."""
    if total_bytes % 2:
        raise ValueError("slab size must be even")
    return np.full(total_bytes // 2, pattern16, dtype=np.uint16).view(np.uint8)
