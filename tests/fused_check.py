"""Tolerance checks of fused GEMM outputs against the oracle's float64 product.

The reference values come from the oracle (gemm_exact / gemm_exact_entries:
the float64 product of the 16-bit operands, and the same product of their
absolute values, obtained by clearing the sign bits), and the rounded value
from the oracle's round-to-nearest-even.  A kernel that accumulates in float32
and rounds once to the 16-bit output type must satisfy, entry by entry,

    |C_gpu - C_exact| <= ulp_out(C_exact) + 2 K 2^-24 sum_k |a_k| |b_k|

(the float32 accumulation error bound plus one rounding), plus the stated bars:
max |error| <= 2e-2 and normwise relative error <= 1e-2.
"""

from __future__ import annotations

import numpy as np

from oracle import (decode_bits, gemm_exact, gemm_exact_entries, round_f64_to_bf16_bits,
                    round_f64_to_f16_bits)

MAX_ABS = 2e-2
MAX_REL = 1e-2


def _round(exact: np.ndarray, dtype: str) -> np.ndarray:
    return round_f64_to_f16_bits(exact) if dtype == "f16" else round_f64_to_bf16_bits(exact)


def _ulp(exact: np.ndarray, dtype: str) -> np.ndarray:
    return (2.0 ** -10 if dtype == "f16" else 2.0 ** -7) * np.maximum(np.abs(exact), 2.0 ** -14)


def check_values(got_bits, exact, absum, K, dtype, max_abs=MAX_ABS, what=""):
    """Every entry within the fp32 bound of exact and within it of the oracle's rounded value; the bars.

    got_bits: uint16 bits from the GPU; exact, absum: float64 arrays of the same shape.
    Returns (max abs error, normwise relative error).
    """
    got = decode_bits(np.asarray(got_bits, dtype=np.uint16), dtype)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - exact)
    ulp = _ulp(exact, dtype)
    bound = ulp + 2 * K * 2.0 ** -24 * absum
    out = err > bound
    assert not out.any(), f"{what}: {np.count_nonzero(out)} entries outside the fp32 accumulation bound " \
                          f"(worst excess {np.max(err - bound):.3e})"
    want = decode_bits(_round(exact, dtype), dtype)          # the oracle's rounded value
    assert np.all(np.abs(want - got) <= ulp + bound), f"{what}: further than the bound from the oracle"
    if max_abs is not None:
        assert err.max() <= max_abs, f"{what}: max abs error {err.max()}"
    rel = float(np.linalg.norm(got - exact) / max(np.linalg.norm(exact), 1e-300))
    assert rel <= MAX_REL, f"{what}: normwise relative error {rel}"
    return float(err.max()), rel


def check_full(got_bits, a_bits, b_bits, dtype, b_layout="nk", max_abs=MAX_ABS, what=""):
    """Every entry of an (M, N) output block against the oracle's whole product."""
    a_bits = np.asarray(a_bits, dtype=np.uint16)
    b_bits = np.asarray(b_bits, dtype=np.uint16)
    exact = gemm_exact(a_bits, b_bits, dtype, b_layout)
    absum = gemm_exact(a_bits & 0x7FFF, b_bits & 0x7FFF, dtype, b_layout)
    return check_values(got_bits, exact, absum, a_bits.shape[1], dtype, max_abs, what)


def check_entries(got_bits, a_bits, b_bits, dtype, rows, cols, b_layout="nk", max_abs=MAX_ABS, what=""):
    """Selected entries (rows[i], cols[i]) against the oracle's one-by-one dot products."""
    a_bits = np.asarray(a_bits, dtype=np.uint16)
    b_bits = np.asarray(b_bits, dtype=np.uint16)
    exact = gemm_exact_entries(a_bits, b_bits, dtype, rows, cols, b_layout)
    absum = gemm_exact_entries(a_bits & 0x7FFF, b_bits & 0x7FFF, dtype, rows, cols, b_layout)
    return check_values(got_bits, exact, absum, a_bits.shape[1], dtype, max_abs, what)


def tile_samples(M: int, N: int, tm: int, tn: int, rng: np.random.Generator):
    """Rows and columns of the four corners and one random interior entry of every tm x tn output tile.

    Tiles on the ragged edges are clipped to the matrix.  Every tile of the
    kernel's grid is therefore read at least five times.
    """
    rows, cols = [], []
    for r0 in range(0, M, tm):
        r1 = min(M, r0 + tm) - 1
        for c0 in range(0, N, tn):
            c1 = min(N, c0 + tn) - 1
            rows += [r0, r0, r1, r1, int(rng.integers(r0, r1 + 1))]
            cols += [c0, c1, c0, c1, int(rng.integers(c0, c1 + 1))]
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)
