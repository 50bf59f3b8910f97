"""Plain CPU oracle: multi-destination all-gather and fused GEMM + all-gather.

TEST INFRASTRUCTURE ONLY -- imported by the test suite, the smoke entry point
and the benchmark's CPU-baseline leg, never by the product path.  It shares no
code, table or constant with the HIP library: it reads plain numpy arrays and
returns plain numpy arrays.

What it computes (sources are the three pages on the iris all-gather):

* all-gather -- ROCm/iris #594, "Multi-GPU CI" and "Local validation": the
  kernel's output must equal torch.distributed.all_gather_into_tensor, i.e.
  every member of the group receives the concatenation, in group order, of
  all members' inputs; logical ranks on one GPU are independent heap regions,
  and the check is a full-heap comparison (outputs, padding, guards and the
  heaps of ranks outside the group).  The tiled kernel, its destination order
  and its launch shape do not change this result, so the oracle is the
  definition itself, written as byte copies.
* all-to-all -- ROCm/iris #594, "Compiler inspection and grouping", and
  ROCm/iris #591, "Hoist the peer heap bases", name the all_to_all collective
  as the next user of the same heap-base machinery; its result is that of
  torch.distributed.all_to_all_single with equal splits: every rank's input
  is W chunks, chunk j goes to member j, and member j's output holds, in
  group order, the chunk j of every rank.  Written as byte copies.
* fused GEMM + all-gather -- ROCm/iris #626, "Summary" and "Assembly" table
  (256x256 fp16 C tile produced by the matmul and stored to every rank): each
  rank's C_j = A_j . B_j, rounded once to the 16-bit output type, then
  gathered exactly as above.  The dot products are formed in float64 (the
  "exact" value up to negligible rounding); the kernel under test accumulates
  in float32 and is compared with this within a tolerance.

Readings of points the pages leave open (each is repeated in the project's
design notes):
* the row block a caller writes is selected by its *group* rank
  g = (rank - rank_start) / rank_stride, so a strided sub-group's output has
  W*M_local rows in group order, as all_gather_into_tensor with a group does;
* inputs and outputs are dense row-major (leading dimension N);
* out_offset is a byte offset that is the same in every rank's region;
* rounding to fp16/bf16 is IEEE round-to-nearest-even, overflow gives +-inf,
  a NaN stays a quiet NaN.

Every function here is pinned by tests/test_oracle.py against hand-written
fixtures, closed forms, library routines and invariants.
"""

from __future__ import annotations

import numpy as np

F16, BF16, F32 = "f16", "bf16", "f32"
ELEM_BYTES = {F16: 2, BF16: 2, F32: 4}


# ---------------------------------------------------------------------------
# all-gather
# ---------------------------------------------------------------------------

def group_members(rank_start: int, rank_stride: int, world: int) -> list[int]:
    """Heap regions of a strided group, in group order.

    ROCm/iris #591, "Hoist the peer heap bases": the group is described by
    rank_start, rank_stride and world_size; member j is rank_start + j*rank_stride.
    """
    return [rank_start + j * rank_stride for j in range(world)]


def all_gather_expected_block(inputs: list[np.ndarray]) -> np.ndarray:
    """The gathered tensor every member must hold: the inputs stacked in group order.

    ROCm/iris #594, "Multi-GPU CI": the reference result is
    all_gather_into_tensor, whose output is the concatenation along dim 0.
    """
    return np.concatenate([np.asarray(x) for x in inputs], axis=0)


def all_gather_oracle(slab: np.ndarray, region_bytes: int, inputs: list[np.ndarray],
                      rank_start: int, rank_stride: int, out_offset: int) -> np.ndarray:
    """Full-heap result of an all-gather by every member of a group.

    slab         -- host copy of the whole heap before the calls, uint8, length
                    R*region_bytes (region r = bytes [r*region_bytes, (r+1)*region_bytes)).
    inputs       -- inputs[j] is group rank j's (M_local, N) array (any dtype).
    out_offset   -- byte offset of the output inside every region.

    Returns a new uint8 array: in every member's region, the W*M_local*N*e bytes
    at out_offset hold the inputs in group order; every other byte is unchanged
    (ROCm/iris #594, "Local validation": outputs, padding, guards and inactive
    heaps are all compared).
    """
    slab = np.asarray(slab, dtype=np.uint8)
    out = slab.copy()
    world = len(inputs)
    members = group_members(rank_start, rank_stride, world)
    regions = [out[h * region_bytes:(h + 1) * region_bytes] for h in members]
    cursor = out_offset
    for j in range(world):
        block = np.ascontiguousarray(inputs[j]).view(np.uint8).reshape(-1)
        store_to_members(regions, cursor, block)     # group rank j's rows follow ranks 0..j-1
        cursor += block.size
    return out


def store_to_members(regions: list[np.ndarray], offset: int, data: np.ndarray) -> None:
    """Write the same bytes at the same offset of every member's region (in place).

    One rank's all-gather is this store with its input at
    out_offset + g*M_local*N*e (ROCm/iris #626, "Summary": the tile is stored
    to every rank's heap at the same symmetric offset).  regions are uint8
    arrays (views into the heap), data a uint8 array.
    """
    n = data.size
    for region in regions:
        np.copyto(region[offset:offset + n], data)


# ---------------------------------------------------------------------------
# all-to-all
# ---------------------------------------------------------------------------

def all_to_all_expected_block(inputs: list[np.ndarray], j: int) -> np.ndarray:
    """What group member j must hold: chunk j of every rank's input, in group order.

    inputs[g] is group rank g's (W*M_chunk, N) array, chunk c being rows
    [c*M_chunk, (c+1)*M_chunk) (all_to_all_single with equal splits).
    """
    world = len(inputs)
    parts = []
    for x in inputs:
        x = np.asarray(x)
        m = x.shape[0] // world
        parts.append(x[j * m:(j + 1) * m])
    return np.concatenate(parts, axis=0)


def all_to_all_oracle(slab: np.ndarray, region_bytes: int, inputs: list[np.ndarray],
                      rank_start: int, rank_stride: int, out_offset: int) -> np.ndarray:
    """Full-heap result of an all-to-all by every member of a group.

    Same conventions as all_gather_oracle; inputs[g] holds W chunks.  In member
    j's region the W*M_chunk*N*e bytes at out_offset hold
    all_to_all_expected_block(inputs, j); every other byte is unchanged.
    """
    slab = np.asarray(slab, dtype=np.uint8)
    out = slab.copy()
    members = group_members(rank_start, rank_stride, len(inputs))
    for j, h in enumerate(members):
        block = np.ascontiguousarray(all_to_all_expected_block(inputs, j)).view(np.uint8).reshape(-1)
        start = h * region_bytes + out_offset
        out[start:start + block.size] = block
    return out


# ---------------------------------------------------------------------------
# 16-bit floating-point encodings
# ---------------------------------------------------------------------------

def _round_to_binary_format(x: np.ndarray, frac_bits: int, exp_bits: int) -> np.ndarray:
    """Bit pattern of the nearest value (ties to even) in a binary IEEE format.

    IEEE 754 round-to-nearest-even: the representable numbers of a binade
    [2^E, 2^(E+1)) are multiples of 2^(E - frac_bits); below the smallest
    normal binade the spacing stays 2^(emin - frac_bits) (gradual underflow).
    A value at or beyond the rounding boundary of the largest finite number
    becomes infinity; a NaN becomes the quiet NaN with the sign kept.
    """
    x = np.asarray(x, dtype=np.float64)
    bias = (1 << (exp_bits - 1)) - 1
    emin, emax = 1 - bias, bias
    exp_all_ones = (1 << exp_bits) - 1
    sign = np.signbit(x).astype(np.uint64)
    a = np.abs(x)
    out = np.zeros(x.shape, dtype=np.uint64)

    nan = np.isnan(a)
    # anything >= 2^(emax+2) is certainly infinite; keeps the scaling below finite
    huge = ~nan & (a >= np.ldexp(1.0, emax + 2))
    work = ~nan & ~huge & (a > 0)

    aw = a[work]
    _, ex = np.frexp(aw)                       # aw = m * 2^ex, m in [0.5, 1)
    E = np.maximum(ex.astype(np.int64) - 1, emin)
    step_exp = E - frac_bits                   # exponent of the spacing in this binade
    q = np.rint(np.ldexp(aw, -step_exp))       # RNE to an integer number of steps
    q = q.astype(np.int64)
    carry = q == (1 << (frac_bits + 1))        # rounded up into the next binade
    E = np.where(carry, E + 1, E)
    q = np.where(carry, q >> 1, q)
    normal = q >= (1 << frac_bits)
    biased = np.where(normal, E + bias, 0)
    frac = np.where(normal, q - (1 << frac_bits), q)
    overflow = normal & (E > emax)
    biased = np.where(overflow, exp_all_ones, biased)
    frac = np.where(overflow, 0, frac)
    out[work] = (biased.astype(np.uint64) << np.uint64(frac_bits)) | frac.astype(np.uint64)

    out[huge] = np.uint64(exp_all_ones) << np.uint64(frac_bits)
    out[nan] = (np.uint64(exp_all_ones) << np.uint64(frac_bits)) | np.uint64(1 << (frac_bits - 1))
    total_bits = 1 + exp_bits + frac_bits
    out |= sign << np.uint64(total_bits - 1)
    return out


def round_f64_to_f16_bits(x) -> np.ndarray:
    """IEEE binary16 bits (uint16) nearest to x, ties to even (1 sign, 5 exponent, 10 fraction bits)."""
    return _round_to_binary_format(x, frac_bits=10, exp_bits=5).astype(np.uint16)


def round_f64_to_bf16_bits(x) -> np.ndarray:
    """bfloat16 bits (uint16) nearest to x, ties to even (1 sign, 8 exponent, 7 fraction bits)."""
    return _round_to_binary_format(x, frac_bits=7, exp_bits=8).astype(np.uint16)


def f16_bits_to_f64(bits) -> np.ndarray:
    """Value of IEEE binary16 bit patterns (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Value of bfloat16 bit patterns: they are the upper 16 bits of a binary32 (exact)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):     # NaN patterns stay NaN
        return u32.view(np.float32).astype(np.float64)


def decode_bits(bits, dtype: str) -> np.ndarray:
    if dtype == F16:
        return f16_bits_to_f64(bits)
    if dtype == BF16:
        return bf16_bits_to_f64(bits)
    raise ValueError(f"16-bit dtype expected, got {dtype!r}")


def _encode(values: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return round_f64_to_f16_bits(values)
    if dtype == BF16:
        return round_f64_to_bf16_bits(values)
    raise ValueError(f"16-bit dtype expected, got {dtype!r}")


# ---------------------------------------------------------------------------
# GEMM and fused GEMM + all-gather
# ---------------------------------------------------------------------------

def _logical_b(b_bits: np.ndarray, dtype: str, b_layout: str) -> np.ndarray:
    """B as a logical (K, N) float64 matrix.

    b_layout "kn": b_bits[k, n] = B(k, n) (row-major K x N).
    b_layout "nk": b_bits[n, k] = B(k, n) (K-contiguous, the transposed weight of a linear layer).
    """
    b = decode_bits(b_bits, dtype)
    if b_layout == "kn":
        return b
    if b_layout == "nk":
        return b.T
    raise ValueError(f"b_layout must be 'kn' or 'nk', got {b_layout!r}")


def gemm_exact(a_bits: np.ndarray, b_bits: np.ndarray, dtype: str, b_layout: str = "nk") -> np.ndarray:
    """The float64 product A . B of 16-bit operands, before any rounding to the output type; (M, N).

    Each product of two 16-bit values is exact in float64; the sums carry
    float64 rounding only, far below the output type's resolution.  This is
    the value gemm_oracle rounds, and the "exact" value against which a
    float32-accumulating kernel's error is measured.  a_bits is the row-major
    (M, K) A.
    """
    a = decode_bits(a_bits, dtype)
    b = _logical_b(b_bits, dtype, b_layout)
    if a.shape[1] != b.shape[0]:
        raise ValueError(f"inner dimensions differ: A is {a.shape}, B is {b.shape}")
    return np.matmul(a, b)


def gemm_oracle(a_bits: np.ndarray, b_bits: np.ndarray, dtype: str, b_layout: str = "nk") -> np.ndarray:
    """C = A . B rounded once to the 16-bit dtype; returns uint16 bits of shape (M, N).

    ROCm/iris #626, "Assembly" table and "Benchmark": the matmul produces an
    fp16 C tile from fp16 operands.  The products and sums are formed in
    float64 (gemm_exact) and rounded once (round-to-nearest-even) to the
    output type.
    """
    return _encode(gemm_exact(a_bits, b_bits, dtype, b_layout), dtype)


def gemm_exact_entries(a_bits: np.ndarray, b_bits: np.ndarray, dtype: str, rows, cols,
                       b_layout: str = "nk") -> np.ndarray:
    """Selected entries C[rows[i], cols[i]] of gemm_exact, each one as its own float64 dot product."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    a = np.asarray(a_bits, dtype=np.uint16)
    b = np.asarray(b_bits, dtype=np.uint16)
    vals = np.empty(rows.size, dtype=np.float64)
    for i, (r, c) in enumerate(zip(rows, cols)):
        a_row = decode_bits(a[r, :], dtype)
        b_col = decode_bits(b[c, :] if b_layout == "nk" else b[:, c], dtype)
        vals[i] = np.dot(a_row, b_col)
    return vals


def gemm_oracle_entries(a_bits: np.ndarray, b_bits: np.ndarray, dtype: str, rows, cols,
                        b_layout: str = "nk") -> np.ndarray:
    """Selected entries C[rows[i], cols[i]] of gemm_oracle, each one as its own float64 dot product.

    For full-size checks where the whole product is too slow on the CPU.
    """
    return _encode(gemm_exact_entries(a_bits, b_bits, dtype, rows, cols, b_layout), dtype)


def gemm_all_gather_oracle(slab: np.ndarray, region_bytes: int, a_list, b_list, dtype: str,
                           rank_start: int, rank_stride: int, out_offset: int,
                           b_layout: str = "nk") -> np.ndarray:
    """Full-heap result of the fused GEMM + all-gather by every member of a group.

    Group rank j computes C_j = A_j . B_j (gemm_oracle) and the C_j are gathered
    exactly as all_gather_oracle gathers plain inputs (ROCm/iris #626, "Summary":
    the same multi-destination store is the matmul's epilogue).
    """
    c_list = [gemm_oracle(a, b, dtype, b_layout) for a, b in zip(a_list, b_list)]
    return all_gather_oracle(slab, region_bytes, c_list, rank_start, rank_stride, out_offset)
