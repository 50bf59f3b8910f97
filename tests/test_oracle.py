"""Pins for the CPU oracle: hand-worked fixtures, closed forms, library routines, invariants.

None of these compares the oracle with itself; each pin would fail for a
plausible mistake (wrong group order, strided-group index, dropped guard,
transposed operand, rounding direction, overflow handling).
"""

import os

import numpy as np
import pytest
import torch

from oracle import (
    F16, BF16,
    all_gather_oracle, all_gather_expected_block, group_members,
    all_to_all_oracle, all_to_all_expected_block,
    round_f64_to_f16_bits, round_f64_to_bf16_bits, f16_bits_to_f64, bf16_bits_to_f64,
    gemm_oracle, gemm_oracle_entries, gemm_all_gather_oracle, gemm_exact, gemm_exact_entries,
)
from gemm_all_gather_amd import inputs as gen

S16 = gen.SENTINEL16


def _read_fixture(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------
# all-gather
# ---------------------------------------------------------------------------

def test_all_gather_hand_worked_strided_example(golden_dir):
    rows = _read_fixture(os.path.join(golden_dir, "all_gather_strided_tiny.txt"))
    kv = {}
    inputs, expect = {}, {}
    for r in rows:
        if r[0] == "input":
            inputs[int(r[1])] = [int(v) for v in r[2:]]
        elif r[0] == "expect":
            expect[int(r[1])] = [S16 if v == "S" else int(v) for v in r[2:]]
        else:
            kv[r[0]] = int(r[1])
    R, words = kv["regions"], kv["region_words"]
    M, N = kv["m_local"], kv["n"]
    slab = np.full(R * words, S16, dtype=np.uint16).view(np.uint8)
    ins = [np.array(inputs[j], dtype=np.uint16).reshape(M, N) for j in sorted(inputs)]
    out = all_gather_oracle(slab, words * 2, ins, kv["rank_start"], kv["rank_stride"],
                            kv["out_offset_bytes"]).view(np.uint16).reshape(R, words)
    for r in range(R):
        assert out[r].tolist() == expect[r], f"region {r}"


def _run_fixture(path, oracle_fn, mkey):
    rows = _read_fixture(path)
    kv, inputs, expect = {}, {}, {}
    for r in rows:
        if r[0] == "input":
            inputs[int(r[1])] = [int(v) for v in r[2:]]
        elif r[0] == "expect":
            expect[int(r[1])] = [S16 if v == "S" else int(v) for v in r[2:]]
        else:
            kv[r[0]] = int(r[1])
    R, words = kv["regions"], kv["region_words"]
    M, N = kv[mkey], kv["n"]
    slab = np.full(R * words, S16, dtype=np.uint16).view(np.uint8)
    ins = [np.array(inputs[j], dtype=np.uint16).reshape(-1, N) for j in sorted(inputs)]
    assert all(x.shape[0] in (M, M * len(ins)) for x in ins)
    out = oracle_fn(slab, words * 2, ins, kv["rank_start"], kv["rank_stride"],
                    kv["out_offset_bytes"]).view(np.uint16).reshape(R, words)
    for r in range(R):
        assert out[r].tolist() == expect[r], f"region {r}"


@pytest.mark.parametrize("name", ["all_to_all_strided_tiny.txt", "all_to_all_w3_tiny.txt"])
def test_all_to_all_hand_worked_examples(golden_dir, name):
    _run_fixture(os.path.join(golden_dir, name), all_to_all_oracle, "m_chunk")


@pytest.mark.parametrize("W,M,N", [(1, 3, 4), (2, 1, 1), (3, 2, 5), (8, 4, 7)])
def test_all_to_all_is_a_block_transpose(W, M, N):
    """Library routine: the result is the (rank, chunk) block matrix transposed.

    Stacking every rank's chunks as X[g, c] and swapping the two block axes
    gives Y[j, g] = X[g, j], member j's output in group order.
    """
    ins = [gen.random_bit_patterns((W * M, N), 2, 31, W, g) for g in range(W)]
    X = np.stack([x.reshape(W, M, N) for x in ins])          # X[g, c, m, n]
    Y = np.swapaxes(X, 0, 1)                                  # Y[j, g, m, n]
    for j in range(W):
        assert np.array_equal(all_to_all_expected_block(ins, j), Y[j].reshape(W * M, N))


@pytest.mark.parametrize("W,start,stride", [(2, 0, 1), (3, 1, 2), (4, 0, 2), (8, 0, 1)])
def test_all_to_all_twice_is_the_identity_and_leaves_the_rest(W, start, stride):
    """Invariants: the exchange is an involution, and only member output blocks change."""
    M, N, e = 3, 6, 2
    R = start + (W - 1) * stride + 2
    blk = M * N * e
    region = W * blk + 96
    off = 32
    slab = gen.random_bit_patterns((R * region // 2,), 2, 17, W, R).view(np.uint8)
    ins = [gen.uniform_pm1((W * M, N), "f16", 5, g) for g in range(W)]
    out = all_to_all_oracle(slab, region, ins, start, stride, off)
    members = group_members(start, stride, W)
    # member outputs, fed back in as inputs, return the original inputs
    outs = [out[h * region + off:h * region + off + W * blk].view(np.uint16).reshape(W * M, N) for h in members]
    back = all_to_all_oracle(out, region, outs, start, stride, off)
    for g, h in enumerate(members):
        got = back[h * region + off:h * region + off + W * blk].view(np.uint16).reshape(W * M, N)
        assert np.array_equal(got, ins[g].view(np.uint16))
    # every byte outside the member output blocks is unchanged
    mask = np.ones(R * region, dtype=bool)
    for h in members:
        mask[h * region + off:h * region + off + W * blk] = False
    assert np.array_equal(out[mask], slab[mask])


def test_all_to_all_single_rank_is_a_copy():
    x = gen.uniform_pm1((5, 9), "bf16", 3, 0)
    slab = np.zeros(4096, dtype=np.uint8)
    out = all_to_all_oracle(slab, 4096, [x], 0, 1, 128)
    assert np.array_equal(out[128:128 + x.nbytes], x.view(np.uint8).reshape(-1))
    assert not out[:128].any() and not out[128 + x.nbytes:].any()


def test_group_members_strided():
    assert group_members(1, 2, 4) == [1, 3, 5, 7]
    assert group_members(0, 1, 8) == list(range(8))
    assert group_members(3, 1, 2) == [3, 4]


@pytest.mark.parametrize("R,W,start,stride", [
    (1, 1, 0, 1), (2, 2, 0, 1), (8, 8, 0, 1), (8, 4, 1, 2), (8, 4, 0, 2), (8, 3, 3, 1), (5, 2, 1, 3),
])
@pytest.mark.parametrize("M,N,dtype", [(3, 5, "f16"), (4, 7, "f32"), (0, 4, "bf16"), (9, 1, "f16")])
def test_all_gather_equals_concatenation_and_leaves_rest(R, W, start, stride, M, N, dtype):
    e = 4 if dtype == "f32" else 2
    blk = M * N * e
    region = W * blk + 64 + 48
    out_offset = 64 - 2 * e   # unaligned to the tile, aligned to the element
    slab = gen.random_bit_patterns((R * region,), 2, 7, R, W).view(np.uint8)
    ins = [gen.uniform_pm1((M, N), dtype, 99, j) for j in range(W)]
    out = all_gather_oracle(slab, region, ins, start, stride, out_offset)
    members = group_members(start, stride, W)
    # library routine: torch.cat in group order is all_gather_into_tensor's result
    gathered = torch.cat([torch.from_numpy(np.ascontiguousarray(x).view(np.uint8).reshape(-1))
                          for x in ins]).numpy()
    assert np.array_equal(gathered, all_gather_expected_block(ins).view(np.uint8).reshape(-1))
    for r in range(R):
        reg_in = slab[r * region:(r + 1) * region]
        reg_out = out[r * region:(r + 1) * region]
        if r in members:
            assert np.array_equal(reg_out[out_offset:out_offset + W * blk], gathered)
            assert np.array_equal(reg_out[:out_offset], reg_in[:out_offset])
            assert np.array_equal(reg_out[out_offset + W * blk:], reg_in[out_offset + W * blk:])
        else:
            assert np.array_equal(reg_out, reg_in)


def test_all_gather_changed_word_count_against_nan_sentinel():
    # 16-bit uniform[-1,1) values can never equal the fp16 NaN sentinel, so the
    # number of changed words after all W calls is exactly W*W*M*N.
    R, W, M, N = 8, 8, 5, 11
    blk = M * N * 2
    region = W * blk + 256
    slab = gen.sentinel_slab(R * region)
    ins = [gen.uniform_pm1((M, N), "f16", 3, j) for j in range(W)]
    out = all_gather_oracle(slab, region, ins, 0, 1, 128)
    changed = np.count_nonzero(out.view(np.uint16) != S16)
    assert changed == W * W * M * N


def test_all_gather_single_rank_is_memcpy():
    x = gen.random_bit_patterns((6, 13), 4, 11)
    slab = np.zeros(6 * 13 * 4 + 32, dtype=np.uint8)
    out = all_gather_oracle(slab, slab.size, [x], 0, 1, 16)
    assert out[16:16 + x.nbytes].tobytes() == x.tobytes()
    assert not out[:16].any() and not out[16 + x.nbytes:].any()


def test_all_gather_group_order_not_region_order():
    # group rank j's rows land at block j even when the members are listed by a stride
    ins = [np.full((1, 2), j + 1, dtype=np.uint16) for j in range(3)]
    region = 3 * 4
    slab = np.zeros(7 * region, dtype=np.uint8)
    out = all_gather_oracle(slab, region, ins, 2, 2, 0).view(np.uint16).reshape(7, 6)
    for r in (2, 4, 6):
        assert out[r].tolist() == [1, 1, 2, 2, 3, 3]
    for r in (0, 1, 3, 5):
        assert out[r].tolist() == [0] * 6


# ---------------------------------------------------------------------------
# 16-bit rounding
# ---------------------------------------------------------------------------

def test_rounding_hand_worked_values(golden_dir):
    for fmt, val, bits in _read_fixture(os.path.join(golden_dir, "round_16bit.txt")):
        fn = round_f64_to_f16_bits if fmt == "f16" else round_f64_to_bf16_bits
        got = int(fn(np.array([float(val)]))[0])
        assert got == int(bits, 16), f"{fmt} {val}: got {got:#06x} want {bits}"


def test_f16_rounding_matches_numpy_direct_double_to_half():
    rng = np.random.default_rng(5)
    mags = np.ldexp(rng.random(200_000) + 0.5, rng.integers(-30, 18, 200_000))
    vals = mags * rng.choice([-1.0, 1.0], mags.size)
    all_halves = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
    finite = all_halves[np.isfinite(all_halves)]
    srt = np.unique(finite)
    mids = (srt[:-1] + srt[1:]) / 2          # exact ties in float64
    vals = np.concatenate([vals, finite, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                           [0.0, -0.0, np.inf, -np.inf, 1e300, -1e300, 1e-300]])
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = round_f64_to_f16_bits(vals)
    assert np.array_equal(got, want)


def test_bf16_rounding_matches_torch_for_float32_inputs():
    rng = np.random.default_rng(6)
    bits = rng.integers(0, 2**32, 400_000, dtype=np.uint64).astype(np.uint32)
    f32 = bits.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = round_f64_to_bf16_bits(f32.astype(np.float64))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_rounding_round_trips_every_finite_pattern_and_ties_go_even(fmt):
    enc = round_f64_to_f16_bits if fmt == "f16" else round_f64_to_bf16_bits
    dec = f16_bits_to_f64 if fmt == "f16" else bf16_bits_to_f64
    pats = np.arange(65536, dtype=np.uint16)
    vals = dec(pats)
    fin = np.isfinite(vals)
    assert np.array_equal(enc(vals[fin]), pats[fin])
    nan_bits = enc(np.array([np.nan, -np.nan]))
    assert all(np.isnan(dec(nan_bits)))
    # ties between adjacent positive finite patterns go to the even pattern
    pos = np.arange(0, 0x7C00 if fmt == "f16" else 0x7F80, dtype=np.uint16)
    lo, hi = dec(pos[:-1]), dec(pos[1:])
    tie = enc((lo + hi) / 2)
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(tie, even)


def test_rounding_is_monotone():
    x = np.sort(np.random.default_rng(8).standard_normal(50_000) * 1000)
    for enc, dec in ((round_f64_to_f16_bits, f16_bits_to_f64), (round_f64_to_bf16_bits, bf16_bits_to_f64)):
        y = dec(enc(x))
        assert np.all(np.diff(y) >= 0)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def _gemm_fixture(golden_dir):
    kv = {r[0]: r[1:] for r in _read_fixture(os.path.join(golden_dir, "gemm_tiny.txt"))}
    a = np.array([float(v) for v in kv["a"]]).reshape(2, 3)
    b = np.array([float(v) for v in kv["b_kn"]]).reshape(3, 2)
    return a, b, kv


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_gemm_hand_worked_product(golden_dir, dtype):
    a, b, kv = _gemm_fixture(golden_dir)
    enc = round_f64_to_f16_bits if dtype == F16 else round_f64_to_bf16_bits
    want = [int(v, 16) for v in kv["c_f16" if dtype == F16 else "c_bf16"]]
    got_kn = gemm_oracle(enc(a), enc(b), dtype, b_layout="kn")
    got_nk = gemm_oracle(enc(a), enc(b.T.copy()), dtype, b_layout="nk")
    assert got_kn.reshape(-1).tolist() == want
    assert got_nk.reshape(-1).tolist() == want


def _int_matmul(a, b):
    M, K = len(a), len(a[0])
    N = len(b[0])
    return [[sum(int(a[i][k]) * int(b[k][j]) for k in range(K)) for j in range(N)] for i in range(M)]


@pytest.mark.parametrize("dtype,lo,hi", [(F16, -3, 3), (BF16, -2, 2)])
@pytest.mark.parametrize("M,N,K", [(5, 7, 9), (1, 3, 33), (6, 2, 50)])
def test_gemm_exact_on_small_integers_against_brute_force(dtype, lo, hi, M, N, K):
    a = gen.small_integers((M, K), dtype, lo, hi, 1, M, N, K)
    b_nk = gen.small_integers((N, K), dtype, lo, hi, 2, M, N, K)
    dec = f16_bits_to_f64 if dtype == F16 else bf16_bits_to_f64
    ai = dec(a).astype(np.int64).tolist()
    bi = dec(b_nk).astype(np.int64).T.tolist()     # logical K x N
    c = np.array(_int_matmul(ai, bi), dtype=np.float64)
    assert np.all(np.abs(c) <= (2048 if dtype == F16 else 256))   # exact in the output type
    got = dec(gemm_oracle(a, b_nk, dtype, "nk"))
    assert np.array_equal(got, c)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_gemm_identity_one_hot_and_zero(dtype):
    K = 24
    a = gen.uniform_pm1((10, K), dtype, 4)
    eye = (round_f64_to_f16_bits if dtype == F16 else round_f64_to_bf16_bits)(np.eye(K))
    assert np.array_equal(gemm_oracle(a, eye, dtype, "nk"), a)          # A . I = A
    b = gen.uniform_pm1((6, K), dtype, 5)                               # N=6 x K, K-contiguous
    idx = np.array([3, 0, 23, 7])
    one_hot = np.zeros((4, K))
    one_hot[np.arange(4), idx] = 1.0
    enc = round_f64_to_f16_bits if dtype == F16 else round_f64_to_bf16_bits
    c = gemm_oracle(enc(one_hot), b, dtype, "nk")
    assert np.array_equal(c, b[:, idx].T)                               # row i = B(idx_i, :)
    z = gemm_oracle(enc(np.zeros((3, K))), b, dtype, "nk")
    assert np.all(z == 0)                                               # +0, not -0


def test_gemm_closed_form_constant_matrices():
    # A = a*ones(M,K), B = b*ones(K,N): every C entry is K*a*b
    K = 1000
    a = round_f64_to_f16_bits(np.full((3, K), 0.5))
    b = round_f64_to_f16_bits(np.full((4, K), -0.25))
    assert np.all(gemm_oracle(a, b, F16, "nk") == round_f64_to_f16_bits(np.array([-125.0]))[0])


def test_gemm_transposed_operand_is_detected():
    a = gen.uniform_pm1((4, 6), F16, 9)
    b_nk = gen.uniform_pm1((5, 6), F16, 10)
    c = f16_bits_to_f64(gemm_oracle(a, b_nk, F16, "nk"))
    ref = f16_bits_to_f64(a) @ f16_bits_to_f64(b_nk).T      # library matmul, float64
    assert np.array_equal(c, f16_bits_to_f64(np.asarray(ref).astype(np.float16).view(np.uint16)))
    with pytest.raises(ValueError):
        gemm_oracle(a, b_nk, F16, "kn")                        # K x N reading of an N x K buffer


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_gemm_within_float32_accumulation_bound(dtype):
    # the kernel accumulates in float32; |fp32 result - exact| <= gamma_K * sum|a||b|
    M, N, K = 16, 24, 512
    a = gen.normal_scaled((M, K), dtype, 1.0, 12)
    b = gen.normal_scaled((N, K), dtype, K ** -0.5, 13)
    dec = f16_bits_to_f64 if dtype == F16 else bf16_bits_to_f64
    exact = dec(a) @ dec(b).T
    c32 = (torch.from_numpy(dec(a).astype(np.float32)) @ torch.from_numpy(dec(b).astype(np.float32)).T).numpy()
    bound = K * 2.0 ** -24 * (np.abs(dec(a)) @ np.abs(dec(b)).T)
    assert np.all(np.abs(c32 - exact) <= bound * 1.0001)
    got = dec(gemm_oracle(a, b, dtype, "nk"))
    ulp_half = np.abs(exact) * (2.0 ** -11 if dtype == F16 else 2.0 ** -8) + 2.0 ** -24
    assert np.all(np.abs(got - exact) <= ulp_half)


@pytest.mark.parametrize("dtype,lo,hi", [(F16, -3, 3), (BF16, -2, 2)])
def test_gemm_exact_is_the_unrounded_product(dtype, lo, hi):
    # K = 700 small integers: sums up to 6300 (fp16) / 2800 (bf16) are not representable in the output
    # type, but the unrounded float64 product holds them exactly; brute force over Python integers
    M, N, K = 4, 5, 700
    a = gen.small_integers((M, K), dtype, lo, hi, 3, M, N, K)
    b_nk = gen.small_integers((N, K), dtype, lo, hi, 4, M, N, K)
    dec = f16_bits_to_f64 if dtype == F16 else bf16_bits_to_f64
    ai = dec(a).astype(np.int64).tolist()
    bi = dec(b_nk).astype(np.int64).T.tolist()
    c = np.array(_int_matmul(ai, bi), dtype=np.float64)
    got = gemm_exact(a, b_nk, dtype, "nk")
    assert got.dtype == np.float64 and np.array_equal(got, c)
    assert np.array_equal(gemm_exact(a, np.ascontiguousarray(b_nk.T), dtype, "kn"), c)
    # clearing the sign bits gives sum |a||b|, the term of the float32 accumulation bound
    absum = np.array(_int_matmul(np.abs(np.array(ai)).tolist(), np.abs(np.array(bi)).tolist()), dtype=np.float64)
    assert np.array_equal(gemm_exact(a & 0x7FFF, b_nk & 0x7FFF, dtype, "nk"), absum)
    # gemm_oracle is this product rounded once
    enc = round_f64_to_f16_bits if dtype == F16 else round_f64_to_bf16_bits
    assert np.array_equal(gemm_oracle(a, b_nk, dtype, "nk"), enc(c))
    rows, cols = np.array([0, 3, 2, 1]), np.array([4, 0, 2, 1])
    assert np.array_equal(gemm_exact_entries(a, b_nk, dtype, rows, cols, "nk"), c[rows, cols])


def test_gemm_entries_match_full_product():
    a = gen.normal_scaled((33, 70), BF16, 1.0, 20)
    b = gen.normal_scaled((17, 70), BF16, 0.1, 21)
    full = gemm_oracle(a, b, BF16, "nk")
    rows = np.array([0, 32, 5, 17, 32])
    cols = np.array([0, 16, 9, 3, 0])
    assert np.array_equal(gemm_oracle_entries(a, b, BF16, rows, cols, "nk"), full[rows, cols])


def test_fused_oracle_places_each_ranks_product_in_group_order(golden_dir):
    a0, b_kn, kv = _gemm_fixture(golden_dir)
    enc = round_f64_to_f16_bits
    a1 = 2 * a0                                                   # rank 1's product is exactly 2x
    c0 = [int(v, 16) for v in kv["c_f16"]]
    c1 = enc(2 * np.array([float(v) for v in kv["c"]])).tolist()
    region = 2 * 4 * 2 + 8
    slab = np.zeros(3 * region, dtype=np.uint8)
    out = gemm_all_gather_oracle(slab, region, [enc(a0), enc(a1)], [enc(b_kn.T.copy())] * 2, F16,
                                 1, 1, 4).view(np.uint16).reshape(3, region // 2)
    for r in (1, 2):
        assert out[r, 2:10].tolist() == c0 + c1
        assert out[r, :2].tolist() == [0, 0] and out[r, 10:].tolist() == [0, 0]
    assert not out[0].any()
