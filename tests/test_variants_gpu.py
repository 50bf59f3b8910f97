"""Parity of the all-gather variants and the all-to-all (through the C ABI) with the CPU oracle.

* destination groups (ag_all_gather_ex, dest_group 1/2/4): ROCm/iris #594,
  "Reviewer performance evaluation" and "Compiler inspection and grouping";
  ROCm/iris #591, "INLINE grouping";
* the partitioned schedule (one destination per program): ROCm/iris #626,
  "Triton CCL all-gather";
* the all-to-all on the same heap machinery: ROCm/iris #594, "Compiler
  inspection and grouping" (result of all_to_all_single with equal splits).

Every comparison is bit-exact over the whole heap: outputs, guard bytes and
the regions of ranks outside the group.
"""

import itertools

import numpy as np
import pytest
import torch

from gemm_all_gather_amd import binding as ag
from gemm_all_gather_amd import inputs as gen
from oracle import all_gather_oracle, all_to_all_oracle
from tests.gpu_util import TorchHeap, log, require_gpu, to_device

pytestmark = pytest.mark.gpu

E = {"f16": 2, "bf16": 2, "f32": 4}


def _compare(got, want, S):
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        raise AssertionError(f"{bad.size} bytes differ; first at {bad[0]} (region {bad[0] // S}, "
                             f"offset {bad[0] % S}): got {got[bad[0]]} want {want[bad[0]]}")


def _gather_ex(R, S, W, start, stride, M, N, dtype, off, tile=(0, 0), programs=0, group=0, sched=0, seed=0,
               streams=False):
    require_gpu()
    log(f"all_gather_ex R={R} S={S} W={W} group=({start},{stride}) M={M} N={N} {dtype} off={off} tile={tile} "
        f"programs={programs} dest_group={group} schedule={sched} seed={seed}")
    th = TorchHeap(R, S)
    try:
        before = th.fill_random(seed + 5)
        ins = [gen.random_bit_patterns((M, N), E[dtype], seed, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        ss = [torch.cuda.Stream() for _ in range(W)] if streams else [None] * W
        for j in range(W):
            ag.all_gather_ex(th.view(start + j * stride), W, start, stride, dev[j], off, M, N, dtype, tile[0],
                             tile[1], programs, group, sched, ss[j])
        torch.cuda.synchronize()
        _compare(th.host(), all_gather_oracle(before, S, ins, start, stride, off), S)
    finally:
        th.close()


def _a2a(R, S, W, start, stride, M, N, dtype, off, tile=(0, 0), programs=0, seed=0, streams=False, sched=0):
    require_gpu()
    log(f"all_to_all R={R} S={S} W={W} group=({start},{stride}) M_chunk={M} N={N} {dtype} off={off} tile={tile} "
        f"programs={programs} seed={seed} schedule={sched}")
    th = TorchHeap(R, S)
    try:
        before = th.fill_random(seed + 9)
        ins = [gen.random_bit_patterns((W * M, N), E[dtype], seed, g) for g in range(W)]
        dev = [to_device(x) for x in ins]
        ss = [torch.cuda.Stream() for _ in range(W)] if streams else [None] * W
        for g in range(W):
            ag.all_to_all_ex(th.view(start + g * stride), W, start, stride, dev[g], off, M, N, dtype, tile[0],
                             tile[1], programs, schedule=sched, stream=ss[g])
        torch.cuda.synchronize()
        _compare(th.host(), all_to_all_oracle(before, S, ins, start, stride, off), S)
    finally:
        th.close()


def _size(W, M, N, e, off, chunks=1):
    return ((off + W * M * N * e * chunks + 512) // 256 + 1) * 256


# ---------------------------------------------------------------------------
# destination groups
# ---------------------------------------------------------------------------

_GROUPED = []
for W, G in [(2, 1), (3, 1), (3, 2), (4, 2), (5, 4), (6, 4), (7, 2), (8, 1), (8, 2), (8, 4)]:
    for M, N, dtype in [(9, 257 * 8, "f16"), (64, 4096, "bf16"), (13, 520, "f32"), (1, 8, "f16")]:
        _GROUPED.append((W, G, M, N, dtype))


@pytest.mark.parametrize("W,G,M,N,dtype", _GROUPED)
def test_destination_groups(W, G, M, N, dtype):
    e = E[dtype]
    start, stride = (1, 1) if W < 8 else (0, 1)
    off = 4 * e * 16
    rng = np.random.default_rng([W, G, M, N])
    tile = [(8, 256), (4, 512), (16, 128)][int(rng.integers(0, 3))] if e == 2 else (8, 256)
    programs = [3, 16, 0][int(rng.integers(0, 3))]
    _gather_ex(8, _size(W, M, N, e, off), W, start, stride, M, N, dtype, off, tile, programs, group=G, seed=W * 10 + G)


def test_destination_groups_strided_subgroup_on_streams():
    _gather_ex(8, _size(4, 100, 1000, 2, 512), 4, 1, 2, 100, 1000, "f16", 512, (8, 256), 32, group=1, seed=3,
               streams=True)


def test_destination_groups_full_size_w8():
    M, N = 1024, 4096
    for G in (1, 2, 4):
        _gather_ex(8, _size(8, M, N, 2, 0), 8, 0, 1, M, N, "f16", 0, (8, 256), 256, group=G, seed=40 + G)


# ---------------------------------------------------------------------------
# partitioned schedule
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("W,start,stride", [(1, 0, 1), (2, 0, 1), (3, 1, 2), (4, 0, 2), (8, 0, 1)])
@pytest.mark.parametrize("M,N,dtype,programs", [(7, 300, "f16", 1), (64, 256, "bf16", 8), (33, 1000, "f32", 24),
                                               (200, 4100, "f16", 256), (0, 64, "f16", 8)])
def test_partitioned_schedule(W, start, stride, M, N, dtype, programs):
    e = E[dtype]
    off = 2 * e * 8
    _gather_ex(8, _size(W, M, N, e, off), W, start, stride, M, N, dtype, off, (8, 256) if e == 2 else (4, 256),
               programs, sched="partitioned", seed=M + N + W)


def test_partitioned_full_size_w8():
    for programs in (64, 128, 256):
        _gather_ex(8, _size(8, 1024, 4096, 2, 0), 8, 0, 1, 1024, 4096, "f16", 0, (8, 256), programs,
                   sched="partitioned", seed=programs)


# ---------------------------------------------------------------------------
# all-to-all
# ---------------------------------------------------------------------------

_A2A = []
_rng = np.random.default_rng(77)
for W, (start, stride), M, N in itertools.product([1, 2, 3, 4, 8], [(0, 1), (1, 2), (3, 1)], [0, 1, 7, 8, 9, 64],
                                                  [1, 3, 8, 255, 256, 257]):
    if start + (W - 1) * stride >= 8:
        continue
    _A2A.append((W, start, stride, M, N))
_A2A = [c for c in _A2A if _rng.random() < 0.3]


@pytest.mark.parametrize("W,start,stride,M,N", _A2A)
def test_all_to_all_tiny_sweep(W, start, stride, M, N):
    rng = np.random.default_rng([W, start, stride, M, N, 1])
    dtype = ["f16", "bf16", "f32"][int(rng.integers(0, 3))]
    e = E[dtype]
    tiles = [(8, 256), (1, 256), (4, 64), (16, 128), (2, 512)] if e == 2 else [(8, 256), (1, 512), (4, 64), (2, 256)]
    first = int(rng.integers(0, len(tiles)))
    programs = [1, 3, 7, 64, 10_000][int(rng.integers(0, 5))]
    off = int(rng.integers(0, 40)) * e
    # the drawn tile first; where a member's vector width rules it out, the next candidate that every
    # member's call accepts (the heap and the inputs are 256-byte aligned, as on the device), so that every
    # case launches the kernel
    chosen = None
    for tile in tiles[first:] + tiles[:first] + [(8, 256)]:
        try:
            for j in range(W):
                ag.plan_all_to_all(ag.Geometry(slab_addr=1 << 32, bytes_per_rank=_size(W, M, N, e, off), n_ranks=8,
                                               rank=start + j * stride, num_cus=256),
                                   W, start, stride, 1 << 44, off, M, N, dtype, tile[0], tile[1], programs)
            chosen = tile
            break
        except ag.AgError as exc:
            assert exc.status == ag.AG_ERR_UNSUPPORTED, exc
    assert chosen is not None
    _a2a(8, _size(W, M, N, e, off), W, start, stride, M, N, dtype, off, chosen, programs, seed=W + M + N)


@pytest.mark.parametrize("W,start,stride", [(3, 1, 2), (8, 0, 1)])
@pytest.mark.parametrize("M,N,dtype,tile,vpt", [(100, 1000, "f16", (32, 256), 4), (77, 4100, "bf16", (16, 512), 8),
                                                (50, 520, "f32", (8, 512), 4), (40, 3000, "f32", (16, 512), 8)])
def test_all_to_all_four_and_eight_vectors_per_thread(W, start, stride, M, N, dtype, tile, vpt):
    """Larger tiles: 4 or 8 vector accesses per thread and chunk tile (ragged rows and columns)."""
    e = E[dtype]
    off = 64
    for programs in (5, 256):
        p = ag.plan_all_to_all(ag.Geometry(slab_addr=1 << 32, bytes_per_rank=_size(W, M, N, e, off), n_ranks=8,
                                           rank=start, num_cus=256), W, start, stride, 1 << 44, off, M, N, dtype,
                               tile[0], tile[1], programs)
        assert p.vectors_per_thread == vpt
        _a2a(8, _size(W, M, N, e, off), W, start, stride, M, N, dtype, off, tile, programs, seed=W + M + programs)


def test_all_to_all_row_view():
    # chunks of 1000 x 4100 fp16: rows of 8200 bytes, chunks of 512,500 16-byte vectors, so the kernel walks
    # them as rows of 4000 elements with 16-byte vectors
    p = ag.plan_all_to_all(ag.Geometry(slab_addr=1 << 32, bytes_per_rank=_size(4, 1000, 4100, 2, 0), n_ranks=8,
                                       rank=1, num_cus=256), 4, 1, 2, 1 << 44, 0, 1000, 4100, "f16", 8, 256, 64)
    assert p.vec_bytes == 16 and (p.tiles_m, p.tiles_n) == (129, 16)
    _a2a(8, _size(4, 1000, 4100, 2, 0), 4, 1, 2, 1000, 4100, "f16", 0, (8, 256), 64, seed=13)


def test_all_to_all_edges_and_streams():
    _a2a(8, _size(4, 125, 4100, 2, 64), 4, 1, 2, 125, 4100, "f16", 64, (8, 256), 64, seed=11, streams=True)
    _a2a(8, _size(8, 13, 520, 4, 0), 8, 0, 1, 13, 520, "f32", 0, (8, 256), 5, seed=12)


@pytest.mark.parametrize("M,N,dtype", [(128, 4096, "f16"), (1024, 4096, "bf16")])
def test_all_to_all_full_size_w8(M, N, dtype):
    for programs in (64, 256):
        _a2a(8, _size(8, M, N, 2, 0), 8, 0, 1, M, N, dtype, 0, (8, 256), programs, seed=programs)


def test_all_to_all_validation():
    require_gpu()
    th = TorchHeap(2, 1 << 20)
    try:
        x = torch.zeros(4096, dtype=torch.uint8, device="cuda")
        with pytest.raises(ag.AgError) as exc:
            ag.all_to_all(th.view(0), 3, 0, 1, x, 0, 4, 8, "f16")         # member 2 past the last region
        assert exc.value.status == ag.AG_ERR_INVALID_ARG
        own = th.view(0).rank_ptr(0, 0)
        with pytest.raises(ag.AgError) as exc:
            ag.all_to_all(th.view(0), 2, 0, 1, own, 0, 4, 8, "f16")       # input inside an output block
        assert exc.value.status == ag.AG_ERR_INVALID_ARG
    finally:
        th.close()


@pytest.mark.parametrize("W,start,stride", [(1, 0, 1), (2, 0, 1), (3, 1, 2), (5, 2, 1), (8, 0, 1)])
@pytest.mark.parametrize("M,N,dtype,tile,programs", [(7, 300, "f16", (8, 256), 1), (64, 256, "bf16", (32, 256), 16),
                                                      (33, 1000, "f32", (8, 256), 24), (9, 264, "f16", (4, 512), 10_000)])
def test_all_to_all_partitioned(W, start, stride, M, N, dtype, tile, programs):
    e = E[dtype]
    off = 64
    _a2a(8, _size(W, M, N, e, off), W, start, stride, M, N, dtype, off, tile, programs, seed=W * 10 + M,
         sched="partitioned")


def test_all_to_all_partitioned_streams_and_full_size():
    _a2a(8, _size(4, 125, 4100, 2, 64), 4, 1, 2, 125, 4100, "f16", 64, (8, 256), 64, seed=13, streams=True,
         sched="partitioned")
    _a2a(8, _size(8, 1024, 4096, 2, 0), 8, 0, 1, 1024, 4096, "f16", 0, (8, 512), 256, seed=14, sched="partitioned")
