"""Parity of the HIP all-gather (through the C ABI) with the CPU oracle.

Bit-exact, full-heap comparisons: outputs, the guard bytes around them and
the regions of ranks outside the group (ROCm/iris #594, "Local validation").
"""

import itertools

import numpy as np
import pytest
import torch

from gemm_all_gather_amd import binding as ag
from gemm_all_gather_amd import inputs as gen
from oracle import all_gather_oracle, all_gather_expected_block, group_members
from tests.gpu_util import TorchHeap, log, require_gpu, run_all_gather, to_device

pytestmark = pytest.mark.gpu

E = {"f16": 2, "bf16": 2, "f32": 4}


def _accepted_tile(th, dev, W, start, stride, out_offset, M, N, dtype, tiles, n_programs):
    """The first tile of the candidates that the planner accepts for every member's call.

    The vector width, and so the set of tiles a call supports, follows the alignment of the input and of
    each member's row block; a case only counts when every call launches a kernel.
    """
    for tile in tiles:
        try:
            for j in range(W):
                v = th.view(start + j * stride)
                ag.plan_all_gather(v.geometry(), W, start, stride, dev[j], out_offset, M, N, dtype, tile[0],
                                   tile[1], n_programs)
            return tile
        except ag.AgError as exc:
            assert exc.status == ag.AG_ERR_UNSUPPORTED and "vectors" in exc.message, exc
    raise AssertionError(f"no candidate tile is accepted: {tiles}")


def _case(R, S, W, start, stride, M, N, dtype, out_offset, tile=(0, 0), n_programs=0, seed=0,
          bits=False, fill_random=False):
    """tile: one (tile_m, tile_n), or a list of candidates (the first one every call accepts runs)."""
    require_gpu()
    log(f"all_gather R={R} S={S} W={W} group=({start},{stride}) M={M} N={N} {dtype} off={out_offset} "
        f"tile={tile} programs={n_programs} seed={seed}")
    th = TorchHeap(R, S)
    try:
        before = th.fill_random(seed + 77) if fill_random else th.host()
        if bits:
            ins = [gen.random_bit_patterns((M, N), E[dtype], seed, j) for j in range(W)]
        else:
            ins = [gen.uniform_pm1((M, N), dtype, seed, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        if isinstance(tile, list):
            tile = _accepted_tile(th, dev, W, start, stride, out_offset, M, N, dtype, tile, n_programs)
            log(f"  tile {tile}")
        run_all_gather(th, dev, W, start, stride, out_offset, M, N, dtype, tile[0], tile[1], n_programs)
        got = th.host()
        want = all_gather_oracle(before, S, ins, start, stride, out_offset)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            raise AssertionError(f"{bad.size} bytes differ; first at {bad[0]} (region {bad[0] // S}, "
                                 f"offset {bad[0] % S}): got {got[bad[0]]} want {want[bad[0]]}")
        return ins, got
    finally:
        th.close()


def test_small_two_ranks_with_sentinel_guards():
    # W=2, 64x256 fp16, 8x256 tile, 4 programs, heap pre-filled with 0x7E00
    R, W, M, N = 2, 2, 64, 256
    S = 256 * 1024
    ins, got = _case(R, S, W, 0, 1, M, N, "f16", out_offset=64 * 1024, tile=(8, 256), n_programs=4, seed=1)
    changed = np.count_nonzero(got.view(np.uint16) != gen.SENTINEL16)
    assert changed == W * W * M * N


_SWEEP = []
_rng = np.random.default_rng(2024)
_groups = [(0, 1), (1, 2), (0, 2), (3, 1)]
for W, (start, stride), M, N in itertools.product([1, 2, 3, 4, 8], _groups, [0, 1, 7, 8, 9, 13, 64],
                                                  [1, 3, 4, 8, 255, 256, 257, 260]):
    if start + (W - 1) * stride >= 8:
        continue
    _SWEEP.append((W, start, stride, M, N))
_SWEEP = [c for i, c in enumerate(_SWEEP) if _rng.random() < 0.35]


@pytest.mark.parametrize("W,start,stride,M,N", _SWEEP)
def test_tiny_sweep(W, start, stride, M, N):
    rng = np.random.default_rng([W, start, stride, M, N])
    dtype = ["f16", "bf16", "f32"][int(rng.integers(0, 3))]
    e = E[dtype]
    tiles = [(8, 256), (1, 256), (4, 64), (16, 128), (2, 512), (32, 64)]
    if e == 4:
        tiles = [(8, 256), (1, 512), (4, 64), (16, 128), (2, 512)]
    first = int(rng.integers(0, len(tiles)))
    # the drawn tile first; where the call's vector width rules it out, the next one the planner accepts
    # (8x256 holds 256 to 2048 vectors at every width, so some tile always runs)
    tiles = tiles[first:] + tiles[:first] + [(8, 256)]
    programs = [1, 3, 4, 7, 64, 10_000][int(rng.integers(0, 6))]
    out_offset = int(rng.integers(0, 40)) * e          # often unaligned to 16 bytes
    S = ((out_offset + W * M * N * e + 300) // 256 + 1) * 256
    _case(8, S, W, start, stride, M, N, dtype, out_offset, tiles, programs, seed=W * 1000 + M)


@pytest.mark.parametrize("n_programs", [64, 128, 256])
def test_w8_1024x4096_fp16(n_programs):
    M, N = 1024, 4096
    S = 8 * M * N * 2 + (2 << 20)
    _case(8, S, 8, 0, 1, M, N, "f16", out_offset=1 << 20, tile=(8, 256), n_programs=n_programs, seed=2)


AG_ALIGN = 256


def test_edge_1000x4100_fp16_partial_tiles():
    M, N = 1000, 4100
    S = ((8 * M * N * 2 + (1 << 20)) // AG_ALIGN + 1) * AG_ALIGN
    _case(8, S, 8, 0, 1, M, N, "f16", out_offset=4096, tile=(8, 256), n_programs=256, seed=3)


def test_edge_strided_group_1000x4100():
    M, N = 1000, 4100
    S = ((4 * M * N * 2 + 8192) // AG_ALIGN + 1) * AG_ALIGN
    _case(8, S, 4, 1, 2, M, N, "f16", out_offset=2048, tile=(8, 256), n_programs=128, seed=4)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_random_bit_patterns_are_copied_bytewise(dtype):
    _case(4, 1 << 20, 4, 0, 1, 37, 300, dtype, out_offset=512, tile=(8, 256), n_programs=5, seed=5,
          bits=True, fill_random=True)


def test_concurrent_streams_match_sequential():
    require_gpu()
    R, W, M, N, dtype = 8, 8, 512, 1024, "bf16"
    S = W * M * N * 2 + 4096
    S = (S // 256 + 1) * 256
    log("concurrent streams W=8 512x1024 bf16")
    ins = [gen.uniform_pm1((M, N), dtype, 6, j) for j in range(W)]
    dev = [to_device(x) for x in ins]
    th = TorchHeap(R, S)
    try:
        before = th.host()
        streams = [torch.cuda.Stream() for _ in range(4)]
        torch.cuda.synchronize()
        for j in range(W):
            ag.all_gather(th.view(j), W, 0, 1, dev[j], 1024, M, N, dtype, 8, 256, 64, streams[j % 4])
        torch.cuda.synchronize()
        got = th.host()
        assert np.array_equal(got, all_gather_oracle(before, S, ins, 0, 1, 1024))
    finally:
        th.close()


def test_in_place_input_is_own_slot():
    require_gpu()
    R, W, M, N, dtype = 4, 4, 33, 520, "f16"
    blk = M * N * 2
    S = ((W * blk + 4096) // 256 + 1) * 256
    off = 2048
    log("in-place all-gather W=4 33x520 f16")
    ins = [gen.uniform_pm1((M, N), dtype, 7, j) for j in range(W)]
    th = TorchHeap(R, S)
    try:
        # place each rank's input in its own slot, then gather in place
        for j in range(W):
            th.region(j)[off + j * blk: off + (j + 1) * blk].copy_(torch.from_numpy(ins[j].view(np.uint8).reshape(-1)))
        before = th.host()
        for j in range(W):
            ptr = th.heap.rank_ptr(j, off + j * blk)
            ag.all_gather(th.view(j), W, 0, 1, ptr, off, M, N, dtype)
        got = th.host()
        assert np.array_equal(got, all_gather_oracle(before, S, ins, 0, 1, off))
    finally:
        th.close()


def test_library_owned_heap_create_and_alloc():
    require_gpu()
    log("ag_heap_create + ag_heap_alloc path")
    R, W, M, N = 4, 4, 100, 300
    big = ag.Heap.create(2, 512 << 20)   # a power-of-two region of 512 MiB gets one more 2 MiB unit
    try:
        assert big.geometry().bytes_per_rank == (512 + 2) << 20 == ag.heap_region_bytes(512 << 20)
    finally:
        big.destroy()
    heap = ag.Heap.create(R, 3 << 20)
    try:
        g = heap.geometry()
        assert g.bytes_per_rank == 4 << 20 and g.n_ranks == R and g.rank == -1
        off_a = heap.alloc(1000)
        off_b = heap.alloc(W * M * N * 2, 4096)
        assert off_a == 0 and off_b == 4096
        with pytest.raises(ag.AgError) as ei:
            heap.alloc(64 << 20)
        assert ei.value.status == ag.AG_ERR_OUT_OF_MEMORY
        # wrap the library's slab in a torch tensor to initialise and read it
        total = R * g.bytes_per_rank

        class _Iface:
            __cuda_array_interface__ = {"shape": (total,), "typestr": "|u1", "data": (g.slab_addr, False),
                                        "version": 3, "strides": None}

        slab = torch.as_tensor(_Iface(), device="cuda")
        slab.fill_(0xA5)
        torch.cuda.synchronize()
        before = slab.cpu().numpy()
        ins = [gen.uniform_pm1((M, N), "f16", 8, j) for j in range(W)]
        dev = [to_device(x) for x in ins]
        views = [heap.view(j) for j in range(W)]
        for j in range(W):
            ag.all_gather(views[j], W, 0, 1, dev[j], off_b, M, N, "f16", 8, 256, 0)
        torch.cuda.synchronize()
        got = slab.cpu().numpy()
        assert np.array_equal(got, all_gather_oracle(before, g.bytes_per_rank, ins, 0, 1, off_b))
        table = torch.empty(R, dtype=torch.int64, device="cuda")

        class _T:
            __cuda_array_interface__ = {"shape": (R,), "typestr": "<i8", "data": (heap.base_table(), False),
                                        "version": 3, "strides": None}

        table.copy_(torch.as_tensor(_T(), device="cuda"))
        assert table.cpu().tolist() == [g.slab_addr + r * g.bytes_per_rank for r in range(R)]
        # ag_heap_info reports what ag_heap_geometry and ag_heap_base_table report, for the root and views
        for h in [heap] + views:
            info, hg = h.info(), h.geometry()
            assert info == {"n_ranks": hg.n_ranks, "rank": hg.rank, "bytes_per_rank": hg.bytes_per_rank,
                            "base_table": h.base_table()}
        assert heap.info()["rank"] == -1 and [v.info()["rank"] for v in views] == list(range(W))
        assert len({v.info()["base_table"] for v in views} | {heap.info()["base_table"]}) == 1
        for v in views:
            v.destroy()
    finally:
        heap.destroy()


def test_wrap_rejects_host_memory_and_short_slabs():
    require_gpu()
    log("ag_heap_wrap validation: host memory, a slab shorter than its regions")
    host = np.zeros(1 << 20, dtype=np.uint8)
    with pytest.raises(ag.AgError) as ei:
        ag.Heap.wrap(host.ctypes.data, 4, 256 << 10)
    assert ei.value.status == ag.AG_ERR_INVALID_ARG
    # a dedicated allocation of 2 MiB (the library's slab of one 2 MiB region) cannot hold 4 regions of 1 MiB
    buf = ag.Heap.create(1, 2 << 20)
    try:
        slab = buf.geometry().slab_addr
        with pytest.raises(ag.AgError) as ei:
            ag.Heap.wrap(slab, 4, 1 << 20)
        assert ei.value.status == ag.AG_ERR_INVALID_ARG and "allocation" in ei.value.message
        with pytest.raises(ag.AgError):
            ag.Heap.wrap(slab + (1 << 20), 2, 1 << 20)        # runs 1 MiB past the end
        h = ag.Heap.wrap(slab, 2, 1 << 20)                    # exactly the allocation
        h.destroy()
        h = ag.Heap.wrap(slab + (1 << 20), 1, 1 << 20)        # its second half
        h.destroy()
    finally:
        buf.destroy()
    # the failed queries leave no error behind for the next launch
    th = TorchHeap(2, 1 << 20)
    try:
        x = to_device(gen.uniform_pm1((16, 256), "f16", 3))
        ag.all_gather(th.view(0), 2, 0, 1, x, 0, 16, 256, "f16")
        torch.cuda.synchronize()
    finally:
        th.close()


_EXPANDABLE = r"""
import os, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
from gemm_all_gather_amd import binding as ag
from gemm_all_gather_amd import inputs as gen
from oracle import all_gather_oracle
R, W, M, N, S = 4, 4, 40, 264, 1 << 20
slab = torch.zeros(R * S, dtype=torch.uint8, device="cuda")
heap = ag.Heap.wrap(slab, R, S)
ins = [gen.uniform_pm1((M, N), "f16", 31, j) for j in range(W)]
dev = [torch.from_numpy(x.view(np.uint8).reshape(-1).copy()).cuda() for x in ins]
before = slab.cpu().numpy()
views = [heap.view(j) for j in range(W)]
for j in range(W):
    ag.all_gather(views[j], W, 0, 1, dev[j], 0, M, N, "f16")
torch.cuda.synchronize()
assert np.array_equal(slab.cpu().numpy(), all_gather_oracle(before, S, ins, 0, 1, 0))
print("expandable-segments slab: bit-exact")
"""


def test_wrap_accepts_expandable_segment_memory():
    """A slab from PyTorch's expandable-segments allocator (memory mapped through the virtual memory API)
    is accepted and gathered bit-exactly (a separate process: the allocator is chosen at start-up)."""
    require_gpu()
    import os
    import subprocess
    import sys
    log("ag_heap_wrap over an expandable-segments allocation (subprocess)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTORCH_HIP_ALLOC_CONF="expandable_segments:True",
               PYTORCH_CUDA_ALLOC_CONF="expandable_segments:True")
    r = subprocess.run([sys.executable, "-c", _EXPANDABLE, root], env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "bit-exact" in r.stdout


def test_launching_entry_point_rejects_invalid_arguments():
    require_gpu()
    log("ag_all_gather validation on the launching entry point")
    th = TorchHeap(4, 1 << 20)
    try:
        x = to_device(gen.uniform_pm1((8, 256), "f16", 9))
        v = th.view(1)
        cases = [
            (dict(W=9), ag.AG_ERR_UNSUPPORTED),
            (dict(W=0), ag.AG_ERR_INVALID_ARG),
            (dict(rank_start=2), ag.AG_ERR_INVALID_ARG),          # rank 1 not in group
            (dict(out_offset=1), ag.AG_ERR_INVALID_ARG),
            (dict(out_offset=1 << 20), ag.AG_ERR_INVALID_ARG),
            (dict(tile_m=3, tile_n=256), ag.AG_ERR_UNSUPPORTED),
            (dict(n_programs=-1), ag.AG_ERR_INVALID_ARG),
            (dict(dtype=7), ag.AG_ERR_INVALID_ARG),
            (dict(input=0), ag.AG_ERR_INVALID_ARG),
        ]
        base = dict(W=4, rank_start=0, rank_stride=1, input=x, out_offset=0, M_local=8, N=256, dtype="f16",
                    tile_m=0, tile_n=0, n_programs=0)
        for over, status in cases:
            kw = dict(base, **over)
            with pytest.raises(ag.AgError) as ei:
                ag.all_gather(v, **kw)
            assert ei.value.status == status, (over, ei.value)
        with pytest.raises(ag.AgError):
            ag.all_gather(th.heap, **base)       # root handle is not a rank view
        torch.cuda.synchronize()
        assert np.all(th.host().view(np.uint16) == gen.SENTINEL16)   # nothing was launched
    finally:
        th.close()


# ---------------------------------------------------------------------------
# full-size workloads: W=8, 16384 x 8192 per rank
# ---------------------------------------------------------------------------

def _full_size(dtype, W, start, stride, M, N, programs_list, seed, orders=("auto", "stride")):
    """Each program count in the library's tile order (tickets at this size) and in the grid stride."""
    require_gpu()
    e = E[dtype]
    blk = M * N * e
    guard = 1 << 20
    S = W * blk + 2 * guard
    R = 8
    members = group_members(start, stride, W)
    log(f"full-size all_gather {dtype} W={W} group=({start},{stride}) {M}x{N}: generating inputs")
    ins = [gen.uniform_pm1((M, N), dtype, seed, j) for j in range(W)]
    dev = [to_device(x) for x in ins]
    expect = to_device(all_gather_expected_block(ins))       # oracle's gathered block, uploaded for comparison
    th = TorchHeap(R, S)
    try:
        for programs, order in itertools.product(programs_list, orders):
            th.fill(gen.SENTINEL16)
            p = ag.plan_all_gather_ex(th.view(start).geometry(), W, start, stride, dev[0], guard, M, N, dtype, 8, 256,
                                      programs, tile_order=order)
            log(f"  n_programs={programs} order={order} -> tile_order {p.tile_order}, {p.tiles_per_ticket} per ticket")
            if order == "auto":
                assert p.tile_order == ag.AG_ORDER_TICKETS
                run_all_gather(th, dev, W, start, stride, guard, M, N, dtype, 8, 256, programs)
            else:
                for j in range(W):
                    ag.all_gather_ex(th.view(start + j * stride), W, start, stride, dev[j], guard, M, N, dtype, 8, 256,
                                     programs, tile_order=order)
            torch.cuda.synchronize()
            sentinel = torch.tensor([np.int16(np.uint16(gen.SENTINEL16).view(np.int16))], device="cuda")
            for r in range(R):
                reg = th.region(r)
                if r in members:
                    assert torch.equal(reg[guard:guard + W * blk], expect), f"region {r} output differs"
                    assert torch.all(reg[:guard].view(torch.int16) == sentinel), f"region {r} front guard"
                    assert torch.all(reg[guard + W * blk:].view(torch.int16) == sentinel), f"region {r} back guard"
                else:
                    assert torch.all(reg.view(torch.int16) == sentinel), f"non-member region {r} touched"
    finally:
        th.close()
        del dev, expect
        torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_full_size_w8_16384x8192(dtype):
    _full_size(dtype, 8, 0, 1, 16384, 8192, [64, 128, 256], seed=10)


def test_full_size_strided_group_16384x8192():
    _full_size("f16", 4, 1, 2, 16384, 8192, [256], seed=11)


# ---------------------------------------------------------------------------
# maximum sizes: blocks on both sides of the ticket kernel's 2 GiB limit, and one past 4 GiB
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,order", [(32760, ag.AG_ORDER_TICKETS), (32776, ag.AG_ORDER_STRIDE),
                                     (65544, ag.AG_ORDER_STRIDE)])
def test_max_size_blocks(M, order):
    """W=2, rows of 64 KiB (N=32768 fp16): tile rows just under 2 GiB per rank (ticket order, 32-bit tile
    offsets), just over (grid stride), and a block past 4 GiB (64-bit tile offsets, descriptor extents
    clamped below 2 GiB).  Both regions' outputs and guards are compared with the oracle's gathered block
    on the device."""
    require_gpu()
    W, N, dtype = 2, 32768, "f16"
    blk = M * N * 2
    guard = 1 << 20
    S = W * blk + 2 * guard
    log(f"max-size all_gather W={W} {M}x{N} {dtype}: {blk / 2 ** 30:.3f} GiB per rank; generating inputs")
    ins = [gen.random_bit_patterns((M, N), 2, 70, M, j) for j in range(W)]
    dev = [to_device(x) for x in ins]
    expect = to_device(all_gather_expected_block(ins))
    del ins
    th = TorchHeap(W, S)
    try:
        p = ag.plan_all_gather_ex(th.view(0).geometry(), W, 0, 1, dev[0], guard, M, N, dtype, 0, 0, 256)
        assert p.tile_order == order
        log(f"  tile order {p.tile_order}, {p.total_tiles} tiles, {p.n_programs} programs: running")
        run_all_gather(th, dev, W, 0, 1, guard, M, N, dtype, 0, 0, 256)
        torch.cuda.synchronize()
        sentinel = torch.tensor([np.int16(np.uint16(gen.SENTINEL16).view(np.int16))], device="cuda")
        for r in range(W):
            reg = th.region(r)
            assert torch.equal(reg[guard:guard + W * blk], expect), f"region {r} output differs"
            assert torch.all(reg[:guard].view(torch.int16) == sentinel), f"region {r} front guard"
            assert torch.all(reg[guard + W * blk:].view(torch.int16) == sentinel), f"region {r} back guard"
    finally:
        th.close()
        del dev, expect
        torch.cuda.empty_cache()
