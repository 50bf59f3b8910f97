"""Host-side checks of libag with no GPU: exported symbols, validation and launch planning.

The ag_plan_* entry points hold every validation and launch decision of
ag_all_gather / ag_gemm_all_gather and touch no device, so they run here on
hand-made heap geometries.
"""

import ctypes
import os
import re

import pytest

from gemm_all_gather_amd import binding as ag

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ag.h")

SLAB = 1 << 32
MiB = 1 << 20


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ag_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert "ag_all_gather" in names and "ag_gemm_all_gather" in names and "ag_heap_create" in names
    lib = ctypes.CDLL(ag.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert ag.version().startswith("libag")


def test_status_strings():
    lib = ag.lib()
    for code, name in ag.STATUS_NAMES.items():
        assert lib.ag_status_string(code).decode() == name
    assert lib.ag_status_string(99).decode() == "AG_ERR_UNKNOWN"


def geom(n_ranks=8, bytes_per_rank=64 * MiB, rank=0, num_cus=256, slab=SLAB):
    return ag.Geometry(slab_addr=slab, bytes_per_rank=bytes_per_rank, n_ranks=n_ranks, rank=rank,
                       num_cus=num_cus)


INPUT = 1 << 44   # a device address far from the slab


def plan(g=None, W=8, start=0, stride=1, inp=INPUT, off=0, M=1024, N=4096, dtype="f16", tm=0, tn=0, progs=0):
    return ag.plan_all_gather(g or geom(), W, start, stride, inp, off, M, N, dtype, tm, tn, progs)


def status_of(fn, *a, **k):
    try:
        fn(*a, **k)
    except ag.AgError as exc:
        return exc.status, exc.message
    return ag.AG_OK, ""


def test_plan_default_workload():
    p = plan(g=geom(rank=3))
    assert (p.tile_m, p.tile_n) == (8, 256)           # 0,0 is the documented 8x256 default
    assert p.group_rank == 3
    assert p.vec_bytes == 16 and p.vectors_per_thread == 1
    assert p.tiles_m == 128 and p.tiles_n == 16 and p.total_tiles == 2048
    assert p.rank_block_offset == 3 * 1024 * 4096 * 2
    assert p.bytes_read == 1024 * 4096 * 2 and p.bytes_written == 8 * p.bytes_read
    assert p.n_programs <= 256 and p.threads % 256 == 0


def test_plan_explicit_tile_is_never_remapped():
    for tm, tn in [(32, 64), (8, 256), (16, 128), (4, 512)]:
        p = plan(tm=tm, tn=tn)
        assert (p.tile_m, p.tile_n) == (tm, tn)


def test_plan_strided_group_uses_group_rank():
    p = plan(g=geom(rank=5), W=4, start=1, stride=2)
    assert p.group_rank == 2
    assert p.rank_block_offset == 2 * 1024 * 4096 * 2


# M = 63: the block's size is N*e*63, a multiple of 16 only when the row is; M = 64 would let the
# kernels view the block as rows of a multiple of 16 bytes (test_plan_row_view)
@pytest.mark.parametrize("N,dtype,inp,off,vec", [
    (4096, "f16", INPUT, 0, 16), (4100, "f16", INPUT, 0, 8), (4098, "f16", INPUT, 0, 4),
    (4097, "f16", INPUT, 0, 2), (4096, "f16", INPUT + 8, 0, 8), (4096, "f16", INPUT, 2, 2),
    (4096, "f32", INPUT, 4, 4), (4097, "f32", INPUT, 0, 4), (4098, "f32", INPUT, 0, 8),
])
def test_plan_vector_width_follows_alignment(N, dtype, inp, off, vec):
    p = plan(N=N, dtype=dtype, inp=inp, off=off, M=63)
    assert p.vec_bytes == vec


# A dense block of M x N elements is M*N*e contiguous bytes.  When rows are not a multiple of 16 bytes
# but the block is (and the input and output block are 16-byte aligned), the kernels walk it as rows of
# cols elements, cols*e a multiple of 16: the divisor of the block's 16-byte vector count nearest N*e/16.
@pytest.mark.parametrize("M,N,dtype,inp,off,vec,tiles", [
    (1000, 4100, "f16", INPUT, 0, 16, (129, 16)),   # 512500 vectors: rows of 500 (4000 elements), 1025 rows
    (64, 4100, "f16", INPUT, 0, 16, None),
    (64, 4097, "f16", INPUT, 0, 16, None),
    (64, 4098, "f32", INPUT, 0, 16, None),
    (64, 4100, "f16", INPUT + 8, 0, 8, (8, 17)),     # input 8-byte aligned: rows as given
    (64, 4100, "f16", INPUT, 8, 8, (8, 17)),         # output block 8-byte aligned
    (1, 4100, "f16", INPUT, 0, 8, (1, 17)),          # one row: 8200 bytes, not a multiple of 16
])
def test_plan_row_view(M, N, dtype, inp, off, vec, tiles):
    p = plan(N=N, dtype=dtype, inp=inp, off=off, M=M)
    assert p.vec_bytes == vec
    if tiles:
        assert (p.tiles_m, p.tiles_n) == tiles
    # the tiles cover the block's bytes exactly once however it is viewed
    e = 4 if dtype == "f32" else 2
    assert p.tiles_m * 8 >= M * N * e // (p.tiles_n * 256 * e) and p.bytes_read == M * N * e


def test_plan_row_view_only_when_the_tile_fits():
    # a 1x256 fp16 tile is 32 vectors of 16 bytes, fewer than 256 threads: the rows stay as given, 2-byte vectors
    p = plan(M=64, N=4097, tm=1, tn=256)
    assert p.vec_bytes == 2 and (p.tiles_m, p.tiles_n) == (64, 17)
    p = plan_a2a(M=16, N=4095, tm=1, tn=256)
    assert p.vec_bytes == 2 and (p.tiles_m, p.tiles_n) == (16, 16)


def test_plan_programs_and_tiles():
    p = plan(M=64, N=256, progs=4)        # 8 tiles over 4 programs
    assert p.total_tiles == 8 and p.n_programs * (p.threads // 256) <= 8
    p = plan(M=1000, N=4100, inp=INPUT + 8)   # partial tiles in both directions (8-byte aligned input)
    assert p.tiles_m == 125 and p.tiles_n == 17
    p = plan(M=8, N=256, progs=10_000)    # more programs than tiles: only one launched
    assert p.n_programs == 1


def test_plan_zero_rows_is_a_noop():
    p = plan(M=0, inp=0)
    assert p.total_tiles == 0 and p.n_programs == 0


@pytest.mark.parametrize("over,status,text", [
    (dict(W=0), ag.AG_ERR_INVALID_ARG, "W"),
    (dict(W=9), ag.AG_ERR_UNSUPPORTED, "W"),
    (dict(start=-1), ag.AG_ERR_INVALID_ARG, "rank_start"),
    (dict(stride=0), ag.AG_ERR_INVALID_ARG, "rank_stride"),
    (dict(W=4, start=1, stride=3), ag.AG_ERR_INVALID_ARG, "past the last region"),
    (dict(W=4, start=1, stride=2), ag.AG_ERR_INVALID_ARG, "not a member"),    # rank 0 not in {1,3,5,7}
    (dict(M=-1), ag.AG_ERR_INVALID_ARG, "M_local"),
    (dict(N=0), ag.AG_ERR_INVALID_ARG, "N"),
    (dict(off=1), ag.AG_ERR_INVALID_ARG, "element size"),
    (dict(off=64 * MiB - 2), ag.AG_ERR_INVALID_ARG, "exceeds the region"),
    (dict(M=1025), ag.AG_ERR_INVALID_ARG, "exceeds the region"),
    (dict(tm=3, tn=256), ag.AG_ERR_UNSUPPORTED, "power of two"),
    (dict(tm=8, tn=0), ag.AG_ERR_INVALID_ARG, "both sides"),
    (dict(tm=512, tn=256), ag.AG_ERR_UNSUPPORTED, "power of two"),
    (dict(tm=1, tn=256), ag.AG_ERR_UNSUPPORTED, "vectors"),                    # 32 vectors < 256
    (dict(tm=64, tn=512), ag.AG_ERR_UNSUPPORTED, "vectors"),                   # 4096 vectors > 2048
    (dict(progs=-1), ag.AG_ERR_INVALID_ARG, "n_programs"),
    (dict(dtype=5), ag.AG_ERR_INVALID_ARG, "dtype"),
    (dict(inp=0), ag.AG_ERR_INVALID_ARG, "NULL"),
    (dict(inp=INPUT + 1), ag.AG_ERR_INVALID_ARG, "aligned"),
])
def test_plan_rejects(over, status, text):
    kw = dict(over)
    got, msg = status_of(plan, **kw)
    assert got == status, (over, got, msg)
    assert text in msg, msg


def test_plan_rejects_bad_geometry_and_root_handle():
    for g, text in [(geom(rank=-1), "not a view"), (geom(rank=8), "not a view"), (geom(n_ranks=0), "n_ranks"),
                    (geom(bytes_per_rank=100), "multiple of 256"), (geom(slab=0), "slab"),
                    (geom(num_cus=0), "num_cus")]:
        got, msg = status_of(plan, g=g)
        assert got == ag.AG_ERR_INVALID_ARG and text in msg, (msg,)


def test_plan_input_overlap_rules():
    S = 64 * MiB
    blk = 1024 * 4096 * 2
    g = geom(rank=2)
    own = SLAB + 2 * S + 2 * blk
    assert plan(g=g, inp=own).group_rank == 2                     # exactly its own slot: in place
    got, msg = status_of(plan, g=g, inp=own + 2)                   # shifted: overlaps
    assert got == ag.AG_ERR_INVALID_ARG and "overlaps" in msg
    got, _ = status_of(plan, g=g, inp=SLAB + 5 * S + 7 * blk)      # inside another member's block
    assert got == ag.AG_ERR_INVALID_ARG
    assert plan(g=geom(rank=1), W=2, start=0, stride=1, inp=SLAB + 5 * S).group_rank == 1   # non-member region


# ---------------------------------------------------------------------------
# fused GEMM + all-gather planning
# ---------------------------------------------------------------------------

A_ADDR, B_ADDR = 1 << 44, 1 << 45


def gplan(g=None, W=8, start=0, stride=1, a=A_ADDR, lda=8192, b=B_ADDR, ldb=8192, off=0, M=1024, N=3584,
          K=8192, dtype="f16", tm=0, tn=0, tk=0, progs=0):
    return ag.plan_gemm_all_gather(g or geom(bytes_per_rank=1 << 30), W, start, stride, a, lda, b, ldb, off,
                                   M, N, K, dtype, tm, tn, tk, progs)


def test_gemm_plan_default_tiles():
    p = gplan()
    assert (p.tile_m, p.tile_n, p.tile_k) == (128, 128, 64)       # 56 tiles of 256^2 cannot fill 256 CUs
    assert p.total_tiles == 8 * 28
    assert p.flops == 2.0 * 1024 * 3584 * 8192
    p = gplan(M=16384)                                             # 256x224: 64 x 16 tiles = 4 rounds of 256
    assert (p.tile_m, p.tile_n) == (256, 224) and p.total_tiles == 64 * 16
    assert p.n_programs == 256
    p = gplan(M=16384, tm=256, tn=256, tk=64)                      # explicit tiles are used as given
    assert (p.tile_m, p.tile_n) == (256, 256) and p.total_tiles == 64 * 14


@pytest.mark.parametrize("over,status", [
    (dict(dtype="f32"), ag.AG_ERR_UNSUPPORTED),
    (dict(K=100), ag.AG_ERR_UNSUPPORTED),
    (dict(N=3585), ag.AG_ERR_UNSUPPORTED),
    (dict(lda=8000), ag.AG_ERR_INVALID_ARG),
    (dict(lda=8196), ag.AG_ERR_UNSUPPORTED),
    (dict(tm=64, tn=64, tk=64), ag.AG_ERR_UNSUPPORTED),
    (dict(off=8), ag.AG_ERR_UNSUPPORTED),
    (dict(a=A_ADDR + 2), ag.AG_ERR_UNSUPPORTED),
    (dict(a=0), ag.AG_ERR_INVALID_ARG),
    (dict(W=9), ag.AG_ERR_UNSUPPORTED),
    (dict(M=40000), ag.AG_ERR_INVALID_ARG),
    (dict(a=SLAB + 256), ag.AG_ERR_INVALID_ARG),      # A inside an output block
])
def test_gemm_plan_rejects(over, status):
    got, msg = status_of(gplan, **over)
    assert got == status, (over, got, msg)


@pytest.mark.parametrize("nbytes,want_mib", [(1, 2), (3 * MiB, 4), (256 * MiB, 256), (510 * MiB + 1, 512 + 2),
                                            (512 * MiB, 514), (1024 * MiB, 1026), (2048 * MiB - 7, 2050),
                                            (2048 * MiB + 1, 2050), (1536 * MiB, 1536), (8 * 16384 * 3584 * 2, 896)])
def test_heap_region_bytes(nbytes, want_mib):
    # whole 2 MiB units, one more when that is a power of two from 512 MiB (the W copies of a tile would
    # alias in the HBM channel interleave)
    assert ag.heap_region_bytes(nbytes) == want_mib * MiB


def test_heap_region_bytes_rejects():
    assert status_of(ag.heap_region_bytes, 0)[0] == ag.AG_ERR_INVALID_ARG
    assert status_of(ag.heap_region_bytes, (1 << 40) + 1)[0] == ag.AG_ERR_INVALID_ARG
    got = ag.lib().ag_heap_region_bytes(MiB, None)
    assert got == ag.AG_ERR_INVALID_ARG


def test_heap_create_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    got, msg = status_of(ag.Heap.create, 2, MiB)
    assert got == ag.AG_ERR_HIP and "hip" in msg.lower()


def test_heap_info_rejects_a_null_handle():
    l = ag.lib()
    n, r, s, t = ctypes.c_int(7), ctypes.c_int(7), ctypes.c_size_t(7), ctypes.c_void_p(7)
    st = l.ag_heap_info(None, ctypes.byref(n), ctypes.byref(r), ctypes.byref(s), ctypes.byref(t))
    assert st == ag.AG_ERR_INVALID_ARG and "heap" in l.ag_last_error_message().decode()
    # nothing is written on failure
    assert (n.value, r.value, s.value, t.value) == (7, 7, 7, 7)


def test_heap_clear_tickets_rejects_a_null_handle():
    l = ag.lib()
    assert l.ag_heap_clear_tickets(None, None) == ag.AG_ERR_INVALID_ARG
    assert "heap" in l.ag_last_error_message().decode()


def test_heap_argument_validation_without_device():
    assert status_of(ag.Heap.create, 0, MiB)[0] == ag.AG_ERR_INVALID_ARG
    assert status_of(ag.Heap.create, 2, 0)[0] == ag.AG_ERR_INVALID_ARG
    assert status_of(ag.Heap.wrap, 0, 2, MiB)[0] == ag.AG_ERR_INVALID_ARG
    assert status_of(ag.Heap.wrap, 1 << 30, 2, 1000)[0] == ag.AG_ERR_INVALID_ARG
    assert status_of(ag.Heap.wrap, (1 << 30) + 8, 2, MiB)[0] == ag.AG_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# all-gather variants: destination groups and the partitioned schedule
# ---------------------------------------------------------------------------

def plan_ex(g=None, W=8, inp=INPUT, off=0, M=1024, N=4096, dtype="f16", tm=0, tn=0, progs=0, group=0, sched=0):
    return ag.plan_all_gather_ex(g or geom(), W, 0, 1, inp, off, M, N, dtype, tm, tn, progs, group, sched)


def test_plan_ex_defaults_equal_plain_plan():
    a, b = plan().as_dict(), plan_ex().as_dict()
    assert a == b
    assert a["dest_group"] == 0 and a["schedule"] == ag.AG_SCHEDULE_TILES


@pytest.mark.parametrize("W,group,applied", [(8, 1, 1), (8, 2, 2), (8, 4, 4), (4, 4, 0), (2, 4, 0), (3, 2, 2),
                                             (1, 1, 0)])
def test_plan_destination_groups(W, group, applied):
    p = plan_ex(g=geom(), W=W, group=group)
    assert p.dest_group == applied
    assert p.bytes_read == 1024 * 4096 * 2 and p.bytes_written == W * p.bytes_read   # grouping moves the same bytes


@pytest.mark.parametrize("kw,status", [
    (dict(group=3), ag.AG_ERR_UNSUPPORTED),
    (dict(group=8), ag.AG_ERR_UNSUPPORTED),
    (dict(group=-1), ag.AG_ERR_INVALID_ARG),
    (dict(group=2, sched=1), ag.AG_ERR_INVALID_ARG),
    (dict(sched=2), ag.AG_ERR_INVALID_ARG),
    (dict(group=2, M=63, N=4097, dtype="f32"), ag.AG_ERR_UNSUPPORTED),   # 4-byte vectors: no grouped kernel
])
def test_plan_ex_rejects(kw, status):
    assert status_of(plan_ex, **kw)[0] == status


def test_plan_ex_rejects_reserved_options():
    o = ag._options(0, 0)
    o.reserved[3] = 1
    p = ag.Plan()
    st = ag.lib().ag_plan_all_gather_ex(ctypes.byref(geom()), 8, 0, 1, INPUT, 0, 1024, 4096, ag.AG_F16, 0, 0, 0,
                                        ctypes.byref(o), ctypes.byref(p))
    assert st == ag.AG_ERR_INVALID_ARG


@pytest.mark.parametrize("W,progs,grid", [(8, 256, 256), (8, 100, 96), (8, 3, 8), (8, 0, 256), (3, 64, 63),
                                          (1, 16, 16)])
def test_plan_partitioned_programs(W, progs, grid):
    p = plan_ex(g=geom(), W=W, progs=progs, sched="partitioned")
    assert p.schedule == ag.AG_SCHEDULE_PARTITIONED
    assert p.n_programs == grid and p.n_programs % W == 0 and p.threads == 256
    blk = 1024 * 4096 * 2
    assert p.bytes_read == W * blk and p.bytes_written == W * blk   # every destination reads the tile itself


def test_plan_partitioned_programs_capped_by_tiles():
    p = plan_ex(W=4, M=8, N=512, progs=256, sched="partitioned")   # 2 tiles of 8x256
    assert p.total_tiles == 2 and p.n_programs == 2 * 4


# ---------------------------------------------------------------------------
# all-to-all
# ---------------------------------------------------------------------------

def plan_a2a(g=None, W=8, start=0, stride=1, inp=INPUT, off=0, M=128, N=4096, dtype="f16", tm=0, tn=0, progs=0):
    return ag.plan_all_to_all(g or geom(), W, start, stride, inp, off, M, N, dtype, tm, tn, progs)


def test_plan_all_to_all_default():
    p = plan_a2a(g=geom(rank=5))
    blk = 128 * 4096 * 2
    assert p.group_rank == 5 and p.rank_block_offset == 5 * blk
    assert p.bytes_read == 8 * blk and p.bytes_written == 8 * blk
    assert (p.tile_m, p.tile_n, p.vec_bytes, p.vectors_per_thread) == (8, 256, 16, 1)
    assert p.total_tiles == 16 * 16 and p.n_programs == 256 and p.threads == 256


def test_plan_all_to_all_strided_group_and_zero_rows():
    p = plan_a2a(g=geom(rank=5), W=4, start=1, stride=2, off=4096)
    assert p.group_rank == 2 and p.rank_block_offset == 4096 + 2 * 128 * 4096 * 2
    z = plan_a2a(M=0)
    assert z.total_tiles == 0 and z.bytes_written == 0


@pytest.mark.parametrize("kw,status", [
    (dict(tm=32, tn=512, dtype="f32"), ag.AG_ERR_UNSUPPORTED),    # 16 vectors per thread: at most 8
    (dict(M=-1), ag.AG_ERR_INVALID_ARG),
    (dict(M=1 << 20), ag.AG_ERR_INVALID_ARG),                     # output block past the region
    (dict(inp=0), ag.AG_ERR_INVALID_ARG),
    (dict(W=9), ag.AG_ERR_UNSUPPORTED),
])
def test_plan_all_to_all_rejects(kw, status):
    assert status_of(plan_a2a, **kw)[0] == status


@pytest.mark.parametrize("N,vec,vpt", [(4096, 16, 1), (4092, 8, 2), (4094, 4, 4), (4095, 2, 8)])
def test_plan_all_to_all_default_tile_fits_every_vector_width(N, vec, vpt):
    p = plan_a2a(M=15, N=N)   # 15 rows: the chunk is a multiple of 16 bytes only when its rows are
    assert (p.vec_bytes, p.vectors_per_thread) == (vec, vpt)


def test_plan_all_to_all_input_may_not_overlap_any_output():
    g = geom(rank=2)
    blk = 128 * 4096 * 2
    own = SLAB + 2 * g.bytes_per_rank + 2 * blk          # this rank's own rows: allowed for the all-gather only
    assert status_of(plan_a2a, g=g, inp=own)[0] == ag.AG_ERR_INVALID_ARG
    assert status_of(plan_a2a, g=g, inp=SLAB + 6 * g.bytes_per_rank + 8 * blk)[0] == ag.AG_OK   # past the block
    assert status_of(plan_a2a, g=g, inp=SLAB + 6 * g.bytes_per_rank + 8 * blk - 2)[0] == ag.AG_ERR_INVALID_ARG


def plan_a2a_ex(g=None, W=8, start=0, stride=1, inp=INPUT, off=0, M=128, N=4096, dtype="f16", tm=0, tn=0, progs=0,
                group=0, sched=0):
    return ag.plan_all_to_all_ex(g or geom(), W, start, stride, inp, off, M, N, dtype, tm, tn, progs,
                                 dest_group=group, schedule=sched)


def test_plan_all_to_all_ex_defaults_equal_the_plain_call():
    a, b = plan_a2a(g=geom(rank=3)), plan_a2a_ex(g=geom(rank=3))
    assert a.as_dict() == b.as_dict()


@pytest.mark.parametrize("W,progs,grid", [(8, 256, 256), (8, 100, 96), (8, 5, 8), (3, 256, 255), (1, 7, 7)])
def test_plan_all_to_all_partitioned_programs(W, progs, grid):
    p = plan_a2a_ex(W=W, progs=progs, sched="partitioned")
    assert p.schedule == ag.AG_SCHEDULE_PARTITIONED
    assert p.n_programs == grid and p.n_programs % W == 0 and p.threads == 256
    blk = 128 * 4096 * 2
    assert p.bytes_read == W * blk and p.bytes_written == W * blk    # every chunk read once


def test_plan_all_to_all_takes_up_to_eight_vectors_per_thread():
    # both schedules hold one chunk tile per step in registers: up to 8 vectors of 16 bytes per thread
    for sched in ("tiles", "partitioned"):
        p = plan_a2a_ex(tm=32, tn=256, sched=sched)
        assert (p.vec_bytes, p.vectors_per_thread) == (16, 4)
        p = plan_a2a_ex(tm=64, tn=256, sched=sched)
        assert (p.vec_bytes, p.vectors_per_thread) == (16, 8)
        assert status_of(plan_a2a_ex, tm=128, tn=256, sched=sched)[0] == ag.AG_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    (dict(group=2), ag.AG_ERR_INVALID_ARG),                          # the all-to-all takes no destination groups
    (dict(group=2, sched="partitioned"), ag.AG_ERR_INVALID_ARG),
    (dict(sched=7), ag.AG_ERR_INVALID_ARG),
])
def test_plan_all_to_all_ex_rejects(kw, status):
    assert status_of(plan_a2a_ex, **kw)[0] == status


# ---------------------------------------------------------------------------
# fused GEMM with B in either layout
# ---------------------------------------------------------------------------

def gplan_ex(g=None, W=8, start=0, stride=1, a=A_ADDR, lda=8192, b=B_ADDR, ldb=3584, off=0, M=1024, N=3584,
             K=8192, dtype="f16", tm=0, tn=0, tk=0, progs=0, layout="n"):
    return ag.plan_gemm_all_gather_ex(g or geom(bytes_per_rank=1 << 30), W, start, stride, a, lda, b, ldb, off,
                                      M, N, K, dtype, tm, tn, tk, progs, b_layout=layout)


def test_gemm_plan_ex_k_layout_equals_the_plain_call():
    assert gplan_ex(ldb=8192, layout="k").as_dict() == gplan().as_dict()
    assert gplan_ex(M=16384, ldb=8192, layout="k").as_dict() == gplan(M=16384).as_dict()


def test_gemm_plan_n_contiguous_tiles():
    assert (gplan_ex().tile_m, gplan_ex().tile_n) == (128, 128)
    p = gplan_ex(M=16384)
    assert (p.tile_m, p.tile_n) == (256, 224) and p.total_tiles == 64 * 16
    assert p.bytes_read == (16384 + 3584) * 8192 * 2


@pytest.mark.parametrize("over,status", [
    (dict(ldb=3000), ag.AG_ERR_INVALID_ARG),              # ldb < N
    (dict(ldb=3588), ag.AG_ERR_UNSUPPORTED),              # not a multiple of 8
    (dict(M=16384, tm=256, tn=256, tk=64), ag.AG_ERR_UNSUPPORTED),   # no 256x256 kernel for this layout
    (dict(ldb=1 << 24, N=8), ag.AG_ERR_UNSUPPORTED),      # one 64-row K stage spans 2 GiB
    (dict(layout=5), ag.AG_ERR_INVALID_ARG),
    (dict(b=SLAB + 512), ag.AG_ERR_INVALID_ARG),         # B inside an output block
])
def test_gemm_plan_n_contiguous_rejects(over, status):
    got, msg = status_of(gplan_ex, **over)
    assert got == status, (over, got, msg)


def test_gemm_plan_n_contiguous_b_may_exceed_2_gib():
    # each K stage gets its own descriptor: only 64 rows of B need 32-bit offsets
    g = geom(bytes_per_rank=1 << 30)
    assert status_of(gplan_ex, g=g, K=65536, lda=65536, ldb=32768, N=32768, b=SLAB + (64 << 30))[0] == ag.AG_OK
    assert status_of(gplan_ex, g=g, ldb=(1 << 24) - 128, N=8)[0] == ag.AG_OK


def test_gemm_plan_n_contiguous_b_extent_is_k_rows():
    # the overlap check covers (K-1)*ldb + N elements of B: a B that ends just before an output block is fine
    g = geom(bytes_per_rank=1 << 30)
    b_bytes = ((8192 - 1) * 3584 + 3584) * 2
    assert status_of(gplan_ex, g=g, b=SLAB - b_bytes)[0] == ag.AG_OK
    assert status_of(gplan_ex, g=g, b=SLAB - b_bytes + 16)[0] == ag.AG_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# tile order of the all-gather's tile schedule: grid stride or tickets
# ---------------------------------------------------------------------------

BIG = dict(M=16384, N=8192)


def _big_geom(e=2, **kw):
    return geom(bytes_per_rank=8 * 16384 * 8192 * e + MiB, **kw)


@pytest.mark.parametrize("progs,ticket,wait", [(256, 3, 1), (0, 3, 1), (512, 3, 1), (192, 4, 1), (191, 4, 0),
                                                (129, 4, 0), (128, 8, 0), (96, 8, 0), (65, 8, 0), (64, 16, 0),
                                                (32, 16, 0)])
def test_plan_tickets_for_long_calls(progs, ticket, wait):
    p = plan(g=_big_geom(), progs=progs, **BIG)
    assert p.tile_order == ag.AG_ORDER_TICKETS and p.tiles_per_ticket == ticket
    assert p.threads == 256 and p.n_programs == (progs or 256)
    assert p.total_tiles == 2048 * 32 and p.vectors_per_thread == 1
    assert p.ticket_wait == wait               # from three quarters of the CUs (192 of 256): drained tickets
    # tiles per ticket: the largest of 16, 8, 4 whose tickets over all programs span at most 1024 tiles
    # (from one program per CU, 3: 12 KiB of 8x256 fp16 tiles, 108 KiB of HBM traffic per ticket at W=8)
    assert p.tiles_per_ticket * p.n_programs <= 1024 or p.tiles_per_ticket <= 4


# every ticket moves at least 96 KiB of HBM traffic (its tiles read once and written W times): one
# counter hands out about one ticket per 12 ns, which bounds small-W calls with small tickets
@pytest.mark.parametrize("W,start,stride,dtype,progs,ticket", [
    (8, 0, 1, "f16", 256, 3), (7, 0, 1, "f16", 256, 3), (6, 0, 1, "f16", 256, 4), (5, 0, 1, "f16", 256, 4),
    (4, 1, 2, "f16", 256, 8), (4, 0, 1, "f16", 192, 8), (3, 0, 1, "f16", 256, 8), (2, 0, 1, "f16", 256, 8),
    (1, 0, 1, "f16", 256, 16), (1, 0, 1, "f16", 128, 16), (2, 0, 1, "f16", 64, 16),
    (8, 0, 1, "f32", 256, 2), (4, 1, 2, "f32", 256, 4), (2, 0, 1, "f32", 256, 4), (1, 0, 1, "f32", 256, 8),
    (4, 0, 1, "f32", 128, 8)])
def test_plan_tiles_per_ticket_move_96_kib(W, start, stride, dtype, progs, ticket):
    e = 4 if dtype == "f32" else 2
    p = plan(g=_big_geom(e=e, rank=start), W=W, start=start, stride=stride, dtype=dtype, progs=progs, **BIG)
    assert p.tile_order == ag.AG_ORDER_TICKETS and p.tiles_per_ticket == ticket
    tile_bytes = 8 * 256 * e
    # at least 96 KiB per ticket wherever a ticket kernel that large exists
    assert ticket * tile_bytes * (1 + W) >= 96 << 10 or ticket == (8 if e == 4 else 16)


@pytest.mark.parametrize("progs,wait", [(256, 1), (128, 1), (96, 1), (95, 0), (64, 0)])
def test_plan_ticket_wait_with_two_vectors_per_thread(progs, wait):
    p = plan(g=_big_geom(e=4), dtype="f32", progs=progs, **BIG)   # 8x256 fp32: two 16-byte vectors
    assert p.vectors_per_thread == 2 and p.tile_order == ag.AG_ORDER_TICKETS
    assert p.ticket_wait == wait               # programs x vectors from three quarters of the CUs


def test_plan_no_tickets_past_2gib_of_tile_rows():
    # 16384 x 32768 fp32 per rank: 2 GiB of input, beyond the ticket kernel's 32-bit tile offsets
    g = geom(bytes_per_rank=8 * 16384 * 32768 * 4 + MiB)
    p = plan(g=g, dtype="f32", progs=256, M=16384, N=32768)
    assert p.tile_order == ag.AG_ORDER_STRIDE
    with pytest.raises(ag.AgError) as exc:
        ag.plan_all_gather_ex(g, 8, 0, 1, INPUT, 0, 16384, 32768, "f32", 0, 0, 256, tile_order="tickets")
    assert exc.value.status == ag.AG_ERR_UNSUPPORTED


def test_plan_tickets_two_vectors_per_thread_at_most_eight():
    p = plan(g=_big_geom(e=4), dtype="f32", progs=64, **BIG)       # 8x256 fp32: two 16-byte vectors
    assert p.vectors_per_thread == 2 and p.tile_order == ag.AG_ORDER_TICKETS and p.tiles_per_ticket == 8
    p = plan(g=_big_geom(), tm=16, tn=512, progs=256, **BIG)        # four vectors per thread: no ticket kernel
    assert p.vectors_per_thread == 4 and p.tile_order == ag.AG_ORDER_STRIDE and p.tiles_per_ticket == 0


def test_plan_short_calls_keep_the_grid_stride():
    p = plan(progs=128)                                            # 1024x4096: 16 tiles per program
    assert p.tile_order == ag.AG_ORDER_STRIDE and p.tiles_per_ticket == 0
    p = ag.plan_all_gather_ex(geom(), 8, 0, 1, INPUT, 0, 1024, 4096, "f16", 0, 0, 128, tile_order="tickets")
    assert p.tile_order == ag.AG_ORDER_TICKETS and p.tiles_per_ticket == 8 and p.n_programs == 128
    p = ag.plan_all_gather_ex(_big_geom(), 8, 0, 1, INPUT, 0, 16384, 8192, "f16", 0, 0, 64, tile_order="stride")
    assert p.tile_order == ag.AG_ORDER_STRIDE and p.threads == 1024      # narrow launch: four slices


def test_plan_ticket_grid_is_capped_by_tickets():
    p = ag.plan_all_gather_ex(geom(), 8, 0, 1, INPUT, 0, 64, 256, "f16", 8, 256, 256, tile_order="tickets")
    assert p.total_tiles == 8 and p.tiles_per_ticket == 3 and p.n_programs == 3     # ceil(8 / 3) tickets


@pytest.mark.parametrize("kw,status", [
    (dict(tile_order="tickets", dest_group=2), ag.AG_ERR_UNSUPPORTED),
    (dict(tile_order="tickets", schedule="partitioned"), ag.AG_ERR_INVALID_ARG),
    (dict(tile_order="stride", schedule="partitioned"), ag.AG_ERR_INVALID_ARG),
    (dict(tile_order=3), ag.AG_ERR_INVALID_ARG),
])
def test_plan_tile_order_rejects(kw, status):
    got, _ = status_of(ag.plan_all_gather_ex, geom(), 8, 0, 1, INPUT, 0, 1024, 4096, "f16", 0, 0, 0, **kw)
    assert got == status


def test_plan_tickets_need_16_byte_vectors():
    # an input 8 bytes off 16-byte alignment gives 8-byte vectors: no ticket kernel
    got, msg = status_of(ag.plan_all_gather_ex, geom(), 8, 0, 1, INPUT + 8, 0, 1024, 4096, "f16", 0, 0, 0,
                         tile_order="tickets")
    assert got == ag.AG_ERR_UNSUPPORTED and "ticket" in msg
    p = ag.plan_all_gather(_big_geom(), 8, 0, 1, INPUT + 8, 0, 16384, 8192, "f16", 0, 0, 256)
    assert p.vec_bytes == 8 and p.tile_order == ag.AG_ORDER_STRIDE


def test_plan_all_to_all_tile_order():
    """The all-to-all's W chunk copies are one sequence of W x (tiles per chunk) tiles shared by the
    programs; in ticket order each tile moves its bytes twice (read, write), so 96 KiB of traffic per
    ticket is 16 tiles of 8x256 fp16 and 8 of 8x512."""
    p = ag.plan_all_to_all_ex(geom(), 8, 0, 1, INPUT, 0, 128, 4096, "f16", 0, 0, 0, tile_order="tickets")
    assert p.tile_order == ag.AG_ORDER_TICKETS and p.tiles_per_ticket == 16
    assert p.total_tiles == 16 * 16 and p.n_programs == 8 * 16 * 16 // 16
    p = ag.plan_all_to_all_ex(geom(), 8, 0, 1, INPUT, 0, 128, 4096, "f16", 8, 512, 0, tile_order="tickets")
    assert p.vectors_per_thread == 2 and p.tiles_per_ticket == 8 and p.n_programs == 8 * 16 * 8 // 8
    p = ag.plan_all_to_all_ex(geom(), 8, 0, 1, INPUT, 0, 128, 4096, "f16", 0, 0, 0, tile_order="stride")
    assert p.tile_order == ag.AG_ORDER_STRIDE and p.n_programs == 256
    # the library's choice: tickets where programs x vectors per thread stay below twice the CU count and
    # there are 64 tiles of the sequence per program and vector
    big = geom(bytes_per_rank=8 * 2048 * 8192 * 2 + MiB)
    for M, N, g, tile, progs, want in ((1024, 4096, geom(), (8, 512), 256, 0), (1024, 4096, geom(), (8, 512), 128, 0),
                                       (1024, 4096, geom(), (8, 512), 64, 8), (1024, 4096, geom(), (8, 256), 192, 16),
                                       (2048, 8192, big, (8, 512), 256, 0), (2048, 8192, big, (8, 512), 192, 8),
                                       (2048, 8192, big, (8, 512), 128, 8), (2048, 8192, big, (8, 256), 256, 16)):
        p = ag.plan_all_to_all(g, 8, 0, 1, INPUT, 0, M, N, "f16", *tile, progs)
        assert p.tiles_per_ticket == want, (M, tile, progs, p.tiles_per_ticket)
        assert p.tile_order == (ag.AG_ORDER_TICKETS if want else ag.AG_ORDER_STRIDE)
    for kw in (dict(schedule="partitioned"), dict(dest_group=2)):
        got, _ = status_of(ag.plan_all_to_all_ex, geom(), 8, 0, 1, INPUT, 0, 128, 4096, "f16", 0, 0, 0,
                           tile_order="tickets", **kw)
        assert got == ag.AG_ERR_INVALID_ARG
