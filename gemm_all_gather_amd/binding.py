"""ctypes binding of libag (include/ag.h): argument marshalling only.

Every function here forwards to the C ABI of the same name; all work on the
device happens in the library's HIP kernels.  There is no fallback: if
libag.so is missing or fails to load, every call raises.

Device memory and streams come from PyTorch (a torch uint8 tensor can serve
as the heap's slab via ``Heap.wrap``); pointers are passed as integers.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libag.so")

AG_OK, AG_ERR_INVALID_ARG, AG_ERR_UNSUPPORTED, AG_ERR_OUT_OF_MEMORY, AG_ERR_HIP = range(5)
STATUS_NAMES = {0: "AG_OK", 1: "AG_ERR_INVALID_ARG", 2: "AG_ERR_UNSUPPORTED",
                3: "AG_ERR_OUT_OF_MEMORY", 4: "AG_ERR_HIP"}
AG_F16, AG_BF16, AG_F32 = 0, 1, 2
DTYPE_CODES = {"f16": AG_F16, "bf16": AG_BF16, "f32": AG_F32}
ELEM_BYTES = {"f16": 2, "bf16": 2, "f32": 4}
AG_MAX_WORLD = 8
AG_NOALLOC_MAX_RANKS = 64
AG_REGION_ALIGN = 2 << 20


class AgError(RuntimeError):
    def __init__(self, status: int, message: str, call: str):
        self.status = status
        self.message = message
        super().__init__(f"{call}: {STATUS_NAMES.get(status, status)}: {message}")


class Geometry(ctypes.Structure):
    _fields_ = [("slab_addr", ctypes.c_uint64), ("bytes_per_rank", ctypes.c_uint64),
                ("n_ranks", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("group_rank", ctypes.c_int32), ("vec_bytes", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("n_programs", ctypes.c_int32), ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("vectors_per_thread", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64), ("total_tiles", ctypes.c_int64),
                ("rank_block_offset", ctypes.c_uint64), ("bytes_read", ctypes.c_uint64),
                ("bytes_written", ctypes.c_uint64), ("flops", ctypes.c_double),
                ("dest_group", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("tile_order", ctypes.c_int32), ("tiles_per_ticket", ctypes.c_int32),
                ("ticket_wait", ctypes.c_int32), ("reserved_plan", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


AG_SCHEDULE_TILES, AG_SCHEDULE_PARTITIONED = 0, 1
SCHEDULES = {"tiles": AG_SCHEDULE_TILES, "partitioned": AG_SCHEDULE_PARTITIONED}
AG_ORDER_AUTO, AG_ORDER_STRIDE, AG_ORDER_TICKETS = 0, 1, 2
TILE_ORDERS = {"auto": AG_ORDER_AUTO, "stride": AG_ORDER_STRIDE, "tickets": AG_ORDER_TICKETS}
AG_B_K_CONTIGUOUS, AG_B_N_CONTIGUOUS = 0, 1
B_LAYOUTS = {"k": AG_B_K_CONTIGUOUS, "n": AG_B_N_CONTIGUOUS}


class CopyOptions(ctypes.Structure):
    _fields_ = [("dest_group", ctypes.c_int32), ("schedule", ctypes.c_int32), ("tile_order", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 5)]


class GemmOptions(ctypes.Structure):
    _fields_ = [("b_layout", ctypes.c_int32), ("reserved", ctypes.c_int32 * 7)]


def _options(dest_group=0, schedule=0, tile_order=0) -> CopyOptions:
    o = CopyOptions()
    o.dest_group = dest_group
    o.schedule = SCHEDULES[schedule] if isinstance(schedule, str) else schedule
    o.tile_order = TILE_ORDERS[tile_order] if isinstance(tile_order, str) else tile_order
    return o


_lib: Optional[ctypes.CDLL] = None

_c_int, _c_size, _c_i64, _c_u64, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
_HEAP_PP = ctypes.POINTER(ctypes.c_void_p)

_SIGNATURES = {
    "ag_heap_region_bytes": [_c_size, ctypes.POINTER(ctypes.c_size_t)],
    "ag_heap_create": [_c_int, _c_size, _HEAP_PP],
    "ag_heap_wrap": [_vp, _c_int, _c_size, _HEAP_PP],
    "ag_heap_view": [_vp, _c_int, _HEAP_PP],
    "ag_heap_destroy": [_vp],
    "ag_heap_alloc": [_vp, _c_size, _c_size, ctypes.POINTER(ctypes.c_size_t)],
    "ag_heap_reset": [_vp],
    "ag_heap_rank_ptr": [_vp, _c_int, _c_size, ctypes.POINTER(ctypes.c_void_p)],
    "ag_heap_base_table": [_vp, ctypes.POINTER(ctypes.c_void_p)],
    "ag_heap_geometry": [_vp, ctypes.POINTER(Geometry)],
    "ag_heap_info": [_vp, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                     ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_void_p)],
    "ag_heap_clear_tickets": [_vp, _vp],
    "ag_all_gather": [_vp, _c_int, _c_int, _c_int, _vp, _c_size, _c_i64, _c_i64, _c_int, _c_int, _c_int,
                      _c_int, _vp],
    "ag_plan_all_gather": [ctypes.POINTER(Geometry), _c_int, _c_int, _c_int, _c_u64, _c_size, _c_i64, _c_i64,
                           _c_int, _c_int, _c_int, _c_int, ctypes.POINTER(Plan)],
    "ag_all_gather_ex": [_vp, _c_int, _c_int, _c_int, _vp, _c_size, _c_i64, _c_i64, _c_int, _c_int, _c_int,
                         _c_int, ctypes.POINTER(CopyOptions), _vp],
    "ag_plan_all_gather_ex": [ctypes.POINTER(Geometry), _c_int, _c_int, _c_int, _c_u64, _c_size, _c_i64, _c_i64,
                              _c_int, _c_int, _c_int, _c_int, ctypes.POINTER(CopyOptions), ctypes.POINTER(Plan)],
    "ag_all_gather_noalloc": [_vp, _c_int, _c_int, _c_int, _vp, _c_size, _c_i64, _c_i64, _c_int, _c_int, _c_int,
                              _c_int, ctypes.POINTER(CopyOptions), _vp],
    "ag_all_to_all": [_vp, _c_int, _c_int, _c_int, _vp, _c_size, _c_i64, _c_i64, _c_int, _c_int, _c_int,
                      _c_int, _vp],
    "ag_plan_all_to_all": [ctypes.POINTER(Geometry), _c_int, _c_int, _c_int, _c_u64, _c_size, _c_i64, _c_i64,
                           _c_int, _c_int, _c_int, _c_int, ctypes.POINTER(Plan)],
    "ag_all_to_all_ex": [_vp, _c_int, _c_int, _c_int, _vp, _c_size, _c_i64, _c_i64, _c_int, _c_int, _c_int,
                         _c_int, ctypes.POINTER(CopyOptions), _vp],
    "ag_plan_all_to_all_ex": [ctypes.POINTER(Geometry), _c_int, _c_int, _c_int, _c_u64, _c_size, _c_i64, _c_i64,
                              _c_int, _c_int, _c_int, _c_int, ctypes.POINTER(CopyOptions), ctypes.POINTER(Plan)],
    "ag_gemm_all_gather": [_vp, _c_int, _c_int, _c_int, _vp, _c_i64, _vp, _c_i64, _c_size, _c_i64, _c_i64,
                           _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int, _vp],
    "ag_plan_gemm_all_gather": [ctypes.POINTER(Geometry), _c_int, _c_int, _c_int, _c_u64, _c_i64, _c_u64, _c_i64,
                                _c_size, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int,
                                ctypes.POINTER(Plan)],
    "ag_gemm_all_gather_ex": [_vp, _c_int, _c_int, _c_int, _vp, _c_i64, _vp, _c_i64, _c_size, _c_i64, _c_i64,
                              _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int, ctypes.POINTER(GemmOptions), _vp],
    "ag_plan_gemm_all_gather_ex": [ctypes.POINTER(Geometry), _c_int, _c_int, _c_int, _c_u64, _c_i64, _c_u64,
                                   _c_i64, _c_size, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   ctypes.POINTER(GemmOptions), ctypes.POINTER(Plan)],
}


def lib() -> ctypes.CDLL:
    """The loaded libag.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gemm_all_gather_amd.build` "
                               "(there is no fallback implementation)")
        l = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        for name in ("ag_status_string", "ag_last_error_message", "ag_version"):
            getattr(l, name).restype = ctypes.c_char_p
        l.ag_status_string.argtypes = [ctypes.c_int]
        _lib = l
    return _lib


def _check(status: int, call: str) -> None:
    if status != AG_OK:
        msg = lib().ag_last_error_message().decode()
        raise AgError(status, msg, call)


def version() -> str:
    return lib().ag_version().decode()


def heap_region_bytes(bytes_per_rank: int) -> int:
    """The region stride ag_heap_create uses for bytes_per_rank (the layout to give ag_heap_wrap too)."""
    out = ctypes.c_size_t(0)
    _check(lib().ag_heap_region_bytes(bytes_per_rank, ctypes.byref(out)), "ag_heap_region_bytes")
    return out.value


def _ptr(x) -> int:
    """Integer device address of a tensor (data_ptr) or an int."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _dtype(d) -> int:
    if isinstance(d, int):
        return d
    if isinstance(d, str):
        return DTYPE_CODES[d]
    import torch
    return {torch.float16: AG_F16, torch.bfloat16: AG_BF16, torch.float32: AG_F32}[d]


class Heap:
    """A handle of the symmetric heap: the root (rank -1) or a view of one rank."""

    def __init__(self, handle: int, keepalive=None):
        self._h = ctypes.c_void_p(handle)
        self._keepalive = keepalive

    @classmethod
    def create(cls, n_ranks: int, bytes_per_rank: int) -> "Heap":
        h = ctypes.c_void_p()
        _check(lib().ag_heap_create(n_ranks, bytes_per_rank, ctypes.byref(h)), "ag_heap_create")
        return cls(h.value)

    @classmethod
    def wrap(cls, slab, n_ranks: int, bytes_per_rank: int) -> "Heap":
        """Heap over caller memory (a device tensor of n_ranks*bytes_per_rank bytes, kept alive here)."""
        h = ctypes.c_void_p()
        _check(lib().ag_heap_wrap(_ptr(slab), n_ranks, bytes_per_rank, ctypes.byref(h)), "ag_heap_wrap")
        return cls(h.value, keepalive=slab)

    def view(self, rank: int) -> "Heap":
        h = ctypes.c_void_p()
        _check(lib().ag_heap_view(self._h, rank, ctypes.byref(h)), "ag_heap_view")
        return Heap(h.value, keepalive=self)

    def destroy(self) -> None:
        if self._h is not None and self._h.value:
            lib().ag_heap_destroy(self._h)
        self._h = None

    close = destroy

    def __del__(self):
        try:
            if self._h is not None and self._h.value and _lib is not None:
                _lib.ag_heap_destroy(self._h)
                self._h = None
        except Exception:
            pass

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise RuntimeError("heap handle already destroyed")
        return self._h

    def alloc(self, nbytes: int, align: int = 256) -> int:
        off = ctypes.c_size_t()
        _check(lib().ag_heap_alloc(self.handle, nbytes, align, ctypes.byref(off)), "ag_heap_alloc")
        return off.value

    def reset(self) -> None:
        _check(lib().ag_heap_reset(self.handle), "ag_heap_reset")

    def rank_ptr(self, rank: int, offset: int = 0) -> int:
        p = ctypes.c_void_p()
        _check(lib().ag_heap_rank_ptr(self.handle, rank, offset, ctypes.byref(p)), "ag_heap_rank_ptr")
        return p.value or 0

    def base_table(self) -> int:
        p = ctypes.c_void_p()
        _check(lib().ag_heap_base_table(self.handle, ctypes.byref(p)), "ag_heap_base_table")
        return p.value or 0

    def geometry(self) -> Geometry:
        g = Geometry()
        _check(lib().ag_heap_geometry(self.handle, ctypes.byref(g)), "ag_heap_geometry")
        return g

    def info(self) -> dict:
        """ag_heap_info: n_ranks, rank (-1 for the root handle), bytes_per_rank, base_table (device address)."""
        n, r, s, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t(), ctypes.c_void_p()
        _check(lib().ag_heap_info(self.handle, ctypes.byref(n), ctypes.byref(r), ctypes.byref(s), ctypes.byref(t)),
               "ag_heap_info")
        return {"n_ranks": n.value, "rank": r.value, "bytes_per_rank": s.value, "base_table": t.value or 0}

    def clear_tickets(self, stream=None) -> None:
        """ag_heap_clear_tickets: zero every rank's tile counters on stream."""
        _check(lib().ag_heap_clear_tickets(self.handle, _stream(stream)), "ag_heap_clear_tickets")


def plan_all_gather(geom: Geometry, W, rank_start, rank_stride, input_addr, out_offset, M_local, N, dtype,
                    tile_m=0, tile_n=0, n_programs=0) -> Plan:
    p = Plan()
    _check(lib().ag_plan_all_gather(ctypes.byref(geom), W, rank_start, rank_stride, _ptr(input_addr), out_offset,
                                    M_local, N, _dtype(dtype), tile_m, tile_n, n_programs, ctypes.byref(p)),
           "ag_plan_all_gather")
    return p


def all_gather(heap: Heap, W, rank_start, rank_stride, input, out_offset, M_local, N, dtype,
               tile_m=0, tile_n=0, n_programs=0, stream=None) -> None:
    _check(lib().ag_all_gather(heap.handle, W, rank_start, rank_stride, _ptr(input), out_offset, M_local, N,
                               _dtype(dtype), tile_m, tile_n, n_programs, _stream(stream)), "ag_all_gather")


def plan_all_gather_ex(geom: Geometry, W, rank_start, rank_stride, input_addr, out_offset, M_local, N, dtype,
                       tile_m=0, tile_n=0, n_programs=0, dest_group=0, schedule=0, tile_order=0) -> Plan:
    p = Plan()
    o = _options(dest_group, schedule, tile_order)
    _check(lib().ag_plan_all_gather_ex(ctypes.byref(geom), W, rank_start, rank_stride, _ptr(input_addr), out_offset,
                                       M_local, N, _dtype(dtype), tile_m, tile_n, n_programs, ctypes.byref(o),
                                       ctypes.byref(p)), "ag_plan_all_gather_ex")
    return p


def all_gather_ex(heap: Heap, W, rank_start, rank_stride, input, out_offset, M_local, N, dtype,
                  tile_m=0, tile_n=0, n_programs=0, dest_group=0, schedule=0, stream=None, tile_order=0) -> None:
    o = _options(dest_group, schedule, tile_order)
    _check(lib().ag_all_gather_ex(heap.handle, W, rank_start, rank_stride, _ptr(input), out_offset, M_local, N,
                                  _dtype(dtype), tile_m, tile_n, n_programs, ctypes.byref(o), _stream(stream)),
           "ag_all_gather_ex")


def all_gather_noalloc(heap: Heap, W, rank_start, rank_stride, input, out_offset, M_local, N, dtype,
                       tile_m=0, tile_n=0, n_programs=0, dest_group=0, schedule=0, stream=None,
                       tile_order=0) -> None:
    """ag_all_gather_noalloc: ag_all_gather_ex whose tile counter is the library's fixed device array."""
    o = _options(dest_group, schedule, tile_order)
    _check(lib().ag_all_gather_noalloc(heap.handle, W, rank_start, rank_stride, _ptr(input), out_offset, M_local, N,
                                       _dtype(dtype), tile_m, tile_n, n_programs, ctypes.byref(o), _stream(stream)),
           "ag_all_gather_noalloc")


def plan_all_to_all(geom: Geometry, W, rank_start, rank_stride, input_addr, out_offset, M_chunk, N, dtype,
                    tile_m=0, tile_n=0, n_programs=0) -> Plan:
    p = Plan()
    _check(lib().ag_plan_all_to_all(ctypes.byref(geom), W, rank_start, rank_stride, _ptr(input_addr), out_offset,
                                    M_chunk, N, _dtype(dtype), tile_m, tile_n, n_programs, ctypes.byref(p)),
           "ag_plan_all_to_all")
    return p


def all_to_all(heap: Heap, W, rank_start, rank_stride, input, out_offset, M_chunk, N, dtype,
               tile_m=0, tile_n=0, n_programs=0, stream=None) -> None:
    _check(lib().ag_all_to_all(heap.handle, W, rank_start, rank_stride, _ptr(input), out_offset, M_chunk, N,
                               _dtype(dtype), tile_m, tile_n, n_programs, _stream(stream)), "ag_all_to_all")


def plan_all_to_all_ex(geom: Geometry, W, rank_start, rank_stride, input_addr, out_offset, M_chunk, N, dtype,
                       tile_m=0, tile_n=0, n_programs=0, dest_group=0, schedule=0, tile_order=0) -> Plan:
    p = Plan()
    o = _options(dest_group, schedule, tile_order)
    _check(lib().ag_plan_all_to_all_ex(ctypes.byref(geom), W, rank_start, rank_stride, _ptr(input_addr), out_offset,
                                       M_chunk, N, _dtype(dtype), tile_m, tile_n, n_programs, ctypes.byref(o),
                                       ctypes.byref(p)), "ag_plan_all_to_all_ex")
    return p


def all_to_all_ex(heap: Heap, W, rank_start, rank_stride, input, out_offset, M_chunk, N, dtype,
                  tile_m=0, tile_n=0, n_programs=0, dest_group=0, schedule=0, stream=None, tile_order=0) -> None:
    o = _options(dest_group, schedule, tile_order)
    _check(lib().ag_all_to_all_ex(heap.handle, W, rank_start, rank_stride, _ptr(input), out_offset, M_chunk, N,
                                  _dtype(dtype), tile_m, tile_n, n_programs, ctypes.byref(o), _stream(stream)),
           "ag_all_to_all_ex")


def plan_gemm_all_gather(geom: Geometry, W, rank_start, rank_stride, a_addr, lda, b_addr, ldb, out_offset,
                         M_local, N, K, dtype, tile_m=0, tile_n=0, tile_k=0, n_programs=0) -> Plan:
    p = Plan()
    _check(lib().ag_plan_gemm_all_gather(ctypes.byref(geom), W, rank_start, rank_stride, _ptr(a_addr), lda,
                                         _ptr(b_addr), ldb, out_offset, M_local, N, K, _dtype(dtype), tile_m,
                                         tile_n, tile_k, n_programs, ctypes.byref(p)), "ag_plan_gemm_all_gather")
    return p


def gemm_all_gather(heap: Heap, W, rank_start, rank_stride, A, lda, B, ldb, out_offset, M_local, N, K, dtype,
                    tile_m=0, tile_n=0, tile_k=0, n_programs=0, stream=None) -> None:
    _check(lib().ag_gemm_all_gather(heap.handle, W, rank_start, rank_stride, _ptr(A), lda, _ptr(B), ldb,
                                    out_offset, M_local, N, K, _dtype(dtype), tile_m, tile_n, tile_k, n_programs,
                                    _stream(stream)), "ag_gemm_all_gather")


def _gemm_options(b_layout=0) -> GemmOptions:
    o = GemmOptions()
    o.b_layout = B_LAYOUTS[b_layout] if isinstance(b_layout, str) else b_layout
    return o


def plan_gemm_all_gather_ex(geom: Geometry, W, rank_start, rank_stride, a_addr, lda, b_addr, ldb, out_offset,
                            M_local, N, K, dtype, tile_m=0, tile_n=0, tile_k=0, n_programs=0, b_layout=0) -> Plan:
    """b_layout: "k" (element (k,n) at B[n*ldb + k]) or "n" (at B[k*ldb + n])."""
    p = Plan()
    o = _gemm_options(b_layout)
    _check(lib().ag_plan_gemm_all_gather_ex(ctypes.byref(geom), W, rank_start, rank_stride, _ptr(a_addr), lda,
                                            _ptr(b_addr), ldb, out_offset, M_local, N, K, _dtype(dtype), tile_m,
                                            tile_n, tile_k, n_programs, ctypes.byref(o), ctypes.byref(p)),
           "ag_plan_gemm_all_gather_ex")
    return p


def gemm_all_gather_ex(heap: Heap, W, rank_start, rank_stride, A, lda, B, ldb, out_offset, M_local, N, K, dtype,
                       tile_m=0, tile_n=0, tile_k=0, n_programs=0, b_layout=0, stream=None) -> None:
    o = _gemm_options(b_layout)
    _check(lib().ag_gemm_all_gather_ex(heap.handle, W, rank_start, rank_stride, _ptr(A), lda, _ptr(B), ldb,
                                       out_offset, M_local, N, K, _dtype(dtype), tile_m, tile_n, tile_k, n_programs,
                                       ctypes.byref(o), _stream(stream)), "ag_gemm_all_gather_ex")
