"""Python binding of libkvdec (ctypes).  Argument marshalling only: every step
of the computation runs in the HIP library.  torch tensors supply device
memory and streams; numpy arrays supply host-side cell lists.

Importing this module loads ``libkvdec.so`` from the package directory and
raises ImportError if it has not been built (``python -m
long_context_decode_kv_amd.build``).  There is no fallback path.
"""

import ctypes
import os

import numpy as np

# torch is imported before the library is loaded so that libkvdec binds to
# the HIP runtime torch already holds (both carry the soname
# libamdhip64.so.7): device pointers and stream handles then come from the
# same runtime instance the kernels are launched through.
import torch  # noqa: F401

from long_context_decode_kv_amd.build import source_hash as _source_hash

# KVDEC_LIB_NAME selects a test build: libkvdec_fi.so (host-side failure
# injection, kvdec_fi_configure), libkvdec_trace.so (phase stamps of the
# one-shot kernel, kvdec_trace_configure) or libkvdec_san.so (planner and validation
# under ASan / UBSan); the product library otherwise
_LIB_NAME = os.environ.get("KVDEC_LIB_NAME", "libkvdec.so")
if _LIB_NAME not in ("libkvdec.so", "libkvdec_fi.so", "libkvdec_trace.so", "libkvdec_san.so"):
    raise ImportError(f"KVDEC_LIB_NAME={_LIB_NAME}: not a build of this package")
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), _LIB_NAME)
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run: python -m long_context_decode_kv_amd.build")
lib = ctypes.CDLL(_LIB_PATH)
LIB_PATH = _LIB_PATH
lib.kvdec_source_hash.argtypes = []
lib.kvdec_source_hash.restype = ctypes.c_char_p
LIB_SOURCE_HASH = lib.kvdec_source_hash().decode()
# a library built from other sources than the ones beside it is never used
if LIB_SOURCE_HASH != _source_hash():
    raise ImportError(f"{_LIB_PATH} was built from other sources (library {LIB_SOURCE_HASH}, sources "
                      f"{_source_hash()}); rebuild: python -m long_context_decode_kv_amd.build")

F16, Q8_B32, Q4_B32 = 0, 1, 2
OK, E_INVALID, E_RANGE, E_UNSUPPORTED, E_WORKSPACE, E_NOMEM, E_DEVICE = 0, -1, -2, -3, -4, -5, -6
TILE_CELLS = 128
KERNEL_AUTO, KERNEL_STREAMED, KERNEL_ONESHOT = 0, 1, 2
MAX_SLOTS = 64

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class Problem(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32), ("n_slots", _i32),
        ("k_type", _i32), ("v_type", _i32), ("scale", ctypes.c_float), ("tiles_per_split", _i32),
        ("capacity_cells", _i64),
        ("cell_begin", _p), ("n_occupied", _p), ("cells", _p), ("cells_off", _p),
        ("tail_begin", _p), ("n_tail", _p),
        ("tail_capacity_cells", _i64), ("tail_chunk_cells", _i64),
        ("tail_ring_depth", _i32), ("n_queries", _i32), ("tail_zero_copy", _i32), ("split_cells", _i32),
        ("max_records", _p), ("kernel", _i32), ("pad0", _i32),
    ]


class IO(ctypes.Structure):
    _fields_ = [
        ("q", _p), ("k", _p), ("v", _p), ("k_scales", _p), ("v_scales", _p),
        ("k_cell_stride", _i64), ("k_head_stride", _i64), ("v_cell_stride", _i64), ("v_head_stride", _i64),
        ("plan_cells", _p),
        ("k_tail", _p), ("v_tail", _p), ("k_tail_scales", _p), ("v_tail_scales", _p),
        ("out", _p), ("lse", _p), ("part_m", _p), ("part_l", _p), ("part_o", _p),
        ("q_pos", _p), ("cell_pos", _p), ("copy_after", _p), ("live_records", _p),
    ]


class PartialC(ctypes.Structure):
    _fields_ = [("m", _p), ("l", _p), ("o", _p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("n_slots", _i32), ("group", _i32), ("n_workgroups", _i32), ("tiles_per_split", _i32),
        ("n_tiles", _i64), ("n_entries", _i64), ("n_tail_chunks", _i64), ("workspace_bytes", _i64),
        ("n_queries", _i32), ("matrix_cores", _i32), ("split_cells", _i32), ("split_unit", _i32),
        ("waves", _i32), ("kernel", _i32), ("split_interleave", _i32), ("ticket_bytes", _i64),
    ]


lib.kvdec_plan.argtypes = [ctypes.POINTER(Problem), _i32, ctypes.POINTER(_p), ctypes.POINTER(ctypes.c_size_t)]
lib.kvdec_plan.restype = ctypes.c_int
lib.kvdec_plan_cells.argtypes = [_p, _p, _p, ctypes.POINTER(_i64)]
lib.kvdec_plan_cells.restype = ctypes.c_int
lib.kvdec_plan_get_info.argtypes = [_p, ctypes.POINTER(PlanInfo)]
lib.kvdec_plan_get_info.restype = ctypes.c_int
lib.kvdec_plan_splits.argtypes = [_p, _p, ctypes.POINTER(_i64)]
lib.kvdec_plan_splits.restype = ctypes.c_int
lib.kvdec_plan_free.argtypes = [_p]
lib.kvdec_plan_free.restype = None
lib.kvdec_attend.argtypes = [_p, ctypes.POINTER(IO), _p, ctypes.c_size_t, _p, _p]
lib.kvdec_attend.restype = ctypes.c_int
lib.kvdec_attend_static.argtypes = [_p, ctypes.POINTER(IO), _p]
lib.kvdec_attend_static.restype = ctypes.c_int
lib.kvdec_merge.argtypes = [_i32, ctypes.POINTER(PartialC), _i64, _i32, _p, _p, _p, _p, _p, _p]
lib.kvdec_merge.restype = ctypes.c_int
lib.kvdec_build_cells.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
lib.kvdec_build_cells.restype = ctypes.c_int
lib.kvdec_strerror.argtypes = [ctypes.c_int]
lib.kvdec_strerror.restype = ctypes.c_char_p
lib.kvdec_last_error.argtypes = []
lib.kvdec_last_error.restype = ctypes.c_char_p
lib.kvdec_version.argtypes = []
lib.kvdec_version.restype = ctypes.c_int

EXPORTED = [
    "kvdec_plan", "kvdec_plan_cells", "kvdec_plan_get_info", "kvdec_plan_splits", "kvdec_plan_free",
    "kvdec_attend", "kvdec_merge", "kvdec_build_cells", "kvdec_strerror", "kvdec_last_error", "kvdec_version",
    "kvdec_source_hash", "kvdec_attend_static",
]

# merge-ticket area at the start of a workspace (one 128-byte line per ticket)
TICKET_AREA_BYTES = 1024 * 1024
# capacity of the library's static scratch array (kvdec_attend_static)
STATIC_TICKET_BYTES = 1024 * 1024
STATIC_WORKSPACE_BYTES = 16 * 1024 * 1024


class KvdecError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib.kvdec_last_error().decode() or lib.kvdec_strerror(status).decode()
        super().__init__(f"{where}: {lib.kvdec_strerror(status).decode()} ({status}): {msg}")


def _check(status, where):
    if status != OK:
        raise KvdecError(status, where)


def _ptr(x):
    """Device or host address of a torch tensor / numpy array / int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """An immutable plan (owns the C handle)."""

    def __init__(self, handle, workspace_bytes, keep):
        self._h = handle
        self.workspace_bytes = int(workspace_bytes)
        self._keep = keep

    @property
    def handle(self):
        return self._h

    def info(self):
        inf = PlanInfo()
        _check(lib.kvdec_plan_get_info(self._h, ctypes.byref(inf)), "kvdec_plan_get_info")
        return {f: getattr(inf, f) for f, _ in PlanInfo._fields_}

    def cells(self):
        """(entries int32, offsets int64 [n_slots + 1]) of an indirect plan."""
        n = _i64()
        _check(lib.kvdec_plan_cells(self._h, None, None, ctypes.byref(n)), "kvdec_plan_cells")
        slots = self.info()["n_slots"]
        entries = np.empty(max(n.value, 1), dtype=np.int32)
        offsets = np.empty(slots + 1, dtype=np.int64)
        _check(lib.kvdec_plan_cells(self._h, entries.ctypes.data, offsets.ctypes.data, ctypes.byref(n)),
               "kvdec_plan_cells")
        return entries[:n.value], offsets

    def splits(self):
        """int64 [n_workgroups, 4]: (slot, kv head, first position, position count)."""
        n = _i64()
        _check(lib.kvdec_plan_splits(self._h, None, ctypes.byref(n)), "kvdec_plan_splits")
        out = np.empty((max(n.value, 1), 4), dtype=np.int64)
        _check(lib.kvdec_plan_splits(self._h, out.ctypes.data, ctypes.byref(n)), "kvdec_plan_splits")
        return out[:n.value]

    def close(self):
        if self._h:
            lib.kvdec_plan_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan(n_q_heads, n_kv_heads, head_dim, n_slots, capacity_cells, *, k_type=F16, v_type=F16, scale=None,
         n_occupied=None, cell_begin=None, cells=None, n_tail=None, tail_begin=None, tail_capacity_cells=0,
         tail_chunk_cells=0, tail_ring_depth=0, tiles_per_split=0, n_cu=0, n_queries=1, tail_zero_copy=False,
         max_records=None, split_cells=0, kernel=KERNEL_AUTO):
    """Build a plan.  ``cells`` is a list of per-slot raw cell arrays
    (indirect mode); otherwise ``n_occupied`` (and optional ``cell_begin``)
    give contiguous ranges.  ``n_queries`` query rows per slot.  ``n_cu=0``
    asks the current HIP device.  ``kernel`` picks the vector-ALU split
    kernel (KERNEL_AUTO, KERNEL_STREAMED, KERNEL_ONESHOT)."""
    keep = []

    def arr64(x):
        if x is None:
            return None
        a = np.ascontiguousarray(np.asarray(x, dtype=np.int64))
        keep.append(a)
        return a.ctypes.data

    p = Problem()
    p.n_q_heads, p.n_kv_heads, p.head_dim, p.n_slots = n_q_heads, n_kv_heads, head_dim, n_slots
    p.k_type, p.v_type = k_type, v_type
    # default 1/sqrt(head_dim); a head_dim the library will reject gets NaN
    p.scale = (1.0 / np.sqrt(head_dim) if head_dim > 0 else float("nan")) if scale is None else scale
    p.tiles_per_split = tiles_per_split
    p.split_cells = split_cells
    p.kernel = kernel
    p.capacity_cells = capacity_cells
    p.cell_begin = arr64(cell_begin)
    p.n_occupied = arr64(n_occupied)
    if cells is not None:
        flat = np.ascontiguousarray(np.concatenate([np.asarray(c, dtype=np.int32).ravel() for c in cells])
                                    if len(cells) else np.zeros(0, np.int32), dtype=np.int32)
        if flat.size == 0:
            flat = np.zeros(1, np.int32)  # non-null pointer for an all-empty list
            off = np.zeros(len(cells) + 1, np.int64)
        else:
            off = np.concatenate([[0], np.cumsum([len(np.asarray(c).ravel()) for c in cells])]).astype(np.int64)
        keep += [flat, off]
        p.cells = flat.ctypes.data
        p.cells_off = off.ctypes.data
    p.tail_begin = arr64(tail_begin)
    p.n_tail = arr64(n_tail)
    p.tail_capacity_cells = tail_capacity_cells
    p.tail_chunk_cells = tail_chunk_cells
    p.tail_ring_depth = tail_ring_depth
    p.n_queries = n_queries
    p.tail_zero_copy = 1 if tail_zero_copy else 0
    if max_records is not None:
        mr = np.ascontiguousarray(np.asarray(max_records, dtype=np.int32))
        keep.append(mr)
        p.max_records = mr.ctypes.data
    h = _p()
    ws = ctypes.c_size_t()
    _check(lib.kvdec_plan(ctypes.byref(p), n_cu, ctypes.byref(h), ctypes.byref(ws)), "kvdec_plan")
    return Plan(h.value, ws.value, None)


def workspace(plan_, device="cuda"):
    """Zero-filled device workspace for ``plan_`` (torch uint8 tensor)."""
    import torch
    return torch.zeros(max(plan_.workspace_bytes, 256), dtype=torch.uint8, device=device)


def _io(q, k, v, out, lse, part, k_scales, v_scales, plan_cells, k_cell_stride, k_head_stride, v_cell_stride,
        v_head_stride, k_tail, v_tail, k_tail_scales, v_tail_scales, q_pos, cell_pos, copy_after, live_records):
    io = IO()
    io.live_records = _ptr(live_records)
    io.q, io.k, io.v = _ptr(q), _ptr(k), _ptr(v)
    io.k_scales, io.v_scales = _ptr(k_scales), _ptr(v_scales)
    io.k_cell_stride, io.k_head_stride = k_cell_stride, k_head_stride
    io.v_cell_stride, io.v_head_stride = v_cell_stride, v_head_stride
    io.plan_cells = _ptr(plan_cells)
    io.k_tail, io.v_tail = _ptr(k_tail), _ptr(v_tail)
    io.k_tail_scales, io.v_tail_scales = _ptr(k_tail_scales), _ptr(v_tail_scales)
    io.out, io.lse = _ptr(out), _ptr(lse)
    if part is not None:
        io.part_m, io.part_l, io.part_o = (_ptr(t) for t in part)
    io.q_pos, io.cell_pos = _ptr(q_pos), _ptr(cell_pos)
    if copy_after is not None:
        io.copy_after = copy_after.cuda_event if hasattr(copy_after, "cuda_event") else int(copy_after)
    return io


def attend(plan_, q, k, v, ws, *, out=None, lse=None, part=None, k_scales=None, v_scales=None, plan_cells=None,
           k_cell_stride=0, k_head_stride=0, v_cell_stride=0, v_head_stride=0, k_tail=None, v_tail=None,
           k_tail_scales=None, v_tail_scales=None, q_pos=None, cell_pos=None, stream=None, copy_stream=None,
           copy_after=None, live_records=None):
    """Enqueue one evaluation (see kvdec_attend in include/kvdec.h).
    ``part`` is an optional (m, l, o) tuple of output tensors; ``q_pos``
    (int32 [slots][n_queries]) and ``cell_pos`` (int32 [capacity]) are the
    positions of the multi-query mask.  ``copy_after`` (a torch.cuda.Event
    or raw hipEvent_t) orders the tail copies after that event instead of
    after all earlier work on the stream.  ``live_records`` (int32 [slots],
    indirect plans) limits each slot to its first segments of entries, e.g.
    the n_records output of build_cells."""
    io = _io(q, k, v, out, lse, part, k_scales, v_scales, plan_cells, k_cell_stride, k_head_stride, v_cell_stride,
             v_head_stride, k_tail, v_tail, k_tail_scales, v_tail_scales, q_pos, cell_pos, copy_after, live_records)
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else int(ws[1])
    wptr = _ptr(ws) if hasattr(ws, "numel") else int(ws[0])
    st = _stream_handle(stream)
    cst = None if copy_stream is None else _stream_handle(copy_stream)
    _check(lib.kvdec_attend(plan_.handle, ctypes.byref(io), wptr, nbytes, st, cst), "kvdec_attend")


def attend_static(plan_, q, k, v, *, out=None, lse=None, part=None, k_scales=None, v_scales=None, plan_cells=None,
                  k_cell_stride=0, k_head_stride=0, v_cell_stride=0, v_head_stride=0, k_tail=None, v_tail=None,
                  k_tail_scales=None, v_tail_scales=None, q_pos=None, cell_pos=None, stream=None, live_records=None):
    """attend() with the library's static per-device scratch in place of a
    workspace (see kvdec_attend_static in include/kvdec.h): allocates
    nothing; calls that may overlap on one GPU race."""
    io = _io(q, k, v, out, lse, part, k_scales, v_scales, plan_cells, k_cell_stride, k_head_stride, v_cell_stride,
             v_head_stride, k_tail, v_tail, k_tail_scales, v_tail_scales, q_pos, cell_pos, None, live_records)
    _check(lib.kvdec_attend_static(plan_.handle, ctypes.byref(io), _stream_handle(stream)), "kvdec_attend_static")


def build_cells(plan_, raw_cells, raw_off, plan_cells, ws, *, n_records=None, stream=None):
    """Build a device-built plan's entries on the device (kvdec_build_cells):
    raw_cells int32 and raw_off int64 [n_slots + 1] device tensors; writes
    plan_cells (int32 [n_entries]) and optionally n_records (int32
    [n_slots + 1])."""
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else int(ws[1])
    wptr = _ptr(ws) if hasattr(ws, "numel") else int(ws[0])
    _check(lib.kvdec_build_cells(plan_.handle, _ptr(raw_cells), _ptr(raw_off), _ptr(plan_cells), _ptr(n_records),
                                 wptr, nbytes, _stream_handle(stream)), "kvdec_build_cells")


def merge(parts, n_rows, head_dim, *, out=None, lse=None, merged=None, stream=None):
    """Log-sum-exp merge of partial sets [(m, l, o), ...] (device tensors)."""
    arr = (PartialC * len(parts))()
    for i, (m, l, o) in enumerate(parts):
        arr[i].m, arr[i].l, arr[i].o = _ptr(m), _ptr(l), _ptr(o)
    mm = ml = mo = None
    if merged is not None:
        mm, ml, mo = (_ptr(t) for t in merged)
    _check(lib.kvdec_merge(len(parts), arr, n_rows, head_dim, _ptr(out), _ptr(lse), mm, ml, mo,
                           _stream_handle(stream)), "kvdec_merge")


def version():
    return lib.kvdec_version()
