"""CPU tests of libkvdec's host side: the library loads and exports every
function include/kvdec.h declares, the planner's compact plan is bit-exact
against the oracle, the split table covers every tile exactly once, and every
error path returns its status before any device work (no GPU needed)."""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle as O
from long_context_decode_kv_amd import kvdec as K
from long_context_decode_kv_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "kvdec.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(kvdec_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(K.lib, name), name
    assert set(names) == set(K.EXPORTED)
    assert K.version() == 10801


def test_probe_library_exports_and_rejects_bad_arguments():
    """The streaming-read probe (include/kvprobe.h) loads, exports what its
    header declares, and rejects invalid arguments before any launch."""
    import ctypes
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "kvprobe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(kvprobe_\w+)\s*\(", text, flags=re.M)))
    assert names == ["kvprobe_lds_workgroups", "kvprobe_read", "kvprobe_read_shape"]
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_decode_kv_amd", "libkvprobe.so"))
    f = lib.kvprobe_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    fake = 1 << 20
    assert f(None, 1024, 4, 4, fake, None) == -1          # null buffer
    assert f(fake, 1000, 4, 4, fake, None) == -1          # not a multiple of 16
    assert f(fake + 8, 1024, 4, 4, fake, None) == -1      # misaligned
    assert f(fake, 1024, 0, 4, fake, None) == -1          # no workgroups
    assert f(fake, 1024, 4, 3, fake, None) == -1          # unsupported unroll
    assert f(fake, 1024, 4, 4, None, None) == -1          # null sink
    g = lib.kvprobe_read_shape
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert g(fake, 1024, 4, 256, 64, 0, fake, None) == -1     # no such register-load shape
    assert g(fake, 1024, 4, 1024, 32, 0, fake, None) == -1    # nor this one
    assert g(fake, 1024, 4, 256, 4, 1, fake, None) == -1      # no such LDS-DMA shape
    assert g(fake, 1024, 0, 512, 8, 0, fake, None) == -1      # no workgroups
    assert g(fake + 4, 1024, 4, 256, 8, 1, fake, None) == -1  # misaligned
    h = lib.kvprobe_lds_workgroups
    h.restype = ctypes.c_int64
    h.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    assert h(53690368, 256, 8) == -(-53690368 // (16 * 256 * 8)) and h(0, 256, 8) == -1


def test_strerror_codes():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert K.lib.kvdec_strerror(code).decode() not in ("", "unknown status")
    assert K.lib.kvdec_strerror(17).decode() == "unknown status"


# ---------------------------------------------------------------- planner

def _plan_cells(lists, capacity, **kw):
    p = K.plan(24, 4, 256, len(lists), capacity, k_type=K.Q8_B32, v_type=K.Q8_B32, cells=lists, n_cu=256, **kw)
    return p, p.cells()


def test_compact_plan_matches_oracle_hand_cases():
    lists = [[5, 130, 5, 7, -1, 129], [300, 0, 1, 2, 257], [639, 128, -1, -1, 639], [], [-1, -1]]
    _, (e, off) = _plan_cells(lists, 640)
    we, woff = O.compact_plan(lists, 640)
    assert np.array_equal(e, we) and np.array_equal(off, woff)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_compact_plan_matches_oracle_random(seed):
    r = synth.rng(100 + seed)
    lengths = [int(x) for x in r.integers(0, 3000, 5)] + [0, 1, 128]
    lists, cap = synth.interleaved_record_lists(lengths, r, shuffle=True, duplicates=40)
    cap += 384  # spare records past the last one
    p, (e, off) = _plan_cells(lists, cap)
    we, woff = O.compact_plan(lists, cap)
    assert np.array_equal(e, we) and np.array_equal(off, woff)
    info = p.info()
    assert info["n_entries"] == len(we)


def test_compact_plan_gqa6_workload_shape():
    lists, cap = synth.interleaved_record_lists([131072, 65536, 20000, 777])
    p, (e, off) = _plan_cells(lists, cap)
    assert cap == 217600 and len(e) == 217600 and int((e == -1).sum()) == 215
    assert list(np.diff(off) // 128) == [1024, 512, 157, 7]


def _split_positions(p, sp):
    """Positions of each row of the split table: a contiguous run, or for an
    interleaved plan the units first, first + U * n_splits, ... of U cells."""
    u = p.info()["split_interleave"]
    if not u:
        return [range(int(p0), int(p0 + n)) for _, _, p0, n in sp]
    per = {}
    for s, g, _, _ in sp:
        per[(int(s), int(g))] = per.get((int(s), int(g)), 0) + 1
    out = []
    for s, g, p0, n in sp:
        stride = u * per[(int(s), int(g))]
        out.append([int(p0) + (i // u) * stride + i % u for i in range(int(n))])
    return out


def _coverage(p, n_per_slot, n_kv):
    """The split table covers every position [0, n) of every (slot, KV head)
    exactly once (contiguous runs, or interleaved units)."""
    sp = p.splits()
    seen = {}
    for (s, g, _, _), ts in zip(sp, _split_positions(p, sp)):
        for t in ts:
            key = (int(s), int(g), int(t))
            assert key not in seen
            seen[key] = 1
    want = {(s, g, t) for s, n in enumerate(n_per_slot) for g in range(n_kv) for t in range(n)}
    assert set(seen) == want
    return sp


@pytest.mark.parametrize("tps,split_cells", [(0, 0), (1, 0), (3, 0), (1000, 0), (0, 96), (7, 32), (0, 4096)])
def test_split_table_covers_every_position_once(tps, split_cells):
    occ = [13100, 0, 1, 128, 129, 40000]
    p = K.plan(32, 8, 128, len(occ), 50000, n_occupied=occ, tiles_per_split=tps, split_cells=split_cells,
               n_cu=256)
    sp = _coverage(p, occ, 8)
    info = p.info()
    unit = info["split_unit"]
    assert unit == 32  # vector-ALU kernel
    want = split_cells or 128 * tps
    for s in range(len(occ)):
        for g in range(8):
            rows = [r for r in sp if r[0] == s and r[1] == g]
            # boundaries on multiples of the unit; pieces differ by at most one unit
            assert all(int(r[2]) % unit == 0 for r in rows)
            counts = [int(r[3]) for r in rows[:-1]]
            if counts:
                assert max(counts) - min(counts) <= unit
            if want:
                assert max(int(r[3]) for r in rows) <= max(want, unit)
    assert info["n_workgroups"] == len(sp)
    assert info["n_tiles"] == sum(-(-n // 128) for n in occ) * 8
    assert info["split_cells"] == max(int(r[3]) for r in sp)


def test_matrix_core_splits_are_whole_tiles():
    occ = [9000, 300]
    p = K.plan(24, 4, 256, 2, 20000, k_type=K.Q8_B32, v_type=K.Q8_B32, n_occupied=occ, cell_begin=[0, 10000],
               split_cells=160, n_cu=256)
    info = p.info()
    assert info["matrix_cores"] == 1 and info["split_unit"] == 128 and info["split_cells"] == 256
    sp = _coverage(p, occ, 4)
    assert all(int(r[2]) % 128 == 0 for r in sp)


@pytest.mark.parametrize("bad", [-32, 48, 1])
def test_split_cells_must_be_multiple_of_32(bad):
    with pytest.raises(K.KvdecError):
        K.plan(32, 8, 128, 1, 4096, n_occupied=[4096], split_cells=bad)


def test_auto_split_fills_device():
    # short f16 contexts at head_dim 128: the one-shot kernel, one split of
    # at most 448 cells per compute unit, on 32-cell boundaries
    for occ, cells in ((8192, 256), (13100, 416), (4096, 128), (1000, 64)):
        info = K.plan(32, 8, 128, 1, 16384, n_occupied=[occ], n_cu=256).info()
        assert info["kernel"] == K.KERNEL_ONESHOT and info["waves"] == 8 and info["split_cells"] == cells
        assert info["n_workgroups"] == 8 * -(-occ // cells) <= 256
    # too long for one split per compute unit: the streamed kernel
    assert K.plan(32, 8, 128, 1, 16384, n_occupied=[16384], n_cu=256).info()["kernel"] == K.KERNEL_STREAMED
    # one-shot splits take every n_splits-th 32-cell unit, covering every position once
    for occ in ([13100], [4096], [1000], [900, 5000, 1, 0, 129]):
        p = K.plan(32, 8, 128, len(occ), 16384 * len(occ), n_occupied=occ, n_cu=256,
                   cell_begin=[16384 * i for i in range(len(occ))])
        assert p.info()["kernel"] == K.KERNEL_ONESHOT and p.info()["split_interleave"] == 32
        sp = _coverage(p, occ, 8)
        assert max(len(ts) for ts in _split_positions(p, sp)) <= p.info()["split_cells"]
    p = K.plan(32, 8, 128, 1, 16384, n_occupied=[8192], n_cu=256, kernel=K.KERNEL_STREAMED)
    info = p.info()
    assert 256 <= info["n_workgroups"] <= 512 and info["waves"] == 4 and info["kernel"] == K.KERNEL_STREAMED
    # short f16 context on the streamed kernel: one eight-wave workgroup per
    # compute unit at most, each split two of its 256-cell steps
    p = K.plan(32, 8, 128, 1, 16384, n_occupied=[13100], n_cu=256, kernel=K.KERNEL_STREAMED)
    info = p.info()
    assert info["waves"] == 8 and info["n_workgroups"] == 208 and info["split_cells"] == 512
    # not for quantized caches, explicit split sizes or head_dim 256
    assert K.plan(32, 8, 128, 1, 16384, n_occupied=[13100], n_cu=256, split_cells=512).info()["waves"] == 4
    assert K.plan(32, 8, 128, 1, 16384, k_type=K.Q8_B32, v_type=K.Q8_B32, n_occupied=[13100],
                  n_cu=256).info()["waves"] == 4
    assert K.plan(16, 8, 256, 1, 16384, n_occupied=[13100], n_cu=256).info()["waves"] == 4
    # matrix-core kernel, short splits: two tiles double to four when that
    # still gives at most one workgroup per compute unit
    # (eight waves, two steps of 256 cells each, for 16-row records at head_dim 128)
    for hq, nq, waves in ((48, 1, 4), (64, 1, 4), (32, 4, 8), (128, 1, 8)):
        info = K.plan(hq, 8, 128, 1, 16384, n_occupied=[13100], n_queries=nq, n_cu=256).info()
        assert info["matrix_cores"] == 1 and info["n_workgroups"] == 208 and info["tiles_per_split"] == 4
        assert info["waves"] == waves
    assert K.plan(32, 8, 128, 1, 16384, n_occupied=[13100], n_queries=4, n_cu=256,
                  split_cells=512).info()["waves"] == 4
    assert K.plan(64, 4, 256, 1, 16384, n_occupied=[13100], n_cu=256).info()["waves"] == 4
    assert K.plan(48, 8, 128, 1, 16384, n_occupied=[8192], n_cu=256).info()["n_workgroups"] == 512
    # five f16 rows: the one-shot kernel, else the matrix-core kernel for
    # short contexts, vector-ALU for long ones
    assert K.plan(40, 8, 128, 1, 16384, n_occupied=[13100], n_cu=256).info()["kernel"] == K.KERNEL_ONESHOT
    assert K.plan(40, 8, 128, 1, 16384, n_occupied=[13100], n_cu=256,
                  kernel=K.KERNEL_STREAMED).info()["matrix_cores"] == 0
    short = K.plan(40, 8, 128, 1, 16384, n_occupied=[16384], n_cu=256).info()
    assert short["matrix_cores"] == 1 and short["tiles_per_split"] == 4
    long_ = K.plan(40, 8, 128, 1, 524288, n_occupied=[524288], n_cu=256).info()
    assert long_["matrix_cores"] == 0 and long_["n_workgroups"] == 256
    assert K.plan(40, 8, 128, 1, 16384, n_occupied=[13100], n_cu=256, split_cells=512).info()["matrix_cores"] == 0
    # long f16 splits on the vector-ALU kernel: one workgroup per compute unit
    p = K.plan(32, 8, 128, 1, 65536, n_occupied=[65536], n_cu=256)
    info = p.info()
    assert info["n_workgroups"] == 256 and info["tiles_per_split"] == 16
    # long f16 splits over more (slot, KV head) pairs than compute units:
    # about eight splits per compute unit
    p = K.plan(32, 8, 128, 36, 36 * 16384, n_occupied=[13100] * 36, cell_begin=[i * 16384 for i in range(36)],
               n_cu=256)
    info = p.info()
    assert info["tiles_per_split"] == 15 and info["n_workgroups"] == 36 * 8 * 7
    p = K.plan(40, 8, 128, 1, 524288, n_occupied=[524288], n_cu=256)
    info = p.info()
    assert info["n_workgroups"] == 256 and info["tiles_per_split"] == 128
    # quantized (matrix-core kernel): about two per compute unit
    p = K.plan(24, 4, 256, 1, 65536, k_type=K.Q8_B32, v_type=K.Q8_B32, n_occupied=[65536], n_cu=256)
    info = p.info()
    assert info["n_workgroups"] == 512 and info["tiles_per_split"] == 4


def test_tail_plan_chunks_and_workspace():
    p = K.plan(32, 8, 128, 1, 40960, n_occupied=[14000], cell_begin=[26960], n_tail=[26960],
               tail_capacity_cells=26960, tail_chunk_cells=2048, tail_ring_depth=4, n_cu=256)
    info = p.info()
    assert info["n_tail_chunks"] == math.ceil(26960 / 2048)
    # ring of 4 slots x 2048 cells x 8 heads x 256 B for each of K and V
    assert info["workspace_bytes"] >= 4 * 2 * 2048 * 8 * 256


# ---------------------------------------------------------------- errors

def _status(fn):
    with pytest.raises(K.KvdecError) as ei:
        fn()
    return ei.value.status


def test_plan_errors():
    base = dict(n_occupied=[10], n_cu=256)
    assert _status(lambda: K.plan(32, 7, 128, 1, 100, **base)) == K.E_INVALID          # not a multiple
    assert _status(lambda: K.plan(34, 2, 128, 1, 100, **base)) == K.E_INVALID          # G = 17
    assert _status(lambda: K.plan(32, 8, 96, 1, 100, **base)) == K.E_INVALID           # head_dim
    assert _status(lambda: K.plan(32, 8, 128, 0, 100, **base)) == K.E_INVALID          # no slots
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, k_type=5, **base)) == K.E_INVALID
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, scale=float("nan"), **base)) == K.E_INVALID
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[101], n_cu=256)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[10], cell_begin=[95], n_cu=256)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, cells=[[3, 100]], n_cu=256)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, cells=[[3, -2]], n_cu=256)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 2, 64, 1, 100, **base)) == K.E_UNSUPPORTED       # G = 16, head_dim 64
    K.plan(32, 2, 128, 1, 100, **base).close()                                           # G = 16 on matrix cores
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, k_type=K.Q8_B32, v_type=K.F16, **base)) == K.E_UNSUPPORTED
    # V stored more finely than K has no kernel; K more finely than V does
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, k_type=K.Q4_B32, v_type=K.Q8_B32, **base)) == K.E_UNSUPPORTED
    for kt, vt in ((K.F16, K.Q8_B32), (K.F16, K.Q4_B32), (K.Q8_B32, K.Q4_B32)):
        K.plan(32, 8, 128, 1, 100, k_type=kt, v_type=vt, **base).close()
    assert _status(lambda: K.plan(32, 8, 128, 65, 100, n_occupied=[1] * 65, n_cu=256)) == K.E_UNSUPPORTED
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, cells=[[1]], n_tail=[1], tail_capacity_cells=1,
                                  n_cu=256)) == K.E_UNSUPPORTED
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[1], n_tail=[5], tail_capacity_cells=4,
                                  n_cu=256)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[1], n_tail=[5], tail_capacity_cells=8,
                                  tail_chunk_cells=100, n_cu=256)) == K.E_INVALID
    # the library keeps the message of the last failure
    assert "tail_chunk_cells" in K.lib.kvdec_last_error().decode()


def test_malformed_ranges_are_rejected():
    """Ranges whose ends overflow int64, offsets that go backwards, record
    budgets and capacities out of range: each is refused with a status code
    (run also under the sanitizer build, where any overflow or out-of-bounds
    read in the planner aborts)."""
    big = 2 ** 63 - 5
    cu = dict(n_cu=256)
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[10], cell_begin=[big], **cu)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[big], cell_begin=[5], **cu)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[-1], **cu)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[1], cell_begin=[-3], **cu)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[1], n_tail=[10], tail_begin=[big],
                                  tail_capacity_cells=100, **cu)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[1], n_tail=[big], tail_begin=[3],
                                  tail_capacity_cells=100, **cu)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[1], n_tail=[-2], tail_capacity_cells=100,
                                  **cu)) == K.E_RANGE
    assert _status(lambda: K.plan(32, 8, 128, 1, 2 ** 62, n_occupied=[1], **cu)) == K.E_INVALID
    assert _status(lambda: K.plan(32, 8, 128, 1, 2 ** 63 - 1, cells=[[1]], **cu)) == K.E_INVALID
    assert _status(lambda: K.plan(32, 8, 128, 1, 100, n_occupied=[1], n_tail=[1], tail_capacity_cells=2 ** 60,
                                  **cu)) == K.E_INVALID
    assert _status(lambda: K.plan(32, 8, 128, 1, -1, n_occupied=[0], **cu)) == K.E_INVALID
    for budget in ([-1], [2 ** 31 - 1], [1, -5]):
        assert _status(lambda: K.plan(24, 4, 256, len(budget), 5000, k_type=K.Q8_B32, v_type=K.Q8_B32,
                                      max_records=budget, **cu)) == K.E_INVALID
    # raw lists with offsets that go backwards or start below zero (the
    # Problem struct filled by hand: the binding only builds valid offsets)
    cells = np.array([1, 2, 3, 4], np.int32)
    for off in ([0, 3, 1], [-1, 2, 4], [2, 1, 4]):
        o = np.array(off, np.int64)
        pr = K.Problem(n_q_heads=32, n_kv_heads=8, head_dim=128, n_slots=2, k_type=K.F16, v_type=K.F16, scale=0.1,
                       capacity_cells=100)
        pr.cells = cells.ctypes.data
        pr.cells_off = o.ctypes.data
        h, ws = ctypes.c_void_p(), ctypes.c_size_t()
        assert K.lib.kvdec_plan(ctypes.byref(pr), 256, ctypes.byref(h), ctypes.byref(ws)) == K.E_INVALID
        assert "cells_off" in K.lib.kvdec_last_error().decode()
    # the planner's memory follows the cells listed, not the capacity
    assert K.plan(32, 8, 128, 1, 2 ** 48, cells=[[1, 2 ** 31 - 1]], **cu).info()["n_entries"] == 256


FAKE = 1 << 20  # an aligned address that is never dereferenced: validation fails first


def test_attend_validation_before_device_work():
    p = K.plan(32, 8, 128, 1, 4096, n_occupied=[4096], n_cu=256)
    ws = (FAKE, p.workspace_bytes)
    args = dict(out=FAKE, stream=0)
    assert _status(lambda: K.attend(p, FAKE, FAKE, FAKE, (0, p.workspace_bytes), **args)) == K.E_WORKSPACE
    assert _status(lambda: K.attend(p, FAKE, FAKE, FAKE, (FAKE, p.workspace_bytes - 1), **args)) == K.E_WORKSPACE
    assert _status(lambda: K.attend(p, FAKE, FAKE, FAKE, (FAKE + 16, p.workspace_bytes), **args)) == K.E_INVALID
    assert _status(lambda: K.attend(p, 0, FAKE, FAKE, ws, **args)) == K.E_INVALID            # no q
    assert _status(lambda: K.attend(p, FAKE, FAKE + 8, FAKE, ws, **args)) == K.E_INVALID     # misaligned k
    assert _status(lambda: K.attend(p, FAKE, 0, FAKE, ws, **args)) == K.E_INVALID            # no k
    assert _status(lambda: K.attend(p, FAKE, FAKE, 0, ws, **args)) == K.E_INVALID            # no v
    assert _status(lambda: K.attend(p, FAKE, FAKE, FAKE, ws, k_cell_stride=24, **args)) == K.E_INVALID
    assert _status(lambda: K.attend(p, FAKE, FAKE, FAKE, ws, stream=0)) == K.E_INVALID       # no output
    assert _status(lambda: K.attend(p, FAKE, FAKE, FAKE, ws, part=(FAKE, FAKE, 0), stream=0)) == K.E_INVALID
    pq = K.plan(24, 4, 256, 1, 4096, k_type=K.Q8_B32, v_type=K.Q8_B32, n_occupied=[10], n_cu=256)
    wsq = (FAKE, pq.workspace_bytes)
    assert _status(lambda: K.attend(pq, FAKE, FAKE, FAKE, wsq, out=FAKE, k_scales=FAKE, stream=0)) == K.E_INVALID
    pi = K.plan(24, 4, 256, 1, 4096, k_type=K.Q4_B32, v_type=K.Q4_B32, cells=[[1, 2]], n_cu=256)
    wsi = (FAKE, pi.workspace_bytes)
    assert _status(lambda: K.attend(pi, FAKE, FAKE, FAKE, wsi, out=FAKE, k_scales=FAKE, v_scales=FAKE, stream=0)) == K.E_INVALID
    pt = K.plan(32, 8, 128, 1, 4096, n_occupied=[10], n_tail=[10], tail_capacity_cells=10, n_cu=256)
    wst = (FAKE, pt.workspace_bytes)
    assert _status(lambda: K.attend(pt, FAKE, FAKE, FAKE, wst, out=FAKE, stream=0)) == K.E_INVALID      # tail arrays missing
    assert _status(lambda: K.attend(p, FAKE, FAKE, FAKE, ws, live_records=FAKE, **args)) == K.E_INVALID  # contiguous
    assert _status(lambda: K.attend(pi, FAKE, FAKE, FAKE, wsi, out=FAKE, k_scales=FAKE, v_scales=FAKE, plan_cells=FAKE,
                                    live_records=FAKE + 2, stream=0)) == K.E_INVALID     # misaligned live_records


def test_no_device_cells_needs_no_cache_arrays():
    """With capacity_cells 0 no split holds a cell or an entry, so k, v,
    their scales and (for an indirect plan, which then has no entries)
    plan_cells may be NULL: the call passes validation and reaches the
    device (which this host lacks); with capacity_cells > 0 they may not."""
    for kind in (K.F16, K.Q8_B32, K.Q4_B32):
        d = 128 if kind == K.F16 else 256
        for p in (K.plan(4 * 2, 2, d, 2, 0, k_type=kind, v_type=kind, n_occupied=[0, 0], n_cu=256),
                  K.plan(4 * 2, 2, d, 2, 0, k_type=kind, v_type=kind, cells=[[], []], n_cu=256)):
            assert p.info()["n_entries"] == 0
            ws = (FAKE, max(p.workspace_bytes, 256))
            st = _status(lambda: K.attend(p, FAKE, 0, 0, ws, out=FAKE, stream=0))
            assert st != K.E_INVALID, K.lib.kvdec_last_error().decode()
    p1 = K.plan(24, 4, 256, 1, 1, k_type=K.Q8_B32, v_type=K.Q8_B32, n_occupied=[0], n_cu=256)
    ws1 = (FAKE, p1.workspace_bytes)
    assert _status(lambda: K.attend(p1, FAKE, 0, 0, ws1, out=FAKE, stream=0)) == K.E_INVALID
    assert "capacity_cells > 0" in K.lib.kvdec_last_error().decode()
    assert _status(lambda: K.attend(p1, FAKE, FAKE, FAKE, ws1, out=FAKE, stream=0)) == K.E_INVALID  # no scales
    pi = K.plan(24, 4, 256, 1, 128, k_type=K.Q8_B32, v_type=K.Q8_B32, cells=[[5]], n_cu=256)
    wsi = (FAKE, pi.workspace_bytes)
    assert _status(lambda: K.attend(pi, FAKE, FAKE, FAKE, wsi, out=FAKE, k_scales=FAKE, v_scales=FAKE,
                                    stream=0)) == K.E_INVALID                               # entries, no plan_cells


def test_ticket_area_fixed_size():
    """Every plan's workspace starts with a merge-ticket area of one 128-byte
    line per ticket, rounded up to KVDEC_TICKET_AREA_BYTES, so plans of up
    to 8192 tickets share one layout of it and can take turns on a workspace."""
    hdr = open(os.path.join(ROOT, "include", "kvdec.h")).read()
    assert "#define KVDEC_TICKET_AREA_BYTES (1024 * 1024)" in hdr and K.TICKET_AREA_BYTES == 1024 * 1024
    plans = [K.plan(32, 8, 128, 1, 16384, n_occupied=[13100], n_cu=256),
             K.plan(32, 8, 128, 2, 16384, n_occupied=[300, 9000], cell_begin=[0, 4096], n_cu=256),
             K.plan(32, 8, 128, 64, 64 * 4096, n_occupied=[4096] * 64, cell_begin=[4096 * s for s in range(64)],
                    n_cu=256),
             K.plan(24, 4, 256, 4, 1 << 18, n_occupied=[131072, 65536, 20000, 777],
                    cell_begin=[0, 131072, 196608, 217088], k_type=K.Q8_B32, v_type=K.Q8_B32, n_cu=256)]
    for p in plans:
        info = p.info()
        assert info["ticket_bytes"] == K.TICKET_AREA_BYTES
        assert p.workspace_bytes > info["ticket_bytes"]
    # 16 slots x 2048 KV heads: 32768 tickets of 128 bytes, exactly 4 areas
    many = K.plan(2048, 2048, 64, 16, 64, n_occupied=[1] * 16, cell_begin=list(range(16)), n_cu=256)
    assert many.info()["ticket_bytes"] == 4 * K.TICKET_AREA_BYTES


def test_attend_static_validation_before_device_work():
    """kvdec_attend_static refuses, before it touches a device, a plan whose
    workspace or merge tickets do not fit the static scratch, a copied tail,
    and bad io; the limits are the header's."""
    hdr = open(os.path.join(ROOT, "include", "kvdec.h")).read()
    assert "#define KVDEC_STATIC_TICKET_BYTES (1024 * 1024)" in hdr and K.STATIC_TICKET_BYTES == 1024 * 1024
    assert "#define KVDEC_STATIC_WORKSPACE_BYTES (16 * 1024 * 1024)" in hdr
    assert K.STATIC_WORKSPACE_BYTES == 16 * 1024 * 1024
    args = dict(out=FAKE, stream=0)
    big = K.plan(32, 8, 128, 1, 262144, n_occupied=[262144], split_cells=64, n_cu=256)
    assert big.workspace_bytes > K.STATIC_WORKSPACE_BYTES
    assert _status(lambda: K.attend_static(big, FAKE, FAKE, FAKE, **args)) == K.E_WORKSPACE
    assert "static scratch" in K.lib.kvdec_last_error().decode()
    # 16 slots x 2048 KV heads: 32768 slot tickets, a workspace that fits
    many = K.plan(2048, 2048, 64, 16, 64, n_occupied=[1] * 16, cell_begin=list(range(16)), n_cu=256)
    assert many.workspace_bytes <= K.STATIC_WORKSPACE_BYTES
    assert _status(lambda: K.attend_static(many, FAKE, FAKE, FAKE, **args)) == K.E_WORKSPACE
    assert "tickets" in K.lib.kvdec_last_error().decode()
    copied = K.plan(32, 8, 128, 1, 4096, n_occupied=[10], n_tail=[10], tail_capacity_cells=10, n_cu=256,
                    tail_chunk_cells=128)
    assert copied.workspace_bytes <= K.STATIC_WORKSPACE_BYTES
    assert _status(lambda: K.attend_static(copied, FAKE, FAKE, FAKE, k_tail=FAKE, v_tail=FAKE, **args)) \
        == K.E_UNSUPPORTED
    ok = K.plan(32, 8, 128, 1, 4096, n_occupied=[4096], n_cu=256)
    assert _status(lambda: K.attend_static(ok, 0, FAKE, FAKE, **args)) == K.E_INVALID          # no q
    assert _status(lambda: K.attend_static(ok, FAKE, FAKE + 8, FAKE, **args)) == K.E_INVALID   # misaligned k
    assert _status(lambda: K.attend_static(ok, FAKE, FAKE, FAKE, stream=0)) == K.E_INVALID     # no output
    zc = K.plan(32, 8, 128, 1, 4096, n_occupied=[10], n_tail=[10], tail_capacity_cells=10, n_cu=256,
                tail_zero_copy=True)
    assert _status(lambda: K.attend_static(zc, FAKE, FAKE, FAKE, **args)) == K.E_INVALID       # tail arrays missing
    assert K.lib.kvdec_attend_static(None, None, None) == K.E_INVALID


def test_merge_validation():
    import ctypes
    arr = (K.PartialC * 1)()
    arr[0].m, arr[0].l, arr[0].o = FAKE, FAKE, FAKE
    f = K.lib.kvdec_merge
    assert f(0, arr, 4, 128, FAKE, None, None, None, None, None) == K.E_INVALID
    assert f(65, arr, 4, 128, FAKE, None, None, None, None, None) == K.E_INVALID
    assert f(1, arr, 4, 0, FAKE, None, None, None, None, None) == K.E_INVALID
    assert f(1, arr, 4, 128, None, None, None, None, None, None) == K.E_INVALID
    assert f(1, arr, 4, 128, None, None, FAKE, FAKE, None, None) == K.E_INVALID
    bad = (K.PartialC * 1)()
    bad[0].m, bad[0].l, bad[0].o = FAKE, None, FAKE
    assert f(1, bad, 4, 128, FAKE, None, None, None, None, None) == K.E_INVALID
    # zero rows: nothing to do, nothing launched
    assert f(1, arr, 0, 128, FAKE, None, None, None, None, None) == K.OK
    del ctypes


def test_multi_query_plans():
    """Several query rows per slot: the matrix-core kernel serves G * n_q <= 16
    rows for head_dim 128 / 256; everything else is refused at plan time."""
    base = dict(n_occupied=[1000], n_cu=256)
    info = K.plan(32, 8, 128, 1, 1000, n_queries=4, **base).info()
    assert info["n_queries"] == 4 and info["matrix_cores"] == 1
    one = K.plan(32, 8, 128, 1, 1000, **base).info()
    assert one["n_queries"] == 1 and one["matrix_cores"] == 0
    assert K.plan(24, 4, 256, 1, 1000, **base).info()["matrix_cores"] == 1   # G = 6
    assert _status(lambda: K.plan(32, 8, 128, 1, 1000, n_queries=9, **base)) == K.E_INVALID
    assert _status(lambda: K.plan(32, 8, 128, 1, 1000, n_queries=-1, **base)) == K.E_INVALID
    assert _status(lambda: K.plan(40, 8, 128, 1, 1000, n_queries=4, **base)) == K.E_UNSUPPORTED  # 20 rows
    assert _status(lambda: K.plan(32, 8, 64, 1, 1000, n_queries=2, **base)) == K.E_UNSUPPORTED   # head_dim 64
    for g, nq in ((1, 8), (2, 8), (4, 4), (8, 2), (16, 1), (3, 5)):
        p = K.plan(8 * g, 8, 256, 2, 1000, n_queries=nq, n_occupied=[1000, 10], n_cu=256)
        assert p.info()["n_queries"] == nq
        p.close()


def test_multi_query_attend_needs_q_pos():
    p = K.plan(32, 8, 128, 1, 1000, n_queries=2, n_occupied=[1000], n_cu=256)
    ws = (FAKE, p.workspace_bytes)
    assert _status(lambda: K.attend(p, FAKE, FAKE, FAKE, ws, out=FAKE, stream=0)) == K.E_INVALID
    assert "q_pos" in K.lib.kvdec_last_error().decode()
    assert _status(lambda: K.attend(p, FAKE, FAKE, FAKE, ws, out=FAKE, q_pos=FAKE, cell_pos=FAKE + 2,
                                    stream=0)) == K.E_INVALID



def test_zero_copy_tail_plan():
    base = dict(n_occupied=[1000], cell_begin=[3000], n_tail=[3000], tail_capacity_cells=3000, n_cu=256,
                tail_chunk_cells=2048)
    staged = K.plan(32, 8, 128, 1, 4000, **base)
    zc = K.plan(32, 8, 128, 1, 4000, tail_zero_copy=True, **base)
    # two chunks: the default depth 4 is clamped to 2 slots of 2048 cells x 8 heads x (K + V) rows
    ring = 2 * 2048 * 8 * 128 * 2 * 2
    assert staged.workspace_bytes - zc.workspace_bytes >= ring
    assert staged.workspace_bytes - zc.workspace_bytes < 2 * ring
    assert zc.info()["n_tail_chunks"] == staged.info()["n_tail_chunks"] == 2
    # default chunk: 32768 cells, one chunk for this tail
    one = K.plan(32, 8, 128, 1, 4000, n_occupied=[1000], cell_begin=[3000], n_tail=[3000], tail_capacity_cells=3000,
                 n_cu=256)
    assert one.info()["n_tail_chunks"] == 1


def test_device_built_plan_shape_and_errors():
    """A device-built indirect plan: max_records segments per slot, no host
    entries, validation of the record budget and of kvdec_build_cells."""
    p = K.plan(24, 4, 256, 3, 5000, k_type=K.Q8_B32, v_type=K.Q8_B32, max_records=[10, 0, 40], n_cu=256)
    info = p.info()
    assert info["n_entries"] == 50 * 128
    n = K._i64()
    offs = np.zeros(4, np.int64)
    assert K.lib.kvdec_plan_cells(p.handle, None, offs.ctypes.data, ctypes.byref(n)) == 0
    assert n.value == 50 * 128 and list(offs) == [0, 1280, 1280, 6400]
    buf = np.zeros(10, np.int32)
    assert K.lib.kvdec_plan_cells(p.handle, buf.ctypes.data, None, ctypes.byref(n)) == K.E_INVALID
    assert _status(lambda: K.plan(24, 4, 256, 1, 5000, k_type=K.Q8_B32, v_type=K.Q8_B32, max_records=[41],
                                  n_cu=256)) == K.E_INVALID                    # > ceil(5000 / 128)
    assert _status(lambda: K.plan(24, 4, 256, 1, 5000, max_records=[-1], n_cu=256)) == K.E_INVALID
    # no cells, no segments (a hole would read row 0 of an empty cache)
    assert _status(lambda: K.plan(24, 4, 256, 1, 0, max_records=[1], n_cu=256)) == K.E_INVALID
    assert K.plan(24, 4, 256, 1, 0, max_records=[0], n_cu=256).info()["n_entries"] == 0
    ws = (FAKE, p.workspace_bytes)
    assert _status(lambda: K.build_cells(p, FAKE, FAKE, FAKE, (FAKE, 16), stream=0)) == K.E_WORKSPACE
    assert _status(lambda: K.build_cells(p, FAKE, FAKE + 4, FAKE, ws, stream=0)) == K.E_INVALID  # raw_off align
    assert _status(lambda: K.build_cells(p, 0, FAKE, FAKE, ws, stream=0)) == K.E_INVALID
    host = K.plan(24, 4, 256, 1, 5000, cells=[[1, 2]], n_cu=256)
    assert _status(lambda: K.build_cells(host, FAKE, FAKE, FAKE, ws, stream=0)) == K.E_INVALID  # not device-built


def test_device_built_splits_fixed_runs_whatever_the_budget():
    """Splits of a device-built plan are runs of split_cells positions from
    the slot's start (the last one ragged), so a larger record budget only
    appends splits: the ones over the records of the smaller budget are the
    same."""
    def table(budget):
        p = K.plan(24, 4, 256, 2, 20000, k_type=K.Q8_B32, v_type=K.Q8_B32, max_records=budget, split_cells=1024,
                   n_cu=256)
        t = p.splits()
        return {(int(s), int(g)): [] for s, g in t[:, :2]}, t
    for tight, generous in (([20, 7], [68, 29]), ([3, 1], [4, 2]), ([33, 9], [140, 30])):
        _, a = table(tight)
        _, b = table(generous)
        for s in range(2):
            ra, rb = a[(a[:, 0] == s) & (a[:, 1] == 0)], b[(b[:, 0] == s) & (b[:, 1] == 0)]
            assert np.all(rb[:, 2] % 1024 == 0) and np.all(ra[:, 2] % 1024 == 0)
            assert np.array_equal(ra[:-1], rb[:len(ra) - 1])        # the same full runs
            assert ra[-1, 2] == rb[len(ra) - 1, 2]                   # the ragged one starts where its run does
            assert ra[:, 3].sum() == tight[s] * 128


def test_failure_injection_only_in_the_test_build():
    """libkvdec_fi.so (the tail streamer's failure-injection switches) is a
    separate test library; the product library has no such entry point."""
    from long_context_decode_kv_amd import build
    fi = ctypes.CDLL(build.FI_LIB)
    assert hasattr(fi, "kvdec_fi_configure") and hasattr(fi, "kvdec_attend")
    assert not hasattr(K.lib, "kvdec_fi_configure")
    fi.kvdec_source_hash.restype = ctypes.c_char_p
    assert fi.kvdec_source_hash().decode() == K.LIB_SOURCE_HASH


def test_phase_trace_only_in_the_diagnostic_build():
    """libkvdec_trace.so (phase stamps of the one-shot kernel) is a separate
    diagnostic library built from the same sources; the product library has
    no trace switch."""
    from long_context_decode_kv_amd import build
    tr = ctypes.CDLL(build.TRACE_LIB)
    assert hasattr(tr, "kvdec_trace_configure") and hasattr(tr, "kvdec_attend")
    assert not hasattr(K.lib, "kvdec_trace_configure")
    tr.kvdec_source_hash.restype = ctypes.c_char_p
    assert tr.kvdec_source_hash().decode() == K.LIB_SOURCE_HASH


def test_build_rejects_kernels_with_scratch():
    """The build parses the compiler's kernel-resource remarks and refuses
    any kernel that needs per-lane scratch memory."""
    from long_context_decode_kv_amd import build
    log = "\n".join([
        "x.h:1:1: remark: Function Name: _Z2k1v [-Rpass-analysis=kernel-resource-usage]",
        "x.h:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.h:9:1: remark: Function Name: _Z2k2v [-Rpass-analysis=kernel-resource-usage]",
        "x.h:9:1: remark:     ScratchSize [bytes/lane]: 188 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build._scratch_kernels(log) == [("_Z2k2v", 188)]


def _draw_plan_request(seed):
    """A seeded kvdec_plan request, valid in most of its fields (each field
    is malformed with probability 0.03): head_dim, group size, KV heads,
    slots, capacity, storage kinds, query rows and one of contiguous ranges,
    host cell lists, a device-built record budget or a window + tail."""
    r = np.random.default_rng(90000 + seed)
    bad = lambda good, badv: badv if r.random() < 0.03 else good  # noqa: E731
    d = bad(int(r.choice([64, 128, 256])), int(r.choice([96, 0])))
    hkv = bad(int(r.choice([1, 2, 4, 8])), int(r.choice([0, 3])))
    g = bad(int(r.choice([1, 2, 3, 4, 5, 6, 8, 16])), 17)
    n_slots = bad(int(r.choice([1, 2, 3, 7, 64])), int(r.choice([0, 65])))
    cap = bad(int(r.choice([0, 1, 127, 128, 129, 5000, 2 ** 20])), -1)
    if d == 64 and g > 8:  # groups above 8 need head_dim 128 or 256
        g = bad(8, g)
    n_q = int(r.choice([1, 1, 1, 2, 4]))
    if d == 64 or g * n_q > 16:  # several query rows: head_dim 128 / 256, at most 16 rows per KV head
        n_q = bad(1, n_q)
    kt = int(r.integers(0, 3))  # K stored at least as finely as V (f16 < int8 < 4-bit)
    kw = dict(k_type=bad(kt, 3), v_type=bad(int(r.integers(kt, 3)), int(r.integers(0, 3))), n_queries=n_q,
              n_cu=int(r.choice([256, 1, 80])))
    ns, c0 = max(n_slots, 0), max(cap, 0)
    mode = int(r.integers(4))
    if mode in (0, 3):
        b = [int(r.integers(0, c0 + 1)) for _ in range(ns)]
        kw["cell_begin"] = [bad(x, -3) for x in b]
        kw["n_occupied"] = [bad(int(r.integers(0, c0 - x + 1)), c0 - x + 1) for x in b]
        if mode == 3:
            kw["n_tail"] = [int(r.choice([0, 1, 300])) for _ in range(ns)]
            kw["tail_begin"] = [bad(int(r.choice([0, 10])), -1) for _ in range(ns)]
            kw["tail_capacity_cells"] = int(r.choice([400, 6000]))
            kw["tail_chunk_cells"] = bad(int(r.choice([128, 512])), 100)
            kw["tail_ring_depth"] = bad(int(r.choice([2, 4])), 17)
            kw["tail_zero_copy"] = bool(r.integers(2))
    elif mode == 1:
        kw["cells"] = [[int(x) for x in r.integers(-1, max(c0, 1), size=int(r.choice([0, 1, 50, 300])))]
                       for _ in range(ns)]
        if ns and r.random() < 0.03:
            kw["cells"][int(r.integers(ns))].append(c0 + 2)  # out of range
    else:
        kw["max_records"] = [bad(int(r.integers(0, -(-c0 // 128) + 1)), -1) for _ in range(ns)]
    if r.integers(3) == 0:
        kw["split_cells"] = bad(int(r.choice([32, 64, 448, 4096])), 33)
    return (g * max(hkv, 1), hkv, d, n_slots, cap), kw, mode


def test_random_plans_split_every_position_once():
    """400 seeded plan requests (_draw_plan_request): a rejected one raises
    with a status and a message; in an accepted one the split table holds
    n_workgroups rows and the splits of every (slot, KV head) cover the
    slot's positions -- its occupied cells, its list's entries or its
    record budget -- exactly once (contiguous runs tile them).  Under the
    sanitized build this also drives the planner's index arithmetic."""
    accepted = 0
    for seed in range(400):
        args, kw, mode = _draw_plan_request(seed)
        try:
            p = K.plan(*args, **kw)
        except K.KvdecError as e:
            assert e.status < 0 and K.lib.kvdec_last_error().decode()
            continue
        accepted += 1
        info, sp = p.info(), p.splits()
        assert len(sp) == info["n_workgroups"] >= 1
        n_slots, hkv = args[3], args[1]
        if mode in (0, 3):
            n = kw["n_occupied"]
        elif mode == 1:
            off = p.cells()[1]
            n = [int(off[s + 1] - off[s]) for s in range(n_slots)]
        else:
            n = [128 * m for m in kw["max_records"]]
        for s in range(n_slots):
            for h in range(hkv):
                rows = sp[(sp[:, 0] == s) & (sp[:, 1] == h)]
                assert len(rows) >= 1 and np.all(rows[:, 3] >= 0), (seed, s, h)
                assert rows[:, 3].sum() == n[s], (seed, s, h, rows[:, 3].sum(), n[s])
                if info["split_interleave"] == 0:
                    runs = rows[np.argsort(rows[:, 2])]
                    ends = runs[:, 2] + runs[:, 3]
                    assert runs[0, 2] == 0 and np.all(runs[1:, 2] == ends[:-1]), (seed, s, h)
    assert accepted >= 150, accepted


def test_phase_timeline_summary_on_built_stamps():
    """summarize() of the phase-trace tool on stamps built by hand (100 MHz
    ticks): 3 layers of 4 workgroups; each layer starts 2000 ticks after the
    previous one, workgroup w enters w ticks late, slot k of every workgroup
    is stamped 100 k ticks after its entry, the per-wave V stamps of wave v
    at 700 + 10 v, and workgroup 3 is the merger (slot 17 at 1500).
    Layer 0 is skipped as warm-up, so every value is known in closed form."""
    from long_context_decode_kv_amd import phase_trace as PT
    L, N = 3, 4
    x = np.zeros((L, N, 32), dtype=np.int64)
    for layer in range(L):
        for w in range(N):
            e = 10_000 + 2000 * layer + w
            x[layer, w, 0] = e
            for k in list(range(1, 17)) + [18, 19, 20, 21, 30, 31]:
                x[layer, w, k] = e + 100 * k
            for v in range(8):
                x[layer, w, 5 + v] = e + 600 + 10 * v
                x[layer, w, 22 + v] = e + 700 + 10 * v
        x[layer, 3, 17] = 10_000 + 2000 * layer + 3 + 1500
    heads = np.array([0, 1, 0, 1])
    s = PT.summarize(x, heads)
    us = PT.TICK_US
    def close(a, b, atol=1e-9):
        return np.allclose(np.asarray(a, float), np.asarray(b, float), rtol=0, atol=atol)
    rounded = 0.0051  # fields the tool rounds to 0.01 us
    # phase k: median over workgroups of (w + 100 k) ticks -> (1.5 + 100 k) ticks; slowest (3 + 100 k)
    for k, name in PT.SLOTS.items():
        want = (1503, 1503) if k == 17 else (1.5 + 100 * k, 3 + 100 * k)
        assert close(s["phases"][name], [t * us for t in want]), name
    assert close(s["waves"]["last V landed by wave"], [(1.5 + 700 + 10 * v) * us for v in range(8)], rounded)
    assert close(s["waves"]["last V landed, slowest of the layer"], (3 + 770) * us)
    # merger chain after its ticket (slot 16 at 1600): slot k at 100 k, slot 17 at 1500
    want = {16: 0, 30: 1400, 18: 200, 31: 1500, 19: 300, 20: 400, 21: 500, 17: -100}
    assert close([s["merge"][name] for _, name in PT.MERGE_SLOTS], [want[k] * us for k, _ in PT.MERGE_SLOTS], rounded)
    assert close(s["gap"], (2000 - 1503) * us)              # next layer's first entry - last merge
    assert close(s["span"], 1503 * us)
    # entry to last V per head: workgroups 0, 2 -> head 0, 1, 3 -> head 1; each 770 ticks
    assert close(s["heads"], [770 * us, 770 * us], rounded)
