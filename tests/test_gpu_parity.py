"""GPU parity: the HIP path through the C ABI against the float64 oracle,
element by element, max |err| <= 2e-3 on out and lse, on seeded inputs that
span several tiles and ragged tails, every compiled group size and head_dim,
f16 / int8 / 4-bit caches, contiguous and indirect (record-grouped, -1 holes)
cells, empty slots, peaked softmax, partial outputs + kvdec_merge, split-count
independence, strided layouts and NaN-poisoned workspace / unused cells."""

import math

import numpy as np
import pytest

import oracle as O
from gpu_cases import Case, check, dev, TOL, TOL_SPLITS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available()
    from long_context_decode_kv_amd import kvdec
    return kvdec


def test_single_layer_4096(K):
    """32 query heads, 8 KV heads, head_dim 128, 4096 contiguous f16 cells."""
    c = Case(1001, 32, 8, 128, occupied=[4096])
    check(*c.run(K), *c.oracle())


def test_ragged_lengths_multi_slot(K):
    occ = [1, 2, 127, 128, 129, 255, 1000, 4099]
    begins = [5, 900, 0, 3000, 128, 17, 2000, 1]
    c = Case(11, 8, 2, 128, occupied=occ, begins=begins)
    check(*c.run(K), *c.oracle())


@pytest.mark.parametrize("d,g,kind,indirect", [(128, 4, O.F16, False), (128, 4, O.F16, True),
                                               (256, 6, O.Q8_B32, False), (256, 6, O.Q4_B32, True)])
def test_maximum_slot_count(K, d, g, kind, indirect):
    """KVDEC_MAX_SLOTS (64) slots in one launch, lengths 0 .. 1500 (empty
    slots, single cells, tile edges), contiguous or an indirect plan with
    shuffled records and duplicates; planner splits at 256 CUs."""
    r = np.random.default_rng(31 + d + kind)
    occ = [int(x) for x in r.choice([0, 1, 2, 127, 128, 129, 300, 700, 1500], size=64)]
    if indirect:
        c = Case(32 + d + kind, 2 * g, 2, d, kind=kind, indirect_lengths=occ, shuffle=True, duplicates=9)
    else:
        c = Case(33 + d + kind, 2 * g, 2, d, kind=kind, occupied=occ,
                 begins=[int(b) for b in np.cumsum([0] + occ[:-1])])
    assert c.n_slots == 64
    check(*c.run(K, n_cu=256), *c.oracle())


@pytest.mark.parametrize("d,g", [(64, 1), (64, 4), (64, 8), (128, 1), (128, 2), (128, 3), (128, 5), (128, 6),
                                 (128, 7), (128, 8), (256, 2), (256, 4), (256, 5), (256, 6), (256, 8),
                                 (128, 12), (128, 16), (256, 9), (256, 16)])
def test_group_sizes_and_head_dims(K, d, g):
    c = Case(20 + d + g, 2 * g, 2, d, occupied=[700, 1500])
    check(*c.run(K), *c.oracle())


def test_empty_slots(K):
    c = Case(12, 8, 2, 128, occupied=[0, 300, 0])
    out, lse = c.run(K)
    wo, wl = c.oracle()
    check(out, lse, wo, wl)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))


@pytest.mark.parametrize("kind", [O.F16, O.Q8_B32, O.Q4_B32], ids=["f16", "int8", "4bit"])
@pytest.mark.parametrize("indirect", [False, True], ids=["contiguous", "indirect"])
def test_no_device_cells_with_null_cache_arrays(K, kind, indirect):
    """capacity_cells 0: k, v, scales and plan_cells passed as NULL, every
    slot empty -- outputs are the empty result (0, lse -inf) and the
    partial triple the merge identity (m -inf, l 0, o 0)."""
    import torch
    d, hkv = (128, 8) if kind == O.F16 else (256, 4)
    hq = 4 * hkv
    kw = dict(cells=[[], [], []]) if indirect else dict(n_occupied=[0, 0, 0])
    p = K.plan(hq, hkv, d, 3, 0, k_type=kind, v_type=kind, n_cu=256, **kw)
    q = dev(np.random.default_rng(31).standard_normal((3, hq, d)).astype(np.float32))
    out = torch.full((3, hq, d), float("nan"), device="cuda")
    lse = torch.full((3, hq), float("nan"), device="cuda")
    pm, pl, po = (torch.full(s, float("nan"), device="cuda") for s in ((3, hq), (3, hq), (3, hq, d)))
    K.attend(p, q, 0, 0, K.workspace(p), out=out, lse=lse, part=(pm, pl, po))
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(torch.isneginf(pm)) and torch.all(pl == 0) and torch.all(po == 0)


@pytest.mark.parametrize("tps", [1, 2, 7, 100000])
def test_split_count_only_changes_rounding(K, tps):
    c = Case(13, 32, 8, 128, occupied=[13100])
    out, lse = c.run(K, tiles_per_split=tps)
    check(out, lse, *c.oracle())


@pytest.mark.parametrize("d,g", [(64, 2), (128, 1), (128, 4), (128, 5), (256, 2), (256, 4)])
@pytest.mark.parametrize("indirect", [False, True])
def test_long_f16_splits(K, d, g, indirect):
    """Splits of several steps, whose later steps are staged through LDS while
    the current one is computed; ragged last step, holes in indirect plans."""
    if indirect:
        c = Case(40 + d + g, 2 * g, 2, d, indirect_lengths=[2900, 1000, 3], shuffle=True, duplicates=7)
    else:
        c = Case(40 + d + g, 2 * g, 2, d, occupied=[2900, 1000, 3])
    check(*c.run(K, tiles_per_split=9), *c.oracle())


@pytest.mark.parametrize("split_cells", [32, 96, 224, 608])
@pytest.mark.parametrize("kind,d,g", [(O.F16, 128, 4), (O.Q8_B32, 128, 2), (O.Q4_B32, 64, 4), (O.F16, 256, 8),
                                      (O.Q8_B32, 256, 6)])
def test_split_boundaries_inside_tiles(K, split_cells, kind, d, g):
    """Splits of 32-cell multiples end inside 128-cell tiles on the
    vector-ALU kernel (whole tiles on the matrix-core kernel); contiguous
    and indirect slots with holes."""
    c = Case(70 + split_cells % 97 + d + g + kind, 2 * g, 2, d, kind=kind, occupied=[3000, 77, 1000])
    p = c.plan(K, split_cells=split_cells)
    assert p.info()["split_unit"] == (128 if p.info()["matrix_cores"] else 32)
    check(*c.run(K, plan=p), *c.oracle())
    ci = Case(71 + split_cells % 97 + d + g + kind, 2 * g, 2, d, kind=kind, indirect_lengths=[2500, 129, 1],
              shuffle=True, duplicates=5)
    check(*ci.run(K, split_cells=split_cells), *ci.oracle())


@pytest.mark.parametrize("d,g,hkv,occ", [(128, 4, 8, [13100]), (128, 1, 8, [12000]), (64, 5, 8, [26000]),
                                         (64, 2, 8, [26000]), (128, 3, 4, [900, 25000, 1])])
def test_eight_wave_workgroups(K, d, g, hkv, occ):
    """Short f16 contexts take one eight-wave workgroup per compute unit with
    two-step splits (512 cells at head_dim 128); ragged last split, a slot
    of one cell."""
    c = Case(500 + d + g + len(occ), g * hkv, hkv, d, occupied=occ)
    p = c.plan(K, n_cu=256, kernel=K.KERNEL_STREAMED)
    assert p.info()["waves"] == 8 and p.info()["kernel"] == K.KERNEL_STREAMED
    check(*c.run(K, plan=p), *c.oracle())


@pytest.mark.parametrize("hq,kind", [(48, O.F16), (64, O.F16), (48, O.Q8_B32), (40, O.F16), (128, O.F16),
                                     (128, O.Q4_B32)])
def test_matrix_core_four_tile_splits(K, hq, kind):
    """Wide groups on a 13100-cell layer: two-tile splits doubled to four
    (208 workgroups at 256 CUs); ragged last split.  Five f16 rows per KV
    head take the matrix-core kernel on a 16384-cell layer (at 13100 cells
    one one-shot split per compute unit covers it)."""
    c = Case(600 + hq + kind, hq, 8, 128, kind=kind, occupied=[16384 if hq == 40 else 13100])
    p = c.plan(K, n_cu=256)
    assert p.info()["matrix_cores"] == 1 and p.info()["tiles_per_split"] == 4
    assert p.info()["waves"] == (8 if hq == 128 else 4)
    check(*c.run(K, plan=p), *c.oracle())


@pytest.mark.parametrize("kind,vkind,indirect", [(O.F16, O.F16, False), (O.F16, O.F16, True),
                                                 (O.Q8_B32, O.Q4_B32, False), (O.Q8_B32, O.Q8_B32, True)])
def test_matrix_core_eight_wave_splits(K, kind, vkind, indirect):
    """16-head groups at head_dim 128 over short contexts: four-tile splits
    as two steps of an eight-wave workgroup; ragged slots (a ragged last
    step, a slot of one cell), contiguous or an indirect plan with shuffled
    records, duplicates and holes."""
    occ = [6000, 5000, 2100, 1]
    if indirect:
        c = Case(640 + kind + vkind, 128, 8, 128, kind=kind, v_kind=vkind, indirect_lengths=occ, shuffle=True,
                 duplicates=9)
    else:
        c = Case(650 + kind + vkind, 128, 8, 128, kind=kind, v_kind=vkind, occupied=occ,
                 begins=[0, 6100, 11200, 13400])
    p = c.plan(K, n_cu=256)
    info = p.info()
    assert info["matrix_cores"] == 1 and info["waves"] == 8 and info["tiles_per_split"] == 4
    check(*c.run(K, plan=p), *c.oracle())


@pytest.mark.parametrize("kind", [O.Q8_B32, O.Q4_B32])
def test_quantized_indirect_interleaved(K, kind):
    """GQA-6, head_dim 256, four slots whose 128-cell records are interleaved,
    raw lists shuffled with duplicates and holes."""
    c = Case(30 + kind, 24, 4, 256, kind=kind, indirect_lengths=[3000, 1500, 777, 1], shuffle=True, duplicates=25)
    check(*c.run(K), *c.oracle())


@pytest.mark.parametrize("kind", [O.Q8_B32, O.Q4_B32])
@pytest.mark.parametrize("d,g", [(128, 4), (128, 8), (64, 2), (256, 6)])
def test_quantized_contiguous(K, kind, d, g):
    c = Case(40 + kind + d + g, 2 * g, 2, d, kind=kind, occupied=[1000, 129])
    check(*c.run(K), *c.oracle())


def test_indirect_f16_with_empty_and_single_cells(K):
    c = Case(14, 16, 4, 128, kind=O.F16, indirect_lengths=[0, 1, 128, 129, 2000], shuffle=True, duplicates=3)
    out, lse = c.run(K)
    check(out, lse, *c.oracle())
    assert np.all(np.isneginf(lse[0]))


def test_peaked_softmax(K):
    """Each KV head's first query head has one cell whose K equals its query
    (rounded to f16): a dominant weight, as with a retrieved needle."""
    c = Case(15, 32, 8, 128, occupied=[13100], peaked=True)
    out, lse = c.run(K)
    wo, wl = c.oracle()
    check(out, lse, wo, wl)
    assert np.max(wl) > 8  # the planted cell dominates


def test_partials_merge_to_whole(K):
    import torch
    c = Case(16, 32, 8, 128, occupied=[5000])
    whole_out, whole_lse = c.run(K)
    # two disjoint ranges -> partials -> kvdec_merge
    c.upload()
    res = []
    for b, n in ((0, 1801), (1801, 3199)):
        p = K.plan(32, 8, 128, 1, c.capacity, n_occupied=[n], cell_begin=[b], scale=c.scale)
        parts = (torch.empty(1, 32, device="cuda"), torch.empty(1, 32, device="cuda"),
                 torch.empty(1, 32, 128, device="cuda"))
        K.attend(p, c.q_d, c.kc_d, c.vc_d, K.workspace(p), part=parts)
        res.append(parts)
    out = torch.empty(1, 32, 128, device="cuda")
    lse = torch.empty(1, 32, device="cuda")
    mm, ml, mo = torch.empty(1, 32, device="cuda"), torch.empty(1, 32, device="cuda"), torch.empty(1, 32, 128, device="cuda")
    K.merge(res, 32, 128, out=out, lse=lse, merged=(mm, ml, mo))
    torch.cuda.synchronize()
    wo, wl = c.oracle()
    check(out.cpu().numpy(), lse.cpu().numpy(), wo, wl)
    check(out.cpu().numpy(), lse.cpu().numpy(), whole_out, whole_lse, tol=TOL_SPLITS)
    # the merged partial reproduces out and lse
    mo_ = mo.cpu().numpy() / ml.cpu().numpy()[..., None]
    assert np.max(np.abs(mo_ - wo)) <= TOL
    assert np.max(np.abs(mm.cpu().numpy() + np.log(ml.cpu().numpy()) - wl)) <= TOL
    # each partial against the oracle's partial of its range
    for (b, n), (pm, pl, po) in zip(((0, 1801), (1801, 3199)), res):
        _, _, op = O.decode_attention(c.q, [((O.F16, c.kc, None), (O.F16, c.vc, None), [np.arange(b, b + n)])], 8,
                                      c.scale, return_partials=True)
        m, l, o = op[0]
        gm, gl, go = pm.cpu().numpy(), pl.cpu().numpy(), po.cpu().numpy()
        assert np.max(np.abs(gm - m)) <= TOL
        # l and o are relative to e^m; compare them rescaled to the oracle's m
        f = np.exp(gm - m)
        assert np.max(np.abs(gl * f / l - 1)) <= TOL
        assert np.max(np.abs(go * f[..., None] / l[..., None] - o / l[..., None])) <= TOL


def test_merge_empty_identity_and_all_empty(K):
    import torch
    rows, d = 5, 64
    r = np.random.default_rng(3)
    m = torch.tensor(r.standard_normal(rows), dtype=torch.float32, device="cuda")
    l = torch.tensor(r.uniform(0.5, 3, rows), dtype=torch.float32, device="cuda")
    o = torch.tensor(r.standard_normal((rows, d)), dtype=torch.float32, device="cuda")
    em = torch.full((rows,), float("-inf"), device="cuda")
    el = torch.zeros(rows, device="cuda")
    eo = torch.zeros(rows, d, device="cuda")
    out = torch.empty(rows, d, device="cuda")
    lse = torch.empty(rows, device="cuda")
    K.merge([(em, el, eo), (m, l, o), (em, el, eo)], rows, d, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.allclose(out, o / l[:, None], atol=1e-6)
    assert torch.allclose(lse, m + torch.log(l), atol=1e-6)
    K.merge([(em, el, eo), (em, el, eo)], rows, d, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_deterministic(K):
    c = Case(17, 32, 8, 128, occupied=[13100])
    a = c.run(K)
    b = c.run(K)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_head_major_strided_layout(K):
    """The same cache stored [kv head][cell][D] through explicit strides."""
    import torch
    c = Case(18, 16, 4, 128, occupied=[3000])
    want = c.run(K)
    p = c.plan(K)
    kh = dev(np.ascontiguousarray(c.kc.transpose(1, 0, 2)))
    vh = dev(np.ascontiguousarray(c.vc.transpose(1, 0, 2)))
    out = torch.empty(1, 16, 128, device="cuda")
    lse = torch.empty(1, 16, device="cuda")
    K.attend(p, c.q_d, kh, vh, K.workspace(p), out=out, lse=lse, k_cell_stride=256, k_head_stride=256 * c.capacity,
             v_cell_stride=256, v_head_stride=256 * c.capacity)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), want[0]) and np.array_equal(lse.cpu().numpy(), want[1])


def test_nan_poisoned_workspace_and_unused_cells(K):
    """Partial records start as NaN and every cell outside the attended set
    holds NaN: nothing of it may reach the output."""
    import torch
    c = Case(19, 24, 4, 256, kind=O.F16, indirect_lengths=[900, 300, 77], shuffle=True, duplicates=5)
    attended = np.zeros(c.capacity, dtype=bool)
    for cells in c.oracle_cells:
        attended[cells[cells >= 0]] = True
    nan16 = np.float16(np.nan).view(np.uint16)
    c.kc[~attended] = nan16
    c.vc[~attended] = nan16
    p = c.plan(K, tiles_per_split=1)
    ws = K.workspace(p)
    tb = p.info()["ticket_bytes"]  # the merge tickets stay zero, the rest is poisoned
    assert tb >= 128 * c.n_slots * c.hkv
    ws[tb:].view(torch.float32).fill_(float("nan"))
    out, lse = c.run(K, plan=p, ws=ws)
    check(out, lse, *c.oracle())


def test_workspace_reuse_across_plans(K):
    """One workspace serves consecutive calls with different plans; tickets
    are back at zero after every call."""
    import torch
    c1 = Case(21, 32, 8, 128, occupied=[6000])
    c2 = Case(22, 32, 8, 128, occupied=[300, 9000])
    p1, p2 = c1.plan(K, tiles_per_split=1), c2.plan(K, tiles_per_split=3)
    ws = K.workspace(p1) if p1.workspace_bytes >= p2.workspace_bytes else K.workspace(p2)
    for _ in range(2):
        check(*c1.run(K, plan=p1, ws=ws), *c1.oracle())
        check(*c2.run(K, plan=p2, ws=ws), *c2.oracle())
    tick = ws[:max(p1.info()["ticket_bytes"], p2.info()["ticket_bytes"])].view(torch.int32)
    assert int(tick.abs().sum()) == 0


@pytest.mark.parametrize("kind,d,g,occ", [(O.Q8_B32, 256, 6, [9000, 300]), (O.F16, 128, 4, [20000]),
                                          (O.F16, 128, 8, [9000, 1]), (O.Q4_B32, 256, 8, [6000])])
def test_two_level_merge(K, kind, d, g, occ):
    """One-tile splits: more splits per KV head than two merge rounds hold,
    so clusters of splits are merged first and the cluster records last."""
    c = Case(60 + d + g + kind, 2 * g, 2, d, kind=kind, occupied=occ)
    out, lse = c.run(K, tiles_per_split=1)
    check(out, lse, *c.oracle())
    # close to a plan whose splits merge in one level (f16 softmax weights
    # are rounded against each stream's own reference maximum, so different
    # split boundaries round differently)
    out1, lse1 = c.run(K, tiles_per_split=max(1, -(-max(occ) // 128) // 8))
    check(out, lse, out1, lse1, tol=1e-3)


MIXED = [(O.F16, O.Q8_B32), (O.F16, O.Q4_B32), (O.Q8_B32, O.Q4_B32)]


@pytest.mark.parametrize("kv", MIXED)
@pytest.mark.parametrize("d,g", [(64, 2), (128, 4), (128, 8), (256, 6)])
def test_mixed_kinds_contiguous(K, kv, d, g):
    """K stored more finely than V (the pages measure int8 K with 4-bit V):
    the VALU kernel (G <= 5) and the matrix-core kernel (G >= 6)."""
    kk, vk = kv
    c = Case(70 + 3 * kk + vk + d + g, 2 * g, 2, d, kind=kk, v_kind=vk, occupied=[1500, 333])
    check(*c.run(K), *c.oracle())


@pytest.mark.parametrize("kv", MIXED)
def test_mixed_kinds_indirect(K, kv):
    kk, vk = kv
    c = Case(80 + 3 * kk + vk, 24, 4, 256, kind=kk, v_kind=vk, indirect_lengths=[2000, 700, 5], shuffle=True,
             duplicates=9)
    check(*c.run(K), *c.oracle())
