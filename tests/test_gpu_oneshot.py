"""GPU parity of the one-shot split kernel (every load of a split issued at
workgroup entry; head_dim 128, f16 K and V, G <= 5, contiguous cells)
against the float64 oracle: every split length a wave can hold (partial
waves, odd counts, the 448-cell maximum), forced split sizes covering each
compiled loads-per-lane instance, all group sizes, 1 to 8 KV heads, several slots, the
device-filling plan of the Qwen3-8B-shaped layer, needles, partial outputs,
strided layouts, poisoned unattended cells, a window with a host tail, an
8-byte-aligned q and graph replays."""

import numpy as np
import pytest

import oracle as O
from gpu_cases import TOL, Case, check, dev, TOL_SPLITS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available()
    from long_context_decode_kv_amd import kvdec
    return kvdec


def oneshot_plan(K, c, **kw):
    p = c.plan(K, kernel=K.KERNEL_ONESHOT, **kw)
    assert p.info()["kernel"] == K.KERNEL_ONESHOT and p.info()["waves"] == 8
    return p


@pytest.mark.parametrize("n", [1, 2, 3, 7, 8, 9, 15, 16, 17, 63, 64, 65, 127, 129, 255, 447, 448])
def test_single_split_lengths(K, n):
    """One split per KV head holding n cells: waves with partial loads, odd
    cell counts (a pair with one real cell), empty waves."""
    c = Case(1100 + n, 32, 8, 128, occupied=[n])
    p = oneshot_plan(K, c, split_cells=448)
    assert p.info()["n_workgroups"] == 8
    check(*c.run(K, plan=p), *c.oracle())


@pytest.mark.parametrize("split_cells", [32, 64, 96, 128, 160, 224, 256, 288, 384, 416, 448])
def test_forced_split_sizes(K, split_cells):
    """Each loads-per-lane instance (splits up to 128, 256, 448 cells) with
    a ragged last split and more splits than one merge round holds."""
    c = Case(1200 + split_cells, 16, 4, 128, occupied=[5003])
    p = oneshot_plan(K, c, split_cells=split_cells)
    assert p.info()["split_cells"] == split_cells
    check(*c.run(K, plan=p), *c.oracle())


@pytest.mark.parametrize("g", [1, 2, 3, 4, 5])
def test_group_sizes_device_filling(K, g):
    """The planner's own choice on a 13100-cell layer of 8 KV heads: one
    split per compute unit."""
    c = Case(1300 + g, 8 * g, 8, 128, occupied=[13100])
    p = c.plan(K, n_cu=256)
    info = p.info()
    assert info["kernel"] == K.KERNEL_ONESHOT and info["n_workgroups"] == 256 and info["split_cells"] == 416
    check(*c.run(K, plan=p), *c.oracle())


@pytest.mark.parametrize("hkv", [1, 2, 3, 5, 6, 7])
def test_kv_head_counts_device_filling(K, hkv):
    """The planner's own choice for 1 to 7 KV heads of 4 query heads each
    on a 6000-cell layer.  Workgroup b runs on XCD b mod 8 and reads KV head
    b mod hkv, so with fewer than 8 KV heads the splits of one head run on
    several XCDs and publish and count their records across them; one KV
    head (94 splits of 64 cells) also takes the two-level merge."""
    c = Case(1310 + hkv, 4 * hkv, hkv, 128, occupied=[6000])
    p = c.plan(K, n_cu=256)
    info = p.info()
    assert info["kernel"] == K.KERNEL_ONESHOT and info["n_workgroups"] <= 256
    per_head = np.bincount(p.splits()[:, 1], minlength=hkv)
    assert np.all(per_head == per_head[0]) and per_head[0] > 8, per_head
    check(*c.run(K, plan=p), *c.oracle())


def test_multi_slot_with_empty_and_single_cells(K):
    c = Case(1401, 16, 4, 128, occupied=[900, 5000, 1, 0, 129], begins=[0, 1000, 6100, 6200, 6300])
    p = oneshot_plan(K, c, split_cells=448)
    out, lse = c.run(K, plan=p)
    check(out, lse, *c.oracle())
    assert np.all(out[3] == 0) and np.all(np.isneginf(lse[3]))


def test_peaked_softmax(K):
    c = Case(1402, 32, 8, 128, occupied=[13100], peaked=True)
    p = c.plan(K, n_cu=256)
    assert p.info()["kernel"] == K.KERNEL_ONESHOT
    out, lse = c.run(K, plan=p)
    wo, wl = c.oracle()
    check(out, lse, wo, wl)
    assert np.max(wl) > 8


def test_matches_streamed_kernel(K):
    """Both vector-ALU kernels on the same 13100-cell layer: close to each
    other (the f16 softmax weights are rounded against each stream's own
    maximum -- per wave here, per cell stream there -- so they differ by a
    re-weighting of up to 2^-11 per weight) and each within the bound of the
    oracle."""
    c = Case(1403, 32, 8, 128, occupied=[13100])
    a = c.run(K, plan=c.plan(K, n_cu=256))
    b = c.run(K, plan=c.plan(K, n_cu=256, kernel=K.KERNEL_STREAMED))
    check(a[0], a[1], b[0], b[1], tol=TOL_SPLITS)
    check(*a, *c.oracle())
    check(*b, *c.oracle())


def test_partials_merge_to_whole(K):
    import torch
    c = Case(1404, 32, 8, 128, occupied=[9000])
    c.upload()
    res = []
    for b, n in ((0, 4001), (4001, 4999)):
        p = K.plan(32, 8, 128, 1, c.capacity, n_occupied=[n], cell_begin=[b], scale=c.scale, n_cu=256)
        assert p.info()["kernel"] == K.KERNEL_ONESHOT
        parts = (torch.empty(1, 32, device="cuda"), torch.empty(1, 32, device="cuda"),
                 torch.empty(1, 32, 128, device="cuda"))
        K.attend(p, c.q_d, c.kc_d, c.vc_d, K.workspace(p), part=parts)
        res.append(parts)
    out = torch.empty(1, 32, 128, device="cuda")
    lse = torch.empty(1, 32, device="cuda")
    K.merge(res, 32, 128, out=out, lse=lse)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), lse.cpu().numpy(), *c.oracle())
    for (b, n), (pm, pl, po) in zip(((0, 4001), (4001, 4999)), res):
        _, _, op = O.decode_attention(c.q, [((O.F16, c.kc, None), (O.F16, c.vc, None), [np.arange(b, b + n)])], 8,
                                      c.scale, return_partials=True)
        m, l, o = op[0]
        gm, gl, go = pm.cpu().numpy(), pl.cpu().numpy(), po.cpu().numpy()
        assert np.max(np.abs(gm - m)) <= TOL
        f = np.exp(gm - m)
        assert np.max(np.abs(gl * f / l - 1)) <= TOL
        assert np.max(np.abs(go * f[..., None] / l[..., None] - o / l[..., None])) <= TOL


def test_head_major_strided_layout(K):
    """[kv head][cell][D] through explicit strides: bit-equal to the dense layout."""
    import torch
    c = Case(1405, 32, 8, 128, occupied=[6000])
    p = c.plan(K, n_cu=256)
    assert p.info()["kernel"] == K.KERNEL_ONESHOT
    want = c.run(K, plan=p)
    kh = dev(np.ascontiguousarray(c.kc.transpose(1, 0, 2)))
    vh = dev(np.ascontiguousarray(c.vc.transpose(1, 0, 2)))
    out = torch.empty(1, 32, 128, device="cuda")
    lse = torch.empty(1, 32, device="cuda")
    K.attend(p, c.q_d, kh, vh, K.workspace(p), out=out, lse=lse, k_cell_stride=256, k_head_stride=256 * c.capacity,
             v_cell_stride=256, v_head_stride=256 * c.capacity)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), want[0]) and np.array_equal(lse.cpu().numpy(), want[1])


def test_nan_poisoned_workspace_and_unattended_cells(K):
    """Cells outside the slots' ranges hold NaN and the partial records start
    as NaN: nothing of it may reach the outputs."""
    import torch
    c = Case(1406, 32, 8, 128, occupied=[3000, 2000], begins=[100, 3300], capacity=5500)
    nan16 = np.float16(np.nan).view(np.uint16)
    keep = np.zeros(c.capacity, dtype=bool)
    keep[100:3100] = True
    keep[3300:5300] = True
    c.kc[~keep] = nan16
    c.vc[~keep] = nan16
    p = c.plan(K, n_cu=256)
    assert p.info()["kernel"] == K.KERNEL_ONESHOT
    ws = K.workspace(p)
    tb = p.info()["ticket_bytes"]  # the merge tickets stay zero, the rest is poisoned
    assert tb >= 128 * c.n_slots * c.hkv
    ws[tb:].view(torch.float32).fill_(float("nan"))
    check(*c.run(K, plan=p, ws=ws), *c.oracle())


def test_q_aligned_to_8_bytes(K):
    """q only 8-byte aligned (the binding's minimum): the one-shot kernel
    reads it in 8-byte pieces."""
    import torch
    c = Case(1407, 32, 8, 128, occupied=[7000])
    p = c.plan(K, n_cu=256)
    assert p.info()["kernel"] == K.KERNEL_ONESHOT
    c.upload()
    buf = torch.empty(c.q_d.numel() + 2, device="cuda")
    q8 = buf[2:].view(c.q_d.shape)
    q8.copy_(c.q_d)
    assert q8.data_ptr() % 16 == 8
    out = torch.empty(1, 32, 128, device="cuda")
    lse = torch.empty(1, 32, device="cuda")
    K.attend(p, q8, c.kc_d, c.vc_d, K.workspace(p), out=out, lse=lse)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), lse.cpu().numpy(), *c.oracle())


def test_graph_replays_equal_eager(K):
    import torch
    c = Case(1408, 32, 8, 128, occupied=[13100])
    p = c.plan(K, n_cu=256)
    assert p.info()["kernel"] == K.KERNEL_ONESHOT
    c.upload()
    ws = K.workspace(p)
    qs = [c.q_d, (c.q_d * 0.5).contiguous(), (-c.q_d).contiguous()]
    outs = [torch.empty(1, 32, 128, device="cuda") for _ in qs]
    lses = [torch.empty(1, 32, device="cuda") for _ in qs]

    def seq():
        for q, o, l in zip(qs, outs, lses):
            K.attend(p, q, c.kc_d, c.vc_d, ws, out=o, lse=l)

    seq()
    torch.cuda.synchronize()
    eager = [(o.clone(), l.clone()) for o, l in zip(outs, lses)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for (eo, el), o, l in zip(eager, outs, lses):
            assert torch.equal(o, eo) and torch.equal(l, el)
    check(eager[0][0].cpu().numpy(), eager[0][1].cpu().numpy(), *c.oracle())
