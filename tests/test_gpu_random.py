"""Seeded random configurations through the C ABI against the float64 oracle:
head_dim, group size, storage kinds (mixed K / V included), slot count and
lengths, contiguous or indirect (shuffled records, duplicates, holes), and
the split choice (planner, tiles_per_split or split_cells, with n_cu 256 so
that the planner's regimes are the ones of the device); a second family is
sized for the planner's device-filling regimes and adds multi-query rows; a
third places K and V with padded and head-major strides; a fourth merges
random partial sets with kvdec_merge.  Every case is a fixed draw, so a
failure names a reproducible configuration."""

import numpy as np
import pytest

import oracle as O
from gpu_cases import Case, check

pytestmark = pytest.mark.gpu

KIND_PAIRS = [(O.F16, O.F16), (O.Q8_B32, O.Q8_B32), (O.Q4_B32, O.Q4_B32), (O.F16, O.Q8_B32), (O.F16, O.Q4_B32),
              (O.Q8_B32, O.Q4_B32)]


def draw(seed):
    r = np.random.default_rng(9000 + seed)
    d = int(r.choice([64, 128, 256]))
    g_max = 8 if d == 64 else 16
    g = int(r.integers(1, g_max + 1))
    hkv = int(r.choice([1, 2, 4]))
    kind, vkind = KIND_PAIRS[int(r.integers(len(KIND_PAIRS)))]
    n_slots = int(r.integers(1, 5))
    lengths = [int(x) for x in r.choice([0, 1, 7, 128, 129, 300, 1000, 2500, 5000], size=n_slots)]
    indirect = bool(r.integers(2))
    split = [{}, {"tiles_per_split": int(r.integers(1, 12))}, {"split_cells": 32 * int(r.integers(1, 40))}][
        int(r.integers(3))]
    return d, g, hkv, kind, vkind, lengths, indirect, split


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available()
    from long_context_decode_kv_amd import kvdec
    return kvdec


@pytest.mark.parametrize("seed", range(48))
def test_random_configuration(K, seed):
    d, g, hkv, kind, vkind, lengths, indirect, split = draw(seed)
    if indirect:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, indirect_lengths=lengths, shuffle=True,
                 duplicates=int(seed % 3) * 4)
    else:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, occupied=lengths,
                 begins=list(np.cumsum([0] + lengths[:-1]) + 3 * seed))
    p = c.plan(K, n_cu=256, **split)
    info = p.info()
    check(*c.run(K, plan=p), *c.oracle())
    assert info["n_workgroups"] >= 1


def draw_filling(seed):
    """Configurations sized so that each of the planner's device-filling
    regimes at 256 CUs applies, in turn by seed: short f16 contexts on
    eight-wave vector-ALU workgroups, 16-row records on eight-wave
    matrix-core workgroups (16-head groups, or 4 heads x 4 query rows),
    long staged f16 splits, and general sizes (any head_dim, kinds, 1-3
    slots, sometimes 2 or 4 query rows)."""
    r = np.random.default_rng(77000 + seed)
    regime = seed % 4
    kind, vkind = KIND_PAIRS[int(r.integers(len(KIND_PAIRS)))]
    n_q = 1
    if regime == 0:
        d, g, hkv, kind, vkind = int(r.choice([64, 128])), int(r.integers(1, 6)), 8, 0, 0
        lengths = [int(r.integers(12000, 16000))]
    elif regime == 1:
        d, hkv = 128, 8
        g, n_q = (16, 1) if r.integers(2) else (4, 4)
        lengths = [int(r.integers(11000, 15000))]
    elif regime == 2:
        d, g, hkv, kind, vkind = 128, int(r.integers(1, 6)), 4, 0, 0
        lengths = [int(r.integers(40000, 60000))]
    else:
        d = int(r.choice([64, 128, 256]))
        g = int(r.integers(1, (8 if d == 64 else 16) + 1))
        hkv = int(r.choice([4, 8]))
        n_slots = int(r.integers(1, 4))
        total = int(r.integers(3000, 30000 if d < 256 else 12000))
        cuts = np.sort(r.integers(0, total, size=n_slots - 1))
        lengths = [int(x) for x in np.diff(np.concatenate([[0], cuts, [total]]))]
        n_q = int(r.choice([1, 1, 2, 4])) if d >= 128 else 1
        if g * n_q > 16:
            n_q = 1
    indirect = bool(r.integers(2)) if regime != 2 else False
    return d, g, hkv, kind, vkind, lengths, indirect, n_q


@pytest.mark.parametrize("seed", range(24))
def test_random_device_filling_configuration(K, seed):
    import torch
    from gpu_cases import dev
    d, g, hkv, kind, vkind, lengths, indirect, n_q = draw_filling(seed)
    if indirect:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, indirect_lengths=lengths, shuffle=True,
                 duplicates=int(seed % 3) * 4)
    else:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, occupied=lengths,
                 begins=list(np.cumsum([0] + lengths[:-1]) + 3 * (seed % 7)))
    if n_q == 1:
        check(*c.run(K, n_cu=256), *c.oracle())
        return
    p = c.plan(K, n_cu=256, n_queries=n_q)
    r = np.random.default_rng(seed)
    q = r.standard_normal((c.n_slots, n_q, c.hq, c.d)).astype(np.float32)
    qp = r.integers(-5, c.capacity + 5, size=(c.n_slots, n_q)).astype(np.int32)
    c.upload()
    out = torch.full((c.n_slots, n_q, c.hq, c.d), float("nan"), device="cuda")
    lse = torch.full((c.n_slots, n_q, c.hq), float("nan"), device="cuda")
    pc = None if c.raw is None else dev(p.cells()[0])
    K.attend(p, dev(q), c.kc_d, c.vc_d, K.workspace(p), out=out, lse=lse, k_scales=c.ks_d, v_scales=c.vs_d,
             plan_cells=pc, q_pos=dev(qp))
    torch.cuda.synchronize()
    want = O.decode_attention_multi(q, [((c.kind, c.kc, c.ks), (c.vkind, c.vc, c.vs), c.oracle_cells)], c.hkv,
                                    c.scale, qp, None)
    check(out.cpu().numpy(), lse.cpu().numpy(), *want)


def place_rows(x, layout, r):
    """The rows of a dense [cell][kv head][row] device array copied into a
    byte buffer with other strides: 'padded' (gaps after each row and each
    cell) or 'headmajor' ([kv head][cell][row], a gap after each head).
    Returns (buffer, cell stride, head stride) in bytes."""
    import torch
    cells, heads = x.shape[0], x.shape[1]
    xb = x.contiguous().view(torch.uint8).view(cells, heads, -1)
    rb = xb.shape[2]
    if layout == "padded":
        hs = rb + 16 * int(r.integers(0, 3))
        cs = hs * heads + 16 * int(r.integers(0, 4))
    else:
        cs, hs = rb, rb * cells + 16 * int(r.integers(0, 2))
    buf = torch.zeros(max(cs * cells, hs * heads) + 64, dtype=torch.uint8, device="cuda")
    for h in range(heads):
        idx = (torch.arange(cells, device="cuda") * cs + h * hs)[:, None] + torch.arange(rb, device="cuda")[None]
        buf[idx.view(-1)] = xb[:, h, :].reshape(-1)
    return buf, cs, hs


@pytest.mark.parametrize("seed", range(16))
def test_random_configuration_strided_layouts(K, seed):
    """A random configuration (draw) with K and V placed densely, with padded
    row and cell strides, and head-major: the three results are bit-equal
    (the same rows, read through the strides) and match the oracle."""
    import torch
    from gpu_cases import dev
    d, g, hkv, kind, vkind, lengths, indirect, split = draw(3000 + seed)
    if indirect:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, indirect_lengths=lengths, shuffle=True)
    else:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, occupied=lengths)
    p = c.plan(K, n_cu=256, **split)
    c.upload()
    pc = None if c.raw is None else dev(p.cells()[0])
    r = np.random.default_rng(seed)
    outs = []
    for layout in ("dense", "padded", "headmajor"):
        kk, vv, kw = c.kc_d, c.vc_d, {}
        if layout != "dense" and c.capacity > 0:
            kk, kcs, khs = place_rows(c.kc_d, layout, r)
            vv, vcs, vhs = place_rows(c.vc_d, layout, r)
            kw = dict(k_cell_stride=kcs, k_head_stride=khs, v_cell_stride=vcs, v_head_stride=vhs)
        out = torch.full((c.n_slots, c.hq, c.d), float("nan"), device="cuda")
        lse = torch.full((c.n_slots, c.hq), float("nan"), device="cuda")
        K.attend(p, c.q_d, kk, vv, K.workspace(p), out=out, lse=lse, k_scales=c.ks_d, v_scales=c.vs_d,
                 plan_cells=pc, **kw)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0]) and np.array_equal(o[1], outs[0][1])
    check(*outs[0], *c.oracle())


@pytest.mark.parametrize("seed", range(16))
def test_random_standalone_merge(K, seed):
    """kvdec_merge of 1-8 random partial sets (rows empty in some sets or in
    all, maxima spread over small and large ranges) against the float64
    log-sum-exp merge."""
    import torch
    from gpu_cases import dev
    r = np.random.default_rng(80000 + seed)
    n_parts, rows, d = int(r.integers(1, 9)), int(r.integers(1, 300)), int(r.choice([64, 128, 256]))
    ms, ls, os_ = [], [], []
    for _ in range(n_parts):
        m = (r.normal(size=rows) * float(r.choice([0.1, 3, 30]))).astype(np.float32)
        l = r.uniform(0.5, 4, size=rows).astype(np.float32)
        empty = r.random(rows) < 0.2
        m[empty], l[empty] = -np.inf, 0
        o = (r.normal(size=(rows, d)) * l[:, None]).astype(np.float32)
        o[empty] = 0
        ms.append(m), ls.append(l), os_.append(o)
    M = np.max(np.stack(ms).astype(np.float64), axis=0)
    Mf = np.where(np.isneginf(M), 0.0, M)
    w = [np.where(np.isneginf(m), 0.0, np.exp(m.astype(np.float64) - Mf)) for m in ms]
    L = sum(l * wi for l, wi in zip(ls, w))
    Ov = sum(o * wi[:, None] for o, wi in zip(os_, w))
    Ls = np.where(L > 0, L, 1.0)
    want_o = np.where(L[:, None] > 0, Ov / Ls[:, None], 0.0)
    want_l = np.where(L > 0, M + np.log(Ls), -np.inf)
    out, lse = torch.empty(rows, d, device="cuda"), torch.empty(rows, device="cuda")
    K.merge([(dev(m), dev(l), dev(o)) for m, l, o in zip(ms, ls, os_)], rows, d, out=out, lse=lse)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), lse.cpu().numpy(), want_o, want_l)
