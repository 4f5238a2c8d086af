"""Seeded random configurations through the C ABI against the float64 oracle:
head_dim, group size, storage kinds (mixed K / V included), slot count and
lengths, contiguous or indirect (shuffled records, duplicates, holes), and
the split choice (planner, tiles_per_split or split_cells, with n_cu 256 so
that the planner's regimes are the ones of the device); a second family is
sized for the planner's device-filling regimes and adds multi-query rows.
Every case is a fixed draw, so a failure names a reproducible configuration."""

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
