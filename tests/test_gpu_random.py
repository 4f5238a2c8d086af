"""Seeded random configurations through the C ABI against the float64 oracle:
head_dim, group size, storage kinds (mixed K / V included), slot count and
lengths, contiguous or indirect (shuffled records, duplicates, holes), and
the split choice (planner, tiles_per_split or split_cells, with n_cu 256 so
that the planner's regimes are the ones of the device).  Every case is a
fixed draw, so a failure names a reproducible configuration."""

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
