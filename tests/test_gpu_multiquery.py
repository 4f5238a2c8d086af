"""GPU parity of multi-query decode attention (several query rows per slot
with a positional mask, as in speculative verification): the HIP path through
the C ABI against the float64 oracle's decode_attention_multi, element by
element, max |err| <= 2e-3 on out and lse."""

import numpy as np
import pytest

import oracle as O
from gpu_cases import Case, check, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available()
    from long_context_decode_kv_amd import kvdec
    return kvdec


def causal_q_pos(c, n_q):
    """Query rows are the slot's last n_q cells (contiguous slots): row t sits
    at the cell index of the (n - n_q + t)-th occupied cell."""
    return np.array([[b + n - n_q + t for t in range(n_q)] for b, n in zip(c.begins, c.occupied)], dtype=np.int32)


def run_mq(K, c, n_q, q, q_pos, cell_pos=None, **kw):
    import torch
    p = c.plan(K, n_queries=n_q, **kw)
    assert p.info()["matrix_cores"] == 1
    c.upload()
    out = torch.full((c.n_slots, n_q, c.hq, c.d), float("nan"), device="cuda")
    lse = torch.full((c.n_slots, n_q, c.hq), float("nan"), device="cuda")
    pc = None if c.raw is None else dev(p.cells()[0])
    K.attend(p, dev(q), c.kc_d, c.vc_d, K.workspace(p), out=out, lse=lse, k_scales=c.ks_d, v_scales=c.vs_d,
             plan_cells=pc, q_pos=dev(q_pos), cell_pos=None if cell_pos is None else dev(cell_pos))
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle_mq(c, q, q_pos, cell_pos=None):
    return O.decode_attention_multi(q, [((c.kind, c.kc, c.ks), (c.vkind, c.vc, c.vs), c.oracle_cells)], c.hkv,
                                    c.scale, q_pos, cell_pos)


def mq_q(seed, c, n_q):
    r = np.random.default_rng(seed)
    return r.standard_normal((c.n_slots, n_q, c.hq, c.d)).astype(np.float32)


@pytest.mark.parametrize("g,n_q,d,kind,vkind", [
    (4, 4, 128, O.F16, O.F16),      # 16 rows
    (4, 2, 128, O.F16, O.F16),      # 8 rows
    (1, 8, 256, O.Q8_B32, O.Q8_B32),
    (8, 2, 128, O.Q4_B32, O.Q4_B32),
    (3, 5, 128, O.Q8_B32, O.Q4_B32),  # 15 rows
    (6, 2, 256, O.F16, O.Q8_B32),
    (2, 3, 256, O.Q4_B32, O.Q4_B32),
])
def test_causal_contiguous(K, g, n_q, d, kind, vkind):
    c = Case(200 + g * 10 + n_q + d, 2 * g, 2, d, kind=kind, v_kind=vkind, occupied=[1500, 300], begins=[0, 1700])
    q = mq_q(1, c, n_q)
    qp = causal_q_pos(c, n_q)
    out, lse = run_mq(K, c, n_q, q, qp)
    check(out, lse, *oracle_mq(c, q, qp))


def test_mask_positions_and_empty_rows(K):
    """Query positions spread over the slot (rows see 0, a few, half, all
    cells); a row before every cell gets out 0 and lse -inf."""
    c = Case(230, 16, 4, 128, occupied=[2000])
    q = mq_q(2, c, 4)
    qp = np.array([[-5, 3, 999, 5000]], dtype=np.int32)
    out, lse = run_mq(K, c, 4, q, qp)
    want = oracle_mq(c, q, qp)
    check(out, lse, *want)
    assert np.all(out[0, 0] == 0) and np.all(np.isneginf(lse[0, 0]))


@pytest.mark.parametrize("kind,vkind", [(O.F16, O.F16), (O.Q8_B32, O.Q4_B32)])
def test_indirect_with_cell_positions(K, kind, vkind):
    """Record-grouped indirect plan (shuffled raw lists, duplicates, holes)
    with explicit cell positions (a random permutation): the mask follows the
    positions, not the cell order."""
    c = Case(240 + kind, 24, 4, 256, kind=kind, v_kind=vkind, indirect_lengths=[1500, 600, 3], shuffle=True,
             duplicates=7)
    r = np.random.default_rng(3)
    cell_pos = (r.permutation(c.capacity) + 100).astype(np.int32)
    q = mq_q(4, c, 2)
    qp = np.array([[100 + c.capacity // 2, 100 + c.capacity], [100 + c.capacity // 3, 99], [1 << 30, 120]],
                  dtype=np.int32)
    out, lse = run_mq(K, c, 2, q, qp, cell_pos)
    check(out, lse, *oracle_mq(c, q, qp, cell_pos))


@pytest.mark.parametrize("kind,vkind,n_q,g", [(O.F16, O.F16, 4, 4), (O.Q8_B32, O.Q4_B32, 2, 8)])
def test_eight_wave_indirect_with_cell_positions(K, kind, vkind, n_q, g):
    """16-row records at head_dim 128 over a short context: the planner's
    four-tile splits on eight-wave workgroups, with a shuffled record plan
    (duplicates, holes) and explicit cell positions."""
    c = Case(280 + n_q, 8 * g, 8, 128, kind=kind, v_kind=vkind, indirect_lengths=[9000, 3000, 1], shuffle=True,
             duplicates=11)
    p = c.plan(K, n_queries=n_q, n_cu=256)
    assert p.info()["waves"] == 8 and p.info()["tiles_per_split"] == 4
    r = np.random.default_rng(8)
    cell_pos = r.permutation(c.capacity).astype(np.int32)
    q = mq_q(9, c, n_q)
    qp = r.integers(-10, c.capacity + 10, size=(c.n_slots, n_q)).astype(np.int32)
    qp[0, 0] = c.capacity  # a row that sees every cell
    out, lse = run_mq(K, c, n_q, q, qp, cell_pos, n_cu=256)
    check(out, lse, *oracle_mq(c, q, qp, cell_pos))


@pytest.mark.parametrize("d,kind", [(256, O.Q8_B32), (128, O.F16)])
def test_two_level_merge_of_16_row_records(K, d, kind):
    """One-tile splits: 16-row records merged through clusters."""
    c = Case(250 + d, 16, 4, d, kind=kind, occupied=[7000])
    q = mq_q(5, c, 4)
    qp = causal_q_pos(c, 4)
    out, lse = run_mq(K, c, 4, q, qp, tiles_per_split=1)
    check(out, lse, *oracle_mq(c, q, qp))


def test_single_query_rows_equal_multi_query_rows(K):
    """With every cell visible, each multi-query row matches the one-row call
    on the same q row (different kernels, same attention)."""
    import torch
    c = Case(260, 32, 8, 128, occupied=[3000])
    q = mq_q(6, c, 2)
    qp = np.full((1, 2), 1 << 30, dtype=np.int32)
    out, lse = run_mq(K, c, 2, q, qp)
    for t in range(2):
        c.q = q[:, t].copy()
        c.upload()
        o1, l1 = c.run(K)
        check(out[:, t], lse[:, t], o1, l1, tol=1e-3)


def test_window_plus_tail_multi_query(K):
    """Resident window + host tail with 4 query rows: tail cells keep their
    tail index as position, window cells their cell index."""
    import torch
    from test_gpu_tail import pinned
    n, t_cells, n_q = 5000, 3100, 4
    c = Case(270, 32, 8, 128, occupied=[n])
    q = mq_q(7, c, n_q)
    qp = np.array([[n - n_q + t for t in range(n_q)]], dtype=np.int32)
    qp[0, 0] = 2000  # one row that sees only part of the tail
    p = K.plan(32, 8, 128, 1, c.capacity, n_occupied=[n - t_cells], cell_begin=[t_cells], n_tail=[t_cells],
               tail_capacity_cells=t_cells, tail_chunk_cells=512, tail_ring_depth=3, n_queries=n_q, scale=c.scale)
    c.upload()
    hk, hv = pinned(c.kc[:t_cells]), pinned(c.vc[:t_cells])
    out = torch.full((1, n_q, 32, 128), float("nan"), device="cuda")
    lse = torch.full((1, n_q, 32), float("nan"), device="cuda")
    K.attend(p, dev(q), c.kc_d, c.vc_d, K.workspace(p), out=out, lse=lse, k_tail=hk, v_tail=hv, q_pos=dev(qp),
             copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    check(out.cpu().numpy(), lse.cpu().numpy(), *oracle_mq(c, q, qp))


MQ_KIND_PAIRS = [(O.F16, O.F16), (O.Q8_B32, O.Q8_B32), (O.Q4_B32, O.Q4_B32), (O.F16, O.Q8_B32),
                 (O.F16, O.Q4_B32), (O.Q8_B32, O.Q4_B32)]


@pytest.mark.parametrize("seed", range(24))
def test_random_multi_query_configuration(K, seed):
    """Seeded random multi-query calls: head_dim, 2-8 query rows, group size
    (rows per KV head at most 16), KV heads, storage kinds, 1-3 slots of
    assorted lengths, contiguous or indirect (with or without cell
    positions), the planner's split or a forced one, and query positions
    causal or anywhere (before the first cell, past the last)."""
    r = np.random.default_rng(60000 + seed)
    d = int(r.choice([128, 256]))
    n_q = int(r.integers(2, 9))
    g = int(r.integers(1, 16 // n_q + 1))
    hkv = int(r.choice([1, 2, 4, 8]))
    kind, vkind = MQ_KIND_PAIRS[int(r.integers(len(MQ_KIND_PAIRS)))]
    n_slots = int(r.integers(1, 4))
    lens = [int(x) for x in r.choice([0, 1, 5, 128, 129, 700, 3000, 9000], size=n_slots)]
    indirect = bool(r.integers(2))
    use_cell_pos = indirect and bool(r.integers(2))
    split = [{}, {"tiles_per_split": int(r.integers(1, 9))}][int(r.integers(2))]
    if indirect:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, indirect_lengths=lens, shuffle=True)
    else:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, occupied=lens,
                 begins=list(np.cumsum([0] + lens[:-1]) + int(r.integers(0, 50))))
    q = mq_q(seed, c, n_q)
    cell_pos = None
    if use_cell_pos:
        cell_pos = r.permutation(c.capacity).astype(np.int32)
        q_pos = r.integers(-3, c.capacity + 3, size=(c.n_slots, n_q)).astype(np.int32)
    elif indirect or not r.integers(2):
        q_pos = r.integers(-3, c.capacity + 3, size=(c.n_slots, n_q)).astype(np.int32)
    else:
        q_pos = causal_q_pos(c, n_q)
    got = run_mq(K, c, n_q, q, q_pos, cell_pos=cell_pos, n_cu=256, **split)
    want = oracle_mq(c, q, q_pos, cell_pos)
    check(got[0].reshape(want[0].shape), got[1].reshape(want[1].shape), *want)
