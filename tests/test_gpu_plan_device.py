"""GPU checks of the device-built indirect plan (kvdec_build_cells): the
entries are bit-exact against the oracle's compact plan of the same raw lists
(padded with -1 segments up to each slot's record budget), the record counts
and dropped entries are reported, and attention through the device-built
plan matches the float64 oracle."""

import numpy as np
import pytest

import oracle as O
from gpu_cases import Case, check, dev
from long_context_decode_kv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available()
    from long_context_decode_kv_amd import kvdec
    return kvdec


def flat(lists):
    off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int64)
    cells = np.concatenate([np.asarray(x, np.int32) for x in lists]) if off[-1] else np.zeros(1, np.int32)
    return cells, off


def build(K, lists, capacity, max_records, hq=24, hkv=4, d=256, kind=O.Q8_B32):
    import torch
    p = K.plan(hq, hkv, d, len(lists), capacity, k_type=kind, v_type=kind, max_records=max_records)
    ws = K.workspace(p)
    cells, off = flat(lists)
    out = torch.full((max(1, p.info()["n_entries"]),), 12345, dtype=torch.int32, device="cuda")
    nrec = torch.full((len(lists) + 1,), -7, dtype=torch.int32, device="cuda")
    K.build_cells(p, dev(cells), dev(off), out, ws, n_records=nrec)
    torch.cuda.synchronize()
    return p, ws, out.cpu().numpy()[:p.info()["n_entries"]], nrec.cpu().numpy()


def expected(lists, capacity, max_records):
    """Oracle compact plan of the in-range entries, each slot padded (or cut)
    to its record budget."""
    want, counts = [], []
    for raw, m in zip(lists, max_records):
        keep = [c for c in raw if -1 <= c < capacity]
        entries, _ = O.compact_plan([keep], capacity)
        n_rec = len(entries) // 128
        counts.append(n_rec)
        seg = entries[:m * 128]
        want.append(np.concatenate([seg, np.full(m * 128 - len(seg), -1, np.int32)]))
    return np.concatenate(want) if want else np.zeros(0, np.int32), counts


def test_entries_bit_exact_against_oracle(K):
    r = synth.rng(300)
    lists, cap = synth.interleaved_record_lists([3000, 1500, 200, 0, 129], r, shuffle=True, duplicates=40)
    lists = [list(x) for x in lists]
    lists[1] += [cap + 5, -3, cap]        # dropped: out of range
    lists[2] += [-1, -1]
    budget = [-(-3000 // 128) + 2, -(-1500 // 128), -(-200 // 128) + 5, 1, 2]
    _, _, got, nrec = build(K, lists, cap, budget)
    want, counts = expected(lists, cap, budget)
    assert np.array_equal(got, want)
    assert list(nrec[:5]) == counts and nrec[5] == 3


def test_budget_overflow_keeps_lowest_records_and_reports_count(K):
    r = synth.rng(301)
    raw = r.permutation(5000)[:3000].tolist()
    budget = [7]
    _, _, got, nrec = build(K, [raw], 5000, budget)
    want, counts = expected([raw], 5000, budget)
    assert np.array_equal(got, want)
    assert nrec[0] == counts[0] > 7


def test_attend_through_device_built_plan_and_rebuild(K):
    """Attention through the device-built plan equals the oracle; rebuilding
    with changed lists on the same workspace (a plan that changes every step)
    stays exact."""
    import torch
    c = Case(302, 24, 4, 256, kind=O.Q8_B32, indirect_lengths=[2500, 800, 7], shuffle=True, duplicates=11)
    budget = [-(-2500 // 128) + 3, -(-800 // 128) + 1, 2]
    p = K.plan(24, 4, 256, 3, c.capacity, k_type=O.Q8_B32, v_type=O.Q8_B32, scale=c.scale, max_records=budget)
    ws = K.workspace(p)
    c.upload()
    entries = torch.empty(p.info()["n_entries"], dtype=torch.int32, device="cuda")
    for step in range(2):
        lists = [list(x) for x in c.raw]
        if step == 1:  # the next step: one more cell per slot, one cell dropped
            lists = [x[1:] + [int(x[0])] for x in lists]
            lists[0].append(int((max(c for c in lists[0] if c >= 0) + 1) % c.capacity))
        cells, off = flat(lists)
        K.build_cells(p, dev(cells), dev(off), entries, ws)
        out = torch.empty(3, 24, 256, device="cuda")
        lse = torch.empty(3, 24, device="cuda")
        K.attend(p, c.q_d, c.kc_d, c.vc_d, ws, out=out, lse=lse, k_scales=c.ks_d, v_scales=c.vs_d,
                 plan_cells=entries)
        torch.cuda.synchronize()
        oc = [O.compact_plan([x], c.capacity)[0] for x in lists]
        wo, wl = O.decode_attention(c.q, [((c.kind, c.kc, c.ks), (c.vkind, c.vc, c.vs), oc)], c.hkv, c.scale)
        check(out.cpu().numpy(), lse.cpu().numpy(), wo, wl)


@pytest.mark.parametrize("kind", [O.Q8_B32, O.Q4_B32])
@pytest.mark.parametrize("size", ["one-level", "two-level"])
def test_generous_budget_bit_equal_to_tight(K, kind, size):
    """The same lists through a tight record budget (each slot's own record
    count) and a generous one, 1024-cell splits, matrix-core kernel: the
    outputs are bit-equal with and without live_records -- a hole segment
    adds nothing, and the extra splits only add empty records to a merge of
    the same shape: every slot has 2 to 32 splits in both plans (one level),
    or more than 32 in both (two levels: clusters of 16 consecutive splits,
    the extra ones empty).  The two-level case (1152 workgroups tight, 2304
    generous) shows the cost of scanning the padding and that live_records
    -- the records in use, as kvdec_build_cells reports them -- removes it."""
    import torch
    r = synth.rng(310 + kind + (0 if size == "one-level" else 20))
    if size == "one-level":
        lists, cap = synth.interleaved_record_lists([4000, 3000, 2500], r, shuffle=True)
    else:
        lists, cap = synth.interleaved_record_lists([131072, 98304, 65536], r)
    _, counts = expected(lists, cap, [0, 0, 0])
    tight = list(counts)
    generous = [min(3 * t + 8 if size == "one-level" else 2 * t, -(-cap // 128)) for t in tight]
    q = synth.gen_q(r, 3, 24, 256)
    kd, ksd = synth.device_quant_cache(330 + kind, kind, cap, 4, 256)
    vd, vsd = synth.device_quant_cache(340 + kind, kind, cap, 4, 256)
    qd = dev(q)
    cells, off = flat(lists)
    res, times = {}, {}
    for name, budget in (("tight", tight), ("generous", generous)):
        p = K.plan(24, 4, 256, 3, cap, k_type=kind, v_type=kind, max_records=budget, split_cells=1024)
        assert p.info()["matrix_cores"] == 1
        per_slot = np.bincount(p.splits()[:, 0], minlength=3) // 4  # split table rows / KV heads
        if size == "one-level":
            assert np.all(per_slot >= 2) and np.all(per_slot <= 32), per_slot
        else:
            assert np.all(per_slot > 32), per_slot
        ws = K.workspace(p)
        pc = torch.empty(p.info()["n_entries"], dtype=torch.int32, device="cuda")
        nrec = torch.empty(4, dtype=torch.int32, device="cuda")
        K.build_cells(p, dev(cells), dev(off), pc, ws, n_records=nrec)
        torch.cuda.synchronize()
        assert list(nrec.cpu().numpy()[:3]) == tight
        for live in (None, nrec):
            out = torch.full((3, 24, 256), float("nan"), device="cuda")
            lse = torch.full((3, 24), float("nan"), device="cuda")

            def call():
                K.attend(p, qd, kd, vd, ws, out=out, lse=lse, k_scales=ksd, v_scales=vsd, plan_cells=pc,
                         live_records=live)

            call()
            torch.cuda.synchronize()
            key = (name, live is not None)
            res[key] = (out.cpu().numpy(), lse.cpu().numpy())
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(20):
                call()
            b.record()
            torch.cuda.synchronize()
            times[key] = a.elapsed_time(b) * 1e3 / 20
    ref = res[("tight", False)]
    for key, got in res.items():
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), key
    # the oracle on the smallest slot (its rows gathered on the device)
    entries = expected(lists, cap, tight)[0]
    bounds = np.concatenate([[0], np.cumsum(tight)]) * 128
    seg = entries[bounds[2]:bounds[3]]
    live_cells = torch.from_numpy(seg[seg >= 0].astype(np.int64)).cuda()
    kh, vh = (t.index_select(0, live_cells).cpu().numpy() for t in (kd, vd))
    ksh, vsh = (t.index_select(0, live_cells).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                for t in (ksd, vsd))
    want = O.decode_attention(q[2:3], [((kind, kh, ksh), (kind, vh, vsh), [np.arange(len(live_cells))])], 4, 1 / 16)
    check(ref[0][2:3], ref[1][2:3], *want)
    print("\nus per call:", {f"{k[0]}{'+live' if k[1] else ''}": round(v, 2) for k, v in times.items()})
    # padding skipped: within 15% of the tight plan's time (plus launch noise)
    assert times[("generous", True)] <= 1.15 * times[("tight", False)] + 3.0
    if size == "two-level":
        # without live_records the padding is scanned: visibly slower
        assert times[("generous", False)] > 1.3 * times[("generous", True)]


def draw_lists(seed):
    """Seeded raw lists for a device-built plan: capacity around record
    edges, 1-5 slots, cells anywhere, as a wrapping run or within a few
    records, with holes, out-of-range entries (below -1, at / past the
    capacity, INT32_MAX) and duplicates inserted; budgets a little under,
    at or over each slot's record count (within 0 .. ceil(capacity / 128))."""
    r = np.random.default_rng(70000 + seed)
    cap = int(r.choice([1, 127, 128, 129, 1000, 5000, 40000]))
    lists = []
    for _ in range(int(r.integers(1, 6))):
        n = int(r.choice([0, 1, 5, 100, 1000, 5000]))
        style = int(r.integers(3))
        if style == 0:
            x = r.integers(0, cap, size=n)
        elif style == 1:
            x = (int(r.integers(0, cap)) + np.arange(n)) % cap
        else:
            recs = r.integers(0, -(-cap // 128), size=max(1, n // 100))
            x = (recs[r.integers(0, len(recs), size=n)] * 128 + r.integers(0, 128, size=n)) % cap
        x = [int(v) for v in x]
        for _ in range(int(r.integers(0, 6))):
            pick = int(r.integers(5))
            v = [-1, -2 - int(r.integers(0, 5)), cap + int(r.integers(0, 5)), x[0] if x else -1, 2 ** 31 - 1][pick]
            x.insert(int(r.integers(0, len(x) + 1)), v)
        lists.append(x)
    need = [len({c // 128 for c in x if 0 <= c < cap}) for x in lists]
    budget = [max(0, min(-(-cap // 128), n + int(r.integers(-2, 4)))) for n in need]
    return lists, cap, budget


@pytest.mark.parametrize("seed", range(32))
def test_random_lists_bit_exact_against_oracle(K, seed):
    lists, cap, budget = draw_lists(seed)
    _, _, got, nrec = build(K, lists, cap, budget)
    want, counts = expected(lists, cap, budget)
    assert np.array_equal(got, want)
    dropped = sum(1 for x in lists for c in x if c < -1 or c >= cap)
    assert list(nrec[:len(lists)]) == counts and nrec[len(lists)] == dropped
