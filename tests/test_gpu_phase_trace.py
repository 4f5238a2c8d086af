"""The diagnostic build libkvdec_trace.so (KVDEC_PHASE_TRACE): its one-shot
kernel computes exactly what the product library computes -- outputs bit
for bit equal, with the stamps on and off -- and the stamps it writes are
ordered as the phases run: every workgroup's own chain, one merging
workgroup per (slot, KV head) with its merge phases in order, and none
outside the launch's workgroups.  The timeline tool's summary runs on them."""

import numpy as np
import pytest

from gpu_cases import Case, check

pytestmark = pytest.mark.gpu

OWN_CHAIN = [0, 1, 2, 3, 4, 13, 14]          # every workgroup of a multi-split group
PUBLISH = [14, 15, 16]                       # ... that publishes a record
MERGE_CHAIN = [16, 30, 18, 31, 19, 20, 21, 17]  # the merging workgroup


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available()
    from long_context_decode_kv_amd import kvdec
    return kvdec


@pytest.fixture(scope="module")
def KT():
    from long_context_decode_kv_amd import phase_trace
    m = phase_trace.load()
    yield m
    m.lib.kvdec_trace_configure(None)


@pytest.mark.parametrize("occupied", [[4000], [300, 9000]], ids=["one-slot", "two-slots"])
def test_trace_build_outputs_and_stamp_order(K, KT, occupied):
    import torch
    c = Case(8800 + len(occupied), 32, 8, 128, occupied=occupied)
    c.upload()
    p = c.plan(K, kernel=K.KERNEL_ONESHOT, n_cu=256)
    pt = c.plan(KT, kernel=KT.KERNEL_ONESHOT, n_cu=256)
    info = p.info()
    assert info["kernel"] == K.KERNEL_ONESHOT and pt.info() == info
    nw = info["n_workgroups"]
    want = c.run(K, plan=p)
    KT.lib.kvdec_trace_configure(None)
    plain = c.run(KT, plan=pt)
    st = torch.zeros(nw * 32 + 64, dtype=torch.int64, device="cuda")  # one spare workgroup's slots past the end
    KT.lib.kvdec_trace_configure(st.data_ptr())
    try:
        traced = c.run(KT, plan=pt)
    finally:
        KT.lib.kvdec_trace_configure(None)
    for got in (plain, traced):
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    check(*traced, *c.oracle())
    x = st.cpu().numpy().astype(np.int64)
    assert not x[nw * 32:].any()  # nothing written past the launch's workgroups
    x = x[:nw * 32].reshape(nw, 32)
    splits = p.splits()  # (slot, KV head, first position, count) per workgroup
    mergers = {}
    for wg in range(nw):
        s, g, _, cnt = (int(v) for v in splits[wg])
        row = x[wg]
        assert row[0] > 0
        multi = sum(1 for r in splits if int(r[0]) == s and int(r[1]) == g) > 1
        if cnt == 0 or not multi:
            continue
        assert all(row[k] > 0 for k in OWN_CHAIN + PUBLISH), (wg, row)
        assert all(row[a] <= row[b] for a, b in zip(OWN_CHAIN, OWN_CHAIN[1:])), (wg, row)
        assert all(row[a] <= row[b] for a, b in zip(PUBLISH, PUBLISH[1:])), (wg, row)
        assert all(row[13] >= row[5 + w] for w in range(8) if row[5 + w] > 0)
        if row[17] > 0:
            assert (s, g) not in mergers
            mergers[(s, g)] = wg
            assert all(row[a] <= row[b] for a, b in zip(MERGE_CHAIN, MERGE_CHAIN[1:])), (wg, row)
    groups = {(int(r[0]), int(r[1])) for r in splits
              if sum(1 for q in splits if q[0] == r[0] and q[1] == r[1]) > 1}
    assert set(mergers) == groups


def test_timeline_summary_runs_on_recorded_stamps(KT):
    """A short run of the timeline tool: two layers of a 4096-cell
    Qwen3-8B-shaped cache, every phase present and ordered on average."""
    from long_context_decode_kv_amd import phase_trace
    info, us_plain, us_traced, x, heads = phase_trace.record(KT, layers=3, occupied=4000, capacity=4096, reps=3)
    assert info["kernel"] == KT.KERNEL_ONESHOT and us_plain > 0 and us_traced > 0
    assert heads.shape == (info["n_workgroups"],) and set(heads.tolist()) == set(range(8))
    s = phase_trace.summarize(x, heads)
    names = list(phase_trace.SLOTS.values())
    assert list(s["phases"]) == names
    meds = [s["phases"][n][0] for n in names]
    assert all(a <= b + 1e-9 for a, b in zip(meds, meds[1:13]))
    m = [s["merge"][n] for _, n in phase_trace.MERGE_SLOTS]
    assert m[0] == 0 and all(a <= b + 1e-9 for a, b in zip(m, m[1:]))
    assert s["span"] > 0 and s["gap"] > 0
    assert len(s["heads"]) == 8 and all(0 < t < s["span"] for t in s["heads"])
