"""kvdec_attend_static (the library's static per-device scratch array in place
of a caller workspace) against kvdec_attend with a workspace of its own, both
through the C ABI: bit-equal outputs on consecutive calls whose plans differ in
kernel, size and workspace layout -- the second call of each pair smaller than
the first -- each also within the bound of the float64 oracle; a zero-copy host
tail; graph capture replays."""

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


def run_static(K, c, p):
    import torch
    if not hasattr(c, "q_d"):
        c.upload()
    out = torch.full((c.n_slots, c.hq, c.d), float("nan"), device="cuda")
    lse = torch.full((c.n_slots, c.hq), float("nan"), device="cuda")
    pc = dev(p.cells()[0]) if c.raw is not None else None
    K.attend_static(p, c.q_d, c.kc_d, c.vc_d, out=out, lse=lse, k_scales=c.ks_d, v_scales=c.vs_d, plan_cells=pc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def same(a, b):
    assert np.array_equal(a[0], b[0], equal_nan=False) and np.array_equal(a[1], b[1])


def test_vector_kernels_second_call_smaller(K):
    """A device-filling one-shot layer (256 splits), then a smaller
    multi-slot streamed-kernel plan (an empty and a one-cell slot), then the
    first again: every call bit-equal to kvdec_attend."""
    big = Case(2101, 32, 8, 128, occupied=[13100])
    small = Case(2102, 16, 4, 128, occupied=[900, 3000, 1, 0], begins=[0, 1000, 4100, 4200])
    pb = big.plan(K, n_cu=256)
    ps = small.plan(K, n_cu=256, kernel=K.KERNEL_STREAMED)
    assert pb.info()["kernel"] == K.KERNEL_ONESHOT and pb.info()["n_workgroups"] == 256
    assert ps.workspace_bytes < pb.workspace_bytes
    for c, p in ((big, pb), (small, ps), (big, pb)):
        got = run_static(K, c, p)
        same(got, c.run(K, plan=p))
        check(*got, *c.oracle())


def test_matrix_core_kernel_second_call_smaller(K):
    """Group 6, head_dim 256 on matrix cores: an int8 indirect plan over
    three slots, then a smaller 4-bit one."""
    big = Case(2103, 24, 4, 256, kind=O.Q8_B32, indirect_lengths=[9000, 3000, 700], shuffle=True)
    small = Case(2104, 24, 4, 256, kind=O.Q4_B32, indirect_lengths=[1500, 200])
    pb, ps = big.plan(K, n_cu=256), small.plan(K, n_cu=256)
    assert pb.info()["matrix_cores"] == 1 and ps.info()["matrix_cores"] == 1
    assert ps.workspace_bytes < pb.workspace_bytes
    for c, p in ((big, pb), (small, ps)):
        got = run_static(K, c, p)
        same(got, c.run(K, plan=p))
        check(*got, *c.oracle())


def test_zero_copy_tail(K):
    """A resident window plus a host tail read in place (pinned, mapped)."""
    import torch

    def pinned(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        t = torch.empty(a.shape, dtype=torch.from_numpy(a[:0]).dtype, pin_memory=True)
        t.copy_(torch.from_numpy(a))
        return t

    c = Case(2105, 32, 8, 128, occupied=[5000])
    t = 3217
    p = K.plan(32, 8, 128, 1, c.capacity, scale=c.scale, n_occupied=[5000 - t], cell_begin=[t], n_tail=[t],
               tail_begin=[0], tail_capacity_cells=t, tail_chunk_cells=1024, tail_zero_copy=True, n_cu=256)
    c.upload()
    hk, hv = pinned(c.kc[:t]), pinned(c.vc[:t])
    res = []
    for static in (False, True):
        out = torch.full((1, 32, 128), float("nan"), device="cuda")
        lse = torch.full((1, 32), float("nan"), device="cuda")
        if static:
            K.attend_static(p, c.q_d, c.kc_d, c.vc_d, out=out, lse=lse, k_tail=hk, v_tail=hv)
        else:
            K.attend(p, c.q_d, c.kc_d, c.vc_d, K.workspace(p), out=out, lse=lse, k_tail=hk, v_tail=hv)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    same(res[1], res[0])
    check(*res[1], *c.oracle())


def test_graph_replays(K):
    """Two static calls of different plans recorded into one graph; replays
    with eager work and synchronizations between them equal the eager
    kvdec_attend results every time."""
    import torch
    a = Case(2106, 32, 8, 128, occupied=[13100]).upload()
    b = Case(2107, 16, 4, 128, occupied=[2000]).upload()
    pa, pb = a.plan(K, n_cu=256), b.plan(K, n_cu=256)
    want = [a.run(K, plan=pa), b.run(K, plan=pb)]
    outs = [torch.empty(1, 32, 128, device="cuda"), torch.empty(1, 16, 128, device="cuda")]
    lses = [torch.empty(1, 32, device="cuda"), torch.empty(1, 16, device="cuda")]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.attend_static(pa, a.q_d, a.kc_d, a.vc_d, out=outs[0], lse=lses[0])
        K.attend_static(pb, b.q_d, b.kc_d, b.vc_d, out=outs[1], lse=lses[1])
    for _ in range(3):
        for o, l in zip(outs, lses):
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for w, o, l in zip(want, outs, lses):
            same((o.cpu().numpy(), l.cpu().numpy()), w)
        # eager work on the same scratch between replays
        same(run_static(K, b, pb), want[1])
