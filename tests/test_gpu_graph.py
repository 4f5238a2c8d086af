"""kvdec_attend captured in a HIP graph (torch.cuda.CUDAGraph), as the
benchmark times it: every replay, with eager work and synchronisations in
between, must give the eager result bit for bit (the tickets left at zero by
each call, the merge order fixed by split index) and match the oracle."""

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


CASES = {
    "f16 G4 eight-wave": dict(args=(61, 32, 8, 128), kw=dict(occupied=[13100]), plan={}),
    "f16 G4 two-level merge": dict(args=(62, 16, 4, 128), kw=dict(occupied=[20000]), plan=dict(tiles_per_split=1)),
    "q8 G6 indirect matrix cores": dict(args=(63, 24, 4, 256), kw=dict(kind=O.Q8_B32, indirect_lengths=[3000, 700, 1],
                                                                        shuffle=True, duplicates=5), plan={}),
    "f16 G16 eight-wave matrix cores": dict(args=(65, 128, 8, 128), kw=dict(occupied=[13100]), plan={}),
    "f16 G5 long staged splits": dict(args=(64, 10, 2, 128), kw=dict(kind=O.F16, occupied=[30000]),
                                      plan=dict(split_cells=4096)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_equal_eager(K, name):
    import torch
    spec = CASES[name]
    c = Case(*spec["args"], **spec["kw"])
    p = c.plan(K, n_cu=256, **spec["plan"])
    c.upload()
    ws = K.workspace(p)
    pc = None if c.raw is None else dev(p.cells()[0])
    # three calls on one workspace per captured sequence, each with its own q
    qs = [c.q_d, (c.q_d * 0.5).contiguous(), (-c.q_d).contiguous()]
    outs = [torch.empty(c.n_slots, c.hq, c.d, device="cuda") for _ in qs]
    lses = [torch.empty(c.n_slots, c.hq, device="cuda") for _ in qs]

    def seq():
        for q, o, l in zip(qs, outs, lses):
            K.attend(p, q, c.kc_d, c.vc_d, ws, out=o, lse=l, k_scales=c.ks_d, v_scales=c.vs_d, plan_cells=pc)

    seq()
    torch.cuda.synchronize()
    eager = [(o.clone(), l.clone()) for o, l in zip(outs, lses)]
    check(eager[0][0].cpu().numpy(), eager[0][1].cpu().numpy(), *c.oracle())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    for rep in range(4):
        for o, l in zip(outs, lses):
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (eo, el), o, l in zip(eager, outs, lses):
            assert torch.equal(o, eo) and torch.equal(l, el), f"replay {rep} differs from eager"
        # eager work between replays on the same workspace
        seq()
        torch.cuda.synchronize()
        for (eo, el), o, l in zip(eager, outs, lses):
            assert torch.equal(o, eo) and torch.equal(l, el)


@pytest.mark.parametrize("seed", range(16))
def test_random_configuration_replays(K, seed):
    """A random configuration (the draw of test_gpu_random) captured once and
    replayed three times, with an eager call on the same workspace after
    each replay: every replay and every eager call bit-equal to the first
    eager call, which matches the oracle."""
    import torch
    from test_gpu_random import draw
    d, g, hkv, kind, vkind, lengths, indirect, split = draw(5000 + seed)
    if indirect:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, indirect_lengths=lengths, shuffle=True)
    else:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, occupied=lengths)
    p = c.plan(K, n_cu=256, **split)
    c.upload()
    pc = None if c.raw is None else dev(p.cells()[0])
    ws = K.workspace(p)
    out = torch.full((c.n_slots, c.hq, c.d), float("nan"), device="cuda")
    lse = torch.full((c.n_slots, c.hq), float("nan"), device="cuda")

    def call():
        K.attend(p, c.q_d, c.kc_d, c.vc_d, ws, out=out, lse=lse, k_scales=c.ks_d, v_scales=c.vs_d, plan_cells=pc)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    want = (out.cpu().numpy().copy(), lse.cpu().numpy().copy())
    check(*want, *c.oracle())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        call()
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        gr.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want[0]) and np.array_equal(lse.cpu().numpy(), want[1])
        call()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want[0]) and np.array_equal(lse.cpu().numpy(), want[1])
