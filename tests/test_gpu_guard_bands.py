"""Guard bands around every buffer a call writes: out, lse, the partial
triple, the workspace (at exactly the plan's workspace_bytes) and the
standalone merge's outputs sit inside larger allocations whose margins hold
a fixed byte pattern; after the call, every margin byte must be unchanged
and the results must match the float64 oracle.  One case per kernel family
and path: the one-shot kernel, the streamed kernel on several slots with
partials, the matrix-core kernel on int8 and 4-bit indirect plans and on
several query rows, a resident window with a host tail, and kvdec_merge;
then seeded random configurations of every planner regime."""

import numpy as np
import pytest

import oracle as O
from gpu_cases import Case, check, dev

pytestmark = pytest.mark.gpu

MARGIN = 4096        # bytes of guard on each side (keeps 256-byte alignment)
PATTERN = 0xA5


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available()
    from long_context_decode_kv_amd import kvdec
    return kvdec


class Guarded:
    """A device buffer of `nbytes` between two MARGIN-byte guards filled with
    PATTERN; the middle is filled with `fill` (a byte) or viewed as `dtype`."""

    def __init__(self, nbytes, fill=PATTERN):
        import torch
        self.nbytes = nbytes
        self.raw = torch.full((nbytes + 2 * MARGIN,), PATTERN, dtype=torch.uint8, device="cuda")
        self.raw[MARGIN:MARGIN + nbytes].fill_(fill)

    def view(self, dtype, shape):
        return self.raw[MARGIN:MARGIN + self.nbytes].view(dtype).view(shape)

    def ptr(self):
        return self.raw.data_ptr() + MARGIN

    def assert_guards_intact(self, what):
        import torch
        torch.cuda.synchronize()
        g = torch.cat([self.raw[:MARGIN], self.raw[MARGIN + self.nbytes:]]).cpu().numpy()
        bad = np.flatnonzero(g != PATTERN)
        assert bad.size == 0, f"{what}: {bad.size} guard bytes overwritten (first at offset {bad[0]})"


def outputs(c, n_q=1, part=False):
    """Guarded out / lse (NaN-filled) and optionally the partial triple."""
    import torch
    rows = c.n_slots * n_q * c.hq
    bufs = {"out": Guarded(rows * c.d * 4, fill=0xFF), "lse": Guarded(rows * 4, fill=0xFF)}
    if part:
        bufs.update({"pm": Guarded(rows * 4, fill=0xFF), "pl": Guarded(rows * 4, fill=0xFF),
                     "po": Guarded(rows * c.d * 4, fill=0xFF)})
    t = {k: b.view(torch.float32, (rows, c.d) if k in ("out", "po") else (rows,)) for k, b in bufs.items()}
    return bufs, t


def guarded_workspace(p):
    ws = Guarded(max(p.workspace_bytes, 256), fill=0)
    return ws, (ws.ptr(), p.workspace_bytes)


def finish(bufs, ws, c, t, n_q=1):
    for k, b in bufs.items():
        b.assert_guards_intact(k)
    ws.assert_guards_intact("workspace")
    return t["out"].cpu().numpy().reshape(c.n_slots * n_q, c.hq, c.d), t["lse"].cpu().numpy().reshape(-1, c.hq)


@pytest.mark.parametrize("kind", ["oneshot", "streamed"])
def test_vector_alu_kernels(K, kind):
    c = Case(9100 + len(kind), 32, 8, 128, occupied=[4000] if kind == "oneshot" else [300, 9000, 17],
             begins=None if kind == "oneshot" else [0, 512, 9600]).upload()
    p = c.plan(K, kernel=K.KERNEL_ONESHOT if kind == "oneshot" else K.KERNEL_STREAMED)
    bufs, t = outputs(c, part=(kind == "streamed"))
    ws, wst = guarded_workspace(p)
    part = (t["pm"], t["pl"], t["po"]) if "pm" in t else None
    K.attend(p, c.q_d, c.kc_d, c.vc_d, wst, out=t["out"], lse=t["lse"], part=part)
    out, lse = finish(bufs, ws, c, t)
    check(out, lse, *c.oracle())
    if part is not None:
        m, l, o = (t[k].cpu().numpy() for k in ("pm", "pl", "po"))
        assert np.all(np.isfinite(l)) and np.all(l > 0)


@pytest.mark.parametrize("kind", [O.Q8_B32, O.Q4_B32], ids=["int8", "4bit"])
def test_matrix_core_kernel_indirect(K, kind):
    import torch
    c = Case(9200 + kind, 24, 4, 256, kind=kind, indirect_lengths=[3000, 777, 1]).upload()
    p = c.plan(K)
    assert p.info()["matrix_cores"] == 1
    bufs, t = outputs(c)
    ws, wst = guarded_workspace(p)
    cells = Guarded(4 * max(len(p.cells()[0]), 1))
    pc = cells.view(torch.int32, (-1,))
    pc.copy_(dev(p.cells()[0].astype(np.int32)))
    K.attend(p, c.q_d, c.kc_d, c.vc_d, wst, out=t["out"], lse=t["lse"], k_scales=c.ks_d, v_scales=c.vs_d,
             plan_cells=pc)
    out, lse = finish(bufs, ws, c, t)
    cells.assert_guards_intact("plan_cells")
    check(out, lse, *c.oracle())


def test_matrix_core_kernel_several_query_rows(K):
    n_q = 4
    c = Case(9300, 32, 8, 128, occupied=[2000, 5000]).upload()
    q = np.random.default_rng(9301).standard_normal((c.n_slots, n_q, c.hq, c.d)).astype(np.float32)
    # query rows at the slots' last n_q cells (both slots start at cell 0)
    qp = np.array([[n - n_q + i for i in range(n_q)] for n in c.occupied], dtype=np.int32)
    p = c.plan(K, n_queries=n_q)
    bufs, t = outputs(c, n_q=n_q)
    ws, wst = guarded_workspace(p)
    K.attend(p, dev(q), c.kc_d, c.vc_d, wst, out=t["out"], lse=t["lse"], q_pos=dev(qp))
    out, lse = finish(bufs, ws, c, t, n_q=n_q)
    want_out, want_lse = O.decode_attention_multi(q, [((c.kind, c.kc, c.ks), (c.vkind, c.vc, c.vs), c.oracle_cells)],
                                                  c.hkv, c.scale, qp, None)
    check(out.reshape(want_out.shape), lse.reshape(want_lse.shape), want_out, want_lse)


def test_window_with_host_tail(K):
    import torch
    ctx, t0 = 5000, 3217
    c = Case(9400, 32, 8, 128, occupied=[ctx]).upload()
    p = K.plan(c.hq, c.hkv, c.d, 1, c.capacity, n_occupied=[ctx - t0], cell_begin=[t0], n_tail=[t0],
               tail_begin=[0], tail_capacity_cells=t0, tail_chunk_cells=512, tail_ring_depth=2)
    hk = torch.empty(c.kc[:t0].shape, dtype=torch.int16, pin_memory=True)
    hv = torch.empty(c.vc[:t0].shape, dtype=torch.int16, pin_memory=True)
    hk.copy_(torch.from_numpy(np.ascontiguousarray(c.kc[:t0]).view(np.int16)))
    hv.copy_(torch.from_numpy(np.ascontiguousarray(c.vc[:t0]).view(np.int16)))
    bufs, t = outputs(c)
    ws, wst = guarded_workspace(p)
    K.attend(p, c.q_d, c.kc_d, c.vc_d, wst, out=t["out"], lse=t["lse"], k_tail=hk, v_tail=hv)
    out, lse = finish(bufs, ws, c, t)
    check(out, lse, *c.oracle())


def test_standalone_merge(K):
    import torch
    rows, d = 40, 128
    r = np.random.default_rng(9500)
    parts, want_m, want_l, want_o = [], [], [], []
    for i in range(3):
        m = r.normal(size=rows).astype(np.float32)
        l = r.uniform(0.5, 2, size=rows).astype(np.float32)
        o = r.normal(size=(rows, d)).astype(np.float32)
        parts.append((dev(m), dev(l), dev(o)))
        want_m.append(m.astype(np.float64)); want_l.append(l.astype(np.float64)); want_o.append(o.astype(np.float64))
    M = np.max(want_m, axis=0)
    L = sum(l * np.exp(m - M) for m, l in zip(want_m, want_l))
    Ov = sum(o * (np.exp(m - M))[:, None] for m, o in zip(want_m, want_o))
    g = {k: Guarded(n, fill=0xFF) for k, n in (("out", rows * d * 4), ("lse", rows * 4), ("mm", rows * 4),
                                              ("ml", rows * 4), ("mo", rows * d * 4))}
    v = {k: b.view(torch.float32, (rows, d) if k in ("out", "mo") else (rows,)) for k, b in g.items()}
    K.merge(parts, rows, d, out=v["out"], lse=v["lse"], merged=(v["mm"], v["ml"], v["mo"]))
    for k, b in g.items():
        b.assert_guards_intact(k)
    check(v["out"].cpu().numpy(), v["lse"].cpu().numpy(), Ov / L[:, None], M + np.log(L))


@pytest.mark.parametrize("seed", range(12))
def test_random_configurations_between_guards(K, seed):
    """Random configurations (the generators of test_gpu_random: general
    draws and draws sized for the planner's regimes, multi-query rows
    included) with out, lse, every third one the partial triple, and the
    workspace between guard margins: no byte outside them changes, and the
    single-query results match the oracle."""
    from test_gpu_random import draw, draw_filling
    if seed % 2 == 0:
        d, g, hkv, kind, vkind, lengths, indirect, split = draw(7000 + seed)
        n_q = 1
    else:
        d, g, hkv, kind, vkind, lengths, indirect, n_q = draw_filling(7000 + seed)
        split = {}
    if indirect:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, indirect_lengths=lengths, shuffle=True)
    else:
        c = Case(seed, g * hkv, hkv, d, kind=kind, v_kind=vkind, occupied=lengths)
    p = c.plan(K, n_cu=256, n_queries=n_q, **split)
    c.upload()
    part = seed % 3 == 0
    bufs, t = outputs(c, n_q=n_q, part=part)
    ws, wst = guarded_workspace(p)
    pc = None if c.raw is None else dev(p.cells()[0])
    q, kw = c.q_d, {}
    if n_q > 1:
        q = dev(np.random.default_rng(seed + 1).standard_normal((c.n_slots, n_q, c.hq, c.d)).astype(np.float32))
        kw = dict(q_pos=dev(np.random.default_rng(seed).integers(-5, c.capacity + 5, size=(c.n_slots, n_q))
                            .astype(np.int32)))
    K.attend(p, q, c.kc_d, c.vc_d, wst, out=t["out"], lse=t["lse"], part=(t["pm"], t["pl"], t["po"]) if part else None,
             k_scales=c.ks_d, v_scales=c.vs_d, plan_cells=pc, **kw)
    out, lse = finish(bufs, ws, c, t, n_q=n_q)
    if n_q == 1:
        check(out, lse, *c.oracle())
