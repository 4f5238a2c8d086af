"""Phase timeline of the one-shot split kernel on the Qwen3-8B-shaped decode
step (36 layers x 32 query / 8 KV heads / head_dim 128, 13100 of 16384
cells, f16 K and V), from the diagnostic build libkvdec_trace.so.

    python -m long_context_decode_kv_amd.phase_trace [--layers 36] [--occupied 13100]

That build is the product's kernels compiled with KVDEC_PHASE_TRACE: thread
0 of every workgroup (lane 0 of every wave for the per-wave slots) writes
the constant 100 MHz clock into 32 slots per workgroup at the phase points
listed in csrc/split_kernels.h.  The step runs as one captured graph, as
bench.py runs it, once with stamps and once without (the difference is the
cost of the stamps themselves).  Times are relative to the first workgroup
entry of each layer, averaged over the layers after the first.
"""

import argparse
import ctypes
import importlib.util
import os

import numpy as np

SLOTS = {0: "entry", 1: "loads issued", 2: "query converted", 3: "scores and maximum", 4: "weights",
         13: "streams merged", 14: "record stores issued", 15: "record stores acknowledged", 16: "ticket returned",
         17: "merge done (merging workgroups)"}
MERGE_SLOTS = [(16, "ticket returned"), (30, "merge entered"), (18, "(m, l) loads issued"),
               (31, "record loads issued"), (19, "(m, l) reduced"), (20, "records accumulated"),
               (21, "columns combined"), (17, "outputs stored")]
TICK_US = 0.01  # s_memrealtime runs at 100 MHz


def load():
    """The binding over libkvdec_trace.so, as a module of its own (the
    product binding, if imported, stays bound to libkvdec.so)."""
    import torch  # noqa: F401  (the binding expects torch's HIP runtime loaded first)
    from long_context_decode_kv_amd import kvdec
    os.environ["KVDEC_LIB_NAME"] = "libkvdec_trace.so"
    try:
        spec = importlib.util.spec_from_file_location("kvdec_trace", kvdec.__file__)
        m = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(m)
    finally:
        del os.environ["KVDEC_LIB_NAME"]
    assert m.LIB_PATH.endswith("libkvdec_trace.so"), m.LIB_PATH
    m.lib.kvdec_trace_configure.argtypes = [ctypes.c_void_p]
    m.lib.kvdec_trace_configure.restype = None
    return m


def record(K, layers=36, occupied=13100, capacity=16384, hq=32, hkv=8, d=128, reps=20):
    """Run the step in a captured graph with and without stamps; return
    (plan info, us per step without stamps, with stamps, stamps int64
    [layers, workgroups, 32] in clock ticks, 0 where a slot was not written,
    the KV head each workgroup reads)."""
    import torch
    from long_context_decode_kv_amd import synth
    ks, vs, qs, outs, lses = [], [], [], [], []
    for layer in range(layers):
        s = 1001 * 100 + layer
        ks.append(synth.device_f16_cache(3 * s, capacity, hkv, d))
        vs.append(synth.device_f16_cache(3 * s + 1, capacity, hkv, d))
        qs.append(synth.device_q(3 * s + 2, 1, hq, d))
        outs.append(torch.empty(1, hq, d, device="cuda"))
        lses.append(torch.empty(1, hq, device="cuda"))
    p = K.plan(hq, hkv, d, 1, capacity, n_occupied=[occupied])
    info = p.info()
    nw = info["n_workgroups"]
    heads = np.asarray(p.splits())[:, 1].astype(np.int64)
    ws = K.workspace(p)
    st = torch.zeros(layers * nw * 32, dtype=torch.int64, device="cuda")

    def step(stamps):
        for layer in range(layers):
            K.lib.kvdec_trace_configure(st.data_ptr() + layer * nw * 32 * 8 if stamps else None)
            K.attend(p, qs[layer], ks[layer], vs[layer], ws, out=outs[layer], lse=lses[layer])
        K.lib.kvdec_trace_configure(None)

    for _ in range(3):
        step(True)
    torch.cuda.synchronize()
    times = {}
    for stamps in (False, True):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(stamps)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        times[stamps] = a.elapsed_time(b) * 1e3 / reps
        if stamps:
            st.zero_()
            g.replay()
            torch.cuda.synchronize()
    x = st.view(layers, nw, 32).cpu().numpy().astype(np.int64)
    return info, times[False], times[True], x, heads


def summarize(x, heads=None):
    """Phase times (us) from the stamps of record(): per slot the median and
    the slowest workgroup, per-wave P.V and last-V times, the merging
    workgroups' chain (us after their ticket), the gap from a layer's last
    merge to the next layer's first entry, and first entry to last merge.
    With `heads` (KV head per workgroup): per KV head, the mean time from a
    workgroup's entry to its last V row landing."""
    L = x.shape[0]
    rel = lambda layer, v: (v - x[layer, :, 0].min()) * TICK_US  # noqa: E731
    out = {"phases": {}, "merge": {}, "waves": {}}
    for k, name in SLOTS.items():
        med, slow = [], []
        for layer in range(1, L):
            v = x[layer, :, k]
            v = v[v > 0]
            if len(v):
                med.append(np.median(rel(layer, v)))
                slow.append(np.max(rel(layer, v)))
        if med:
            out["phases"][name] = (float(np.mean(med)), float(np.mean(slow)))
    pv = np.array([rel(layer, x[layer, :, 5:13]) for layer in range(1, L)])
    vl = np.array([rel(layer, x[layer, :, 22:30]) for layer in range(1, L)])
    out["waves"]["P.V done by wave"] = [round(float(t), 2) for t in pv.mean((0, 1))]
    out["waves"]["last V landed by wave"] = [round(float(t), 2) for t in vl.mean((0, 1))]
    out["waves"]["last V landed, slowest wave of a workgroup (mean over workgroups)"] = float(vl.max(2).mean())
    out["waves"]["last V landed, slowest of the layer"] = float(vl.max((1, 2)).mean())
    chain = []
    for layer in range(1, L):
        m = x[layer, :, 17] > 0
        t = x[layer, m][:, [k for k, _ in MERGE_SLOTS]].astype(np.int64)
        chain.append(((t - t[:, :1]) * TICK_US).mean(0))
    out["merge"] = {name: round(float(t), 2) for (_, name), t in zip(MERGE_SLOTS, np.mean(chain, 0))}
    gap = [(x[layer + 1, :, 0].min() - x[layer, :, 17].max()) * TICK_US for layer in range(1, L - 1)]
    out["gap"] = float(np.mean(gap))
    out["span"] = float(np.mean([(x[layer, :, 17].max() - x[layer, :, 0].min()) * TICK_US for layer in range(1, L)]))
    if heads is not None:
        own = np.array([(x[layer, :, 22:30].max(1) - x[layer, :, 0]) * TICK_US for layer in range(1, L)]).mean(0)
        out["heads"] = [round(float(own[heads == h].mean()), 2) for h in range(int(heads.max()) + 1)]
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--occupied", type=int, default=13100)
    args = ap.parse_args(argv)
    K = load()
    info, us_plain, us_traced, x, heads = record(K, layers=args.layers, occupied=args.occupied)
    print(f"library source hash {K.LIB_SOURCE_HASH}; plan: {info['n_workgroups']} workgroups, "
          f"{info['split_cells']} cells per split, kernel {info['kernel']}")
    print(f"step without stamps {us_plain:.1f} us ({us_plain / args.layers:.2f} us / layer), "
          f"with stamps {us_traced:.1f} us ({us_traced / args.layers:.2f} us / layer)")
    s = summarize(x, heads)
    print("phase (us after the layer's first workgroup entry)   median   slowest workgroup")
    for name, (med, slow) in s["phases"].items():
        print(f"  {name:48s} {med:7.2f}   {slow:7.2f}")
    for name, v in s["waves"].items():
        print(f"  {name}: {v if isinstance(v, list) else round(v, 2)}")
    print("merging workgroups, us after their ticket returned:")
    for name, t in s["merge"].items():
        print(f"  {name:48s} {t:7.2f}")
    print(f"entry to last V landed, mean per KV head: {s['heads']}")
    print(f"gap from a layer's last merge to the next layer's first entry: {s['gap']:.2f} us")
    print(f"first entry to last merge done: {s['span']:.2f} us")


if __name__ == "__main__":
    main()
