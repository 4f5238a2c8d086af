"""Decode-attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode graph|eager]

A step is one decode step of attention over the whole model: for every layer
one kvdec_attend call (plan -> split kernel with fused log-sum-exp merge)
over that layer's own resident KV cache, q and outputs.  Inputs are resident
in HBM before the timed region.  Prints one JSON line on stdout; progress
goes to stderr.

Workloads (synthetic N(0, 1) data of the named model's attention shape):
  single-4096       one layer (32 q heads, 8 KV heads, head_dim 128, 4096
                    f16 cells) per step, rotated over 32 cache copies
  qwen3-8b-ctx16k   36 layers x (32 q heads, 8 KV heads, head_dim 128),
                    13100 occupied cells of a 16384-cell f16 cache (default)
  qwen2.5-14b-1m    48 layers x (40 q / 8 KV heads, head_dim 128), 524288
                    cells of f16 K/V (96 GiB)
  gqa6-q8 / gqa6-q4 one layer, 24 q / 4 KV heads, head_dim 256, four slots of
                    131072 / 65536 / 20000 / 777 cells in interleaved 128-cell
                    records, block-scaled int8 / 4-bit K and V
  gqa6-q8k-q4v      the same with int8 K and 4-bit V
  rolling-ctx40960  qwen3-8b shape at ctx 40960: newest 14000 cells resident,
                    oldest 26960 streamed from pinned host memory per layer
                    (-prefetch: cross-layer prefetch through two workspaces;
                    -zerocopy: kernels read the pinned tail in place)
  qwen3-8b-ctx16k-verify4
                    the qwen3-8b-ctx16k caches with 4 query rows per step
                    (speculative verification, causal positional mask)
  qwen3-8b-ctx16k-1launch
                    secondary figure for the qwen3-8b-ctx16k data: all 36
                    layers as 36 slots of ONE kvdec_attend call (ignores the
                    layer-to-layer dependency of a real decode step)
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
KIND = {0: "f16", 1: "q8", 2: "q4"}
KDESC = {0: "f16", 1: "int8+f16 scale/32", 2: "4-bit+f16 scale/32"}


def measure_h2d(torch, nbytes=256 << 20, reps=5):
    """Pinned host -> device copy rate (GB/s) of one large hipMemcpyAsync."""
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        d.copy_(h, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    return round(nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9, 2)


# launch shapes of the read-ceiling sweep: (LDS DMA?, threads, loads in
# flight per thread, workgroups or None for the LDS-DMA grid)
CEILING_SHAPES = ([(0, t, u, w) for t, us in ((256, (4, 8, 16, 32)), (512, (4, 8, 16, 32)), (1024, (4, 8, 16)))
                   for u in us for w in (256, 512, 1024, 2048, 4096)] +
                  [(1, t, n, None) for t, n in ((256, 8), (256, 16), (256, 32), (512, 8), (512, 16), (1024, 4),
                                                (1024, 8))])


def measure_read_ceiling(torch, nbytes, launches):
    """Streaming-read ceiling for the same bytes per launch and launches per
    step: `launches` back-to-back reads (kvprobe_read_shape, 16-byte loads)
    of distinct buffers of `nbytes` each, rotated over >= 1 GiB so the 256 MB
    MALL cannot serve repeats, over a sweep of launch shapes (register loads
    with 256 to 1024 threads, 4 to 32 loads in flight, 256 to 4096
    workgroups; LDS DMA of each thread's whole share at entry).  Returns
    (GB/s, us per launch, shape) of the best, and a dict with the best of
    each load method and the number of shapes tried."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_decode_kv_amd", "libkvprobe.so"))
    f = lib.kvprobe_read_shape
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p]
    g = lib.kvprobe_lds_workgroups
    g.restype = ctypes.c_int64
    g.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    nb = -(-nbytes // 16) * 16
    copies = max(2, -(-(1 << 30) // nb))
    reps = max(2, -(-(20 << 30) // (nb * launches)))
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    grids = {sh: (sh[3] if not sh[0] else g(nb, sh[1], sh[2])) for sh in CEILING_SHAPES}
    sink = torch.empty(max(grids[sh] * sh[1] for sh in CEILING_SHAPES), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best, per_method = None, {}
    for sh in CEILING_SHAPES:
        lds, t, u, w = sh

        def run(n):
            k = 0
            for _ in range(n):
                for _ in range(launches):
                    rc = f(bufs[k % copies].data_ptr(), nb, w or 0, t, u, lds, sink.data_ptr(), stream.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"kvprobe_read_shape{sh} failed: {rc}")
                    k += 1
            return k
        run(1)
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        k = run(reps)
        e.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(e) * 1e3 / k
        desc = (f"{grids[sh]} workgroups x {t} threads, " +
                (f"{u} loads of 16 B in flight per thread" if not lds else f"{u} LDS-DMA loads of 16 B per thread at entry"))
        rec = (round(nb / (us * 1e-6) / 1e9, 1), round(us, 3), desc)
        m = "lds_dma" if lds else "register_loads"
        if m not in per_method or us < per_method[m][1]:
            per_method[m] = rec
        if best is None or us < best[1]:
            best = rec
    del bufs
    return best, {"shapes_tried": len(CEILING_SHAPES),
                  "best_by_method": {m: {"gbs": r[0], "us_per_launch": r[1], "shape": r[2]} for m, r in per_method.items()}}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- workloads

class Workload:
    name = ""
    layers = 1
    hq = hkv = d = 0
    kind = 0

    def algorithmic_bytes_per_launch(self):
        raise NotImplementedError


def kv_row_bytes(kind, d):
    return {0: 2 * d, 1: d, 2: d // 2}[kind]


def scale_row_bytes(kind, d):
    return 0 if kind == 0 else 2 * (d // 32)


def algorithmic_bytes(n_cells_attended, hkv, d, kind, n_slots, hq, plan_entries=0, v_kind=None):
    """Bytes the method must move for one evaluation: the attended cells' K
    and V codes and scales, the indirect plan (4 B per entry), q (fp32) and
    out (fp32).  Unoccupied cells, hole cells, partials and re-reads are not
    counted."""
    vk = kind if v_kind is None else v_kind
    kv = n_cells_attended * hkv * (kv_row_bytes(kind, d) + scale_row_bytes(kind, d) + kv_row_bytes(vk, d) +
                                   scale_row_bytes(vk, d))
    return kv + 4 * plan_entries + 2 * 4 * n_slots * hq * d


class ContiguousModel(Workload):
    split_cells = 0  # planner's choice unless --split-cells
    kernel = 0       # vector-ALU split kernel: planner's choice unless --kernel

    def __init__(self, name, layers, hq, hkv, d, capacity, occupied, n_q=1):
        self.name, self.layers, self.hq, self.hkv, self.d = name, layers, hq, hkv, d
        self.capacity, self.occupied, self.kind, self.n_q = capacity, occupied, 0, n_q

    def config(self):
        c = {"workload": self.name, "layers": self.layers, "q_heads": self.hq, "kv_heads": self.hkv,
             "head_dim": self.d, "cells_occupied": self.occupied, "cells_capacity": self.capacity,
             "batch": 1, "kv_dtype": "f16", "cells_per_tile": 128}
        if self.split_cells:
            c["split_cells"] = self.split_cells
        if self.kernel:
            c["kernel_forced"] = {1: "streamed", 2: "one-shot"}[self.kernel]
        if self.n_q > 1:
            c.update({"query_rows_per_slot": self.n_q, "mask": "causal: row t at the position of occupied cell "
                                                                "n - n_q + t (speculative verification)"})
        return c

    def algorithmic_bytes_per_launch(self):
        return algorithmic_bytes(self.occupied, self.hkv, self.d, 0, self.n_q, self.hq)

    def setup(self, K, torch, seed0):
        from long_context_decode_kv_amd import synth
        self.k, self.v, self.q, self.out, self.lse = [], [], [], [], []
        for layer in range(self.layers):
            s = seed0 * 100 + layer
            self.k.append(synth.device_f16_cache(3 * s, self.capacity, self.hkv, self.d))
            self.v.append(synth.device_f16_cache(3 * s + 1, self.capacity, self.hkv, self.d))
            self.q.append(synth.device_q(3 * s + 2, self.n_q, self.hq, self.d))
            self.out.append(torch.empty(self.n_q, self.hq, self.d, device="cuda"))
            self.lse.append(torch.empty(self.n_q, self.hq, device="cuda"))
            if layer % 8 == 7:
                log(f"  generated {layer + 1}/{self.layers} layers")
        self.plan = K.plan(self.hq, self.hkv, self.d, 1, self.capacity, n_occupied=[self.occupied],
                           n_queries=self.n_q, split_cells=self.split_cells, kernel=self.kernel)
        self.ws = K.workspace(self.plan)
        self.q_pos = None
        if self.n_q > 1:
            self.q_pos = torch.arange(self.occupied - self.n_q, self.occupied, dtype=torch.int32, device="cuda")

    def launch(self, K, layer):
        K.attend(self.plan, self.q[layer], self.k[layer], self.v[layer], self.ws, out=self.out[layer],
                 lse=self.lse[layer], q_pos=self.q_pos)

    def stored_layer(self, layer):
        """The stored tensors of one layer: (q, K, V) device views of the
        attended cells."""
        return self.q[layer], self.k[layer][:self.occupied], self.v[layer][:self.occupied]

    def oracle_sample(self, budget_s, max_layers=None):
        """Time the float64 oracle on host copies of the exact stored tensors
        (device-to-host copies timed apart): whole layers, in order, until
        the budget is spent (at least one).  Returns (layers, oracle seconds,
        description, copy seconds)."""
        import numpy as np
        import torch
        import oracle as O
        max_layers = max_layers or self.layers
        done, el, d2h = 0, 0.0, 0.0
        while True:
            t0 = time.perf_counter()
            qd, kd, vd = self.stored_layer(done % self.layers)
            q = qd.cpu().numpy()
            kc = kd.cpu().numpy().view(np.uint16)
            vc = vd.cpu().numpy().view(np.uint16)
            torch.cuda.synchronize()
            d2h += time.perf_counter() - t0
            regions = [((O.F16, kc, None), (O.F16, vc, None), [np.arange(kc.shape[0])])]
            t0 = time.perf_counter()
            if self.n_q > 1:
                qp = np.arange(self.occupied - self.n_q, self.occupied)[None]
                O.decode_attention_multi(q[None], regions, self.hkv, 1 / math.sqrt(self.d), qp)
            else:
                O.decode_attention(q, regions, self.hkv, 1 / math.sqrt(self.d))
            el += time.perf_counter() - t0
            done += 1
            if el >= budget_s or done >= max_layers:
                return done, el, f"{done} of {max_layers} layers, host copies of the stored tensors (full layer " \
                                 f"each: {self.occupied} cells x {self.hkv} KV heads x {self.hq} q heads)", d2h


class Gqa6Quant(Workload):
    """One launch over four slots (131072 / 65536 / 20000 / 777 cells) whose
    128-cell records are interleaved in one cache, block-scaled K and V.
    ``copies`` independent caches are rotated so repeated steps cannot be
    served from the 256 MB MALL."""

    cycle = 4  # steps per captured cycle (one launch per step, caches rotated)

    def __init__(self, name, kind, copies=4, v_kind=None):
        self.name, self.kind, self.layers = name, kind, copies
        self.v_kind = kind if v_kind is None else v_kind
        self.hq, self.hkv, self.d = 24, 4, 256
        self.lengths = [131072, 65536, 20000, 777]

    def config(self):
        return {"workload": self.name, "q_heads": 24, "kv_heads": 4, "head_dim": 256, "slots": 4,
                "cells_per_slot": self.lengths,
                "kv_dtype": ("K " if self.v_kind != self.kind else "") + KDESC[self.kind] +
                            (" / V " + KDESC[self.v_kind] if self.v_kind != self.kind else ""),
                "indirect_plan": "128-cell records interleaved round-robin across slots, -1 holes",
                "rotated_cache_copies": self.layers}

    def algorithmic_bytes_per_launch(self):
        return algorithmic_bytes(sum(self.lengths), self.hkv, self.d, self.kind, 4, self.hq, self.n_entries,
                                 self.v_kind)

    def setup(self, K, torch, seed0):
        import numpy as np
        from long_context_decode_kv_amd import synth
        lists, cap = synth.interleaved_record_lists(self.lengths)
        t0 = time.perf_counter()
        self.plan = K.plan(24, 4, 256, 4, cap, k_type=self.kind, v_type=self.v_kind, cells=lists)
        entries, offs = self.plan.cells()
        self.n_entries = len(entries)
        self.plan_cells = torch.from_numpy(entries).cuda()
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3
        # the same plan built on the device from the raw lists (kvdec_build_cells)
        budget = [int(offs[i + 1] - offs[i]) // 128 for i in range(4)]
        dplan = K.plan(24, 4, 256, 4, cap, k_type=self.kind, v_type=self.v_kind, max_records=budget)
        dws = K.workspace(dplan)
        raw = torch.from_numpy(np.concatenate([np.asarray(x, np.int32) for x in lists])).cuda()
        raw_off = torch.from_numpy(np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int64)).cuda()
        dcells = torch.empty(dplan.info()["n_entries"], dtype=torch.int32, device="cuda")
        K.build_cells(dplan, raw, raw_off, dcells, dws)
        torch.cuda.synchronize()
        assert torch.equal(dcells, self.plan_cells)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(20):
            K.build_cells(dplan, raw, raw_off, dcells, dws)
        b.record()
        torch.cuda.synchronize()
        self.plan_build = {"raw_entries": int(raw.numel()), "plan_entries": self.n_entries,
                           "host_kvdec_plan_and_upload_ms": round(host_ms, 3),
                           "device_kvdec_build_cells_us": round(a.elapsed_time(b) * 1e3 / 20, 2)}
        self.k, self.v, self.q, self.out, self.lse = [], [], [], [], []
        for c in range(self.layers):
            s = seed0 * 100 + c
            self.k.append(synth.device_quant_cache(3 * s, self.kind, cap, 4, 256))
            self.v.append(synth.device_quant_cache(3 * s + 1, self.v_kind, cap, 4, 256))
            self.q.append(synth.device_q(3 * s + 2, 4, 24, 256))
            self.out.append(torch.empty(4, 24, 256, device="cuda"))
            self.lse.append(torch.empty(4, 24, device="cuda"))
        self.ws = K.workspace(self.plan)

    def extra(self):
        return {"plan_build": self.plan_build}

    def launch(self, K, i):
        K.attend(self.plan, self.q[i], self.k[i][0], self.v[i][0], self.ws, out=self.out[i], lse=self.lse[i],
                 k_scales=self.k[i][1], v_scales=self.v[i][1], plan_cells=self.plan_cells)

    def oracle_sample(self, budget_s):
        """The oracle on host copies of the stored cache rows of the
        20000-cell slot (gathered on the device through the plan's entries,
        copy timed apart), scaled by cell count to all four slots."""
        import numpy as np
        import torch
        import oracle as O
        entries, offs = self.plan.cells()
        cells = entries[offs[2]:offs[3]]
        cells = cells[cells >= 0]
        n = len(cells)
        t0 = time.perf_counter()
        idx = torch.from_numpy(cells.astype(np.int64)).cuda()
        q = self.q[0][2:3].cpu().numpy()
        kc, ks = (t.index_select(0, idx).cpu().numpy() for t in self.k[0])
        vc, vs = (t.index_select(0, idx).cpu().numpy() for t in self.v[0])
        torch.cuda.synchronize()
        d2h = time.perf_counter() - t0
        ks, vs = ks.view(np.uint16), vs.view(np.uint16)
        t0 = time.perf_counter()
        done = 0
        while True:
            O.decode_attention(q, [((self.kind, kc, ks), (self.v_kind, vc, vs), [np.arange(n)])], 4, 1 / 16)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget_s or done >= 4:
                break
        total = el / (done * n) * sum(self.lengths)
        return 1, total, f"the {n}-cell slot x 4 KV heads x 24 q heads, host copies of its stored rows, timed " \
                         f"{done}x ({el:.1f} s), scaled by cell count to all {sum(self.lengths)} attended cells", d2h


class RollingWindow(ContiguousModel):
    eager_only = True  # host-tail copies and events are enqueued per call
    """Qwen3-8B shape at ctx 40960: per layer the newest 14000 cells are
    resident and the oldest 26960 stream from pinned host memory through the
    workspace ring (copy stream + events), merged by log-sum-exp."""

    chunk = 0  # tail cells per chunk (bench.py --tail-chunk); 0: the whole tail (the library's default chunking)

    def __init__(self, name="rolling-ctx40960", mode="staged"):
        super().__init__(name, 36, 32, 8, 128, 40960, 40960)
        self.window, self.tail, self.mode = 14000, 26960, mode
        if not self.chunk:
            self.chunk = -(-self.tail // 128) * 128

    def config(self):
        c = super().config()
        c.update({"cells_resident_window": self.window, "cells_host_tail": self.tail, "tail_chunk_cells": self.chunk,
                  "ring_depth": 4, "tail_mode": {
                      "staged": "copies into a workspace ring; each call's copies wait for earlier work",
                      "prefetch": "copies into a ring; layers alternate two workspaces and each call's copies "
                                  "wait only for the call two layers back (cross-layer prefetch)",
                      "zerocopy": "chunk kernels read the pinned host tail in place"}[self.mode]})
        return c

    def algorithmic_bytes_per_launch(self):
        return algorithmic_bytes(self.occupied, self.hkv, self.d, 0, 1, self.hq)

    def pcie_bytes_per_launch(self):
        return 2 * self.tail * self.hkv * self.d * 2

    def setup(self, K, torch, seed0):
        from long_context_decode_kv_amd import synth
        self.k, self.v, self.q, self.out, self.lse, self.hk, self.hv = [], [], [], [], [], [], []
        for layer in range(self.layers):
            s = seed0 * 100 + layer
            kd = synth.device_f16_cache(3 * s, self.capacity, self.hkv, self.d)
            vd = synth.device_f16_cache(3 * s + 1, self.capacity, self.hkv, self.d)
            hk = torch.empty((self.tail, self.hkv, self.d), dtype=torch.float16, pin_memory=True)
            hv = torch.empty((self.tail, self.hkv, self.d), dtype=torch.float16, pin_memory=True)
            hk.copy_(kd[:self.tail])
            hv.copy_(vd[:self.tail])
            self.k.append(kd)
            self.v.append(vd)
            self.hk.append(hk)
            self.hv.append(hv)
            self.q.append(synth.device_q(3 * s + 2, 1, self.hq, self.d))
            self.out.append(torch.empty(1, self.hq, self.d, device="cuda"))
            self.lse.append(torch.empty(1, self.hq, device="cuda"))
        self.plan = K.plan(self.hq, self.hkv, self.d, 1, self.capacity, n_occupied=[self.window],
                           cell_begin=[self.tail], n_tail=[self.tail], tail_capacity_cells=self.tail,
                           tail_chunk_cells=self.chunk, tail_ring_depth=4, tail_zero_copy=self.mode == "zerocopy")
        self.ws = [K.workspace(self.plan) for _ in range(2 if self.mode == "prefetch" else 1)]
        self.ev = [torch.cuda.Event() for _ in range(2)]
        self.copy_stream = torch.cuda.Stream()
        self.window_plan = K.plan(self.hq, self.hkv, self.d, 1, self.capacity, n_occupied=[self.window],
                                  cell_begin=[self.tail])
        self.window_ws = K.workspace(self.window_plan)

    def launch(self, K, layer):
        pre = self.mode == "prefetch"
        K.attend(self.plan, self.q[layer], self.k[layer], self.v[layer], self.ws[layer % 2 if pre else 0],
                 out=self.out[layer], lse=self.lse[layer], k_tail=self.hk[layer], v_tail=self.hv[layer],
                 copy_stream=self.copy_stream, copy_after=self.ev[layer % 2] if pre else None)
        if pre:
            self.ev[layer % 2].record()

    def resident_only_us(self, K, torch, reps=5):
        """Step time of the resident windows alone (no tail): the first term
        of t = resident + tail bytes / link rate."""
        def step():
            for layer in range(self.layers):
                K.attend(self.window_plan, self.q[layer], self.k[layer], self.v[layer], self.window_ws,
                         out=self.out[layer], lse=self.lse[layer])
        step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            step()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps


class ContiguousModelOneLaunch(ContiguousModel):
    """Secondary figure: every layer of a ContiguousModel as one slot of a
    single launch (one cache allocation, layer l's cells at l * capacity)."""

    def __init__(self, name, layers, hq, hkv, d, capacity, occupied):
        super().__init__(name, layers, hq, hkv, d, capacity, occupied)
        self.model_layers, self.layers = layers, 1

    def config(self):
        c = super().config()
        c.update({"layers": self.model_layers, "launch": f"all {self.model_layers} layers as slots of one call",
                  "figure": "secondary: ignores the layer-to-layer dependency of a real decode step"})
        return c

    def algorithmic_bytes_per_launch(self):
        return algorithmic_bytes(self.occupied * self.model_layers, self.hkv, self.d, 0, self.model_layers, self.hq)

    def setup(self, K, torch, seed0):
        from long_context_decode_kv_amd import synth
        L, cap = self.model_layers, self.capacity
        kc = torch.empty((L * cap, self.hkv, self.d), dtype=torch.float16, device="cuda")
        vc = torch.empty_like(kc)
        q = torch.empty((L, self.hq, self.d), device="cuda")
        for layer in range(L):
            s = seed0 * 100 + layer
            synth.device_f16_cache(3 * s, cap, self.hkv, self.d, out=kc[layer * cap:(layer + 1) * cap])
            synth.device_f16_cache(3 * s + 1, cap, self.hkv, self.d, out=vc[layer * cap:(layer + 1) * cap])
            q[layer] = synth.device_q(3 * s + 2, 1, self.hq, self.d)[0]
        self.k, self.v, self.q = [kc], [vc], [q]
        self.out = [torch.empty(L, self.hq, self.d, device="cuda")]
        self.lse = [torch.empty(L, self.hq, device="cuda")]
        self.plan = K.plan(self.hq, self.hkv, self.d, L, L * cap, n_occupied=[self.occupied] * L,
                           split_cells=self.split_cells,
                           cell_begin=[layer * cap for layer in range(L)])
        self.ws = K.workspace(self.plan)
        self.q_pos = None

    def stored_layer(self, layer):
        cap = self.capacity
        return self.q[0][layer:layer + 1], self.k[0][layer * cap:layer * cap + self.occupied], \
            self.v[0][layer * cap:layer * cap + self.occupied]

    def oracle_sample(self, budget_s):
        saved, self.layers = self.layers, self.model_layers
        try:
            done, el, sample, d2h = super().oracle_sample(budget_s, self.model_layers)
        finally:
            self.layers = saved
        return done / self.model_layers, el, sample, d2h


class RotatedLayer(ContiguousModel):
    """One layer per step, rotated over ``copies`` independent caches (over
    the 256 MB MALL in total) so that repeated steps read HBM."""

    def __init__(self, name, copies, hq, hkv, d, occupied):
        super().__init__(name, copies, hq, hkv, d, occupied, occupied)
        self.cycle = copies

    def config(self):
        c = super().config()
        c.update({"layers": 1, "rotated_cache_copies": self.layers,
                  "rotated_bytes": self.layers * self.occupied * self.hkv * self.d * 4})
        return c


WORKLOADS = {
    "single-4096": lambda: RotatedLayer("single-4096", 32, 32, 8, 128, 4096),
    "qwen3-8b-ctx16k": lambda: ContiguousModel("qwen3-8b-ctx16k", 36, 32, 8, 128, 16384, 13100),
    "qwen2.5-14b-1m": lambda: ContiguousModel("qwen2.5-14b-1m", 48, 40, 8, 128, 524288, 524288),
    "gqa6-q8": lambda: Gqa6Quant("gqa6-q8", 1),
    "gqa6-q4": lambda: Gqa6Quant("gqa6-q4", 2),
    "gqa6-q8k-q4v": lambda: Gqa6Quant("gqa6-q8k-q4v", 1, v_kind=2),
    "rolling-ctx40960": lambda: RollingWindow(),
    "rolling-ctx40960-prefetch": lambda: RollingWindow("rolling-ctx40960-prefetch", "prefetch"),
    "rolling-ctx40960-zerocopy": lambda: RollingWindow("rolling-ctx40960-zerocopy", "zerocopy"),
    "qwen3-8b-ctx16k-verify4": lambda: ContiguousModel("qwen3-8b-ctx16k-verify4", 36, 32, 8, 128, 16384, 13100,
                                                        n_q=4),
    "qwen3-8b-ctx16k-1launch": lambda: ContiguousModelOneLaunch("qwen3-8b-ctx16k-1launch", 36, 32, 8, 128, 16384,
                                                                13100),
}


# ---------------------------------------------------------------- traffic from committed counters

def strip_c_comments(text):
    """C / C++ source without its comments and with runs of whitespace
    collapsed, string and character literals kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_source_hash():
    """Hash of the code (comments and layout ignored) of every source that
    decides what the split and merge kernels do -- the kernels, the planner
    that picks their launch shape, and the dispatch -- and of the flags
    particular sources are compiled with."""
    import glob
    csrc = os.path.join(ROOT, "long_context_decode_kv_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*.hip"))) + [os.path.join(csrc, f) for f in
                                                              ("split_kernels.h", "internal.h", "plan.cpp",
                                                               "api.cpp")]
    h = hashlib.sha256()
    for f in files:
        if os.path.basename(f) != "probe.hip":
            h.update(strip_c_comments(open(f, encoding="utf-8").read()).encode())
    from long_context_decode_kv_amd.build import SOURCE_FLAGS  # per-source compiler flags change the code too
    h.update(repr(sorted(SOURCE_FLAGS.items())).encode())
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per dispatch from the committed rocprofv3 --pmc summary of
    this workload, if it was taken with the current kernel source."""
    import glob
    paths = glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}_pmc.txt"))
    if len(paths) != 1:
        return None
    text = open(paths[0]).read()
    m = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    t = re.search(r"hbm_bytes_per_dispatch:\s*([0-9.]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def kernel_label(wl, info):
    """Name of the split-kernel instance a workload's plan launches."""
    kv, vv = KIND[wl.kind], KIND[getattr(wl, "v_kind", wl.kind)]
    g = wl.hq // wl.hkv
    if info.get("matrix_cores"):
        return "split_mfma_kernel<%d,rows %d,%s,%s,%d waves>" % (wl.d, g * getattr(wl, "n_q", 1), kv, vv,
                                                                 info.get("waves", 4))
    if info.get("kernel") == 2:
        cw = (-(-info["split_cells"] // 8) + 1) & ~1
        jm = -(-cw // 8)
        return "split_oneshot_kernel<%d,%d>" % (g, 2 if jm <= 2 else (4 if jm <= 4 else 7))
    return "split_kernel<%d,%d,%s,%s,%d waves>" % (wl.d, g, kv, vv, info.get("waves", 4))


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3-8b-ctx16k", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="graph", choices=["graph", "eager"])
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true", help="skip the streaming-read ceiling (profiling runs)")
    ap.add_argument("--split-cells", type=int, default=0,
                    help="cells per split for the contiguous-model workloads (multiple of 32; 0: planner)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "streamed", "oneshot"],
                    help="vector-ALU split kernel for the contiguous-model workloads (default: the planner's choice)")
    ap.add_argument("--tail-chunk", type=int, default=0,
                    help="host-tail cells per chunk (rolling workloads; 0: the whole tail in one chunk)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the path shards by KV head, "
              f"layer or cell range with one small partial exchange, but no multi-GPU code is built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_decode_kv_amd.build import ensure_built
    ensure_built()
    from long_context_decode_kv_amd import kvdec as K
    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    RollingWindow.chunk = args.tail_chunk
    ContiguousModel.split_cells = args.split_cells
    ContiguousModel.kernel = {"auto": 0, "streamed": 1, "oneshot": 2}[args.kernel]
    wl = WORKLOADS[args.workload]()
    log(f"[bench] workload {wl.name}: generating inputs on the device")
    wl.setup(K, torch, 1001)
    torch.cuda.synchronize()
    info = wl.plan.info()
    log(f"[bench] plan: {info}")
    stream = torch.cuda.current_stream()

    cycle = getattr(wl, "cycle", 1)          # steps covered by one pass over the launch list
    launches_per_step = wl.layers // cycle
    mode = "eager" if getattr(wl, "eager_only", False) else args.mode

    def one_cycle():
        for layer in range(wl.layers):
            wl.launch(K, layer)

    # warm-up (eager), then optional graph capture of one cycle
    for _ in range(max(1, args.warmup // cycle)):
        one_cycle()
    torch.cuda.synchronize()
    graph = None
    if mode == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_cycle()
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup // cycle)):
            graph.replay()
        torch.cuda.synchronize()

    # timed region 1: whole steps
    n_cycles = max(1, args.steps // cycle)
    steps = n_cycles * cycle
    log(f"[bench] timing {steps} steps ({mode})")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_cycles + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs[0].record(stream)
    for c in range(n_cycles):
        if graph is not None:
            graph.replay()
        else:
            one_cycle()
        evs[c + 1].record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms_per_step = evs[0].elapsed_time(evs[-1]) / steps
    per_cycle = sorted(evs[c].elapsed_time(evs[c + 1]) * 1e3 / cycle for c in range(n_cycles))  # us per step

    def pct(p):
        return round(per_cycle[min(len(per_cycle) - 1, int(p * len(per_cycle)))], 2)

    # timed region 2: every launch bracketed by its own events on its stream
    # (adds the dispatch overhead of an isolated launch)
    reps = max(1, min(n_cycles, 20 // cycle if cycle > 1 else 20))
    n_ev = reps * wl.layers
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    torch.cuda.synchronize()
    i = 0
    for _ in range(reps):
        for layer in range(wl.layers):
            starts[i].record(stream)
            wl.launch(K, layer)
            ends[i].record(stream)
            i += 1
    torch.cuda.synchronize()
    durs = sorted(s_.elapsed_time(e_) * 1e3 for s_, e_ in zip(starts, ends))  # microseconds
    bracketed_us = sum(durs) / len(durs)
    # average launch duration over timed region 1: a step is nothing but
    # back-to-back launches on one stream
    avg_us = ms_per_step * 1e3 / launches_per_step

    bytes_launch = wl.algorithmic_bytes_per_launch()
    bytes_step = bytes_launch * launches_per_step
    gbs = bytes_step / (ms_per_step * 1e-3) / 1e9
    achieved = bytes_launch / (avg_us * 1e-6) / 1e9
    traffic = committed_traffic(wl.name)
    ceiling = None
    if not args.no_read_ceiling:
        (c_gbs, c_us, c_shape), c_sweep = measure_read_ceiling(torch, bytes_launch, launches_per_step)
        ceiling = {"method": "kvprobe_read_shape: plain 16-byte streaming read of the same bytes per launch, same "
                             "launches per step, best of a sweep of launch shapes",
                   "shape": c_shape, "gbs": c_gbs, "us_per_launch": c_us, "frac_of_ceiling": round(achieved / c_gbs, 4),
                   **c_sweep}

    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info
        layers_done, el, sample, d2h = wl.oracle_sample(args.cpu_budget)
        pools = threadpool_info()
        threads = max([p.get("num_threads", 1) for p in pools] + [1])
        blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in pools
                                 if p.get("user_api") == "blas"}))
        cpu = {"value": round(bytes_launch * layers_done / el / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "sample": sample + f"; {el:.1f} s float64 numpy on the host",
               "blas": blas or None, "host_cpus": os.cpu_count(),
               "us_per_step_extrapolated": round(el / layers_done * launches_per_step * 1e6, 1),
               "d2h_copy_s": round(d2h, 4),
               "d2h_note": "device-to-host copies of the stored tensors, timed apart from the oracle"}
        # the same oracle on one thread, where one unit of the sample stays short
        if el / layers_done * threads < 20.0:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                d1, e1, s1, _ = wl.oracle_sample(min(4.0, args.cpu_budget / 3))
            cpu["value_1thread"] = round(bytes_launch * d1 / e1 / 1e9, 4)
            cpu["sample_1thread"] = s1 + f"; {e1:.1f} s on 1 thread"

    res = {
        "metric": "decode-attention µs/step and effective KV GB/s (fraction of HBM peak)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ({0: "f16 KV", 1: "int8 KV (f16 scale per 32)", 2: "4-bit KV (f16 scale per 32)"}[wl.kind]
                  if getattr(wl, "v_kind", wl.kind) == wl.kind else
                  f"{KIND[wl.kind]} K / {KIND[wl.v_kind]} V (f16 scale per 32)") + ", fp32 accumulate",
        "data": "synthetic: q ~ N(0,1); K, V ~ N(0,1) rounded to f16 or block-encoded; seeded on-device generator",
        "config": dict(wl.config(), mode=mode, workgroups_per_launch=info["n_workgroups"],
                       tiles_per_split=info["tiles_per_split"], cells_per_split=info["split_cells"]),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": kernel_label(wl, info),
                     "algorithmic_bytes_per_launch": bytes_launch, "launches_per_step": launches_per_step,
                     "avg_launch_us": round(avg_us, 3), "isolated_launch_event_us": round(bracketed_us, 3),
                     "read_ceiling": ceiling},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall_s, 4),
        "kernel_source_sha256_16": kernel_source_hash(),
        "library_source_hash": K.LIB_SOURCE_HASH,
    }
    if hasattr(wl, "extra"):
        res.update(wl.extra())
    if hasattr(wl, "pcie_bytes_per_launch"):
        pb = wl.pcie_bytes_per_launch() * launches_per_step
        link = measure_h2d(torch)
        resident_us = wl.resident_only_us(K, torch)
        model_us = resident_us + pb / (link * 1e9) * 1e6
        res["pcie"] = {"h2d_bytes_per_step": pb, "h2d_gbs_effective": round(pb / (ms_per_step * 1e-3) / 1e9, 2),
                       "link_gbs_measured": link, "frac_of_link": round(pb / (ms_per_step * 1e-3) / 1e9 / link, 4),
                       "resident_only_us_per_step": round(resident_us, 1),
                       "model_us_per_step": round(model_us, 1),
                       "model": "t = resident_only + tail_bytes / link rate",
                       "residual_vs_model": round(ms_per_step * 1e3 / model_us - 1, 4)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
