"""Decode-attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode graph|eager]

A step is one decode step of attention over the whole model: for every layer
one kvdec_attend call (plan -> split kernel with fused log-sum-exp merge)
over that layer's own resident KV cache, q and outputs.  Inputs are resident
in HBM before the timed region.  Prints one JSON line on stdout; progress
goes to stderr.

Workloads (synthetic N(0, 1) data of the named model's attention shape):
  qwen3-8b-ctx16k   36 layers x (32 q heads, 8 KV heads, head_dim 128),
                    13100 occupied cells of a 16384-cell f16 cache (default)
  qwen2.5-14b-1m    48 layers x (40 q / 8 KV heads, head_dim 128), 524288
                    cells of f16 K/V (96 GiB)
  gqa6-q8 / gqa6-q4 one layer, 24 q / 4 KV heads, head_dim 256, four slots of
                    131072 / 65536 / 20000 / 777 cells in interleaved 128-cell
                    records, block-scaled int8 / 4-bit K and V
  rolling-ctx40960  qwen3-8b shape at ctx 40960: newest 14000 cells resident,
                    oldest 26960 streamed from pinned host memory per layer
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


def algorithmic_bytes(n_cells_attended, hkv, d, kind, n_slots, hq, plan_entries=0):
    """Bytes the method must move for one evaluation: the attended cells' K
    and V codes and scales, the indirect plan (4 B per entry), q (fp32) and
    out (fp32).  Unoccupied cells, hole cells, partials and re-reads are not
    counted."""
    kv = 2 * n_cells_attended * hkv * (kv_row_bytes(kind, d) + scale_row_bytes(kind, d))
    return kv + 4 * plan_entries + 2 * 4 * n_slots * hq * d


class ContiguousModel(Workload):
    def __init__(self, name, layers, hq, hkv, d, capacity, occupied):
        self.name, self.layers, self.hq, self.hkv, self.d = name, layers, hq, hkv, d
        self.capacity, self.occupied, self.kind = capacity, occupied, 0

    def config(self):
        return {"workload": self.name, "layers": self.layers, "q_heads": self.hq, "kv_heads": self.hkv,
                "head_dim": self.d, "cells_occupied": self.occupied, "cells_capacity": self.capacity,
                "batch": 1, "kv_dtype": "f16", "cells_per_tile": 128}

    def algorithmic_bytes_per_launch(self):
        return algorithmic_bytes(self.occupied, self.hkv, self.d, 0, 1, self.hq)

    def setup(self, K, torch, seed0):
        from long_context_decode_kv_amd import synth
        self.k, self.v, self.q, self.out, self.lse = [], [], [], [], []
        for layer in range(self.layers):
            s = seed0 * 100 + layer
            self.k.append(synth.device_f16_cache(3 * s, self.capacity, self.hkv, self.d))
            self.v.append(synth.device_f16_cache(3 * s + 1, self.capacity, self.hkv, self.d))
            self.q.append(synth.device_q(3 * s + 2, 1, self.hq, self.d))
            self.out.append(torch.empty(1, self.hq, self.d, device="cuda"))
            self.lse.append(torch.empty(1, self.hq, device="cuda"))
            if layer % 8 == 7:
                log(f"  generated {layer + 1}/{self.layers} layers")
        self.plan = K.plan(self.hq, self.hkv, self.d, 1, self.capacity, n_occupied=[self.occupied])
        self.ws = K.workspace(self.plan)

    def launch(self, K, layer):
        K.attend(self.plan, self.q[layer], self.k[layer], self.v[layer], self.ws, out=self.out[layer],
                 lse=self.lse[layer])

    def oracle_sample(self, budget_s):
        """Time the float64 oracle on host copies of the workload's shape:
        whole layers until the budget is spent (at least one)."""
        import numpy as np
        import oracle as O
        from long_context_decode_kv_amd import synth
        r = synth.rng(99)
        q = synth.gen_q(r, 1, self.hq, self.d)
        kc = synth.gen_f16_cache(r, self.occupied, self.hkv, self.d)
        vc = synth.gen_f16_cache(r, self.occupied, self.hkv, self.d)
        cells = [np.arange(self.occupied)]
        done, t0 = 0, time.perf_counter()
        while True:
            O.decode_attention(q, [((O.F16, kc, None), (O.F16, vc, None), cells)], self.hkv, 1 / math.sqrt(self.d))
            done += 1
            el = time.perf_counter() - t0
            if el >= budget_s or done >= self.layers:
                return done, el, f"{done} of {self.layers} layers (full layer each: {self.occupied} cells x " \
                                 f"{self.hkv} KV heads x {self.hq} q heads)"


WORKLOADS = {
    "qwen3-8b-ctx16k": lambda: ContiguousModel("qwen3-8b-ctx16k", 36, 32, 8, 128, 16384, 13100),
    "qwen2.5-14b-1m": lambda: ContiguousModel("qwen2.5-14b-1m", 48, 40, 8, 128, 524288, 524288),
}


# ---------------------------------------------------------------- traffic from committed counters

def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("kernels.hip", "internal.h"):
        h.update(open(os.path.join(ROOT, "long_context_decode_kv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per dispatch from the committed rocprofv3 --pmc summary of
    this workload, if it was taken with the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"split_kernel_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    t = re.search(r"hbm_bytes_per_dispatch:\s*([0-9.]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


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
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the path shards by KV head, "
              f"layer or cell range with one small partial exchange, but no multi-GPU code is built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_decode_kv_amd import kvdec as K
    torch.cuda.set_device(0)
    wl = WORKLOADS[args.workload]()
    log(f"[bench] workload {wl.name}: generating inputs on the device")
    wl.setup(K, torch, 1001)
    torch.cuda.synchronize()
    info = wl.plan.info()
    log(f"[bench] plan: {info}")
    stream = torch.cuda.current_stream()

    def step():
        for layer in range(wl.layers):
            wl.launch(K, layer)

    # warm-up (eager), then optional graph capture of one step
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.mode == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()

    # timed region 1: whole steps
    log(f"[bench] timing {args.steps} steps ({args.mode})")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # timed region 2: every split-kernel launch bracketed by its own events on
    # its stream (adds the dispatch overhead of an isolated launch)
    n_ev = min(args.steps, 20) * wl.layers
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    torch.cuda.synchronize()
    i = 0
    for _ in range(min(args.steps, 20)):
        for layer in range(wl.layers):
            starts[i].record(stream)
            wl.launch(K, layer)
            ends[i].record(stream)
            i += 1
    torch.cuda.synchronize()
    durs = sorted(s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends))  # microseconds
    bracketed_us = sum(durs) / len(durs)
    # average launch duration over timed region 1: the step is nothing but
    # back-to-back split-kernel launches on one stream
    avg_us = ms_per_step * 1e3 / wl.layers

    bytes_launch = wl.algorithmic_bytes_per_launch()
    bytes_step = bytes_launch * wl.layers
    gbs = bytes_step / (ms_per_step * 1e-3) / 1e9
    achieved = bytes_launch / (avg_us * 1e-6) / 1e9
    traffic = committed_traffic(wl.name)

    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info
        layers_done, el, sample = wl.oracle_sample(args.cpu_budget)
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        cpu = {"value": round(bytes_launch * layers_done / el / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "sample": sample + f"; {el:.1f} s float64 numpy on the host",
               "us_per_step_extrapolated": round(el / layers_done * wl.layers * 1e6, 1)}

    res = {
        "metric": "decode-attention µs/step and effective KV GB/s (fraction of HBM peak)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 KV, fp32 accumulate",
        "data": "synthetic: q, K, V ~ N(0,1), K/V rounded to f16, seeded on-device generator",
        "config": dict(wl.config(), mode=args.mode, workgroups_per_launch=info["n_workgroups"],
                       tiles_per_split=info["tiles_per_split"]),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "split_kernel<128,%d,f16,f16>" % (wl.hq // wl.hkv),
                     "algorithmic_bytes_per_launch": bytes_launch, "launches_per_step": wl.layers,
                     "avg_launch_us": round(avg_us, 3), "isolated_launch_event_us": round(bracketed_us, 3)},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall_s, 4),
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
