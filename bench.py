"""PPSA decode-step benchmark on one MI355X.

Times whole decode steps (every layer of the schedule: full, full + top-k
selection, sparse) through the C ABI entry point ppsa_decode_step, with all
inputs resident in HBM, and prints one JSON line: achieved KV GB/s (the
algorithmic K+V bytes a step must read, divided by the step time), step
microseconds, the fraction of the 8 TB/s HBM peak, a per-layer-kind
breakdown, the roofline of the dominant kernel and the float64 CPU oracle
timed over the same decode step on one host thread.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "PPSA decode-step attention µs and achieved KV GB/s (% of HBM peak)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--breakdown-steps", type=int, default=None)
    p.add_argument("--copy-probe", action="store_true", help="also time a plain device copy of known size")
    return p.parse_args()


class OracleTimer:
    """Times the float64 oracle over the whole decode step, one layer at a time as layers are generated."""

    def __init__(self, wl, seq_lens):
        import oracle

        self.oracle = oracle
        self.wl = wl
        self.seq_lens = seq_lens
        self.scale = oracle.default_scale(wl.head_dim)
        self.sel = None
        self.secs = 0.0

    def __call__(self, layer, q, K, V):
        import threadpoolctl

        kind = self.wl.schedule()[layer]
        t0 = time.perf_counter()
        with threadpoolctl.threadpool_limits(1):
            _, self.sel, _ = self.oracle.decode_layer(kind, q, K, V, self.seq_lens, self.wl.group, self.wl.topk,
                                                      self.scale, self.wl.dtype, self.sel)
        self.secs += time.perf_counter() - t0

    def result(self, step_bytes):
        return {"value": round(step_bytes / self.secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "step_us": round(self.secs * 1e6, 1),
                "sample": f"the whole decode step ({self.wl.layers} layers, all {self.wl.batch * self.wl.kv_heads} "
                          f"(batch, KV head) units) on 1 thread, {self.secs:.1f} s; inputs generated outside the "
                          f"timed calls"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the PPSA path here is single-GPU",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import position_persistent_sparse_amd as ppsa
    import synth
    from synth import torch_io

    wl = synth.WORKLOADS[args.workload or synth.BENCH_WORKLOAD]
    dev = torch.device("cuda:0")
    gen = synth.Generator(wl)
    timer = None if args.no_cpu_baseline else OracleTimer(wl, gen.seq_lens)
    log(f"generating {wl.name}: {wl.layers} layers, B={wl.batch}, Hq={wl.q_heads}, Hkv={wl.kv_heads}, "
        f"N={wl.max_len}, k={wl.topk}, {wl.dtype}" + ("" if timer is None else "; timing the oracle per layer"))
    t0 = time.time()
    q, k, v, lens, _ = torch_io.upload(wl, gen, dev, keep_layers=set(), visit=timer)
    torch.cuda.synchronize()
    log(f"inputs resident on {torch.cuda.get_device_name(dev)} after {time.time() - t0:.1f} s")

    sched = wl.schedule()
    n_sel = sched.count("X")
    dims = ppsa.make_dims(wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim, wl.max_len, torch_io.torch_dtype(wl))
    ws = ppsa.alloc_workspace(dims, wl.topk, dev)
    out = torch.empty_like(q)
    idx = torch.empty((n_sel, wl.batch, wl.kv_heads, wl.topk), dtype=torch.int32, device=dev)
    codes = ppsa.schedule_codes(sched)

    def step():
        ppsa.decode_step(sched, q, k, v, lens, wl.topk, out=out, idx=idx, workspace=ws, sched_codes=codes)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    step_bytes = synth.step_kv_bytes(wl, gen.seq_lens)
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us, {gbs:.1f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of peak)")

    # Per-layer-kind breakdown: the same kernels, one entry-point call per layer, HIP events around each call on
    # the stream the kernels run on (torch's current stream).
    bsteps = args.breakdown_steps or max(3, min(args.steps, 10))
    per_kind = {"F": [], "X": [], "S": []}
    stream = torch.cuda.current_stream(dev)
    for it in range(bsteps + 1):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(wl.layers + 1)]
        evs[0].record(stream)
        sel = -1
        for layer, kind in enumerate(sched):
            if kind == "F":
                ppsa.full_attn(q[layer], k[layer], v[layer], lens, out=out[layer], workspace=ws)
            elif kind == "X":
                sel += 1
                ppsa.full_attn_select(q[layer], k[layer], v[layer], lens, wl.topk, out=out[layer], idx=idx[sel],
                                      workspace=ws)
            else:
                ppsa.sparse_attn(q[layer], k[layer], v[layer], lens, idx[sel], out=out[layer], workspace=ws)
            evs[layer + 1].record(stream)
        torch.cuda.synchronize()
        if it == 0:
            continue  # warm-up pass
        for layer, kind in enumerate(sched):
            per_kind[kind].append(evs[layer].elapsed_time(evs[layer + 1]) * 1e3)
    avg = {kk: float(np.mean(vv)) for kk, vv in per_kind.items() if vv}
    layer_bytes = {kk: synth.layer_kv_bytes(wl, kk, gen.seq_lens) for kk in avg}
    totals = {kk: avg[kk] * sched.count(kk) for kk in avg}
    breakdown = {kk: {"layers": sched.count(kk), "us_per_layer": round(avg[kk], 2),
                      "GB_per_s": round(layer_bytes[kk] / (avg[kk] * 1e-6) / 1e9, 1),
                      "hbm_frac": round(layer_bytes[kk] / (avg[kk] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
                 for kk in avg}
    sel_overhead_us = n_sel * (avg.get("X", 0.0) - avg.get("F", avg.get("X", 0.0)))
    dominant = max(("F", "S"), key=lambda kk: totals.get(kk, 0.0))
    if dominant == "F" and "F" not in avg:
        dominant = "X"
    kname = {"F": "full attention layer (split-N attention + combine)",
             "X": "full attention + selection layer",
             "S": "sparse attention layer (gathered split attention + combine)"}[dominant]
    achieved = layer_bytes[dominant] / (avg[dominant] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "bytes_per_launch": layer_bytes[dominant], "us_per_launch": round(avg[dominant], 2)}

    copy_probe = None
    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 10
        copy_probe = {"bytes_read": n, "bytes_written": n, "us": round(us, 1),
                      "GB_per_s_read_plus_write": round(2 * n / (us * 1e-6) / 1e9, 1)}
        del src, dst

    cpu = None if timer is None else timer.result(step_bytes)

    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: seeded N(0,1) q/K/V with 4 sinks + k/2 heavy-hitter keys per (batch, KV head)",
        "config": {"workload": wl.name, "layers": wl.layers, "batch": wl.batch, "q_heads": wl.q_heads,
                   "kv_heads": wl.kv_heads, "head_dim": wl.head_dim, "seq_len": wl.max_len, "topk": wl.topk,
                   "select_layers": list(wl.select_layers), "parallelism": "single GPU"},
        "step_us": round(ms_per_step * 1e3, 1),
        "kv_bytes_per_step": step_bytes,
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "selection_overhead_frac": round(sel_overhead_us / (ms_per_step * 1e3), 4),
        "breakdown": breakdown,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if copy_probe:
        result["copy_probe"] = copy_probe
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
