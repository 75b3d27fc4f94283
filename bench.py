"""PPSA decode-step benchmark on one MI355X.

Times whole decode steps (every layer of the schedule: full, full + top-k
selection, sparse) through the C ABI entry point ppsa_decode_step, with all
inputs resident in HBM, and prints one JSON line: achieved KV GB/s (the
algorithmic K+V bytes a step must read, divided by the step time), step
microseconds, the fraction of the 8 TB/s HBM peak, per-kernel durations from
the library's launch timing (HIP events around each launch, on the stream the
kernels run on), the roofline of the dominant kernel, the float64 CPU oracle
timed over the same decode step on one host thread, and two comparison
schedules over the same inputs (every layer full; a selection at every layer
after the first two) with PPSA's speedup over each.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "PPSA decode-step attention µs and achieved KV GB/s (% of HBM peak)"
EVICT_BYTES = 1 << 30  # written between per-step timings: larger than the last-level cache
# Sources of the matrix-core attention kernel: the HBM traffic counted for it holds only while they are unchanged.
ATTN_SOURCES = ("attn_mfma.hip", "attn_epilogue.h", "device_common.h", "ppsa_internal.h")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", action="store_true", help="also time a plain 1 GiB device copy (PMC calibration)")
    p.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing (counter-collection runs)")
    p.add_argument("--no-comparison", action="store_true", help="skip the dense and select-every-layer schedules")
    p.add_argument("--no-multi-token", action="store_true", help="skip the multi-token (append + step) timing")
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


def attn_source_digest():
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(ROOT, "position_persistent_sparse_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload, kernel_key):
    """HBM bytes per launch of `kernel_key` from the committed counter summary, or (None, reason)."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None, f"no counter summary for {workload}"
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None, f"{os.path.basename(path)} has no json block"
    rec = json.loads(m.group(1))
    if rec.get("kernel_key") != kernel_key:
        return None, f"counters were taken for {rec.get('kernel_key')}, not {kernel_key}"
    if rec.get("source_sha256") != attn_source_digest():
        return None, "attention kernel sources changed since the counters were taken"
    b = (rec["fetch_kib_per_dispatch"] * rec["fetch_scale"] + rec["write_kib_per_dispatch"] * rec["write_scale"]) * 1024
    return int(round(b)), os.path.basename(path)


def percentile(xs, p):
    import numpy as np

    return float(np.percentile(np.asarray(xs), p))


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
    stream = torch.cuda.current_stream(dev)
    step_bytes = synth.step_kv_bytes(wl, gen.seq_lens)

    def step():
        ppsa.decode_step(sched, q, k, v, lens, wl.topk, out=out, idx=idx, workspace=ws, sched_codes=codes)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # 1. The timed region: K back-to-back steps.
    start, end = ev(), ev()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us, {gbs:.1f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of peak)")

    # 2. Per-step times, each step preceded (outside its events) by a 1 GiB write that evicts the caches.
    scratch = torch.empty(EVICT_BYTES, dtype=torch.uint8, device=dev)
    per_step = []
    for i in range(args.steps):
        scratch.fill_(i & 0xFF)
        e0, e1 = ev(), ev()
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        per_step.append(e0.elapsed_time(e1) * 1e3)
    del scratch
    log(f"evicted steps: median {percentile(per_step, 50):.1f} us")

    # 3. Per-kernel durations: the library's launch timing (two HIP events around each launch).
    launches_per_step = 2 * len(sched) + n_sel
    ppsa.timing_enable(launches_per_step * args.steps)
    try:
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        timed = ppsa.timing_read()
    finally:
        ppsa.timing_enable(0)
    instrumented_us = e0.elapsed_time(e1) * 1e3 / args.steps
    kernels = {}
    for key in ppsa.KERNEL_KEYS:
        n, ms = timed[key]
        if n:
            kernels[key] = {"launches_per_step": round(n / args.steps, 2), "us_per_launch": round(ms * 1e3 / n, 2),
                            "us_per_step": round(ms * 1e3 / args.steps, 1)}
    layer_bytes = {"attn_full": synth.layer_kv_bytes(wl, "F", gen.seq_lens),
                   "attn_full_scores": synth.layer_kv_bytes(wl, "X", gen.seq_lens),
                   "attn_sparse": synth.layer_kv_bytes(wl, "S", gen.seq_lens)}
    for key, b in layer_bytes.items():
        if key in kernels:
            gb = b / (kernels[key]["us_per_launch"] * 1e-6) / 1e9
            kernels[key].update({"kv_bytes_per_launch": b, "GB_per_s": round(gb, 1),
                                 "hbm_frac": round(gb / HBM_PEAK_GBS, 4)})

    # 4. The same step replayed from a captured HIP graph.
    graph_us = None
    try:
        if args.no_graph:
            raise RuntimeError("skipped (--no-graph)")
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_us = round(e0.elapsed_time(e1) * 1e3 / args.steps, 1)
        del graph
    except Exception as exc:  # reported, never fatal: the eager step is the measurement
        log(f"graph replay not measured: {exc}")

    # 5. Comparison schedules over the same inputs: every layer full (the dense decode step TidalDecode
    # is measured against) and a selection at every layer after the first two.
    comparison = {}
    for name, sch in (("dense", ["F"] * wl.layers), ("select_every_layer", ["F", "F"] + ["X"] * (wl.layers - 2))):
        if args.no_comparison or wl.layers < 3:
            break
        c_codes = ppsa.schedule_codes(sch)
        n_x = sch.count("X")
        c_idx = torch.empty((max(n_x, 1), wl.batch, wl.kv_heads, wl.topk), dtype=torch.int32, device=dev)

        def c_step():
            ppsa.decode_step(sch, q, k, v, lens, wl.topk, out=out, idx=c_idx if n_x else None, workspace=ws,
                             sched_codes=c_codes)

        c_step()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(args.steps):
            c_step()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        comparison[name] = {"schedule": "".join(sch), "step_us": round(us, 1),
                            "ppsa_speedup": round(us / (ms_per_step * 1e3), 3)}
        del c_idx
    def overlap(a, b):
        """Mean over (selection layer, batch row, KV head) of the fraction of set a also in set b."""
        fr = []
        for sel_i in range(a.shape[0]):
            for bb in range(a.shape[1]):
                for hh in range(a.shape[2]):
                    x, y = a[sel_i, bb, hh], b[sel_i, bb, hh]
                    x = x[x >= 0]
                    if x.numel():
                        fr.append(float(torch.isin(x, y[y >= 0]).float().mean()))
        return round(sum(fr) / max(len(fr), 1), 4)

    if not args.no_comparison and n_sel:
        step()
        torch.cuda.synchronize()
        idx_default = idx.clone()
        # Selection variant: one set per batch row over all of its query heads (same schedule and inputs).
        def shared_step():
            ppsa.decode_step(sched, q, k, v, lens, wl.topk, out=out, idx=idx, workspace=ws, sched_codes=codes,
                             select_mode="shared")

        shared_step()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(args.steps):
            shared_step()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        comparison["shared_selection"] = {"schedule": "".join(sched), "select_mode": "shared", "step_us": round(us, 1),
                                          "ppsa_speedup": round(us / (ms_per_step * 1e3), 3),
                                          "overlap_with_default_set": overlap(idx_default, idx)}

        def softmax_step():
            ppsa.decode_step(sched, q, k, v, lens, wl.topk, out=out, idx=idx, workspace=ws, sched_codes=codes,
                             select_mode="softmax")

        softmax_step()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(args.steps):
            softmax_step()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        comparison["softmax_selection"] = {"schedule": "".join(sched), "select_mode": "softmax",
                                           "step_us": round(us, 1), "ppsa_speedup": round(us / (ms_per_step * 1e3), 3),
                                           "overlap_with_default_set": overlap(idx_default, idx)}

        # Coverage budget instead of a fixed k (capped at k): prune the lowest-mass tail past tau.
        tau = 0.8

        def coverage_step():
            ppsa.decode_step(sched, q, k, v, lens, wl.topk, out=out, idx=idx, workspace=ws, sched_codes=codes,
                             select_mode="coverage", coverage_tau=tau)

        coverage_step()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(args.steps):
            coverage_step()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        kept = (idx >= 0).sum(dim=-1).float()
        comparison["coverage_selection"] = {"schedule": "".join(sched), "select_mode": "coverage", "tau": tau,
                                            "cap": wl.topk, "step_us": round(us, 1),
                                            "ppsa_speedup": round(us / (ms_per_step * 1e3), 3),
                                            "kept_per_unit": {"mean": round(float(kept.mean()), 1),
                                                              "min": int(kept.min()), "max": int(kept.max())}}
    if comparison:
        log("comparison: " + ", ".join(f"{kk} {vv['step_us']} us" for kk, vv in comparison.items()))

    # 6. Multi-token decode (last: it writes cache rows): T tokens, each appending its K/V rows and then
    # running the step, each batch row starting T rows short of its length so that every token has room.
    multi = None
    if not args.no_multi_token:
        T = args.steps
        lens_mt = torch.clamp(lens - T, min=0).to(torch.int32)
        kn = torch.randn((wl.layers, wl.batch, wl.kv_heads, wl.head_dim), device=dev).to(k.dtype)
        vn = torch.randn_like(kn)

        def token():
            ppsa.append_kv(kn, vn, k, v, lens_mt)
            ppsa.decode_step(sched, q, k, v, lens_mt, wl.topk, out=out, idx=idx, workspace=ws, sched_codes=codes)

        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(T):
            token()
        e1.record(stream)
        torch.cuda.synchronize()
        ok = bool(torch.equal(lens_mt, torch.clamp(lens - T, min=0).to(torch.int32) + T))
        multi = {"tokens": T, "us_per_token": round(e0.elapsed_time(e1) * 1e3 / T, 1),
                 "start_lengths": "each batch row T rows short of its length", "lengths_grew_by_tokens": ok}
        log(f"multi-token decode: {multi['us_per_token']} us per token (append + step)")

    # Roofline of the attention kernel with the largest share of the step.
    attn_keys = [kk for kk in layer_bytes if kk in kernels]
    dom = max(attn_keys, key=lambda kk: kernels[kk]["us_per_step"])
    traffic, traffic_src = measured_traffic(wl.name, dom)
    roofline = {"bound": "hbm", "kernel": f"{dom}: {ppsa.timing_kernel_name(ppsa.KERNEL_KEYS.index(dom))}",
                "achieved": kernels[dom]["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": kernels[dom]["hbm_frac"], "traffic": traffic, "traffic_source": traffic_src,
                "bytes_per_launch": layer_bytes[dom], "us_per_launch": kernels[dom]["us_per_launch"],
                "launches_per_step": kernels[dom]["launches_per_step"]}

    sel_us = kernels.get("select", {}).get("us_per_step", 0.0)
    if "attn_full_scores" in kernels and "attn_full" in kernels:
        sel_us += n_sel * (kernels["attn_full_scores"]["us_per_launch"] - kernels["attn_full"]["us_per_launch"])

    copy_probe = None
    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        e1.record(stream)
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
        "step_us_evicted": {"median": round(percentile(per_step, 50), 1), "p10": round(percentile(per_step, 10), 1),
                            "p90": round(percentile(per_step, 90), 1)},
        "step_us_graph_replay": graph_us,
        "step_us_with_launch_timing": round(instrumented_us, 1),
        "selection_overhead_frac": round(sel_us / (ms_per_step * 1e3), 4),
        "comparison_schedules": comparison or None,
        "multi_token_decode": multi,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if copy_probe:
        result["copy_probe"] = copy_probe
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
