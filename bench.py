"""PPSA decode-step benchmark on one MI355X.

Times whole decode steps (every layer of the schedule: full, full + top-k
selection, sparse) through the C ABI entry point ppsa_decode_step, with all
inputs resident in HBM, and prints one JSON line.

Headline (`value`, `ms_per_step`): the workload the metric is quoted on
(LLaMA-3-8B GQA, 32K context): K steps, each preceded (outside its HIP
events) by two reads of a 1 GiB buffer that evict the last-level cache and
the L2s, reported as the median; `value` is the algorithmic K+V
bytes of one step over that median. The same K steps back to back without
eviction are reported beside it (`step_us_back_to_back`).

The line also carries: per-kernel durations from the library's launch timing
(HIP events around each launch, on the launch stream) and per-layer figures
(attention launch plus its merge launch, and the two launches apart, each
back to back in a captured graph); the roofline of the dominant kernel
against the 8 TB/s peak and against the read bandwidth this GPU reaches
(`roofline.achievable`, from the read probe; `achievable_same_size`, a read
of the launch's own size), its duration taken from the
graph of its launches (an event pair around every launch adds its marker
packets to the launch); the sparse kernel over its load-only twin; measurement probes (read ceiling, launch floor); a parity
summary of the timed outputs on sampled (batch row, KV head) units against
the float64 oracle; the oracle itself timed on the host cores
(`cpu_baseline`); comparison schedules, selection variants and a multi-token
decode on the headline workload; and `workloads`: the other four
configurations and one GPU's share of the two GQA shapes under 8-way KV-head
sharding, timed the same way.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--workloads all|none|NAME,...]
                    [--no-cpu-baseline] [--no-probes] [--no-parity] [--no-graph] [--no-comparison]
                    [--no-multi-token] [--copy-probe]
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
EVICT_BYTES = 1 << 30  # read between per-step timings: larger than the last-level cache
# Sources of the attention kernels: HBM traffic counted for a kernel holds only while they are unchanged.
ATTN_SOURCES = ("attn_mfma.hip", "attn_sparse.hip", "mfma_tile.h", "sparse_gather.h", "attn_epilogue.h",
                "device_common.h", "ppsa_internal.h")
# Host threads the oracle may use: at most 16, one GPU's share of a multi-GPU host.
CPU_THREADS_CAP = 16


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=None, help="headline workload (default: the metric's configuration)")
    p.add_argument("--workloads", default="all", help="other workloads to time: all, none or a comma list")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-probes", action="store_true")
    p.add_argument("--no-parity", action="store_true")
    p.add_argument("--copy-probe", action="store_true", help="also time a plain 1 GiB device copy (PMC calibration)")
    p.add_argument("--no-graph", action="store_true",
                   help="skip every timing taken through a captured graph (counter-collection runs)")
    p.add_argument("--no-comparison", action="store_true", help="skip the dense and select-every-layer schedules")
    p.add_argument("--no-multi-token", action="store_true", help="skip the multi-token (append + step) timing")
    return p.parse_args()


def percentile(xs, p):
    import numpy as np

    return float(np.percentile(np.asarray(xs), p))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(CPU_THREADS_CAP, n))


class OracleTimer:
    """Times the float64 oracle over the whole decode step, layer by layer as the layers are generated
    (generation outside the timed calls), with the (batch row, KV head) units of a layer spread over a
    pool of host threads (numpy releases the GIL in its array work; BLAS is held to one thread per
    worker). Each unit keeps its own selection state across layers."""

    def __init__(self, wl, seq_lens, threads):
        import numpy as np

        import oracle

        self.np = np
        self.oracle = oracle
        self.wl = wl
        self.seq_lens = np.asarray(seq_lens)
        self.threads = threads
        self.scale = oracle.default_scale(wl.head_dim)
        self.sel = {}
        self.secs = 0.0
        self.pool = None
        if threads > 1:
            from concurrent.futures import ThreadPoolExecutor

            self.pool = ThreadPoolExecutor(max_workers=threads)

    def _unit(self, kind, q, K, V, b, h):
        wl, g = self.wl, self.wl.group
        out, sel, _ = self.oracle.decode_layer(kind, q[b:b + 1, h * g:(h + 1) * g], K[b:b + 1, h:h + 1],
                                               V[b:b + 1, h:h + 1], self.seq_lens[b:b + 1], g, wl.topk,
                                               self.scale, wl.dtype, self.sel.get((b, h)))
        if sel is not None:
            self.sel[(b, h)] = sel
        return out

    def __call__(self, layer, q, K, V):
        import threadpoolctl

        kind = self.wl.schedule()[layer]
        units = [(b, h) for b in range(self.wl.batch) for h in range(self.wl.kv_heads)]
        with threadpoolctl.threadpool_limits(1):
            t0 = time.perf_counter()
            if self.pool is None:
                for b, h in units:
                    self._unit(kind, q, K, V, b, h)
            else:
                list(self.pool.map(lambda u: self._unit(kind, q, K, V, u[0], u[1]), units))
            self.secs += time.perf_counter() - t0

    def close(self):
        if self.pool is not None:
            self.pool.shutdown()

    def result(self, step_bytes):
        wl = self.wl
        return {"value": round(step_bytes / self.secs / 1e9, 4), "unit": "GB/s", "cores": self.threads,
                "kind": "oracle", "step_us": round(self.secs * 1e6, 1), "cpu_model": cpu_model(),
                "sample": f"the whole decode step ({wl.layers} layers, all {wl.batch * wl.kv_heads} (batch, KV "
                          f"head) units, float64), {self.secs:.2f} s on {self.threads} host thread(s), units of a "
                          f"layer spread over the threads; inputs generated outside the timed calls"}


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


class Bench:
    """Shared GPU state: the stream, an eviction buffer, a sink for probes."""

    def __init__(self, args):
        import torch

        import position_persistent_sparse_amd as ppsa

        self.torch = torch
        self.ppsa = ppsa
        self.args = args
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream(self.dev)
        self.sink = torch.zeros(16, dtype=torch.int32, device=self.dev)
        self.scratch = None

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def evict(self, i):
        """A plain read of 1 GiB: the last-level cache and the L2s then hold clean, unrelated lines (a write
        would leave dirty lines whose write-back the next step would pay)."""
        if self.scratch is None:
            self.scratch = self.torch.ones(EVICT_BYTES, dtype=self.torch.uint8, device=self.dev)
        # Twice: the GPU is still reading when the host enqueues the step, so no idle gap falls inside the
        # step's events.
        self.ppsa.probe_read(self.scratch, False, self.sink)
        self.ppsa.probe_read(self.scratch, False, self.sink)

    def graph_time(self, fn, calls, replays=3):
        """µs per call of `calls` calls captured in one HIP graph and replayed back to back (no host work
        between the launches)."""
        torch = self.torch
        side = torch.cuda.Stream(self.dev)
        side.wait_stream(self.stream)
        with torch.cuda.stream(side):
            fn(0)
        self.stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(calls):
                fn(i)
        graph.replay()
        us = self.time_loop(lambda i: graph.replay(), replays) / calls
        del graph
        return us

    def time_loop(self, fn, reps):
        """Back-to-back: µs per call over `reps` calls, bracketed by events on the launch stream."""
        torch = self.torch
        torch.cuda.synchronize()
        e0, e1 = self.ev(), self.ev()
        e0.record(self.stream)
        for i in range(reps):
            fn(i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def time_each(self, fn, reps, evict=False):
        """µs of each call, each bracketed by its own events (eviction outside them when asked); one
        synchronisation before and after the whole loop."""
        torch = self.torch
        torch.cuda.synchronize()
        pairs = []
        for i in range(reps):
            if evict:
                self.evict(i)
            e0, e1 = self.ev(), self.ev()
            e0.record(self.stream)
            fn(i)
            e1.record(self.stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in pairs]

    def probes(self):
        """The read ceiling of this GPU, the fixed cost of a launch, and the read of a sparse layer's size."""
        torch, ppsa = self.torch, self.ppsa
        res = {}
        n = 4 << 30
        buf = torch.empty(n, dtype=torch.uint8, device=self.dev)
        buf.fill_(1)
        for nt in (True, False):
            ppsa.probe_read(buf, nt, self.sink)
            us = self.time_loop(lambda i: ppsa.probe_read(buf, nt, self.sink), 5)
            res["read_4GiB_" + ("nontemporal" if nt else "plain")] = {"us": round(us, 1),
                                                                    "GB_per_s": round(n / us / 1e3, 1)}
        # 64 MiB reads (a sparse layer's K+V bytes at the LLaMA-3-8B 32K shape), each from a new part of the
        # 4 GiB buffer, so that none is served by the last-level cache.
        part = 64 << 20
        views = [buf[i * part:(i + 1) * part] for i in range(n // part)]
        us = self.graph_time(lambda i: ppsa.probe_read(views[i % len(views)], True, self.sink), len(views))
        res["read_64MiB_nontemporal"] = {"us": round(us, 2), "GB_per_s": round(part / us / 1e3, 1),
                                         "timing": "back to back in a captured graph"}
        del views, buf
        for groups, threads in ((512, 256), (64, 512)):
            key = f"empty_kernel_{groups}x{threads}"
            rec = {"us_per_launch_graph": round(self.graph_time(lambda i: ppsa.probe_empty(groups, threads, self.sink),
                                                                100), 2),
                   "us_per_launch_python_loop": round(
                       self.time_loop(lambda i: ppsa.probe_empty(groups, threads, self.sink), 200), 2)}
            res[key] = rec
        torch.cuda.synchronize()
        return res


class WorkloadRun:
    """One workload: inputs resident on the GPU, the step timed, kernels and layers timed, parity sampled."""

    def __init__(self, bench, wl, headline, oracle_threads):
        import numpy as np

        import synth
        from synth import torch_io

        self.b = bench
        self.wl = wl
        self.np = np
        self.synth = synth
        torch, ppsa = bench.torch, bench.ppsa
        self.gen = synth.Generator(wl)
        self.sched = wl.schedule()
        self.n_sel = self.sched.count("X")
        self.units = self._sample_units(4 if headline else 2)
        self.timer = None
        if oracle_threads:
            self.timer = OracleTimer(wl, self.gen.seq_lens, oracle_threads)
        log(f"generating {wl.name}: {wl.layers} layers, B={wl.batch}, Hq={wl.q_heads}, Hkv={wl.kv_heads}, "
            f"N={wl.max_len}, k={wl.topk}, {wl.dtype}"
            + ("" if self.timer is None else f"; timing the oracle per layer on {oracle_threads} thread(s)"))
        t0 = time.time()
        keep = None if bench.args.no_parity else set(range(wl.layers))
        self.q, self.k, self.v, self.lens, self.host = torch_io.upload(
            wl, self.gen, bench.dev, keep_layers=keep if keep is not None else set(),
            keep_units=self.units, visit=self.timer)
        if self.timer is not None:
            self.timer.close()
        torch.cuda.synchronize()
        log(f"{wl.name}: inputs resident after {time.time() - t0:.1f} s")
        self.dims = ppsa.make_dims(wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim, wl.max_len,
                                   torch_io.torch_dtype(wl))
        self.ws = ppsa.alloc_workspace(self.dims, wl.topk, bench.dev)
        self.out = torch.empty_like(self.q)
        self.idx = torch.empty((max(self.n_sel, 1), wl.batch, wl.kv_heads, wl.topk), dtype=torch.int32,
                               device=bench.dev)
        self.codes = ppsa.schedule_codes(self.sched)
        self.step_bytes = synth.step_kv_bytes(wl, self.gen.seq_lens)

    def _sample_units(self, count):
        wl = self.wl
        units = [(b, h) for b in range(wl.batch) for h in range(wl.kv_heads)]
        if len(units) <= count:
            return units
        stride = len(units) / count
        return [units[int(i * stride + stride / 2)] for i in range(count)]

    def step(self, *_):
        self.b.ppsa.decode_step(self.sched, self.q, self.k, self.v, self.lens, self.wl.topk, out=self.out,
                                idx=self.idx if self.n_sel else None, workspace=self.ws, sched_codes=self.codes)

    def free(self):
        del self.q, self.k, self.v, self.ws, self.out, self.idx, self.host
        self.b.torch.cuda.empty_cache()

    def time_steps(self, steps, warmup):
        for _ in range(warmup):
            self.step()
        evicted = self.b.time_each(self.step, steps, evict=True)
        b2b = self.b.time_loop(self.step, steps)
        return evicted, b2b

    def kernel_times(self, steps):
        """Per-kernel durations from the library's launch timing over `steps` steps."""
        ppsa = self.b.ppsa
        launches_per_step = 2 * len(self.sched) + self.n_sel
        ppsa.timing_enable(launches_per_step * steps)
        try:
            us = self.b.time_loop(self.step, steps)
            timed = ppsa.timing_read()
        finally:
            ppsa.timing_enable(0)
        kernels = {}
        for key in ppsa.KERNEL_KEYS:
            n, ms = timed[key]
            if n:
                kernels[key] = {"launches_per_step": round(n / steps, 2), "us_per_launch": round(ms * 1e3 / n, 2),
                                "us_per_step": round(ms * 1e3 / steps, 1)}
        wl, lens = self.wl, self.gen.seq_lens
        self.layer_bytes = {"attn_full": self.synth.layer_kv_bytes(wl, "F", lens),
                            "attn_full_scores": self.synth.layer_kv_bytes(wl, "X", lens),
                            "attn_sparse": self.synth.layer_kv_bytes(wl, "S", lens)}
        for key, nbytes in self.layer_bytes.items():
            if key in kernels:
                gb = nbytes / (kernels[key]["us_per_launch"] * 1e-6) / 1e9
                kernels[key].update({"kv_bytes_per_launch": nbytes, "GB_per_s": round(gb, 1),
                                     "hbm_frac": round(gb / HBM_PEAK_GBS, 4)})
        return kernels, us

    def layer_times(self, kernels):
        """Per layer kind: the attention launch plus the merge launch that follows it (when the layer's
        units have several splits), from the event brackets, and the layers timed back to back through
        the single-layer entry points."""
        ppsa = self.b.ppsa
        n_f, n_s = self.sched.count("F"), self.sched.count("S")
        n_comb = kernels.get("combine", {}).get("launches_per_step", 0)
        comb_us = kernels.get("combine", {}).get("us_per_launch", 0.0)
        full_merged = n_comb in (n_f, n_f + n_s) and n_f > 0
        sparse_merged = n_comb in (n_s, n_f + n_s) and n_s > 0
        res = {}
        if "attn_full" in kernels:
            us = kernels["attn_full"]["us_per_launch"] + (comb_us if full_merged else 0.0)
            res["full_layer"] = {"events_us": round(us, 2), "merge_launch": full_merged,
                                 "GB_per_s": round(self.layer_bytes["attn_full"] / us / 1e3, 1)}
        if "attn_full_scores" in kernels and "select" in kernels:
            us = kernels["attn_full_scores"]["us_per_launch"] + kernels["select"]["us_per_step"] / max(self.n_sel, 1)
            res["selection_layer"] = {"events_us": round(us, 2), "note": "attention + score write, then top-k "
                                      "(whose first launch also merges the layer's partials; rows over 32768 "
                                      "positions take two selection launches)"}
        if "attn_sparse" in kernels:
            us = kernels["attn_sparse"]["us_per_launch"] + (comb_us if sparse_merged else 0.0)
            graphs = not self.b.args.no_graph
            res["sparse_layer"] = {"events_us": round(us, 2), "merge_launch": sparse_merged,
                                   "GB_per_s": round(self.layer_bytes["attn_sparse"] / us / 1e3, 1),
                                   "hbm_frac": round(self.layer_bytes["attn_sparse"] / us / 1e3 / HBM_PEAK_GBS, 4)}
            # The sparse layers of a step back to back through ppsa_sparse_attn (kernel + merge launch).
            s_layers = [layer for layer, kind in enumerate(self.sched) if kind == "S"]
            sel_of = {}
            sel = -1
            for layer, kind in enumerate(self.sched):
                if kind == "X":
                    sel += 1
                sel_of[layer] = sel
            outs = self.out

            def one(i):
                layer = s_layers[i % len(s_layers)]
                ppsa.sparse_attn(self.q[layer], self.k[layer], self.v[layer], self.lens, self.idx[sel_of[layer]],
                                 out=outs[layer], workspace=self.ws)

            if not graphs:
                return res
            # At least 28 launches per graph, cycling through the step's sparse layers, so that the
            # replay's own fixed cost is spread as in the benchmark workload.
            n_calls = max(len(s_layers), 28)
            self.step()
            us = self.b.graph_time(one, n_calls)
            nbytes = self.layer_bytes["attn_sparse"]
            rec = res["sparse_layer"]
            rec["back_to_back_us"] = round(us, 2)
            rec["back_to_back_GB_per_s"] = round(nbytes / us / 1e3, 1)
            rec["back_to_back_timing"] = "the step's sparse layers through ppsa_sparse_attn (kernel and merge " \
                                         "launch), captured in a graph"

            # The same layers' two launches apart (ppsa_sparse_attn_phases): the attention kernel alone, then
            # the merge launch alone, each back to back in a graph.
            def phase(ph):
                def run_one(i):
                    layer = s_layers[i % len(s_layers)]
                    ppsa.sparse_attn(self.q[layer], self.k[layer], self.v[layer], self.lens,
                                     self.idx[sel_of[layer]], out=outs[layer], workspace=self.ws, phases=ph)
                return run_one

            k_us = self.b.graph_time(phase(ppsa.PHASE_ATTN), n_calls)
            rec["kernel_back_to_back_us"] = round(k_us, 2)
            rec["kernel_back_to_back_GB_per_s"] = round(nbytes / k_us / 1e3, 1)
            if sparse_merged:
                rec["merge_back_to_back_us"] = round(self.b.graph_time(phase(ppsa.PHASE_MERGE), n_calls), 2)
            self.step()
        return res

    def gather_twin(self):
        """The sparse kernel's load-only twin over this step's sparse layers (event-bracketed like the
        launch timing)."""
        ppsa = self.b.ppsa
        s_layers = [layer for layer, kind in enumerate(self.sched) if kind == "S"]
        if not s_layers or self.wl.dtype != "bf16" or self.wl.head_dim != 128:
            return None
        sel_of, sel = {}, -1
        for layer, kind in enumerate(self.sched):
            if kind == "X":
                sel += 1
            sel_of[layer] = sel
        self.step()

        def one(i):
            layer = s_layers[i % len(s_layers)]
            ppsa.probe_gather(self.k[layer], self.v[layer], self.lens, self.idx[sel_of[layer]], self.wl.q_heads,
                              self.b.sink)

        us = self.b.graph_time(one, max(2 * len(s_layers), 56))
        nbytes = self.synth.layer_kv_bytes(self.wl, "S", self.gen.seq_lens)
        return {"us_per_launch": round(us, 2), "GB_per_s": round(nbytes / us / 1e3, 1), "kv_bytes_per_launch": nbytes,
                "timing": "back to back over the step's sparse layers (each its own K/V, as in the step), "
                          "captured in a graph: from the previous launch's end to this one's"}

    def parity(self):
        """The timed step's outputs on the sampled units against the float64 oracle: per layer kind the
        max abs error, the relative L2 error, and at selection layers the band rule (positions inside the
        1e-3 band counted). Sparse layers are evaluated on the GPU's own selection."""
        if self.b.args.no_parity:
            return None
        import oracle
        from oracle import compare
        from synth import torch_io

        np, wl = self.np, self.wl
        self.step()
        self.b.torch.cuda.synchronize()
        out = torch_io.from_torch(self.out)
        out = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if wl.dtype == "bf16" \
            else out.astype(np.float64)
        idx = self.idx.cpu().numpy()
        scale = oracle.default_scale(wl.head_dim)
        g = wl.group
        acc = {k: {"max_abs": 0.0, "err2": 0.0, "ref2": 0.0, "layers": 0} for k in ("F", "X", "S")}
        band_pos, sel_ok = 0, True
        sel_i = -1
        for layer, kind in enumerate(self.sched):
            if kind == "X":
                sel_i += 1
            for (b, h) in self.units:
                qg, kb, vb = self.host[layer][(b, h)]
                n = int(self.gen.seq_lens[b])
                selection = idx[sel_i, b, h][None, None] if kind == "S" else None
                want, _, oscores = oracle.decode_layer(kind, qg[None], kb[None, None], vb[None, None],
                                                       np.array([n]), g, wl.topk, scale, wl.dtype, selection)
                got = out[layer, b, h * g:(h + 1) * g]
                err = np.abs(got - want[0])
                a = acc[kind]
                a["max_abs"] = max(a["max_abs"], float(err.max()))
                a["err2"] += float(np.sum(err ** 2))
                a["ref2"] += float(np.sum(want[0] ** 2))
                if kind == "X":
                    ok, _, inband = compare.check_selection_band(idx[sel_i, b, h], oscores[0, 0], n, wl.topk)
                    sel_ok &= ok
                    band_pos += inband
            acc[kind]["layers"] += 1
        tol = 1e-5 if wl.dtype == "f32" else 2e-2
        res = {"units": [list(u) for u in self.units], "tolerance_max_abs": tol, "selection_band_rule_ok": sel_ok,
               "band_positions": band_pos}
        ok = sel_ok
        for kind, name in (("F", "full"), ("X", "selection"), ("S", "sparse")):
            a = acc[kind]
            if a["layers"]:
                rel = (a["err2"] / a["ref2"]) ** 0.5 if a["ref2"] > 0 else 0.0
                res[name] = {"layers": a["layers"], "max_abs": float(f"{a['max_abs']:.3e}"),
                             "rel_l2": float(f"{rel:.3e}")}
                ok &= a["max_abs"] <= tol
        res["ok"] = bool(ok)
        return res

    def summary(self, steps, warmup, with_twin=True):
        """Step, kernel and layer timings plus parity: the record of one workload."""
        evicted, b2b = self.time_steps(steps, warmup)
        med = percentile(evicted, 50)
        kernels, instrumented = self.kernel_times(steps)
        sel_us = kernels.get("select", {}).get("us_per_step", 0.0)
        if "attn_full_scores" in kernels and "attn_full" in kernels:
            sel_us += self.n_sel * (kernels["attn_full_scores"]["us_per_launch"] - kernels["attn_full"]["us_per_launch"])
        rec = {"workload": self.wl.name, "layers": self.wl.layers, "batch": self.wl.batch,
               "q_heads": self.wl.q_heads, "kv_heads": self.wl.kv_heads, "head_dim": self.wl.head_dim,
               "seq_len": self.wl.max_len, "seq_lens": "ragged " + str(self.gen.seq_lens.tolist())
               if self.wl.ragged else self.wl.max_len, "topk": self.wl.topk, "dtype": self.wl.dtype,
               "schedule": "".join(self.sched), "kv_bytes_per_step": self.step_bytes,
               "step_us": round(med, 1),
               "step_us_evicted": {"median": round(med, 1), "p10": round(percentile(evicted, 10), 1),
                                   "p90": round(percentile(evicted, 90), 1)},
               "step_us_back_to_back": round(b2b, 1),
               "GB_per_s": round(self.step_bytes / med / 1e3, 1),
               "hbm_frac": round(self.step_bytes / med / 1e3 / HBM_PEAK_GBS, 4),
               "step_us_with_launch_timing": round(instrumented, 1),
               "selection_overhead_frac": round(sel_us / med, 4),
               "kernels": kernels, "layers_timed": self.layer_times(kernels)}
        if with_twin and not self.b.args.no_graph:
            twin = self.gather_twin()
            sl = rec["layers_timed"].get("sparse_layer", {})
            if twin and "kernel_back_to_back_us" in sl:
                twin["sparse_kernel_over_twin"] = round(sl["kernel_back_to_back_us"] / twin["us_per_launch"], 3)
                twin["ratio_timing"] = "both back to back in a graph over the step's sparse layers"
            rec["gather_twin"] = twin
        rec["parity"] = self.parity()
        return rec


def comparison_schedules(run, steps, base_us):
    """Dense and select-every-layer schedules, and the selection variants, over the same inputs."""
    ppsa, torch, wl = run.b.ppsa, run.b.torch, run.wl
    comparison = {}
    for name, sch in (("dense", ["F"] * wl.layers), ("select_every_layer", ["F", "F"] + ["X"] * (wl.layers - 2))):
        c_codes = ppsa.schedule_codes(sch)
        n_x = sch.count("X")
        c_idx = torch.empty((max(n_x, 1), wl.batch, wl.kv_heads, wl.topk), dtype=torch.int32, device=run.b.dev)

        def c_step(*_):
            ppsa.decode_step(sch, run.q, run.k, run.v, run.lens, wl.topk, out=run.out, idx=c_idx if n_x else None,
                             workspace=run.ws, sched_codes=c_codes)

        c_step()
        us = run.b.time_loop(c_step, steps)
        comparison[name] = {"schedule": "".join(sch), "step_us": round(us, 1), "ppsa_speedup": round(us / base_us, 3)}
        del c_idx

    def overlap(a, b):
        """Mean over (selection layer, batch row, KV head) of the fraction of set a also in set b."""
        fr = []
        for s in range(a.shape[0]):
            for bb in range(a.shape[1]):
                for hh in range(a.shape[2]):
                    x, y = a[s, bb, hh], b[s, bb, hh]
                    x = x[x >= 0]
                    if x.numel():
                        fr.append(float(torch.isin(x, y[y >= 0]).float().mean()))
        return round(sum(fr) / max(len(fr), 1), 4)

    run.step()
    torch.cuda.synchronize()
    idx_default = run.idx.clone()
    for mode, extra in (("shared", {}), ("softmax", {}), ("coverage", {"coverage_tau": 0.8})):
        def v_step(*_):
            ppsa.decode_step(run.sched, run.q, run.k, run.v, run.lens, wl.topk, out=run.out, idx=run.idx,
                             workspace=run.ws, sched_codes=run.codes, select_mode=mode, **extra)

        v_step()
        us = run.b.time_loop(v_step, steps)
        rec = {"schedule": "".join(run.sched), "select_mode": mode, "step_us": round(us, 1),
               "ppsa_speedup": round(us / base_us, 3), "overlap_with_default_set": overlap(idx_default, run.idx)}
        if mode == "coverage":
            kept = (run.idx >= 0).sum(dim=-1).float()
            rec.update({"tau": 0.8, "cap": wl.topk, "kept_per_unit": {"mean": round(float(kept.mean()), 1),
                                                                       "min": int(kept.min()), "max": int(kept.max())}})
        comparison[mode + "_selection"] = rec
    run.step()
    return comparison


def graph_replay(run, steps):
    torch = run.b.torch
    try:
        side = torch.cuda.Stream(run.b.dev)
        side.wait_stream(run.b.stream)
        with torch.cuda.stream(side):
            run.step()
        run.b.stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run.step()
        graph.replay()
        us = run.b.time_loop(lambda i: graph.replay(), steps)
        del graph
        return round(us, 1)
    except Exception as exc:  # reported, never fatal: the eager step is the measurement
        log(f"graph replay not measured: {exc}")
        return None


def multi_token(run, steps):
    """T tokens, each appending its K/V rows and then running the step, each batch row starting T rows short
    of its length so that every token has room (last: it writes cache rows)."""
    torch, ppsa, wl = run.b.torch, run.b.ppsa, run.wl
    T = steps
    lens_mt = torch.clamp(run.lens - T, min=0).to(torch.int32)
    kn = torch.randn((wl.layers, wl.batch, wl.kv_heads, wl.head_dim), device=run.b.dev).to(run.k.dtype)
    vn = torch.randn_like(kn)

    def token(*_):
        ppsa.append_kv(kn, vn, run.k, run.v, lens_mt)
        ppsa.decode_step(run.sched, run.q, run.k, run.v, lens_mt, wl.topk, out=run.out, idx=run.idx,
                         workspace=run.ws, sched_codes=run.codes)

    us = run.b.time_loop(token, T)
    ok = bool(torch.equal(lens_mt, torch.clamp(run.lens - T, min=0).to(torch.int32) + T))
    return {"tokens": T, "us_per_token": round(us, 1), "start_lengths": "each batch row T rows short of its length",
            "lengths_grew_by_tokens": ok}


def one_thread_oracle(wl):
    """The oracle over the whole step of a small workload on one host thread (baseline plan: C1 and C2)."""
    import synth

    gen = synth.Generator(wl)
    timer = OracleTimer(wl, gen.seq_lens, 1)
    kb = vb = None
    for layer in range(wl.layers):
        kb, vb = gen.kv(layer, kb, vb)
        timer(layer, gen.q(layer), kb, vb)
    nbytes = synth.step_kv_bytes(wl, gen.seq_lens)
    return {"value": round(nbytes / timer.secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "step_us": round(timer.secs * 1e6, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the PPSA path here is single-GPU",
              file=sys.stderr)
        sys.exit(2)

    import synth

    bench = Bench(args)
    probes = None
    if not args.no_probes:
        probes = bench.probes()
        log("probes: " + json.dumps(probes))

    # Headline workload.
    wl = synth.WORKLOADS[args.workload or synth.BENCH_WORKLOAD]
    threads = 0 if args.no_cpu_baseline else host_threads()
    run = WorkloadRun(bench, wl, headline=True, oracle_threads=threads)
    rec = run.summary(args.steps, args.warmup)
    ms_per_step = rec["step_us"] / 1e3
    log(f"{wl.name}: step {rec['step_us']} us evicted median ({rec['GB_per_s']} GB/s, {rec['hbm_frac']:.1%} of peak), "
        f"{rec['step_us_back_to_back']} us back to back")
    kernels = rec["kernels"]
    graph_us = None if args.no_graph else graph_replay(run, args.steps)
    comparison = None
    if not args.no_comparison and run.n_sel and wl.layers >= 3:
        comparison = comparison_schedules(run, args.steps, rec["step_us_back_to_back"])
        log("comparison: " + ", ".join(f"{kk} {vv['step_us']} us" for kk, vv in comparison.items()))
    multi = None if args.no_multi_token else multi_token(run, args.steps)
    cpu = None if run.timer is None else run.timer.result(run.step_bytes)

    # Roofline of the attention kernel with the largest share of the step.
    attn_keys = [kk for kk in run.layer_bytes if kk in kernels]
    dom = max(attn_keys, key=lambda kk: kernels[kk]["us_per_step"])
    traffic, traffic_src = measured_traffic(wl.name, dom)
    achievable = None if probes is None else probes["read_4GiB_nontemporal"]["GB_per_s"]
    # Launch duration: for the sparse kernel the graph-timed back-to-back figure (events around the replay of
    # the step's sparse launches, on the launch stream); the library's per-launch event pairs add the cost of
    # their own marker packets to every launch and are reported beside it.
    nbytes = run.layer_bytes[dom]
    sl = rec["layers_timed"].get("sparse_layer", {})
    if dom == "attn_sparse" and "kernel_back_to_back_us" in sl:
        us_launch, timing_src = sl["kernel_back_to_back_us"], "graph of the step's sparse attention launches " \
                                "(ppsa_sparse_attn_phases, attention phase), back to back, events around the replay"
    else:
        us_launch, timing_src = kernels[dom]["us_per_launch"], "library launch timing (events around each launch)"
    achieved = round(nbytes / us_launch / 1e3, 1)
    # The read ceiling at this launch's own size (a 64 MiB read back to back in a graph: one launch's ramp and
    # drain included), when the probe read that many bytes.
    same_size = None
    if probes is not None and nbytes == 64 << 20:
        same_size = probes["read_64MiB_nontemporal"]["GB_per_s"]
    roofline = {"bound": "hbm", "kernel": f"{dom}: {bench.ppsa.timing_kernel_name(bench.ppsa.KERNEL_KEYS.index(dom))}",
                "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "traffic_source": traffic_src,
                "achievable": achievable,
                "frac_of_achievable": None if achievable is None else round(achieved / achievable, 4),
                "achievable_same_size": same_size,
                "frac_of_achievable_same_size": None if same_size is None else round(achieved / same_size, 4),
                "bytes_per_launch": nbytes, "us_per_launch": us_launch, "us_per_launch_timing": timing_src,
                "us_per_launch_event_pairs": kernels[dom]["us_per_launch"],
                "launches_per_step": kernels[dom]["launches_per_step"]}
    layer_key = {"attn_sparse": "sparse_layer", "attn_full": "full_layer"}.get(dom)
    if layer_key and layer_key in rec["layers_timed"]:
        roofline["with_merge_launch"] = rec["layers_timed"][layer_key]
    run.free()
    del run

    # The other workloads, timed the same way (no comparison schedules; oracle baselines on one thread for
    # the two small ones, as the baseline plan asks).
    others = {}
    names = [] if args.workloads == "none" else (
        [n for n in synth.WORKLOADS if n != wl.name] if args.workloads == "all" else args.workloads.split(","))
    for name in names:
        other = synth.WORKLOADS[name]
        r = WorkloadRun(bench, other, headline=False, oracle_threads=0)
        o = r.summary(args.steps, min(args.warmup, 2))
        log(f"{name}: step {o['step_us']} us evicted median ({o['GB_per_s']} GB/s, {o['hbm_frac']:.1%}), "
            f"{o['step_us_back_to_back']} us back to back; parity ok={None if o['parity'] is None else o['parity']['ok']}")
        r.free()
        del r
        if not args.no_cpu_baseline and name in ("tiny-f32", "llama2-7b-10k"):
            o["cpu_baseline_one_thread"] = one_thread_oracle(other)
        others[name] = o

    copy_probe = None
    if args.copy_probe:
        torch = bench.torch
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=bench.dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        us = bench.time_loop(lambda i: dst.copy_(src), 10)
        copy_probe = {"bytes_read": n, "bytes_written": n, "us": round(us, 1),
                      "GB_per_s_read_plus_write": round(2 * n / (us * 1e-6) / 1e9, 1)}
        del src, dst

    result = {
        "metric": METRIC,
        "value": rec["GB_per_s"],
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
        "timing": "value and ms_per_step: median of the steps, each timed after a 1 GiB cache-evicting read; "
                  "step_us_back_to_back: the same steps without eviction",
        "step_us": rec["step_us"],
        "step_us_evicted": rec["step_us_evicted"],
        "step_us_back_to_back": rec["step_us_back_to_back"],
        "step_us_graph_replay": graph_us,
        "step_us_with_launch_timing": rec["step_us_with_launch_timing"],
        "kv_bytes_per_step": rec["kv_bytes_per_step"],
        "hbm_frac": rec["hbm_frac"],
        "selection_overhead_frac": rec["selection_overhead_frac"],
        "kernels": kernels,
        "layers_timed": rec["layers_timed"],
        "gather_twin": rec.get("gather_twin"),
        "parity": rec["parity"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "probes": probes,
        "comparison_schedules": comparison,
        "multi_token_decode": multi,
        "workloads": others or None,
    }
    if copy_probe:
        result["copy_probe"] = copy_probe
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
