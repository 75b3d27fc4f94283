"""GPU checks of the launch-timing instrumentation and of decode steps
replayed from a captured HIP graph (both used by the benchmark)."""
import sys

import pytest
import torch

import position_persistent_sparse_amd as ppsa
import synth
from synth import torch_io

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
WL = synth.WORKLOADS["llama3-8b-gqa-32k"].with_(layers=8, batch=2, q_heads=8, kv_heads=2, max_len=6000,
                                                topk=1024, select_layers=(2, 5))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def inputs():
    gen = synth.Generator(WL)
    q, k, v, lens, _ = torch_io.upload(WL, gen, DEV, keep_layers=set())
    return q, k, v, lens


def run_step(inputs, out, idx, ws):
    q, k, v, lens = inputs
    ppsa.decode_step(WL.schedule(), q, k, v, lens, WL.topk, out=out, idx=idx, workspace=ws)


def buffers(inputs):
    q = inputs[0]
    n_sel = WL.schedule().count("X")
    dims = ppsa.make_dims(WL.batch, WL.q_heads, WL.kv_heads, WL.head_dim, WL.max_len, q.dtype)
    out = torch.empty_like(q)
    idx = torch.empty((n_sel, WL.batch, WL.kv_heads, WL.topk), dtype=torch.int32, device=DEV)
    return out, idx, ppsa.alloc_workspace(dims, WL.topk, DEV)


def test_launch_timing_counts_and_results(inputs):
    sched = WL.schedule()
    say(f"[timing] schedule {''.join(sched)} B={WL.batch} N={WL.max_len} k={WL.topk}")
    out0, idx0, ws = buffers(inputs)
    run_step(inputs, out0, idx0, ws)
    torch.cuda.synchronize()
    out1, idx1, _ = buffers(inputs)
    ppsa.timing_enable(64)
    try:
        run_step(inputs, out1, idx1, ws)
        res = ppsa.timing_read()
        # Fewer pairs than launches: the rest are dropped, never waited on.
        ppsa.timing_enable(3)
        run_step(inputs, out1, idx1, ws)
        small = ppsa.timing_read()
    finally:
        ppsa.timing_enable(0)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16)) and torch.equal(idx0, idx1)
    n_f, n_x, n_s = sched.count("F"), sched.count("X"), sched.count("S")
    assert res["attn_full"][0] == n_f and res["attn_full_scores"][0] == n_x and res["attn_sparse"][0] == n_s
    assert res["select"][0] == n_x
    # Every layer of this shape is cut into several splits; a selection layer's merge runs inside its
    # selection launch, every other layer has a merge launch of its own.
    assert res["combine"][0] == len(sched) - n_x
    assert res["dropped"] == 0
    for key in ppsa.KERNEL_KEYS:
        if key in ("append", "softmax_scores", "coverage"):  # not part of a default decode step
            assert res[key] == (0, 0.0)
        else:
            assert res[key][1] > 0.0, key
    launches = n_f + n_x + n_s + res["combine"][0] + res["select"][0]
    assert sum(small[k][0] for k in ppsa.KERNEL_KEYS) == 3 and small["dropped"] == launches - 3
    say(f"[timing] ok: {res}")


def test_graph_replay_matches_eager(inputs):
    say("[graph] capture one decode step, replay 3 times")
    out_e, idx_e, ws = buffers(inputs)
    run_step(inputs, out_e, idx_e, ws)
    torch.cuda.synchronize()
    out_g, idx_g, ws_g = buffers(inputs)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_step(inputs, out_g, idx_g, ws_g)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_step(inputs, out_g, idx_g, ws_g)
    for rep in range(3):
        out_g.fill_(0)
        idx_g.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_e.view(torch.int16), out_g.view(torch.int16)), rep
        assert torch.equal(idx_e, idx_g), rep
        run_step(inputs, out_e, idx_e, ws)  # eager work between replays
        torch.cuda.synchronize()
    say("[graph] ok")
