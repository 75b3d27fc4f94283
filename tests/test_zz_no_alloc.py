"""GPU check of ppsa_decode_step_static, the decode step that allocates nothing (its workspace is the
library's static device scratch): through the C ABI, its outputs and selected indices must equal
ppsa_decode_step's on the same inputs, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents), and the selection layers must also pass the oracle's band
rule. It runs alone in a fresh process as well as after the other tests."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
import position_persistent_sparse_amd as ppsa
import synth
from synth import torch_io

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(name, wl):
    gen = synth.Generator(wl)
    sched = wl.schedule()
    say(f"[static] {name}: L={wl.layers} B={wl.batch} Hq={wl.q_heads} Hkv={wl.kv_heads} N={wl.max_len} "
        f"k={wl.topk} {wl.dtype} schedule {''.join(sched)}")
    q, k, v, lens, host = torch_io.upload(wl, gen, DEV)
    out_ref, idx_ref = ppsa.decode_step(sched, q, k, v, lens, wl.topk)
    out_s = torch.full_like(q, float("nan"))
    idx_s = torch.full_like(idx_ref, -7)
    ppsa.decode_step_static(sched, q, k, v, lens, wl.topk, out=out_s, idx=idx_s)
    torch.cuda.synchronize()
    # Same kernels, same plan, same order of arithmetic: bit-identical.
    assert torch.equal(idx_s, idx_ref), name
    assert torch.equal(out_s.view(torch.int16) if out_s.dtype == torch.bfloat16 else out_s,
                       out_ref.view(torch.int16) if out_ref.dtype == torch.bfloat16 else out_ref), name
    # The selections also hold against the oracle's scores (band rule of the parity bar).
    idx_h = idx_s.cpu().numpy()
    scale = oracle.default_scale(wl.head_dim)
    sel_i = -1
    for layer, kind in enumerate(sched):
        if kind != "X":
            continue
        sel_i += 1
        qh, kh, vh = host[layer]
        _, _, oscores = oracle.decode_layer(kind, qh, kh, vh, gen.seq_lens, wl.group, wl.topk, scale, wl.dtype,
                                            None)
        for b in range(wl.batch):
            for h in range(wl.kv_heads):
                ok, msg, _ = compare.check_selection_band(idx_h[sel_i, b, h], oscores[b, h], int(gen.seq_lens[b]),
                                                          wl.topk)
                assert ok, f"{name} layer {layer} b={b} h={h}: {msg}"
    say(f"[static] {name}: identical to the workspace entry point")


def test_static_scratch_step_matches_workspace_step_twice():
    big = synth.WORKLOADS["llama3-8b-gqa-32k"].with_(layers=6, batch=2, q_heads=8, kv_heads=2, max_len=6000,
                                                     topk=1024, select_layers=(2, 4))
    small = synth.WORKLOADS["llama3-70b-ragged-10k"].with_(layers=5, batch=3, q_heads=8, kv_heads=1, max_len=900,
                                                           min_len=500, topk=128, select_layers=(2, 3))
    _case("first call", big)
    _case("second call, smaller", small)
