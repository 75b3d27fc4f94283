"""GPU parity of the multi-token decode: ppsa_append_kv then ppsa_decode_step
once per token, against the oracle's append_kv / decode_steps."""
import sys

import numpy as np
import pytest
import torch

import oracle
import position_persistent_sparse_amd as ppsa
import synth
from synth import torch_io

from gpu_parity import check_layer

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def storage(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return synth.round_bf16(x) if dtype == "bf16" else x


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_append_kv_rows_and_lengths_exact(dtype, d):
    rng = np.random.default_rng(5 + d)
    L, B, Hkv, n_max = 3, 5, 2, 40
    lens0 = np.array([39, 40, 0, 17, -3], dtype=np.int32)  # one row of room, full, empty, middle, negative
    say(f"[append] {dtype} d={d} L={L} B={B} Hkv={Hkv} Nmax={n_max} lens={lens0.tolist()}")
    K = storage(rng, (L, B, Hkv, n_max, d), dtype)
    V = storage(rng, (L, B, Hkv, n_max, d), dtype)
    kt, vt = torch_io.to_torch(K.copy()).to(DEV), torch_io.to_torch(V.copy()).to(DEV)
    lens = torch.from_numpy(lens0.copy()).to(DEV)
    Kh, Vh = [K[layer].copy() for layer in range(L)], [V[layer].copy() for layer in range(L)]
    lens_h = lens0
    overflow = torch.zeros(1, dtype=torch.int32, device=DEV)
    dropped = 0
    for step in range(2):
        kn, vn = storage(rng, (L, B, Hkv, d), dtype), storage(rng, (L, B, Hkv, d), dtype)
        ppsa.append_kv(torch_io.to_torch(kn).to(DEV), torch_io.to_torch(vn).to(DEV), kt, vt, lens, overflow=overflow)
        dropped += int(np.sum(np.clip(lens_h, 0, n_max) == n_max))  # rows already full drop this token
        lens_h = oracle.append_kv(Kh, Vh, lens_h, kn, vn)
        torch.cuda.synchronize()
        assert lens.cpu().numpy().tolist() == lens_h.tolist(), step
        np.testing.assert_array_equal(torch_io.from_torch(kt), np.stack(Kh))
        np.testing.assert_array_equal(torch_io.from_torch(vt), np.stack(Vh))
        assert int(overflow.item()) == dropped, step
    assert lens_h.tolist() == [40, 40, 2, 19, 2]
    assert dropped == 3  # the full row twice, the row with one slot of room on the second token


def test_multi_token_decode_matches_oracle():
    wl = synth.WORKLOADS["llama3-70b-ragged-10k"].with_(layers=6, batch=3, q_heads=16, kv_heads=2, max_len=2100,
                                                        min_len=1500, topk=256, select_layers=(2, 4))
    gen = synth.Generator(wl)
    rng = np.random.default_rng(2024)
    T = 3
    say(f"[multistep] {T} tokens, L={wl.layers} B={wl.batch} Hq={wl.q_heads} Hkv={wl.kv_heads} "
        f"N={wl.max_len} k={wl.topk} lens={gen.seq_lens.tolist()}")
    q0, k, v, lens, host = torch_io.upload(wl, gen, DEV)
    Kh = [host[layer][1].copy() for layer in range(wl.layers)]
    Vh = [host[layer][2].copy() for layer in range(wl.layers)]
    lens_h = gen.seq_lens.copy()
    sched = wl.schedule()
    shape_q = (wl.layers, wl.batch, wl.q_heads, wl.head_dim)
    shape_kv = (wl.layers, wl.batch, wl.kv_heads, wl.head_dim)
    worst = 0.0
    for t in range(T):
        q_t = storage(rng, shape_q, "bf16")
        kn, vn = storage(rng, shape_kv, "bf16"), storage(rng, shape_kv, "bf16")
        ppsa.append_kv(torch_io.to_torch(kn).to(DEV), torch_io.to_torch(vn).to(DEV), k, v, lens)
        scores = torch.full((2, wl.batch, wl.kv_heads, wl.max_len), float("nan"), dtype=torch.float32, device=DEV)
        out, idx = ppsa.decode_step(sched, torch_io.to_torch(q_t).to(DEV), k, v, lens, wl.topk, scores=scores)
        torch.cuda.synchronize()
        lens_h = oracle.append_kv(Kh, Vh, lens_h, kn, vn)
        assert lens.cpu().numpy().tolist() == lens_h.tolist()
        out_h = torch_io.from_torch(out)
        out_h = (out_h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        idx_h, sc_h = idx.cpu().numpy(), scores.cpu().numpy()
        sel = -1
        for layer, kind in enumerate(sched):
            if kind == "X":
                sel += 1
            worst = max(worst, check_layer(kind, wl, q_t[layer], Kh[layer], Vh[layer], lens_h, out_h[layer],
                                           idx_h[sel] if sel >= 0 else None, sc_h[sel] if kind == "X" else None,
                                           idx_h[sel] if sel >= 0 else None, f"token {t} layer {layer} ({kind})"))
        say(f"[multistep] token {t}: lens {lens_h.tolist()} ok")
    say(f"[multistep] ok, max abs error {worst:.3e}")
