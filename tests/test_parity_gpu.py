"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Reduced workloads keep every shape trait of the benchmark workloads (dtype,
head_dim, group size, ragged lengths, two selection layers) at sizes the
oracle finishes in seconds, spanning several split tiles and a ragged tail.
The full-size test runs the benchmark workload in the launch configuration
the benchmark times and checks sampled (batch row, KV head) units.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
import position_persistent_sparse_amd as ppsa
import synth
from synth import torch_io

from gpu_parity import check_layer, check_output

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

REDUCED = {
    "tiny-f32": synth.WORKLOADS["tiny-f32"],
    "llama2-7b-10k": synth.WORKLOADS["llama2-7b-10k"].with_(layers=9, q_heads=4, kv_heads=4, max_len=3001,
                                                             topk=512, select_layers=(2, 7)),
    "llama3-8b-gqa-32k": synth.WORKLOADS["llama3-8b-gqa-32k"].with_(layers=8, batch=2, q_heads=8, kv_heads=2,
                                                                     max_len=6000, topk=1024,
                                                                     select_layers=(2, 5)),
    "llama2-7b-100k": synth.WORKLOADS["llama2-7b-100k"].with_(layers=6, q_heads=2, kv_heads=2, max_len=20000,
                                                               topk=2048, select_layers=(2, 4)),
    "llama3-70b-ragged-10k": synth.WORKLOADS["llama3-70b-ragged-10k"].with_(layers=6, batch=3, q_heads=16,
                                                                             kv_heads=2, max_len=2100,
                                                                             min_len=1500, topk=256,
                                                                             select_layers=(2, 4)),
}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def widen_out(out, wl):
    if wl.dtype == "bf16":
        return (out.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return out.astype(np.float64)


def check_step(wl, gen, name):
    say(f"[parity] {name}: shape L={wl.layers} B={wl.batch} Hq={wl.q_heads} Hkv={wl.kv_heads} "
        f"N={wl.max_len} k={wl.topk} {wl.dtype} lens={gen.seq_lens.tolist()}")
    q, k, v, lens, host = torch_io.upload(wl, gen, DEV)
    n_sel = wl.schedule().count("X")
    scores = None
    if n_sel:
        scores = torch.full((n_sel, wl.batch, wl.kv_heads, wl.max_len), float("nan"), dtype=torch.float32,
                            device=DEV)
    out, idx = ppsa.decode_step(wl.schedule(), q, k, v, lens, wl.topk, scores=scores)
    torch.cuda.synchronize()
    out_h = widen_out(torch_io.from_torch(out), wl)
    idx_h = idx.cpu().numpy() if n_sel else None
    sc_h = scores.cpu().numpy() if n_sel else None
    sel = -1
    worst = 0.0
    for layer, kind in enumerate(wl.schedule()):
        if kind == "X":
            sel += 1
        qh, kh, vh = host[layer]
        worst = max(worst, check_layer(kind, wl, qh, kh, vh, gen.seq_lens, out_h[layer],
                                       idx_h[sel] if sel >= 0 else None, sc_h[sel] if kind == "X" else None,
                                       idx_h[sel] if sel >= 0 else None, f"{name} layer {layer} ({kind})"))
    say(f"[parity] {name}: ok, max abs error {worst:.3e}")
    return out, idx


@pytest.mark.parametrize("name", list(REDUCED))
def test_decode_step_reduced(name):
    wl = REDUCED[name]
    check_step(wl, synth.Generator(wl), name)


@pytest.mark.parametrize("kind", ["dense", "select-every-layer"])
def test_comparison_schedules(kind):
    """The two comparison schedules the benchmark times: every layer full (the dense baseline) and a
    selection at every layer after the first two (a per-layer selection cost)."""
    base = REDUCED["llama3-8b-gqa-32k"]
    wl = base.with_(select_layers=() if kind == "dense" else tuple(range(2, base.layers)))
    check_step(wl, synth.Generator(wl), f"{kind} {''.join(wl.schedule())}")


def test_padding_poison_and_determinism():
    wl = REDUCED["llama3-70b-ragged-10k"]
    gen = synth.Generator(wl, pad_mode=synth.PAD_NAN)
    out1, idx1 = check_step(wl, gen, "ragged+NaN padding")
    q, k, v, lens, _ = torch_io.upload(wl, gen, DEV)
    out2, idx2 = ppsa.decode_step(wl.schedule(), q, k, v, lens, wl.topk)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), "outputs differ between two runs"
    assert torch.equal(idx1, idx2)


def test_edge_lengths_and_budget():
    # One empty row, one single row, one row shorter than k, one at Nmax.
    wl = synth.WORKLOADS["llama2-7b-10k"].with_(layers=4, batch=4, q_heads=4, kv_heads=2, max_len=700, topk=300,
                                                select_layers=(2,))
    gen = synth.Generator(wl, seq_lens=[0, 1, 200, 700], pad_mode=synth.PAD_NAN)
    out, idx = check_step(wl, gen, "edge lengths")
    o = out.float().cpu().numpy()
    assert np.all(o[:, 0] == 0.0)
    i = idx.cpu().numpy()
    assert np.all(i[0, 0] == -1)
    assert list(i[0, 1, 0, :2]) == [0, -1]
    assert np.all(i[0, 2, :, :200] == np.arange(200)) and np.all(i[0, 2, :, 200:] == -1)


@pytest.mark.parametrize("dtype,d,g", [("bf16", 64, 3), ("f32", 128, 2), ("bf16", 128, 16), ("f32", 64, 5)])
def test_other_shapes(dtype, d, g):
    wl = synth.Workload("shape", layers=5, batch=2, q_heads=2 * g, kv_heads=2, head_dim=d, max_len=777, topk=100,
                        dtype=dtype, select_layers=(2, 3), seed=77, min_len=500)
    check_step(wl, synth.Generator(wl), f"{dtype} d={d} g={g}")


@pytest.mark.parametrize("g", [1, 8, 16])
def test_multi_split_sparse_groups(g):
    """Sparse layers cut into several splits per unit (the streaming launch, K rows loaded whole and
    moved to the matrix-core operand layout through LDS) at group sizes besides the benchmark's 4:
    ragged lengths, a budget that is not a multiple of the 32-row tile, NaN padding."""
    wl = synth.Workload("msplit", layers=5, batch=2, q_heads=2 * g, kv_heads=2, head_dim=128, max_len=3000,
                        topk=1000, dtype="bf16", select_layers=(2, 3), seed=91, min_len=2200)
    check_step(wl, synth.Generator(wl, pad_mode=synth.PAD_NAN), f"multi-split sparse g={g}")


def test_q_zero_ties_select_prefix():
    wl = synth.WORKLOADS["llama3-8b-gqa-32k"].with_(layers=3, batch=1, q_heads=8, kv_heads=2, max_len=1500,
                                                    topk=333, select_layers=(2,))
    gen = synth.Generator(wl)
    q, k, v, lens, _ = torch_io.upload(wl, gen, DEV)
    q.zero_()
    out, idx = ppsa.decode_step(wl.schedule(), q, k, v, lens, wl.topk)
    torch.cuda.synchronize()
    i = idx.cpu().numpy()
    assert np.all(i[0] == np.arange(333)[None, None, :])
    # q = 0: every weight equal, so each output is the mean of the live V rows.
    vh = torch_io.from_torch(v[2])
    mean = ((vh.astype(np.uint32) << 16).view(np.float32).astype(np.float64)).mean(axis=2)
    got = widen_out(torch_io.from_torch(out[2]), wl)
    for h in range(8):
        check_output(got[0, h], mean[0, h // 4], "bf16", f"q=0 mean head {h}")


def test_sparse_with_k_equal_n_matches_full():
    wl = synth.WORKLOADS["llama3-8b-gqa-32k"].with_(layers=1, batch=2, q_heads=8, kv_heads=2, max_len=1200,
                                                    topk=1200, select_layers=())
    gen = synth.Generator(wl, seq_lens=[1200, 1111])
    q, k, v, lens, _ = torch_io.upload(wl, gen, DEV)
    full = ppsa.full_attn(q[0], k[0], v[0], lens)
    idx = torch.arange(1200, dtype=torch.int32, device=DEV).flip(0).repeat(2, 2, 1).contiguous()
    sp = ppsa.sparse_attn(q[0], k[0], v[0], lens, idx)
    torch.cuda.synchronize()
    a = widen_out(torch_io.from_torch(full), wl)
    b = widen_out(torch_io.from_torch(sp), wl)
    assert np.abs(a - b).max() <= 2 ** -8 * np.abs(a).max() + 1e-6


@pytest.mark.parametrize("topk", [96, 1000])
def test_sparse_phases_compose_to_the_layer(topk):
    """The attention launch and the merge launch called apart (ppsa_sparse_attn_phases) give the same bits
    as the whole layer, with one split per unit (96 slots: the attention launch writes out itself) and with
    several (1000 slots: the merge completes out)."""
    wl = synth.WORKLOADS["llama3-8b-gqa-32k"].with_(layers=1, batch=2, q_heads=8, kv_heads=2, max_len=3000,
                                                    topk=topk, select_layers=())
    gen = synth.Generator(wl, seq_lens=[3000, 2222])
    q, k, v, lens, _ = torch_io.upload(wl, gen, DEV)
    rng = np.random.default_rng(12)
    idx = torch.from_numpy(np.sort(rng.integers(0, 2222, size=(2, 2, topk)), axis=2).astype(np.int32)).to(DEV)
    whole = ppsa.sparse_attn(q[0], k[0], v[0], lens, idx)
    ws = ppsa.alloc_workspace(ppsa.make_dims(2, 8, 2, 128, 3000, torch.bfloat16), topk, torch.device(DEV))
    out = torch.full_like(q[0], float("nan"))
    ppsa.sparse_attn(q[0], k[0], v[0], lens, idx, out=out, workspace=ws, phases=ppsa.PHASE_ATTN)
    ppsa.sparse_attn(q[0], k[0], v[0], lens, idx, out=out, workspace=ws, phases=ppsa.PHASE_MERGE)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), whole.view(torch.int16))


def test_sparse_invalid_and_repeated_entries():
    wl = synth.WORKLOADS["tiny-f32"].with_(layers=1, batch=1, q_heads=4, kv_heads=2, max_len=300, topk=40,
                                           select_layers=())
    gen = synth.Generator(wl, seq_lens=[250], pad_mode=synth.PAD_NAN)
    q, k, v, lens, host = torch_io.upload(wl, gen, DEV)
    rng = np.random.default_rng(4)
    idx_h = rng.integers(-5, 300, size=(1, 2, 40)).astype(np.int32)
    idx_h[0, 0, :6] = 17  # repeated entry
    out = ppsa.sparse_attn(q[0], k[0], v[0], lens, torch.from_numpy(idx_h).to(DEV))
    torch.cuda.synchronize()
    qh, kh, vh = host[0]
    scale = oracle.default_scale(wl.head_dim)
    for h in range(2):
        want = oracle.sparse_attention(qh[0, 2 * h:2 * h + 2].astype(np.float64), kh[0, h].astype(np.float64),
                                       vh[0, h].astype(np.float64), idx_h[0, h], 250, scale)
        check_output(out[0, 2 * h:2 * h + 2].cpu().numpy(), want, "f32", f"sparse invalid/repeat h={h}")


def test_select_topk_on_crafted_scores():
    B, H, N = 2, 3, 5000
    rng = np.random.default_rng(8)
    s = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 2.0], dtype=np.float32), size=(B, H, N))
    s[1, 2] = rng.standard_normal(N).astype(np.float32)
    s[0, 1, 4000:] = np.nan  # past seq_lens[0]: never read
    lens = np.array([4000, 5000], dtype=np.int32)
    for k in (1, 17, 1000, 3999, 4000, 4500):
        idx = ppsa.select_topk(torch.from_numpy(s).to(DEV), torch.from_numpy(lens).to(DEV), k)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for b in range(B):
            for h in range(H):
                n = int(lens[b])
                want = oracle.select_topk(s[b, h, :n], k)
                assert sorted(got[b, h][got[b, h] >= 0].tolist()) == sorted(want[want >= 0].tolist()), (k, b, h)
                assert np.all(got[b, h][min(k, n):] == -1)


@pytest.mark.parametrize("n,kind", [(40000, "normal"), (9000, "tied"), (70000, "tied"), (32768, "normal"),
                                    (5000, "two-values"), (20000, "cluster"), (12000, "outlier"), (9000, "inf"),
                                    (6000, "huge"), (102400, "cluster"), (131072, "tied"), (140000, "normal")])
def test_select_topk_paths(n, kind):
    """Register-resident rows (n <= 32768) and re-read rows: up to four super-rounds the output comes
    from the masks kept by the candidate pass (40000, 70000, 102400), beyond that from a third read
    (140000); rows over 65536 also in two launches (chunks, then their winners); threshold bucket resolved by radix digits over its candidates (normal, two-values,
    cluster, huge: a range too wide for float32 puts every score in one bucket) or over all keys
    (tied, outlier: bucket larger than the LDS list)."""
    rng = np.random.default_rng(n)
    B, H = 2, 3
    if kind == "normal":
        s = (rng.standard_normal((B, H, n)) * 2).astype(np.float32)
    elif kind == "tied":
        s = np.full((B, H, n), 0.75, dtype=np.float32)
        s[..., rng.integers(0, n, size=n // 50)] = 3.0
        s[..., rng.integers(0, n, size=n // 50)] = -1.0
    elif kind == "cluster":  # 5000 scores inside one bucket around the 4096-th largest
        s = rng.uniform(0.0, 1.0, size=(B, H, n)).astype(np.float32)
        s[..., rng.permutation(n)[:5000]] = (0.9 + 1e-5 * rng.uniform(size=5000)).astype(np.float32)
    elif kind == "outlier":
        s = (rng.standard_normal((B, H, n)) * 2).astype(np.float32)
        s[..., 7], s[..., 11] = 1e30, -1e30
    elif kind == "inf":
        s = (rng.standard_normal((B, H, n)) * 2).astype(np.float32)
        s[..., rng.integers(0, n, size=40)] = np.inf
        s[..., rng.integers(0, n, size=40)] = -np.inf
    elif kind == "huge":
        s = rng.uniform(-3e38, 3e38, size=(B, H, n)).astype(np.float32)
    else:
        s = rng.choice(np.array([1.0, 2.0], dtype=np.float32), size=(B, H, n))
    lens = np.array([n, n - 333], dtype=np.int32)
    # Rows over 65536 positions: both the two-launch form (top-k per chunk, then over the chunks'
    # winners; used when a workspace is given and the winners fit one super-round) and one launch.
    for two_stage in ((True, False) if n > 65536 else (True,)):
        for k in (1, 257, 4096, n - 400):
            idx = ppsa.select_topk(torch.from_numpy(s).to(DEV), torch.from_numpy(lens).to(DEV), k,
                                   two_stage=two_stage)
            torch.cuda.synchronize()
            got = idx.cpu().numpy()
            for b in range(B):
                for h in range(H):
                    m = int(lens[b])
                    want = oracle.select_topk(s[b, h, :m], k)
                    g = got[b, h]
                    assert np.array_equal(np.sort(g[g >= 0]), np.sort(want[want >= 0])), (n, kind, k, b, h, two_stage)
                    assert np.all(np.diff(g[g >= 0]) > 0) and np.all(g[min(k, m):] == -1)


def test_select_two_launch_with_empty_and_partial_chunks():
    """Two-launch selection (140000 positions: five chunks of 28000) on rows whose live lengths leave
    whole chunks empty, one chunk partly live, and a budget above some chunks' live counts: the set is
    the oracle's, bit for bit, and the same as the one-launch set."""
    rng = np.random.default_rng(31)
    B, H, N = 4, 2, 140000
    s = (rng.standard_normal((B, H, N)) * 2).astype(np.float32)
    s[1, :, 20000:20010] = 50.0  # ties among the largest, inside the only live chunk of row 1
    lens = np.array([N, 30000, 56001, 28000], dtype=np.int32)
    st, lt = torch.from_numpy(s).to(DEV), torch.from_numpy(lens).to(DEV)
    for k in (1000, 4096, 6000):
        two = ppsa.select_topk(st, lt, k, two_stage=True).cpu().numpy()
        one = ppsa.select_topk(st, lt, k, two_stage=False).cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(two, one), k
        for b in range(B):
            for h in range(H):
                want = oracle.select_topk(s[b, h, :lens[b]], k)
                g = two[b, h]
                assert np.array_equal(np.sort(g[g >= 0]), np.sort(want[want >= 0])), (k, b, h)
                assert np.all(np.diff(g[g >= 0]) > 0) and np.all(g[min(k, lens[b]):] == -1)


FULL_SIZE_UNITS = {
    "llama3-8b-gqa-32k": [(0, 0), (1, 3), (2, 5), (3, 7)],
    "llama2-7b-10k": [(0, 0), (0, 17), (0, 31)],
    "llama2-7b-100k": [(0, 0), (0, 21)],
    "llama3-70b-ragged-10k": [(0, 0), (3, 4), (7, 7)],
    "llama3-8b-gqa-32k-tp8": [(0, 0), (3, 0)],
    "llama3-70b-ragged-10k-tp8": [(1, 0), (6, 0)],
}


@pytest.mark.parametrize("name", list(FULL_SIZE_UNITS))
def test_full_size_workload_sampled(name):
    """Every multi-layer workload at its full size, in the launch configuration the benchmark times;
    sampled (batch row, KV head) units checked layer by layer against the oracle."""
    wl = synth.WORKLOADS[name]
    gen = synth.Generator(wl)
    units = FULL_SIZE_UNITS[name]
    say(f"[parity] full-size {wl.name}: generating {wl.layers} layers, B={wl.batch} Hkv={wl.kv_heads} "
        f"N={wl.max_len} k={wl.topk}, units {units}")
    q, k, v, lens, host = torch_io.upload(wl, gen, DEV, keep_units=units,
                                          progress=lambda layer: say(f"[parity]   layer {layer} resident")
                                          if layer % 8 == 7 else None)
    n_sel = wl.schedule().count("X")
    scores = torch.empty((n_sel, wl.batch, wl.kv_heads, wl.max_len), dtype=torch.float32, device=DEV)
    ws = ppsa.alloc_workspace(ppsa.make_dims(wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim, wl.max_len,
                                             torch.bfloat16), wl.topk, DEV)
    out, idx = ppsa.decode_step(wl.schedule(), q, k, v, lens, wl.topk, scores=scores, workspace=ws)
    torch.cuda.synchronize()
    say("[parity] full-size: step done, checking sampled units")
    out_h = widen_out(torch_io.from_torch(out), wl)
    idx_h, sc_h = idx.cpu().numpy(), scores.cpu().numpy()
    g = wl.group
    sel = -1
    worst = 0.0
    for layer, kind in enumerate(wl.schedule()):
        if kind == "X":
            sel += 1
        for (b, h) in units:
            qg, kh, vh = host[layer][(b, h)]
            sub = wl.with_(batch=1, q_heads=g, kv_heads=1)
            worst = max(worst, check_layer(
                kind, sub, qg[None], kh[None, None], vh[None, None], gen.seq_lens[b:b + 1],
                out_h[layer, b, h * g:(h + 1) * g][None], idx_h[sel, b:b + 1, h:h + 1] if sel >= 0 else None,
                sc_h[sel, b:b + 1, h:h + 1] if kind == "X" else None,
                idx_h[sel, b:b + 1, h:h + 1] if sel >= 0 else None, f"full-size layer {layer} unit {(b, h)}"))
    say(f"[parity] full-size {wl.name}: ok, max abs error {worst:.3e}")


def test_selection_layer_at_score_staging_cap_sampled():
    """Group 16 with 32 units at N = 70000: the planner's 8832-row splits exceed the 8192 rows whose
    scores one workgroup can stage in LDS, so splits are capped at 8192 rows (9 per unit, ragged last
    one). Scores, selection and outputs of sampled units are checked."""
    wl = synth.Workload("score-cap", layers=3, batch=4, q_heads=128, kv_heads=8, head_dim=128, max_len=70000,
                        topk=512, dtype="bf16", select_layers=(2,), seed=91, min_len=60000)
    gen = synth.Generator(wl)
    units = [(0, 0), (3, 7)]
    say(f"[parity] score-cap: B={wl.batch} Hq={wl.q_heads} Hkv={wl.kv_heads} N={wl.max_len} "
        f"lens={gen.seq_lens.tolist()}")
    q, k, v, lens, host = torch_io.upload(wl, gen, DEV, keep_layers={2}, keep_units=units)
    scores = torch.full((1, wl.batch, wl.kv_heads, wl.max_len), float("nan"), dtype=torch.float32, device=DEV)
    out, idx = ppsa.decode_step(wl.schedule(), q, k, v, lens, wl.topk, scores=scores)
    torch.cuda.synchronize()
    out_h = widen_out(torch_io.from_torch(out), wl)
    idx_h, sc_h = idx.cpu().numpy(), scores.cpu().numpy()
    g = wl.group
    for (b, h) in units:
        qg, kh, vh = host[2][(b, h)]
        sub = wl.with_(batch=1, q_heads=g, kv_heads=1)
        check_layer("X", sub, qg[None], kh[None, None], vh[None, None], gen.seq_lens[b:b + 1],
                    out_h[2, b, h * g:(h + 1) * g][None], idx_h[0, b:b + 1, h:h + 1], sc_h[0, b:b + 1, h:h + 1],
                    idx_h[0, b:b + 1, h:h + 1], f"score-cap unit {(b, h)}")
    n_min = int(gen.seq_lens.min())
    assert np.all(np.isfinite(sc_h[0, :, :, :n_min])), "a live score was not written"
    say("[parity] score-cap: ok")


@pytest.mark.parametrize("name", ["llama3-8b-gqa-32k", "llama3-70b-ragged-10k"])
def test_decode_step_shared_selection(name):
    """Head-shared selection (one set per batch row over the sum of all query heads' logits): the set is
    checked with the band rule against the oracle's shared scores and is the same for every KV head;
    outputs are checked layer by layer, sparse layers against the GPU's own set."""
    wl = REDUCED[name]
    gen = synth.Generator(wl)
    say(f"[parity] shared selection {name}: lens={gen.seq_lens.tolist()}")
    q, k, v, lens, host = torch_io.upload(wl, gen, DEV)
    out, idx = ppsa.decode_step(wl.schedule(), q, k, v, lens, wl.topk, select_mode="shared")
    torch.cuda.synchronize()
    out_h = widen_out(torch_io.from_torch(out), wl)
    idx_h = idx.cpu().numpy()
    scale = oracle.default_scale(wl.head_dim)
    sel = -1
    for layer, kind in enumerate(wl.schedule()):
        qh, kh, vh = host[layer]
        if kind == "X":
            sel += 1
            check_layer("F", wl, qh, kh, vh, gen.seq_lens, out_h[layer], None, None, None,
                        f"shared {name} layer {layer} (X output)")
            for b in range(wl.batch):
                n = min(max(int(gen.seq_lens[b]), 0), wl.max_len)
                s = oracle.shared_selection_scores(oracle.widen(qh[b], wl.dtype), oracle.widen(kh[b, :, :n], wl.dtype),
                                                   n, wl.group, scale)
                ok, msg, _ = compare.check_selection_band(idx_h[sel, b, 0], s, n, wl.topk)
                assert ok, f"shared {name} layer {layer} b={b}: {msg}"
                for h in range(1, wl.kv_heads):
                    assert np.array_equal(idx_h[sel, b, h], idx_h[sel, b, 0]), (layer, b, h)
        else:
            check_layer(kind, wl, qh, kh, vh, gen.seq_lens, out_h[layer], None, None,
                        idx_h[sel] if sel >= 0 else None, f"shared {name} layer {layer} ({kind})")
    say(f"[parity] shared selection {name}: ok")


@pytest.mark.parametrize("n", [3000, 40000])
def test_select_topk_shared_exact(n):
    """The head-shared select ranks the float32 sum of the KV heads' scores, added in head order; the same
    sum formed in numpy gives the exact expected set (ties included)."""
    rng = np.random.default_rng(n + 1)
    B, H = 3, 4
    s = rng.choice(np.array([-1.0, 0.0, 0.25, 0.5, 1.5], dtype=np.float32), size=(B, H, n))
    s[1] = (rng.standard_normal((H, n)) * 2).astype(np.float32)
    lens = np.array([n, n - 77, 1000], dtype=np.int32)
    tot = s[:, 0].copy()
    for h in range(1, H):
        tot = (tot + s[:, h]).astype(np.float32)
    for k in (1, 500, 2999):
        idx = ppsa.select_topk(torch.from_numpy(s).to(DEV), torch.from_numpy(lens).to(DEV), k, mode="shared")
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for b in range(B):
            m = int(lens[b])
            want = oracle.select_topk(tot[b, :m], k)
            for h in range(H):
                assert np.array_equal(got[b, h], np.sort(want[want >= 0]).tolist() + [-1] * (k - min(k, m))), (n, k, b, h)


@pytest.mark.parametrize("name", ["tiny-f32", "llama3-8b-gqa-32k", "llama3-70b-ragged-10k", "llama2-7b-10k"])
def test_decode_step_softmax_selection(name):
    """Softmax-weight selection (a group ranks a position by the sum of its heads' softmax weights). The
    written scores are within 1e-4 relative of the oracle's (logits carry ~1e-6 relative float32 error,
    exp2 and the normaliser about as much, so 1e-4 leaves a tenfold margin); the set passes the band
    rule with a band of 1e-4 of s_k and is exactly the top-k of its own scores; outputs are checked
    layer by layer, sparse layers against the GPU's own set. Covers the vector-ALU path (fp32, group 1),
    split and single-split matrix-core launches (groups 4 and 8), and group 1 with a row length that is
    not a multiple of 4 (3001: head logits and scores stored one float at a time)."""
    wl = REDUCED[name]
    gen = synth.Generator(wl)
    say(f"[parity] softmax selection {name}: lens={gen.seq_lens.tolist()}")
    q, k, v, lens, host = torch_io.upload(wl, gen, DEV)
    n_sel = wl.schedule().count("X")
    scores = torch.full((n_sel, wl.batch, wl.kv_heads, wl.max_len), float("nan"), dtype=torch.float32, device=DEV)
    out, idx = ppsa.decode_step(wl.schedule(), q, k, v, lens, wl.topk, scores=scores, select_mode="softmax")
    torch.cuda.synchronize()
    out_h = widen_out(torch_io.from_torch(out), wl)
    idx_h, sc_h = idx.cpu().numpy(), scores.cpu().numpy()
    scale = oracle.default_scale(wl.head_dim)
    g = wl.group
    sel = -1
    for layer, kind in enumerate(wl.schedule()):
        qh, kh, vh = host[layer]
        if kind == "X":
            sel += 1
            check_layer("F", wl, qh, kh, vh, gen.seq_lens, out_h[layer], None, None, None,
                        f"softmax {name} layer {layer} (X output)")
            for b in range(wl.batch):
                n = min(max(int(gen.seq_lens[b]), 0), wl.max_len)
                for h in range(wl.kv_heads):
                    ref = oracle.softmax_selection_scores(oracle.widen(qh[b, h * g:(h + 1) * g], wl.dtype),
                                                          oracle.widen(kh[b, h], wl.dtype), n, scale).astype(np.float64)
                    got = sc_h[sel, b, h, :n].astype(np.float64)
                    assert np.all(np.abs(got - ref) <= 1e-4 * np.abs(ref) + 1e-12), (layer, b, h)
                    ok, msg, _ = compare.check_selection_band(idx_h[sel, b, h], ref, n, wl.topk, band=0.0, rel_band=1e-4)
                    assert ok, f"softmax {name} layer {layer} b={b} h={h}: {msg}"
                    assert compare.check_selection_exact(idx_h[sel, b, h], sc_h[sel, b, h], n, wl.topk), (layer, b, h)
        else:
            check_layer(kind, wl, qh, kh, vh, gen.seq_lens, out_h[layer], None, None,
                        idx_h[sel] if sel >= 0 else None, f"softmax {name} layer {layer} ({kind})")
    say(f"[parity] softmax selection {name}: ok")


@pytest.mark.parametrize("name,tau,cap", [("tiny-f32", 0.2, None), ("llama3-8b-gqa-32k", 0.1, None),
                                          ("llama3-70b-ragged-10k", 0.5, None), ("llama3-8b-gqa-32k", 0.1, 64)])
def test_decode_step_coverage_budget(name, tau, cap):
    """Coverage budget: per unit, the lowest-mass positions are pruned until their mass exceeds tau; the
    kept count must sit at a crossing of the oracle's cumulative mass within 2e-4 (masses carry 1e-4
    relative error from the softmax-weight sums), the set must pass the relative band rule for that
    count and be exactly the top of the GPU's own scores; outputs are checked layer by layer. With a
    cap (topk below the budget) the set is the top-cap positions."""
    base = REDUCED[name]
    wl = base.with_(topk=cap if cap else base.max_len)
    gen = synth.Generator(wl)
    say(f"[parity] coverage {name} tau={tau} topk={wl.topk}: lens={gen.seq_lens.tolist()}")
    q, k, v, lens, host = torch_io.upload(wl, gen, DEV)
    n_sel = wl.schedule().count("X")
    scores = torch.full((n_sel, wl.batch, wl.kv_heads, wl.max_len), float("nan"), dtype=torch.float32, device=DEV)
    out, idx = ppsa.decode_step(wl.schedule(), q, k, v, lens, wl.topk, scores=scores, select_mode="coverage",
                                coverage_tau=tau)
    torch.cuda.synchronize()
    out_h = widen_out(torch_io.from_torch(out), wl)
    idx_h, sc_h = idx.cpu().numpy(), scores.cpu().numpy()
    scale = oracle.default_scale(wl.head_dim)
    g = wl.group
    sel = -1
    kept = []
    for layer, kind in enumerate(wl.schedule()):
        qh, kh, vh = host[layer]
        if kind != "X":
            check_layer(kind, wl, qh, kh, vh, gen.seq_lens, out_h[layer], None, None,
                        idx_h[sel] if sel >= 0 else None, f"coverage {name} layer {layer} ({kind})")
            continue
        sel += 1
        check_layer("F", wl, qh, kh, vh, gen.seq_lens, out_h[layer], None, None, None,
                    f"coverage {name} layer {layer} (X output)")
        for b in range(wl.batch):
            n = min(max(int(gen.seq_lens[b]), 0), wl.max_len)
            for h in range(wl.kv_heads):
                ref = oracle.softmax_selection_scores(oracle.widen(qh[b, h * g:(h + 1) * g], wl.dtype),
                                                      oracle.widen(kh[b, h], wl.dtype), n, scale)
                row = idx_h[sel, b, h]
                k_gpu = int(np.sum(row >= 0))
                assert np.all(row[k_gpu:] == -1)
                if cap is None:
                    m = ref.astype(np.float64) / g
                    csum = np.concatenate([[0.0], np.cumsum(m[np.lexsort((-np.arange(n), m))])])
                    p = n - k_gpu  # pruned count
                    thr = tau * csum[-1]
                    assert p >= 1 and csum[p - 1] <= thr + 2e-4 and csum[p] > thr - 2e-4, (layer, b, h, p)
                    assert abs(k_gpu - oracle.coverage_budget(ref, g, tau)) <= max(3, n // 100), (layer, b, h)
                else:
                    assert k_gpu == min(cap, oracle.coverage_budget(ref, g, tau)), (layer, b, h)
                kept.append(k_gpu)
                ok, msg, _ = compare.check_selection_band(row, ref, n, k_gpu, band=0.0, rel_band=1e-4)
                assert ok, f"coverage {name} layer {layer} b={b} h={h}: {msg}"
                assert compare.check_selection_exact(row, sc_h[sel, b, h], n, k_gpu), (layer, b, h)
    say(f"[parity] coverage {name} tau={tau}: ok, kept per unit {min(kept)}..{max(kept)}")


def test_results_do_not_depend_on_the_split_plan():
    """One reduced LLaMA-3-8B-shaped step (group 4, several selection and sparse layers) under three split
    plans -- automatic, many small splits, and one split per (batch row, KV head) -- through the planner
    override: identical selections, and outputs that differ by at most the rounding the plans may
    legitimately change (the weights' bf16 rounding, relative to each split's own running max, moves an
    output by at most 2^-7 of the attention of |V|, and the output's own rounding by one bf16 spacing)."""
    wl = REDUCED["llama3-8b-gqa-32k"].with_(layers=6, select_layers=(2, 4))
    gen = synth.Generator(wl)
    say(f"[splits] L={wl.layers} B={wl.batch} Hq={wl.q_heads} Hkv={wl.kv_heads} N={wl.max_len} k={wl.topk}")
    q, k, v, lens, host = torch_io.upload(wl, gen, DEV)
    results = {}
    plans = {"automatic": (0, 0), "small splits": (128, 128), "one split": (wl.max_len, wl.topk)}
    try:
        for name, (fr, sr) in plans.items():
            ppsa.set_split_rows(fr, sr)
            out, idx = ppsa.decode_step(wl.schedule(), q, k, v, lens, wl.topk)
            torch.cuda.synchronize()
            results[name] = (widen_out(torch_io.from_torch(out), wl), idx.cpu().numpy())
    finally:
        ppsa.set_split_rows(0, 0)
    scale = oracle.default_scale(wl.head_dim)
    ref_out, ref_idx = results["automatic"]
    sel = -1
    for layer, kind in enumerate(wl.schedule()):
        if kind == "X":
            sel += 1
        qh, kh, vh = host[layer]
        selection = ref_idx[sel] if kind == "S" else None
        absw, _, _ = oracle.decode_layer(kind, qh, kh, np.asarray(vh) & np.uint16(0x7FFF), gen.seq_lens, wl.group,
                                         wl.topk, scale, wl.dtype, selection)
        for name, (o, i) in results.items():
            assert np.array_equal(i, ref_idx), f"{name}: selections differ"
            diff = np.abs(o[layer] - ref_out[layer])
            bound = 2 * (2.0 ** -7 * 1.01 * absw) + 2 * (2.0 ** -8) * np.abs(ref_out[layer]) + 2e-5
            bad = int(np.sum(diff > bound))
            assert bad == 0, f"{name} layer {layer} ({kind}): {bad} elements differ beyond the rounding bound"
    say("[splits] ok: three plans agree")
