"""Host-side logic: byte accounting and schedules, against the page's figures."""
import json
import os

import numpy as np

from synth import WORKLOADS, kv_cache_bytes, schedule_for, step_kv_bytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_kv_cache_size_page_example():
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_size.json")))
    got = kv_cache_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["tokens"], g["bytes_per_element"])
    assert got == g["printed_total_bytes_binary"] == 64 * 2 ** 30


def test_schedule_matches_framework_figure():
    g = json.load(open(os.path.join(GOLDEN, "decode_schedule.json")))
    for ex in g["examples"]:
        assert "".join(schedule_for(ex["layers"], (2, ex["middle"]))) == ex["kinds"]


def test_two_selections_per_step():
    for wl in WORKLOADS.values():
        sched = wl.schedule()
        assert sched.count("X") == 2
        assert sched[0] == sched[1] == "F"
        assert sched.index("X") == 2


def test_step_bytes_fixed_length_workloads():
    want = {"tiny-f32": 17825792, "llama2-7b-10k": 905969664, "llama3-8b-gqa-32k": 4026531840,
            "llama2-7b-100k": 7650410496}
    for name, b in want.items():
        wl = WORKLOADS[name]
        assert step_kv_bytes(wl, [wl.max_len] * wl.batch) == b


def test_step_bytes_ragged():
    wl = WORKLOADS["llama3-70b-ragged-10k"]
    lens = np.full(wl.batch, 9216)
    per_full = 2 * wl.batch * wl.kv_heads * 9216 * 256
    per_sparse = 2 * wl.batch * wl.kv_heads * 256 * 256
    assert step_kv_bytes(wl, lens) == 4 * per_full + 76 * per_sparse == 1845493760


def test_sharded_workloads_are_kv_head_zero_of_their_shape():
    """The 8-way KV-head shards reproduce the whole shape's KV head 0 and its query heads bit for bit
    (same seed, counter-based generator), so their timings are one GPU's share of that shape."""
    from synth import Generator
    for shard, whole in (("llama3-8b-gqa-32k-tp8", "llama3-8b-gqa-32k"),
                         ("llama3-70b-ragged-10k-tp8", "llama3-70b-ragged-10k")):
        kw = dict(layers=4, max_len=2048, topk=256)
        ws, ww = WORKLOADS[shard], WORKLOADS[whole]
        if ww.ragged:
            kw["min_len"] = 1500
        gs, gw = Generator(ws.with_(**kw)), Generator(ww.with_(**kw))
        assert ws.kv_heads == 1 and ws.q_heads == ww.group and ws.batch == ww.batch
        assert gs.seq_lens.tolist() == gw.seq_lens.tolist()
        layer = 3
        assert np.array_equal(gs.q(layer), gw.q(layer)[:, :ws.q_heads])
        ks, vs = gs.kv(layer, None, None)
        kw_, vw = gw.kv(layer, None, None)
        assert np.array_equal(ks, kw_[:, :1]) and np.array_equal(vs, vw[:, :1])


def test_hbm_traffic_record_matches_the_attention_sources():
    """The committed FETCH_SIZE / WRITE_SIZE record of the headline sparse kernel was taken on the
    attention sources as they are now (their sha256 is stored with it and checked by the benchmark), and
    it counts close to the algorithmic bytes: 2 k d e per (batch row, KV head), 32 units, plus slot
    entries, q and partials. A change to those sources has to come with new counters."""
    import bench
    nbytes, source = bench.measured_traffic("llama3-8b-gqa-32k", "attn_sparse")
    assert nbytes is not None, source
    algorithmic = 2 * 4 * 8 * 4096 * 128 * 2
    assert 1.0 <= nbytes / algorithmic < 1.1, nbytes / algorithmic
