"""The seeded generator: determinism, shapes and the heavy-hitter structure."""
import numpy as np

import synth
from synth import Generator, WORKLOADS


def _f(x, dtype):
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x


def test_round_bf16_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0, 3.14159265, 65504.0], dtype=np.float32)
    assert list(synth.round_bf16(vals)) == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x4049, 0x4780]


def test_deterministic_and_layer_dependent():
    wl = WORKLOADS["tiny-f32"]
    a, b = Generator(wl), Generator(wl)
    np.testing.assert_array_equal(a.q(3), b.q(3))
    ka, va = a.kv(2)
    kb, vb = b.kv(2)
    np.testing.assert_array_equal(ka, kb)
    np.testing.assert_array_equal(va, vb)
    assert not np.array_equal(a.kv(3)[0], ka)
    assert not np.array_equal(Generator(wl, seed=5).q(3), a.q(3))


def test_heavy_positions_structure():
    wl = WORKLOADS["llama3-70b-ragged-10k"].with_(layers=2, batch=3)
    g = Generator(wl)
    for b in range(wl.batch):
        assert wl.min_len <= g.seq_lens[b] <= wl.max_len
        for h in range(wl.kv_heads):
            hs = g.heavy_set(b, h)
            assert len(hs) == 4 + wl.topk // 2
            assert list(hs[:4]) == [0, 1, 2, 3]
            assert len(set(hs.tolist())) == len(hs)
            assert hs.min() >= 0 and hs.max() < g.seq_lens[b]
    np.testing.assert_allclose(np.linalg.norm(g.u, axis=1), 1.0, atol=1e-6)


def test_key_bias_lands_on_heavy_rows_in_every_layer():
    wl = WORKLOADS["llama2-7b-10k"].with_(layers=3, kv_heads=2, q_heads=2, max_len=2048, topk=128)
    g = Generator(wl)
    for layer in (0, 2):
        K, V = g.kv(layer)
        for h in range(2):
            proj = _f(K[0, h], "bf16") @ g.u[h]
            hs = g.heavy_set(0, h)
            mask = np.zeros(wl.max_len, bool)
            mask[hs] = True
            assert abs(proj[mask].mean() - 3.0) < 0.3
            assert abs(proj[~mask].mean()) < 0.1
        q = _f(g.q(layer), "bf16")
        assert abs((q[0, 0] @ g.u[0]) - 1.0) < 4.0  # N(0,1) + 1 along u


def test_normal_moments():
    wl = WORKLOADS["llama2-7b-10k"].with_(kv_heads=1, q_heads=1, max_len=8192)
    K, V = Generator(wl).kv(0)
    v = _f(V, "bf16").astype(np.float64).ravel()
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01


def test_padding_modes():
    wl = WORKLOADS["tiny-f32"].with_(batch=2)
    g = Generator(wl, seq_lens=[1000, 7], pad_mode=synth.PAD_NAN)
    K, V = g.kv(0)
    assert np.isnan(K[1, :, 7:]).all() and np.isfinite(K[1, :, :7]).all()
    assert np.isnan(V[0, :, 1000:]).all() and np.isfinite(V[0, :, :1000]).all()
    z = Generator(wl, seq_lens=[1000, 7]).kv(0)[0]
    assert (z[1, :, 7:] == 0).all()
    np.testing.assert_array_equal(z[:, :, :7], K[:, :, :7])
