"""Pins for the float64 oracle: each check ties it to something other than itself.

Kinds of pin (none re-types the oracle's own formula):
  - brute force: top-k by rank counting and by exhaustive subset search;
  - a library routine: torch's float64 scaled_dot_product_attention and
    torch.sort(stable=True);
  - closed forms: q = 0 (uniform weights), one row, two rows (logistic
    weights), one dominant key, exact bf16 bit patterns;
  - invariants: softmax rows sum to one, PPSA with k = N equals full
    attention, the sparse output ignores the order of the index list;
  - multi-step decode against attention over a cache built by concatenating
    the new tokens' rows, and a dominant new key that must be selected.
The mutation test at the bottom plants plausible mistakes in the oracle and
checks that at least one pin fails for each.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ppsa_oracle as O

RNG = np.random.default_rng(20241007)


# --------------------------------------------------------------------------- helpers (independent of oracle)

def rank_select(scores, k):
    """Brute force: n is selected iff fewer than k positions outrank it (higher score, or equal and lower index)."""
    s = [float(x) for x in scores]
    n = len(s)
    chosen = []
    for i in range(n):
        r = sum(1 for j in range(n) if s[j] > s[i] or (s[j] == s[i] and j < i))
        if r < k:
            chosen.append(i)
    return sorted(chosen)


def torch_attention(q, K, V, scale=None):
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, None]
    Kt = torch.from_numpy(np.asarray(K, dtype=np.float64))[None, None]
    Vt = torch.from_numpy(np.asarray(V, dtype=np.float64))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return out[0, 0].numpy()


def as_set(idx):
    return sorted(int(i) for i in idx if i >= 0)


# --------------------------------------------------------------------------- pins

def pin_bf16_bits():
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0000, 0x8000, 0x4049, 0x7F80, 0x0001], dtype=np.uint16)
    want = [1.0, -2.0, 0.5, 0.0, -0.0, 3.140625, math.inf, 2.0 ** -133]
    got = O.widen(bits, "bf16")
    for g, w in zip(got, want):
        assert g == w and math.copysign(1.0, g) == math.copysign(1.0, w)


def pin_select_rank_definition():
    rng = np.random.default_rng(7)
    for n in range(1, 25):
        for trial in range(3):
            vals = np.array([-1.5, -0.0, 0.0, 0.25, 2.0, 2.0], dtype=np.float32)
            s = rng.choice(vals, size=n) if trial else rng.standard_normal(n).astype(np.float32)
            for k in range(1, n + 4):
                got = O.select_topk(s, k)
                assert got.shape == (k,)
                assert np.all(got[min(k, n):] == -1)
                assert as_set(got) == rank_select(s, k)


def pin_select_exhaustive_subsets():
    rng = np.random.default_rng(11)
    for n in range(1, 10):
        s = rng.integers(-2, 3, size=n).astype(np.float32)
        for k in range(1, n + 1):
            best = None
            for sub in itertools.combinations(range(n), k):
                key = (sum(float(s[i]) for i in sub), tuple(-i for i in sub))
                if best is None or key > best[0]:
                    best = (key, sub)
            assert as_set(O.select_topk(s, k)) == list(best[1])


def pin_select_vs_torch_sort():
    rng = np.random.default_rng(3)
    for n in (1, 5, 64, 257):
        s = rng.integers(-4, 5, size=n).astype(np.float32) * 0.5
        order = torch.sort(torch.from_numpy(s), descending=True, stable=True).indices.numpy()
        for k in (1, n // 2 + 1, n):
            assert list(O.select_topk(s, k)[:k]) == list(order[:k])


def pin_q_zero_selects_prefix():
    K = RNG.standard_normal((40, 16))
    q = np.zeros((3, 16))
    s = O.selection_scores(q, K, 40, 0.25)
    for k in (1, 7, 40):
        assert as_set(O.select_topk(s, k)) == list(range(k))


def pin_full_vs_torch_sdpa():
    rng = np.random.default_rng(5)
    for g, n, d in ((1, 1, 8), (1, 17, 64), (4, 33, 128), (8, 5, 64)):
        q = rng.standard_normal((g, d))
        K = rng.standard_normal((n + 3, d))
        V = rng.standard_normal((n + 3, d))
        got = O.full_attention(q, K, V, n, O.default_scale(d))
        want = torch_attention(q, K[:n], V[:n])
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def pin_q_zero_mean():
    K = RNG.standard_normal((20, 8))
    V = RNG.standard_normal((20, 8))
    got = O.full_attention(np.zeros((2, 8)), K, V, 13, 0.3)
    np.testing.assert_allclose(got, np.tile(V[:13].mean(axis=0), (2, 1)), rtol=0, atol=1e-14)


def pin_single_row():
    K = RNG.standard_normal((4, 8))
    V = RNG.standard_normal((4, 8))
    got = O.full_attention(RNG.standard_normal((3, 8)), K, V, 1, 0.3)
    np.testing.assert_array_equal(got, np.tile(V[0], (3, 1)))


def pin_two_rows_closed_form():
    # q=(1,2), K0=(3,0), K1=(0,1), d=2: logits 3/sqrt2 and 2/sqrt2, gap 1/sqrt2.
    q = np.array([[1.0, 2.0]])
    K = np.array([[3.0, 0.0], [0.0, 1.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    w0 = 1.0 / (1.0 + math.exp(-1.0 / math.sqrt(2.0)))
    got = O.full_attention(q, K, V, 2, O.default_scale(2))
    np.testing.assert_allclose(got, [[w0, 1.0 - w0]], rtol=0, atol=1e-15)


def pin_dominant_key():
    d = 16
    q = np.zeros((1, d))
    q[0, 3] = 1.0
    K = RNG.standard_normal((30, d)) * 0.1
    K[17, 3] = 200.0  # logit gap > 40 at scale 1/4
    V = RNG.standard_normal((30, d))
    got = O.full_attention(q, K, V, 30, O.default_scale(d))
    np.testing.assert_allclose(got[0], V[17], rtol=0, atol=1e-15)


def pin_softmax_rows_sum_to_one():
    for scale in (0.01, 1.0, 30.0):
        a = RNG.standard_normal((5, 300)) * scale
        w = O.softmax_weights(a)
        assert np.all(w >= 0)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def pin_group_score_is_sum_of_heads():
    # Two query heads picking coordinates 0 and 1: score[n] = (K[n,0] + K[n,1]) * scale, one float32 rounding.
    K = np.array([[1.0, 2.0, 9.0], [0.5, -4.0, 9.0], [1e-3, 1e-3, 9.0]])
    q = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]])
    s = O.selection_scores(q, K, 3, 0.5)
    assert s.dtype == np.float32
    assert list(s) == [np.float32(1.5), np.float32(-1.75), np.float32(1e-3)]
    assert as_set(O.select_topk(s, 2)) == [0, 2]


def pin_sparse_equals_full_when_k_is_n():
    rng = np.random.default_rng(9)
    L, B, Hkv, g, N, d = 5, 2, 2, 2, 24, 16
    q = rng.standard_normal((L, B, Hkv * g, d)).astype(np.float32)
    kv = [(rng.standard_normal((B, Hkv, N, d)).astype(np.float32),
           rng.standard_normal((B, Hkv, N, d)).astype(np.float32)) for _ in range(L)]
    lens = np.array([N, N - 5])
    outs, _ = O.decode_step(["F", "X", "S", "S", "X"], q, lambda l: kv[l], lens, g, N, O.default_scale(d), "f32")
    for layer in range(L):
        for b in range(B):
            for h in range(Hkv):
                n = lens[b]
                want = torch_attention(q[layer, b, h * g:(h + 1) * g], kv[layer][0][b, h, :n], kv[layer][1][b, h, :n])
                np.testing.assert_allclose(outs[layer, b, h * g:(h + 1) * g], want, rtol=0, atol=1e-12)


def pin_sparse_permutation_invariant():
    q = RNG.standard_normal((2, 8))
    K = RNG.standard_normal((50, 8))
    V = RNG.standard_normal((50, 8))
    idx = np.array([40, 3, 17, 22, 8, 9])
    a = O.sparse_attention(q, K, V, idx, 50, 0.3)
    b = O.sparse_attention(q, K, V, idx[::-1].copy(), 50, 0.3)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
    want = torch_attention(q, K[np.sort(idx)], V[np.sort(idx)], scale=0.3)
    np.testing.assert_allclose(a, want, rtol=0, atol=1e-12)


def pin_sparse_skips_invalid_and_counts_repeats():
    # Rows 0 and 1, with row 0 listed twice: weights 2e^a0 : e^a1.
    q = np.array([[1.0, 0.0]])
    K = np.array([[1.0, 0.0], [0.0, 0.0], [5.0, 5.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0], [7.0, 7.0]])
    idx = np.array([0, -1, 1, 0, 2, 9])  # 2 is past n_live=2, 9 past the cache
    got = O.sparse_attention(q, K, V, idx, 2, 1.0)
    w0 = 2 * math.e / (2 * math.e + 1.0)
    np.testing.assert_allclose(got, [[w0, 1.0 - w0]], rtol=0, atol=1e-15)


def pin_reuse_most_recent_selection():
    rng = np.random.default_rng(21)
    L, B, Hkv, g, N, d, k = 6, 1, 2, 2, 40, 8, 5
    sched = ["F", "X", "S", "X", "S", "S"]
    q = rng.standard_normal((L, B, Hkv * g, d)).astype(np.float32)
    kv = [(rng.standard_normal((B, Hkv, N, d)).astype(np.float32),
           rng.standard_normal((B, Hkv, N, d)).astype(np.float32)) for _ in range(L)]
    lens = np.array([N])
    scale = O.default_scale(d)
    outs, sels = O.decode_step(sched, q, lambda l: kv[l], lens, g, k, scale, "f32")
    assert len(sels) == 2
    current = None
    for layer, kind in enumerate(sched):
        for h in range(Hkv):
            qh = q[layer, 0, h * g:(h + 1) * g].astype(np.float64)
            K = kv[layer][0][0, h].astype(np.float64)
            V = kv[layer][1][0, h].astype(np.float64)
            if kind == "X":
                sc = (torch.from_numpy(qh) @ torch.from_numpy(K).T).numpy().sum(axis=0) * scale
                chosen = rank_select(sc.astype(np.float32), k)
                assert as_set(sels[0 if layer == 1 else 1][0, h]) == chosen
                if h == Hkv - 1:
                    current = "layer%d" % layer
            if kind == "S":
                src = sels[0] if current == "layer1" else sels[1]
                rows = as_set(src[0, h])
                want = torch_attention(qh, K[rows], V[rows], scale=scale)
                np.testing.assert_allclose(outs[layer, 0, h * g:(h + 1) * g], want, rtol=0, atol=1e-12)
    assert as_set(sels[0][0, 0]) != as_set(sels[1][0, 0])  # the two selections differ on this input


def pin_empty_and_short():
    q = RNG.standard_normal((2, 8))
    K = RNG.standard_normal((6, 8))
    V = RNG.standard_normal((6, 8))
    np.testing.assert_array_equal(O.full_attention(q, K, V, 0, 0.3), np.zeros((2, 8)))
    assert list(O.select_topk(np.zeros(0, np.float32), 3)) == [-1, -1, -1]
    s = np.array([0.5, -1.0, 2.0], dtype=np.float32)
    assert list(O.select_topk(s, 5)) == [2, 0, 1, -1, -1]


def _multistep_case(schedule, topk=3):
    L, B, Hkv, g, d, n_max, T = len(schedule), 2, 2, 2, 8, 10, 3
    lens0 = np.array([6, 9])
    K = [RNG.standard_normal((B, Hkv, n_max, d)).astype(np.float32) for _ in range(L)]
    V = [RNG.standard_normal((B, Hkv, n_max, d)).astype(np.float32) for _ in range(L)]
    q = RNG.standard_normal((T, L, B, Hkv * g, d)).astype(np.float32)
    kn = RNG.standard_normal((T, L, B, Hkv, d)).astype(np.float32)
    vn = RNG.standard_normal((T, L, B, Hkv, d)).astype(np.float32)
    K0, V0 = [x.copy() for x in K], [x.copy() for x in V]
    outs, sels, lens = O.decode_steps(schedule, q, K, V, lens0, kn, vn, g, topk, 0.35, "f32")
    return (L, B, Hkv, g, d, n_max, T, lens0, K0, V0, q, kn, vn), outs, sels, lens


def pin_multistep_full_vs_torch_sdpa_on_concatenated_cache():
    """T full-attention steps with appends equal attention over the original rows followed by the new
    tokens' rows, built by concatenation (a cache that fills up stops taking rows)."""
    (L, B, Hkv, g, d, n_max, T, lens0, K0, V0, q, kn, vn), outs, _, lens = _multistep_case(["F", "F"])
    for b in range(B):
        taken = min(T, n_max - int(lens0[b]))
        assert int(lens[b]) == int(lens0[b]) + taken
        for t in range(T):
            m = min(t + 1, taken)
            for layer in range(L):
                for h in range(Hkv):
                    Kc = np.concatenate([K0[layer][b, h, :lens0[b]], kn[:m, layer, b, h]])
                    Vc = np.concatenate([V0[layer][b, h, :lens0[b]], vn[:m, layer, b, h]])
                    want = torch_attention(q[t, layer, b, h * g:(h + 1) * g], Kc, Vc, 0.35)
                    np.testing.assert_allclose(outs[t, layer, b, h * g:(h + 1) * g], want, rtol=1e-12, atol=1e-12)


def pin_multistep_new_dominant_key_is_selected():
    """A new token whose key dominates every query is the single selected position at its step."""
    L, B, Hkv, g, d, n_max = 3, 1, 1, 2, 4, 12
    K = [RNG.standard_normal((B, Hkv, n_max, d)).astype(np.float32) for _ in range(L)]
    V = [RNG.standard_normal((B, Hkv, n_max, d)).astype(np.float32) for _ in range(L)]
    q = np.ones((2, L, B, g, d), dtype=np.float32)
    kn = np.zeros((2, L, B, Hkv, d), dtype=np.float32)
    kn[1] = 50.0  # step 1's token dominates; step 0's token has logit 0
    vn = RNG.standard_normal((2, L, B, Hkv, d)).astype(np.float32)
    _, sels, lens = O.decode_steps(["F", "F", "X"], q, K, V, np.array([7]), kn, vn, g, 1, 0.5, "f32")
    assert int(lens[0]) == 9
    assert as_set(sels[1][0][0, 0]) == [8]


def pin_append_into_full_cache_changes_nothing():
    K = [RNG.standard_normal((1, 2, 5, 4)).astype(np.float32)]
    V = [RNG.standard_normal((1, 2, 5, 4)).astype(np.float32)]
    K0, V0 = K[0].copy(), V[0].copy()
    lens = O.append_kv(K, V, np.array([5]), np.ones((1, 1, 2, 4), np.float32), np.ones((1, 1, 2, 4), np.float32))
    assert int(lens[0]) == 5
    np.testing.assert_array_equal(K[0], K0)
    np.testing.assert_array_equal(V[0], V0)


def pin_shared_selection_brute_force():
    """Head-shared selection: the set ranks positions by the sum, over every query head of the batch row,
    of its logit against its own KV head's key, written out as plain loops; every KV head gets that set."""
    B, Hkv, g, d, n_max, k, scale = 2, 3, 2, 5, 9, 4, 0.4
    q = RNG.standard_normal((B, Hkv * g, d)).astype(np.float32)
    K = RNG.standard_normal((B, Hkv, n_max, d)).astype(np.float32)
    V = RNG.standard_normal((B, Hkv, n_max, d)).astype(np.float32)
    lens = [9, 6]
    _, sel, _ = O.decode_layer("X", q, K, V, lens, g, k, scale, "f32", None, "shared")
    for b in range(B):
        total = []
        for n in range(lens[b]):
            acc = 0.0
            for hq in range(Hkv * g):
                acc += sum(float(q[b, hq, i]) * float(K[b, hq // g, n, i]) for i in range(d)) * scale
            total.append(np.float32(acc))
        want = rank_select(total, k)
        for h in range(Hkv):
            assert as_set(sel[b, h]) == want, (b, h)


def pin_shared_equals_per_head_with_one_kv_head():
    q = RNG.standard_normal((2, 4, 6)).astype(np.float32)
    K = RNG.standard_normal((2, 1, 11, 6)).astype(np.float32)
    V = RNG.standard_normal((2, 1, 11, 6)).astype(np.float32)
    _, a, _ = O.decode_layer("X", q, K, V, [11, 8], 4, 5, 0.3, "f32", None, "kv_head")
    _, b, _ = O.decode_layer("X", q, K, V, [11, 8], 4, 5, 0.3, "f32", None, "shared")
    np.testing.assert_array_equal(a, b)


def pin_softmax_selection_brute_force():
    """Softmax-weight selection: each head's weights written out with math.exp, summed over the group."""
    B, Hkv, g, d, n_max, k, scale = 1, 2, 3, 4, 8, 3, 0.7
    q = RNG.standard_normal((B, Hkv * g, d)).astype(np.float32) * 2
    K = RNG.standard_normal((B, Hkv, n_max, d)).astype(np.float32)
    V = RNG.standard_normal((B, Hkv, n_max, d)).astype(np.float32)
    _, sel, sc = O.decode_layer("X", q, K, V, [7], g, k, scale, "f32", None, "softmax")
    for h in range(Hkv):
        tot = [0.0] * 7
        for hq in range(h * g, (h + 1) * g):
            a = [sum(float(q[0, hq, i]) * float(K[0, h, n, i]) for i in range(d)) * scale for n in range(7)]
            z = sum(math.exp(x - max(a)) for x in a)
            for n in range(7):
                tot[n] += math.exp(a[n] - max(a)) / z
        want = [np.float32(x) for x in tot]
        np.testing.assert_allclose(sc[0, h, :7], want, rtol=1e-6)
        assert as_set(sel[0, h]) == rank_select(want, k)


def pin_softmax_selection_group_one_orders_like_logits():
    q = RNG.standard_normal((2, 3, 6)).astype(np.float32)
    K = RNG.standard_normal((2, 3, 20, 6)).astype(np.float32)
    V = RNG.standard_normal((2, 3, 20, 6)).astype(np.float32)
    _, a, _ = O.decode_layer("X", q, K, V, [20, 13], 1, 6, 0.4, "f32", None, "kv_head")
    _, b, _ = O.decode_layer("X", q, K, V, [20, 13], 1, 6, 0.4, "f32", None, "softmax")
    np.testing.assert_array_equal(a, b)


def pin_coverage_uniform_closed_form():
    """q = 0 gives every position the same mass 1/n; pruning until the pruned mass exceeds tau takes
    floor(tau n) + 1 positions, from the highest position down."""
    n, g = 8, 2
    q = np.zeros((1, g, 4), np.float32)
    K = RNG.standard_normal((1, 1, n, 4)).astype(np.float32)
    V = RNG.standard_normal((1, 1, n, 4)).astype(np.float32)
    for tau, kept in ((0.25, 5), (0.0, 7), (0.5, 3), (0.9, 0)):
        _, sel, _ = O.decode_layer("X", q, K, V, [n], g, n, 1.0, "f32", None, "coverage", tau)
        assert as_set(sel[0, 0]) == list(range(kept)), (tau, as_set(sel[0, 0]))


def pin_coverage_brute_force():
    """Random masses: sort ascending (equal masses from the higher position), prune while the pruned
    mass has not yet exceeded tau of the total, keep the rest -- written out as a loop."""
    g, n = 3, 11
    q = RNG.standard_normal((1, g, 5)).astype(np.float32)
    K = RNG.standard_normal((1, 1, n, 5)).astype(np.float32)
    V = RNG.standard_normal((1, 1, n, 5)).astype(np.float32)
    for tau in (0.05, 0.3, 0.7):
        _, sel, sc = O.decode_layer("X", q, K, V, [n], g, n, 0.8, "f32", None, "coverage", tau)
        m = [float(x) / g for x in sc[0, 0, :n]]
        order = sorted(range(n), key=lambda i: (m[i], -i))
        total, pruned, acc = sum(m), [], 0.0
        for i in order:
            if acc > tau * total:
                break
            acc += m[i]
            pruned.append(i)
        assert as_set(sel[0, 0]) == sorted(set(range(n)) - set(pruned)), tau


PINS = [pin_bf16_bits, pin_select_rank_definition, pin_select_exhaustive_subsets, pin_select_vs_torch_sort,
        pin_q_zero_selects_prefix, pin_full_vs_torch_sdpa, pin_q_zero_mean, pin_single_row,
        pin_two_rows_closed_form, pin_dominant_key, pin_softmax_rows_sum_to_one, pin_group_score_is_sum_of_heads,
        pin_sparse_equals_full_when_k_is_n, pin_sparse_permutation_invariant,
        pin_sparse_skips_invalid_and_counts_repeats, pin_reuse_most_recent_selection, pin_empty_and_short,
        pin_multistep_full_vs_torch_sdpa_on_concatenated_cache, pin_multistep_new_dominant_key_is_selected,
        pin_append_into_full_cache_changes_nothing, pin_shared_selection_brute_force,
        pin_shared_equals_per_head_with_one_kv_head, pin_softmax_selection_brute_force,
        pin_softmax_selection_group_one_orders_like_logits, pin_coverage_uniform_closed_form,
        pin_coverage_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# --------------------------------------------------------------------------- mutation check of the pins

def _mut_no_scale(q, K, scale):
    return q @ K.T


def _mut_ties_high(scores, k):
    s = np.asarray(scores, dtype=np.float32).astype(np.float64)
    n = s.shape[0]
    k_eff = min(int(k), n)
    order = (n - 1 - np.argsort(-s[::-1], kind="stable"))[:k_eff]
    out = np.full(int(k), -1, dtype=np.int64)
    out[:k_eff] = order
    return out


def _mut_mean_group(q, K, n_live, scale):
    return O.logits(q, K[:n_live], scale).mean(axis=0).astype(np.float32)


def _mut_swapped_kv(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], V.shape[1]))
    return O.softmax_weights(O.logits(q, V, scale)) @ K


def _mut_no_renorm(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], V.shape[1]))
    a = O.logits(q, K, scale)
    return np.exp(a - a.max(axis=-1, keepdims=True)) @ V


_orig_decode_layer = O.decode_layer


def _mut_first_selection(kind, q, K, V, seq_lens, group, topk, scale, dtype, selection=None, select_mode="kv_head",
                         coverage_tau=0.0):
    out, sel, sc = _orig_decode_layer(kind, q, K, V, seq_lens, group, topk, scale, dtype, selection, select_mode,
                                      coverage_tau)
    if kind == "X" and selection is not None:
        sel = selection  # keeps reusing the first set
    return out, sel, sc


def _mut_append_over_last_row(K_layers, V_layers, seq_lens, k_new, v_new):
    n_max = K_layers[0].shape[2]
    lens = np.array([min(max(int(n), 0), n_max) for n in seq_lens])
    for b, n in enumerate(lens):
        if 0 < n < n_max:
            for layer in range(len(K_layers)):
                K_layers[layer][b, :, n - 1, :] = k_new[layer, b]
                V_layers[layer][b, :, n - 1, :] = v_new[layer, b]
    return np.minimum(lens + 1, n_max)


_orig_append = O.append_kv


def _mut_append_without_growth(K_layers, V_layers, seq_lens, k_new, v_new):
    _orig_append(K_layers, V_layers, seq_lens, k_new, v_new)
    return np.asarray(seq_lens, dtype=np.int64)


def _mut_shared_first_head(q_all, K_all, n_live, group, scale):
    return O.logits(q_all[:group], K_all[0, :n_live], scale).sum(axis=0).astype(np.float32)


def _mut_softmax_unnormalised(q, K, n_live, scale):
    a = O.logits(q, K[:n_live], scale)
    return np.exp(a - a.max(axis=1, keepdims=True)).sum(axis=0).astype(np.float32)


def _mut_coverage_reaching(scores, group, tau):
    m = np.asarray(scores, dtype=np.float32).astype(np.float64) / group
    n = m.shape[0]
    if n == 0:
        return 0
    csum = np.cumsum(m[np.lexsort((-np.arange(n), m))])
    over = np.nonzero(csum >= tau * csum[-1])[0]  # stops on reaching tau instead of exceeding it
    return 0 if over.size == 0 else int(n - (over[0] + 1))


MUTANTS = {
    "drop_scale": ("logits", _mut_no_scale),
    "ties_to_higher_index": ("select_topk", _mut_ties_high),
    "group_mean_not_sum": ("selection_scores", _mut_mean_group),
    "swapped_k_and_v": ("attend", _mut_swapped_kv),
    "no_renormalisation": ("attend", _mut_no_renorm),
    "reuse_first_selection": ("decode_layer", _mut_first_selection),
    "append_over_last_row": ("append_kv", _mut_append_over_last_row),
    "append_without_growth": ("append_kv", _mut_append_without_growth),
    "shared_score_of_first_head_only": ("shared_selection_scores", _mut_shared_first_head),
    "softmax_weights_not_normalised": ("softmax_selection_scores", _mut_softmax_unnormalised),
    "coverage_stops_on_reaching_tau": ("coverage_budget", _mut_coverage_reaching),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
