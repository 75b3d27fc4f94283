"""Float64 CPU oracle of the PPSA decode step.

TEST INFRASTRUCTURE. This module is the plain, slow, obviously correct
statement of what the decode step computes. Only the test-suite, the smoke
check in __graft_entry__ and the CPU-baseline leg of bench.py may import it;
the HIP library and its Python binding never do, and it shares no code with
them. Inputs come from the seeded generator in `synth`.

Source: the paper-review page "TidalDecode: Fast and Accurate LLM Decoding
with Position Persistent Sparse Attention" (arXiv 2410.05076).
  [S2]  section 2 "Core idea", solution overview: a decode step uses three
        layer kinds -- full attention in the first layers, full attention
        plus token selection right after them and at one middle layer, and
        PPSA (attention over the pre-selected tokens only) everywhere else.
  [S3F] section 3 "Technical architecture", decode-step framework figure:
        layers 0-1 full, layer 2 full + top-k selection, layers up to the
        middle layer reuse that set, the middle layer re-selects, the rest
        reuse the new set.
  [S3E] section 3, PPSA paragraph, attention equation: A = Q K^T / sqrt(d),
        H = softmax(A) V. The page prints "Q_i K_i"; the transpose is the
        only reading that type-checks.
  [S3P] section 3, PPSA paragraph: later layers reuse the token set of the
        preceding selection layer instead of selecting per layer and head.
  [S2D] section 2 "Core idea", problem definition: decoding produces one
        token at a time against a KV cache that grows with every token.

Readings where the page is silent (each repeated in the design notes):
  R-score  the selection ranks positions by the raw logit q.k/sqrt(d); for a
           GQA group the logits of its query heads are summed, and that sum
           is rounded once to float32 -- the score both sides rank.
  R-unit   one selected set per (batch row, KV head); a sparse layer applies
           it to the same (batch row, KV head) index.
  R-ties   equal scores go to the lower position; -0.0 equals +0.0.
  R-keff   k_eff = min(k, N_b) positions are selected, the rest of the k
           slots hold -1.
  R-empty  attention over zero positions is the zero vector.
  R-mask   the single decode query attends every live row [0, N_b) with no
           causal mask (the cache already holds the current token).
  R-renorm a sparse layer renormalises the softmax over the selected rows.
  R-multi  a sparse index list is taken as given: entries outside [0, N_b)
           are skipped, a repeated entry counts once per occurrence.
  R-lens   a length outside [0, Nmax] is clamped into it.
  R-shared (selection variant, off by default) one set per batch row,
           ranked by the float32 rounding of the sum over all of the row's
           query heads of the raw logit (each head against its own KV head's
           key at that position) and applied to every KV head.
  R-softmax (selection variant, off by default) one set per (batch row,
           KV head), ranked by the float32 rounding of the sum over the
           group's query heads of the softmax weight each head gives the
           position in this layer's full attention.
  R-cover  (selection variant, off by default; the token-sparse page's
           dynamic token coverage) with masses m_n = softmax-weight sum / group
           (about 1 in total), positions are pruned in ascending mass order,
           equal masses from the higher position, until the pruned mass
           exceeds tau times the total; the rest are kept (at most k), ranked
           like any selection.
  R-append a decode step first stores the new token's K and V rows at
           position N_b of every layer and KV head, and N_b becomes N_b + 1;
           the step's attention then sees them. A full cache (N_b = Nmax)
           takes no row and keeps N_b = Nmax.

Parity pins: every function here is pinned by tests/test_oracle_pins.py
against brute force, closed forms, invariants and a library routine (torch
scaled-dot-product attention in float64).
"""
from __future__ import annotations

import numpy as np

FULL, FULL_SELECT, SPARSE = "F", "X", "S"


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage to float64: 'bf16' arrays are uint16 bit patterns, 'f32' are float32."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def default_scale(head_dim: int) -> float:
    """1/sqrt(d) of the attention equation [S3E]."""
    return 1.0 / np.sqrt(float(head_dim))


def logits(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """A[h, n] = (sum_i q[h, i] K[n, i]) * scale  [S3E].  q [g, d], K [n, d]."""
    return (q @ K.T) * scale


def softmax_weights(a: np.ndarray) -> np.ndarray:
    """Row-wise softmax of A [S3E] (max-subtracted, which leaves it unchanged)."""
    m = a.max(axis=-1, keepdims=True)
    e = np.exp(a - m)
    return e / e.sum(axis=-1, keepdims=True)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """H = softmax(q K^T * scale) V over the rows given [S3E]; no rows -> zeros (R-empty)."""
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], V.shape[1]), dtype=np.float64)
    return softmax_weights(logits(q, K, scale)) @ V


def full_attention(q, K, V, n_live: int, scale: float) -> np.ndarray:
    """Full attention of one (batch row, KV head) unit over rows [0, n_live) (R-mask)."""
    return attend(q, K[:n_live], V[:n_live], scale)


def selection_scores(q, K, n_live: int, scale: float) -> np.ndarray:
    """float32 score per live position: sum over the group's query heads of the logit (R-score)."""
    return logits(q, K[:n_live], scale).sum(axis=0).astype(np.float32)


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """The k_eff highest-scoring positions, ties to the lower position, -1 padded to k.

    A stable sort on the negated score keeps equal scores in position order
    (R-ties); -0.0 and +0.0 compare equal under it. Output is in rank order.
    """
    s = np.asarray(scores, dtype=np.float32).astype(np.float64)
    k_eff = min(int(k), s.shape[0])
    order = np.argsort(-s, kind="stable")[:k_eff]
    out = np.full(int(k), -1, dtype=np.int64)
    out[:k_eff] = order
    return out


def sparse_attention(q, K, V, idx, n_live: int, scale: float) -> np.ndarray:
    """Attention over the listed positions only, renormalised over them (R-renorm, R-multi) [S3P]."""
    idx = np.asarray(idx, dtype=np.int64)
    keep = idx[(idx >= 0) & (idx < n_live)]
    return attend(q, K[keep], V[keep], scale)


def shared_selection_scores(q_all, K_all, n_live: int, group: int, scale: float) -> np.ndarray:
    """float32 score per live position summed over every query head of a batch row (R-shared).
    q_all [Hq, d] and K_all [Hkv, N, d] in float64."""
    total = np.zeros(n_live, dtype=np.float64)
    for h in range(K_all.shape[0]):
        total += logits(q_all[h * group:(h + 1) * group], K_all[h, :n_live], scale).sum(axis=0)
    return total.astype(np.float32)


def softmax_selection_scores(q, K, n_live: int, scale: float) -> np.ndarray:
    """float32 score per live position: sum over the group's query heads of their softmax weights (R-softmax)."""
    if n_live == 0:
        return np.zeros(0, dtype=np.float32)
    return softmax_weights(logits(q, K[:n_live], scale)).sum(axis=0).astype(np.float32)


def coverage_budget(scores: np.ndarray, group: int, tau: float) -> int:
    """Positions kept by the coverage rule (R-cover): n minus the smallest count p of lowest-mass
    positions whose mass sum exceeds tau * total; 0 when no count does."""
    m = np.asarray(scores, dtype=np.float32).astype(np.float64) / group
    n = m.shape[0]
    if n == 0:
        return 0
    order = np.lexsort((-np.arange(n), m))  # mass ascending, then position descending
    csum = np.cumsum(m[order])
    over = np.nonzero(csum > tau * csum[-1])[0]
    return 0 if over.size == 0 else int(n - (over[0] + 1))


def decode_layer(kind: str, q, K, V, seq_lens, group: int, topk: int, scale: float, dtype: str,
                 selection=None, select_mode: str = "kv_head", coverage_tau: float = 0.0):
    """One layer of the decode step [S2, S3F].

    q [B, Hq, d], K and V [B, Hkv, Nmax, d] in storage form; `selection`
    [B, Hkv, k] is the most recent selected set (needed by SPARSE layers).
    Returns (out [B, Hq, d] float64, selection after this layer, scores or None).
    """
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    assert Hq == Hkv * group
    out = np.zeros((B, Hq, d), dtype=np.float64)
    new_sel = None if selection is None else np.array(selection, copy=True)
    scores = None
    if kind == FULL_SELECT:
        new_sel = np.full((B, Hkv, topk), -1, dtype=np.int64)
        scores = np.zeros((B, Hkv, K.shape[2]), dtype=np.float32)
    if kind == SPARSE and selection is None:
        raise ValueError("a sparse layer needs an earlier selection layer")
    for b in range(B):
        n = min(max(int(seq_lens[b]), 0), K.shape[2])  # live rows, clamped to the cache
        for h in range(Hkv):
            heads = slice(h * group, (h + 1) * group)
            qg = widen(q[b, heads], dtype)
            if kind == SPARSE:
                rows = np.asarray(selection[b, h], dtype=np.int64)
                keep = rows[(rows >= 0) & (rows < n)]
                Kb = widen(K[b, h, keep], dtype)
                Vb = widen(V[b, h, keep], dtype)
                out[b, heads] = attend(qg, Kb, Vb, scale)
            else:
                Kb = widen(K[b, h, :n], dtype)
                Vb = widen(V[b, h, :n], dtype)
                out[b, heads] = attend(qg, Kb, Vb, scale)
                if kind == FULL_SELECT:
                    if select_mode in ("softmax", "coverage"):
                        s = softmax_selection_scores(qg, Kb, n, scale)
                    else:
                        s = selection_scores(qg, Kb, n, scale)
                    scores[b, h, :n] = s
                    if select_mode == "coverage":
                        kk = min(coverage_budget(s, group, coverage_tau), topk)
                        new_sel[b, h, :kk] = select_topk(s, kk)[:kk]
                    else:
                        new_sel[b, h] = select_topk(s, topk)
        if kind == FULL_SELECT and select_mode == "shared":
            s = shared_selection_scores(widen(q[b], dtype), widen(K[b, :, :n], dtype), n, group, scale)
            new_sel[b, :] = select_topk(s, topk)
    return out, new_sel, scores


def decode_step(schedule, q_layers, kv_layers, seq_lens, group: int, topk: int, scale: float, dtype: str,
                select_mode: str = "kv_head", coverage_tau: float = 0.0):
    """Whole decode step: run `schedule` (list of F/X/S) over per-layer inputs.

    q_layers[l] is [B, Hq, d]; kv_layers(l) returns (K, V) for layer l.
    Returns (outs [L, B, Hq, d], selections made at X layers in order).
    """
    outs, sels = [], []
    selection = None
    for layer, kind in enumerate(schedule):
        K, V = kv_layers(layer)
        out, selection, _ = decode_layer(kind, q_layers[layer], K, V, seq_lens, group, topk, scale, dtype,
                                         selection, select_mode, coverage_tau)
        outs.append(out)
        if kind == FULL_SELECT:
            sels.append(selection)
    return np.stack(outs), sels



def append_kv(K_layers, V_layers, seq_lens, k_new, v_new):
    """Store one new token's rows and grow the lengths [S2D] (R-append, R-lens).

    K_layers / V_layers: per-layer storage arrays [B, Hkv, Nmax, d], updated
    in place; k_new / v_new [L, B, Hkv, d] in the same storage type.
    Returns the new lengths (int64 [B]).
    """
    n_max = K_layers[0].shape[2]
    new_lens = np.empty(len(seq_lens), dtype=np.int64)
    for b, n in enumerate(seq_lens):
        n = min(max(int(n), 0), n_max)
        if n == n_max:
            new_lens[b] = n_max
            continue
        for layer in range(len(K_layers)):
            K_layers[layer][b, :, n, :] = k_new[layer, b]
            V_layers[layer][b, :, n, :] = v_new[layer, b]
        new_lens[b] = n + 1
    return new_lens


def decode_steps(schedule, q_steps, K_layers, V_layers, seq_lens, k_new_steps, v_new_steps, group: int, topk: int,
                 scale: float, dtype: str):
    """T decode steps, each appending its token's rows before its layers run [S2D].

    q_steps [T, L, B, Hq, d]; k_new_steps / v_new_steps [T, L, B, Hkv, d];
    K_layers / V_layers as in append_kv (updated in place).
    Returns (outs [T, L, B, Hq, d], selections per step, final lengths).
    """
    lens = np.asarray(seq_lens)
    outs, sels = [], []
    for t in range(len(q_steps)):
        lens = append_kv(K_layers, V_layers, lens, k_new_steps[t], v_new_steps[t])
        out, sel = decode_step(schedule, q_steps[t], lambda layer: (K_layers[layer], V_layers[layer]), lens,
                               group, topk, scale, dtype)
        outs.append(out)
        sels.append(sel)
    return np.stack(outs), sels, lens
