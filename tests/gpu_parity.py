"""Shared GPU-vs-oracle checking for the parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np

import oracle
from oracle import compare

TOL = {"f32": 1e-5, "bf16": 2e-2}


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_output(got, want, dtype, where):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), f"{where}: non-finite output"
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dtype], f"{where}: max abs error {worst:.3e} > {TOL[dtype]}"
    if dtype == "bf16":
        # Stricter internal bound: one bf16 spacing of the exact value plus 1e-4.
        bound = bf16_ulp(want) + 1e-4
        bad = int(np.sum(err > bound))
        assert bad == 0, f"{where}: {bad} elements beyond one bf16 spacing (+1e-4)"
    return worst


def check_layer(kind, wl, q, K, V, seq_lens, gpu_out, gpu_idx, gpu_scores, selection, where):
    """Check one layer of one (or all) unit(s) in storage form.

    q [B,Hq,d], K/V [B,Hkv,N,d]. `selection` is the set a sparse layer used
    (the GPU's own, already checked at its selection layer).
    Returns max abs error.
    """
    scale = oracle.default_scale(wl.head_dim)
    want, _, oscores = oracle.decode_layer(kind, q, K, V, seq_lens, wl.group, wl.topk, scale, wl.dtype,
                                           selection if kind == "S" else None)
    err = check_output(gpu_out, want, wl.dtype, where)
    if kind == "X":
        for b in range(q.shape[0]):
            n = min(max(int(seq_lens[b]), 0), K.shape[2])
            for h in range(K.shape[1]):
                ok, msg, _ = compare.check_selection_band(gpu_idx[b, h], oscores[b, h], n, wl.topk)
                assert ok, f"{where} b={b} h={h}: {msg}"
                if gpu_scores is not None:
                    s_gpu = np.asarray(gpu_scores[b, h, :n], dtype=np.float64)
                    s_ref = oscores[b, h, :n].astype(np.float64)
                    assert np.all(np.abs(s_gpu - s_ref) <= 1e-3 + 1e-5 * np.abs(s_ref)), f"{where}: scores drift"
                    assert compare.check_selection_exact(gpu_idx[b, h], gpu_scores[b, h], n, wl.topk), \
                        f"{where} b={b} h={h}: selection is not the exact top-k of the written scores"
                live = gpu_idx[b, h][gpu_idx[b, h] >= 0]
                assert np.all(np.diff(live) > 0), f"{where}: positions not ascending"
    return err
