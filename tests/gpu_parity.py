"""Shared GPU-vs-oracle checking for the parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np

import oracle
from oracle import compare

TOL = {"f32": 1e-5, "bf16": 2e-2}
# Relative L2 error of a bf16 layer output: the output rounding alone is at most half a bf16 spacing
# (2^-9 relative) per element, the weight rounding adds about as much again at most, so a layer's
# error vector stays under 2^-8 of the reference's norm; a precision regression would not.
REL_L2_BF16 = 2.0 ** -8


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_output(got, want, dtype, where, abs_weighted=None):
    """Official gate: max abs error <= TOL[dtype].

    bf16 also gets a per-element bound derived from the arithmetic: the
    softmax weights may be rounded to bf16 (relative error <= 2^-8 each,
    so each normalised weight moves by <= ~2^-7 of itself), which moves an
    output by at most 2^-7 * sum_j w_j |V_j| (`abs_weighted`, the attention
    of |V|); the output is then rounded to bf16 (<= one spacing), plus 1e-5
    for float32 accumulation.
    """
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), f"{where}: non-finite output"
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dtype], f"{where}: max abs error {worst:.3e} > {TOL[dtype]}"
    ref_norm = float(np.linalg.norm(want))
    if dtype == "bf16" and ref_norm > 0.0:
        rel = float(np.linalg.norm(got - want)) / ref_norm
        assert rel <= REL_L2_BF16, f"{where}: relative L2 error {rel:.3e} > 2^-8"
    if dtype == "bf16" and abs_weighted is not None:
        bound = 2.0 ** -7 * 1.01 * abs_weighted + bf16_ulp(want) + 1e-5
        bad = int(np.sum(err > bound))
        assert bad == 0, f"{where}: {bad} elements beyond the weight-rounding bound (worst excess " \
                         f"{float(np.max(err - bound)):.3e})"
    return worst


def abs_storage(x, dtype):
    """|x| in storage form: clear the bf16 sign bit, or np.abs for float32."""
    return (np.asarray(x) & np.uint16(0x7FFF)) if dtype == "bf16" else np.abs(x)


def check_layer(kind, wl, q, K, V, seq_lens, gpu_out, gpu_idx, gpu_scores, selection, where):
    """Check one layer of one (or all) unit(s) in storage form.

    q [B,Hq,d], K/V [B,Hkv,N,d]. `selection` is the set a sparse layer used
    (the GPU's own, already checked at its selection layer).
    Returns max abs error.
    """
    scale = oracle.default_scale(wl.head_dim)
    want, _, oscores = oracle.decode_layer(kind, q, K, V, seq_lens, wl.group, wl.topk, scale, wl.dtype,
                                           selection if kind == "S" else None)
    absw = None
    if wl.dtype == "bf16":
        absw, _, _ = oracle.decode_layer(kind, q, K, abs_storage(V, wl.dtype), seq_lens, wl.group, wl.topk, scale,
                                         wl.dtype, selection if kind == "S" else None)
    err = check_output(gpu_out, want, wl.dtype, where, absw)
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
