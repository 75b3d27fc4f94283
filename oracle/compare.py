"""Comparison rules between the HIP path's results and the oracle (test infrastructure).

Selection: several index sets can be correct when scores nearly tie, so a
GPU set is checked against the oracle's float32 scores with a band: with
s_k the k-th largest oracle score, every position scoring above s_k + band
must be selected, none scoring below s_k - band may be, positions inside the
band are free; the set must hold exactly k_eff = min(k, N) distinct live
positions. Independently, the GPU set must be exactly the top-k (ties to
the lower position) of the GPU's own written scores.
"""
from __future__ import annotations

import numpy as np

from .ppsa_oracle import select_topk


def live_set(idx) -> list:
    return sorted(int(i) for i in np.asarray(idx).ravel() if i >= 0)


def check_selection_band(gpu_idx, oracle_scores, n_live: int, k: int, band: float = 1e-3, rel_band: float = 0.0):
    """Returns (ok, message, positions inside the band). The band is band + rel_band * |s_k|."""
    gpu_idx = np.asarray(gpu_idx)
    s = np.asarray(oracle_scores, dtype=np.float32)[:n_live].astype(np.float64)
    k_eff = min(k, n_live)
    chosen = gpu_idx[gpu_idx >= 0]
    if len(chosen) != k_eff or len(set(chosen.tolist())) != k_eff:
        return False, f"{len(chosen)} entries / {len(set(chosen.tolist()))} distinct, want {k_eff}", 0
    if np.any(gpu_idx[k_eff:] != -1) if gpu_idx.shape[0] > k_eff else False:
        return False, "slots past k_eff are not -1", 0
    if k_eff == 0:
        return True, "empty", 0
    if chosen.min() < 0 or chosen.max() >= n_live:
        return False, "position outside the live range", 0
    sk = np.sort(s)[::-1][k_eff - 1]
    band = band + rel_band * abs(sk)
    sel = np.zeros(n_live, bool)
    sel[chosen] = True
    must = s > sk + band
    never = s < sk - band
    if np.any(must & ~sel):
        return False, f"missing {int(np.sum(must & ~sel))} positions above the band", 0
    if np.any(never & sel):
        return False, f"selected {int(np.sum(never & sel))} positions below the band", 0
    return True, "ok", int(np.sum(~must & ~never))


def check_selection_exact(gpu_idx, gpu_scores, n_live: int, k: int):
    """GPU set == exact top-k (ties to lower position) of the GPU's own float32 scores."""
    want = live_set(select_topk(np.asarray(gpu_scores, dtype=np.float32)[:n_live], k))
    got = live_set(gpu_idx)
    return got == want
