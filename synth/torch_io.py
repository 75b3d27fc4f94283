"""Move generated inputs into torch device tensors (layer by layer)."""
from __future__ import annotations

import numpy as np
import torch


def torch_dtype(wl) -> torch.dtype:
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def to_torch(x: np.ndarray) -> torch.Tensor:
    """float32 arrays stay float32; uint16 bf16 bit patterns become bfloat16 (bit-exact)."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(x)


def from_torch(t: torch.Tensor) -> np.ndarray:
    """Inverse of to_torch, on the CPU."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload(wl, gen, device, keep_layers=None, keep_units=None, progress=None, visit=None):
    """Generate every layer and copy it to `device`.

    Returns (q [L,B,Hq,d], k, v [L,B,Hkv,N,d], seq_lens [B] int32, host) where
    host[layer] = (q, K, V) numpy arrays for layers in keep_layers (all if
    None), restricted to the (b, h) pairs in keep_units when given (as dicts
    {(b, h): (q_group, K_unit, V_unit)}). visit(layer, q, K, V), if given,
    sees each layer's host arrays before their buffers are reused.
    """
    L, B, Hq, Hkv, N, d = wl.layers, wl.batch, wl.q_heads, wl.kv_heads, wl.max_len, wl.head_dim
    dt = torch_dtype(wl)
    q = torch.empty((L, B, Hq, d), dtype=dt, device=device)
    k = torch.empty((L, B, Hkv, N, d), dtype=dt, device=device)
    v = torch.empty((L, B, Hkv, N, d), dtype=dt, device=device)
    host = {}
    kb = vb = None
    for layer in range(L):
        qh = gen.q(layer)
        kb, vb = gen.kv(layer, kb, vb)
        q[layer].copy_(to_torch(qh))
        k[layer].copy_(to_torch(kb))
        v[layer].copy_(to_torch(vb))
        if keep_layers is None or layer in keep_layers:
            if keep_units is None:
                host[layer] = (qh, kb.copy(), vb.copy())
            else:
                g = wl.group
                host[layer] = {(b, h): (qh[b, h * g:(h + 1) * g].copy(), kb[b, h].copy(), vb[b, h].copy())
                               for (b, h) in keep_units}
        if visit:
            visit(layer, qh, kb, vb)
        if progress:
            progress(layer)
    lens = torch.from_numpy(gen.seq_lens.copy()).to(device)
    return q, k, v, lens, host
