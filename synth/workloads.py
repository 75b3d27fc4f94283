"""Decode-step workload shapes for the PPSA benchmarks and tests.

Each workload is a synthetic stand-in for one of the model/context settings
that the TidalDecode paper-review page evaluates (section 5, "Experimental
results": LLaMA-2-7B / LongChat at 10K-100K context, LLaMA-3-8B with token
budget 4096, LLaMA-3-70B at 10K with budget 256). No weights or datasets are
used: inputs come from the seeded generator in this package.

The schedule follows the decode-step overview figure of the same page
(section 3, "Overall framework"): every layer before the first selection
layer runs full attention, each selection layer runs full attention plus
top-k selection, every other layer runs sparse attention over the most
recent selection.
"""
from __future__ import annotations

from dataclasses import dataclass, field

FULL, FULL_SELECT, SPARSE = "F", "X", "S"


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    max_len: int
    topk: int
    dtype: str  # "f32" or "bf16": q, K, V and the attention output
    select_layers: tuple
    seed: int
    min_len: int = 0  # < max_len means ragged lengths, uniform in [min_len, max_len]
    key_bias: float = 3.0
    q_bias: float = 1.0
    sinks: int = field(default=4)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def ragged(self) -> bool:
        return 0 < self.min_len < self.max_len

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def heavy_random(self) -> int:
        """Random heavy-hitter positions per (batch, KV head): half the budget."""
        return self.topk // 2

    def schedule(self) -> list:
        return schedule_for(self.layers, self.select_layers)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def schedule_for(layers: int, select_layers) -> list:
    """Per-layer kinds: F before the first selection, X at selections, S after."""
    sel = sorted(set(int(s) for s in select_layers))
    out = []
    seen = False
    for layer in range(layers):
        if layer in sel:
            out.append(FULL_SELECT)
            seen = True
        elif not seen:
            out.append(FULL)
        else:
            out.append(SPARSE)
    return out


WORKLOADS = {
    "tiny-f32": Workload("tiny-f32", layers=8, batch=1, q_heads=8, kv_heads=8, head_dim=64, max_len=1024,
                         topk=64, dtype="f32", select_layers=(2, 4), seed=1001),
    "llama2-7b-10k": Workload("llama2-7b-10k", layers=32, batch=1, q_heads=32, kv_heads=32, head_dim=128,
                              max_len=10240, topk=512, dtype="bf16", select_layers=(2, 7), seed=1002),
    "llama3-8b-gqa-32k": Workload("llama3-8b-gqa-32k", layers=32, batch=4, q_heads=32, kv_heads=8,
                                  head_dim=128, max_len=32768, topk=4096, dtype="bf16",
                                  select_layers=(2, 14), seed=1003),
    "llama2-7b-100k": Workload("llama2-7b-100k", layers=32, batch=1, q_heads=32, kv_heads=32, head_dim=128,
                               max_len=102400, topk=2048, dtype="bf16", select_layers=(2, 7), seed=1004),
    "llama3-70b-ragged-10k": Workload("llama3-70b-ragged-10k", layers=80, batch=8, q_heads=64, kv_heads=8,
                                      head_dim=128, max_len=10240, min_len=8192, topk=256, dtype="bf16",
                                      select_layers=(2, 14), seed=1005),
    # One GPU's share of the two GQA shapes under 8-way sharding over KV heads (every GPU holds one KV
    # head and its query heads for the whole batch; attention and selection need no exchange). Same
    # seed as the whole shape: the inputs and lengths are exactly its KV head 0 and query heads 0..g-1.
    "llama3-8b-gqa-32k-tp8": Workload("llama3-8b-gqa-32k-tp8", layers=32, batch=4, q_heads=4, kv_heads=1,
                                      head_dim=128, max_len=32768, topk=4096, dtype="bf16",
                                      select_layers=(2, 14), seed=1003),
    "llama3-70b-ragged-10k-tp8": Workload("llama3-70b-ragged-10k-tp8", layers=80, batch=8, q_heads=8, kv_heads=1,
                                          head_dim=128, max_len=10240, min_len=8192, topk=256, dtype="bf16",
                                          select_layers=(2, 14), seed=1005),
}

# The workload the benchmark times by default: the LLaMA-3-8B GQA shape at 32K.
BENCH_WORKLOAD = "llama3-8b-gqa-32k"


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, elem_bytes: int) -> int:
    """Bytes of a K plus V cache: layers x heads x dim x tokens x element x 2."""
    return layers * kv_heads * head_dim * seq_len * elem_bytes * 2


def layer_kv_bytes(wl: Workload, kind: str, seq_lens) -> int:
    """K+V bytes one layer must read: every live row (F, X) or k rows per (b, h) (S)."""
    row = wl.head_dim * wl.elem_bytes
    if kind == SPARSE:
        rows = sum(min(wl.topk, int(n)) for n in seq_lens) * wl.kv_heads
    else:
        rows = sum(int(n) for n in seq_lens) * wl.kv_heads
    return 2 * rows * row


def step_kv_bytes(wl: Workload, seq_lens) -> int:
    """Algorithmic K+V bytes of one decode step over the whole schedule."""
    return sum(layer_kv_bytes(wl, kind, seq_lens) for kind in wl.schedule())
