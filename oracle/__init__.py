"""Float64 CPU oracle of the PPSA decode step -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package. It shares no code with the HIP library.
"""
from .ppsa_oracle import (FULL, FULL_SELECT, SPARSE, append_kv, attend, coverage_budget, decode_layer, decode_step,
                          decode_steps, default_scale,
                          full_attention, logits, select_topk, selection_scores, softmax_weights,
                          shared_selection_scores, softmax_selection_scores, sparse_attention, widen)

__all__ = ["FULL", "FULL_SELECT", "SPARSE", "append_kv", "attend", "coverage_budget", "decode_layer", "decode_step",
           "decode_steps",
           "default_scale",
           "full_attention", "logits", "select_topk", "selection_scores", "softmax_weights",
           "shared_selection_scores", "softmax_selection_scores", "sparse_attention", "widen"]
