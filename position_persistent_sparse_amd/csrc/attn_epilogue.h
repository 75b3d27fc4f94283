// Output helpers shared by the attention kernels (gfx950).
//
// A split either writes the attention output itself (when the unit has a
// single split) or leaves its partial (m, l, o) per query head for the merge
// pass (combine.hip): m is the largest logit it saw (log2 units, -inf if
// none), l = sum 2^(x - m), o = sum 2^(x - m) V[row].
#pragma once

#include "device_common.h"
#include "ppsa_internal.h"

namespace ppsa {

__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = bf16_round(v); }

// Index of (b, query head of kv's group h, split s) in the partial arrays.
__device__ __forceinline__ size_t part_row(const AttnArgs& a, int b, int kv, int h, int s) {
  return ((size_t)b * a.q_heads + (size_t)kv * a.group + h) * a.splits + s;
}

}  // namespace ppsa
