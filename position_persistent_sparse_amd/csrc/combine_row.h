// Merge of one (batch row, query head)'s split partials by one 64-lane wave (gfx950), used by the
// selection launch, which merges a selection layer's rows in extra workgroups beside the top-k work
// (the merge pass of the other layers, combine.hip, spreads each row over a workgroup instead).
//
// Each split s leaves m_s (max logit, log2 units), l_s = sum 2^(x - m_s) and o_s = sum
// 2^(x - m_s) V[row]. The softmax over the union of the splits is
//   out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),   M = max_s m_s,
// the attention equation of the TidalDecode review page (section 3, PPSA paragraph) evaluated in
// pieces. A row with no live position (M = -inf) outputs zeros.
#pragma once

#include <math.h>

#include "device_common.h"
#include "ppsa_internal.h"

namespace ppsa {
namespace merge {

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = bf16_round(v); }

// Value of lane L as a wave-uniform scalar.
__device__ __forceinline__ float lane_value(float x, int L) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), L));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f32<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f32<0x140>(x));  // row_mirror: every lane of a row holds the row's max
  return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)), fmaxf(lane_value(x, 32), lane_value(x, 48)));
}

__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);  // every lane of a row holds the row's sum
  return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

// Merges row `row` (lane = this thread's lane in its wave; the whole wave calls it). Every lane
// issues the partial-output loads of its dims for the first 16 splits before the max is known; the
// lanes then hold one split's (m, l) each, the max and the normaliser are wave reductions (DPP
// within rows of 16 lanes, then the four row results read as scalars), and each split's weight
// reaches the lanes as a scalar (v_readlane), not through the LDS crossbar. Summation order is
// fixed, so results are bitwise reproducible.
template <typename T, int D>
__device__ __forceinline__ void combine_row(const CombineArgs& a, int row, int lane) {
  constexpr int kDims = D / kWave;  // dims per lane: 1 (D = 64) or 2 (D = 128)
  constexpr int kB = 16;            // splits whose partial outputs are loaded per batch
  const int S = a.splits;
  const float* pm = a.part_m + (size_t)row * S;
  const float* pl = a.part_l + (size_t)row * S;
  const float* po = a.part_o + (size_t)row * S * D + lane;
  // First batch of partial outputs in flight before the max is known.
  float v[kB][kDims];
#pragma unroll
  for (int j = 0; j < kB; ++j)
#pragma unroll
    for (int e = 0; e < kDims; ++e) v[j][e] = j < S ? po[(size_t)j * D + kWave * e] : 0.0f;
  float mx = -INFINITY;
  for (int s = lane; s < S; s += kWave) mx = fmaxf(mx, pm[s]);
  mx = wave_max(mx);
  const float ms = mx == -INFINITY ? 0.0f : mx;
  float lsum = 0.0f, acc[kDims];
#pragma unroll
  for (int e = 0; e < kDims; ++e) acc[e] = 0.0f;
  for (int s0 = 0; s0 < S; s0 += kWave) {
    const int s = s0 + lane;
    float w = 0.0f;
    if (s < S) {
      w = __builtin_amdgcn_exp2f(pm[s] - ms);  // -inf (empty split) gives 0
      lsum += pl[s] * w;
    }
    for (int b0 = s0; b0 < min(S, s0 + kWave); b0 += kB) {
      if (b0 != 0) {
#pragma unroll
        for (int j = 0; j < kB; ++j)
#pragma unroll
          for (int e = 0; e < kDims; ++e) v[j][e] = b0 + j < S ? po[(size_t)(b0 + j) * D + kWave * e] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const float wj = lane_value(w, b0 - s0 + j);  // b0 - s0 is a multiple of 16: constant lanes per batch
#pragma unroll
        for (int e = 0; e < kDims; ++e) acc[e] += v[j][e] * wj;
      }
    }
  }
  lsum = wave_sum(lsum);
#pragma unroll
  for (int e = 0; e < kDims; ++e)
    store_out(reinterpret_cast<T*>(a.out) + (size_t)row * D + lane + kWave * e, lsum > 0.0f ? acc[e] / lsum : 0.0f);
}

}  // namespace merge
}  // namespace ppsa
