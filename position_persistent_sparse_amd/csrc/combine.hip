// Merge pass of split attention partials (gfx950): one 256-thread workgroup per (batch row, query
// head).
//
// Each split s leaves m_s (max logit, log2 units), l_s = sum 2^(x - m_s) and o_s = sum 2^(x - m_s)
// V[row]; the softmax over the union of the splits is
//   out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),   M = max_s m_s,
// the attention equation of the TidalDecode review page (section 3, PPSA paragraph) evaluated in
// pieces. A row with no live position (M = -inf) outputs zeros.
//
// The pass moves about 1 % of a layer's bytes, so its cost is latency: thread (sg, dq) takes the
// four dims 4 dq .. 4 dq + 3 of the splits sg, sg + SG, sg + 2 SG, ... and issues all their loads
// (m, l and 16 bytes of o per split, eight splits per batch) before it uses any, folds them into a
// running (max, sum, weighted o), and the SG split groups then meet once in LDS. One memory round
// trip and one barrier per row (the wave-per-row merge the selection launch runs, combine_row.h,
// waits on its max before loading the normalisers; as a launch of its own this workgroup form took
// about 0.5 us less per sparse layer at the LLaMA-3-8B 32K and LLaMA-2-7B 100K shapes). The
// summation order is fixed, so results are bitwise reproducible.
#include <math.h>

#include "device_common.h"
#include "ppsa.h"
#include "ppsa_internal.h"

namespace ppsa {
namespace {

constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 8;  // splits per thread whose loads are in flight together

__device__ __forceinline__ void store4(float* p, float4 r, float l) {
  *reinterpret_cast<float4*>(p) = make_float4(r.x / l, r.y / l, r.z / l, r.w / l);
}
__device__ __forceinline__ void store4(uint16_t* p, float4 r, float l) {
  const uint32_t lo = (uint32_t)bf16_round(r.x / l) | ((uint32_t)bf16_round(r.y / l) << 16);
  const uint32_t hi = (uint32_t)bf16_round(r.z / l) | ((uint32_t)bf16_round(r.w / l) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

__device__ __forceinline__ void axpy4(float4& acc, const float4 v, float w) {
  acc.x += v.x * w;
  acc.y += v.y * w;
  acc.z += v.z * w;
  acc.w += v.w * w;
}

template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(CombineArgs a) {
  constexpr int kQ = D / 4;                 // dim quads per row
  constexpr int kSG = kMergeThreads / kQ;   // split groups: 8 (D = 128) or 16 (D = 64)
  __shared__ float sm_m[kSG], sm_l[kSG];
  __shared__ float4 sm_o[kSG][kQ];
  const int row = blockIdx.x, t = threadIdx.x;
  const int dq = t % kQ, sg = t / kQ;
  const int S = a.splits;
  const float* pm = a.part_m + (size_t)row * S;
  const float* pl = a.part_l + (size_t)row * S;
  const float4* po = reinterpret_cast<const float4*>(a.part_o + (size_t)row * S * D) + dq;

  float M = -INFINITY, L = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = sg; s0 < S; s0 += kSG * kMergeBatch) {
    float m[kMergeBatch], l[kMergeBatch];
    float4 v[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int s = s0 + j * kSG;
      const bool ok = s < S;
      m[j] = ok ? pm[s] : -INFINITY;
      l[j] = ok ? pl[s] : 0.0f;
      v[j] = ok ? po[(size_t)s * kQ] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) mb = fmaxf(mb, m[j]);
    const float ms = mb == -INFINITY ? 0.0f : mb;  // no live row yet: every weight below is 0
    const float c = __builtin_amdgcn_exp2f(M - ms);
    L *= c;
    o.x *= c;
    o.y *= c;
    o.z *= c;
    o.w *= c;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const float w = __builtin_amdgcn_exp2f(m[j] - ms);
      L += l[j] * w;
      axpy4(o, v[j], w);
    }
    M = mb;
  }
  if (dq == 0) {
    sm_m[sg] = M;
    sm_l[sg] = L;
  }
  sm_o[sg][dq] = o;
  __syncthreads();
  if (t >= kQ) return;
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSG; ++i) mx = fmaxf(mx, sm_m[i]);
  const float ms = mx == -INFINITY ? 0.0f : mx;
  float lt = 0.0f;
  float4 r = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int i = 0; i < kSG; ++i) {
    const float w = __builtin_amdgcn_exp2f(sm_m[i] - ms);
    lt += sm_l[i] * w;
    axpy4(r, sm_o[i][t], w);
  }
  T* out = reinterpret_cast<T*>(a.out) + (size_t)row * D + 4 * t;
  if (lt > 0.0f)
    store4(out, r, lt);
  else
    store4(out, make_float4(0.0f, 0.0f, 0.0f, 0.0f), 1.0f);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int dtype, int head_dim, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.splits < 1 || a.splits > kMaxSplitsPerUnit) return hipErrorInvalidValue;
  const dim3 grid(a.rows), block(kMergeThreads);
  if (dtype == PPSA_BF16) {
    if (head_dim == 128) merge_kernel<uint16_t, 128><<<grid, block, 0, stream>>>(a);
    else if (head_dim == 64) merge_kernel<uint16_t, 64><<<grid, block, 0, stream>>>(a);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 128) merge_kernel<float, 128><<<grid, block, 0, stream>>>(a);
    else if (head_dim == 64) merge_kernel<float, 64><<<grid, block, 0, stream>>>(a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ppsa
