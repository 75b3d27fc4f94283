// Merge of split attention partials (gfx950).
//
// Each split s of a (batch row, query head) leaves m_s (max logit, log2
// units), l_s = sum 2^(x - m_s) and o_s = sum 2^(x - m_s) V[row]. The
// softmax over the union of the splits is
//   out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),   M = max_s m_s,
// i.e. the attention equation of the TidalDecode review page (section 3,
// PPSA paragraph) evaluated in pieces. A row with no live position
// (M = -inf) outputs zeros.
//
// The pass moves about 0.5-1 % of a layer's bytes, so it is latency bound:
// one 256-thread workgroup per (b, query head); every thread issues all of
// its partial-output loads before waiting (threads t and t+128 take the
// even / odd splits of dim t%128), while wave 0 loads the (m, l) pairs and
// turns them into weights in LDS. Summation order is fixed, so results are
// bitwise reproducible.
#include <math.h>

#include "device_common.h"
#include "ppsa.h"
#include "ppsa_internal.h"

namespace ppsa {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 32;  // partial loads in flight per thread and trip

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = bf16_round(v); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  static_assert(kThreads % D == 0, "threads per dim must be whole");
  constexpr int kLanesPerDim = kThreads / D;  // 2 for D = 128, 4 for D = 64
  __shared__ float sm_w[kMaxSplitsPerUnit];
  __shared__ float sm_part[kThreads];
  __shared__ float sm_norm;

  const int row = blockIdx.x, tid = threadIdx.x;
  const int S = a.splits;
  const int d = tid % D, sub = tid / D;
  const float* pm = a.part_m + (size_t)row * S;
  const float* pl = a.part_l + (size_t)row * S;
  const float* po = a.part_o + (size_t)row * S * D + d;

  if (tid < kWave) {
    float mv[kMaxSplitsPerUnit / kWave], lv[kMaxSplitsPerUnit / kWave];
#pragma unroll
    for (int i = 0; i < kMaxSplitsPerUnit / kWave; ++i) {
      const int s = tid + i * kWave;
      mv[i] = s < S ? pm[s] : -INFINITY;
      lv[i] = s < S ? pl[s] : 0.0f;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxSplitsPerUnit / kWave; ++i) mx = fmaxf(mx, mv[i]);
    mx = wave_max(mx);
    const float ms = mx == -INFINITY ? 0.0f : mx;
    float ls = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxSplitsPerUnit / kWave; ++i) {
      const int s = tid + i * kWave;
      const float w = __builtin_amdgcn_exp2f(mv[i] - ms);  // -inf (empty split) gives 0
      if (s < S) sm_w[s] = w;
      ls += lv[i] * w;
    }
    ls = wave_sum(ls);
    if (tid == 0) sm_norm = ls;
  }

  // Splits sub, sub + kLanesPerDim, ... of dim d: the first batch of loads is
  // issued before the barrier that publishes the weights.
  constexpr int kStride = kBatch * kLanesPerDim;
  float v[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int s = sub + j * kLanesPerDim;
    v[j] = s < S ? po[(size_t)s * D] : 0.0f;
  }
  __syncthreads();
  float acc = 0.0f;
  for (int s0 = sub;;) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = s0 + j * kLanesPerDim;
      if (s < S) acc += v[j] * sm_w[s];
    }
    s0 += kStride;
    if (s0 >= S) break;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = s0 + j * kLanesPerDim;
      v[j] = s < S ? po[(size_t)s * D] : 0.0f;
    }
  }
  sm_part[tid] = acc;
  __syncthreads();
  if (sub == 0) {
    float tot = acc;
#pragma unroll
    for (int j = 1; j < kLanesPerDim; ++j) tot += sm_part[tid + j * D];
    const float L = sm_norm;
    store_out(reinterpret_cast<T*>(a.out) + (size_t)row * D + d, L > 0.0f ? tot / L : 0.0f);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int dtype, int head_dim, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.splits < 1 || a.splits > kMaxSplitsPerUnit) return hipErrorInvalidValue;
  const dim3 grid(a.rows), block(kThreads);
  if (dtype == PPSA_BF16) {
    if (head_dim == 128) combine_kernel<uint16_t, 128><<<grid, block, 0, stream>>>(a);
    else if (head_dim == 64) combine_kernel<uint16_t, 64><<<grid, block, 0, stream>>>(a);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 128) combine_kernel<float, 128><<<grid, block, 0, stream>>>(a);
    else if (head_dim == 64) combine_kernel<float, 64><<<grid, block, 0, stream>>>(a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ppsa
