// Softmax-weight selection scores (gfx950), the selection variant in which a
// GQA group ranks a position by the sum over its query heads of the softmax
// weight each head gives it, rather than by the sum of raw logits.
//
// Input: every query head's logit of every live row (log2 units), written by
// the full attention pass of the same layer. The weight of row n for head h
// is 2^(x_n - M) / L with M the head's largest logit and L = sum 2^(x - M)
// over the live rows: the attention equation's softmax (TidalDecode review
// page, section 3, PPSA paragraph). Two launches:
//  1. one workgroup per (batch row, query head) finds M, then L, from the
//     stored logits (per-thread partial sums over strided rows, then a tree
//     across the workgroup, so the float32 sum of N terms carries an error of
//     about (N/256 + 8) units in the last place at most);
//  2. one thread per (batch row, KV head, position) sums the group's weights
//     in head order.
// The normaliser is recomputed here rather than taken from the attention
// pass, whose normaliser sums the bf16-rounded weights of its PV product.
#include <math.h>

#include "device_common.h"
#include "ppsa_internal.h"

namespace ppsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

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

__global__ __launch_bounds__(kThreads) void softmax_stats_kernel(SoftmaxScoreArgs a) {
  __shared__ float sm[kWaves];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int b = row / a.q_heads;
  const int n_live = min(max(a.seq_lens[b], 0), a.max_len);
  const float* x = a.head_logits + (size_t)row * a.max_len;
  float m = -INFINITY;
  for (int i = tid; i < n_live; i += kThreads) m = fmaxf(m, x[i]);
  m = wave_max(m);
  if (lane == 0) sm[wave] = m;
  __syncthreads();
  m = sm[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, sm[w]);
  __syncthreads();
  float l = 0.0f;
  for (int i = tid; i < n_live; i += kThreads) l += __builtin_amdgcn_exp2f(x[i] - m);
  l = wave_sum(l);
  if (lane == 0) sm[wave] = l;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += sm[w];
    a.stat_m[row] = m;
    a.stat_l[row] = tot;
  }
}

__global__ __launch_bounds__(kThreads) void softmax_scores_kernel(SoftmaxScoreArgs a) {
  const int kv = blockIdx.y, b = blockIdx.z;
  const int pos = blockIdx.x * kThreads + threadIdx.x;
  const int n_live = min(max(a.seq_lens[b], 0), a.max_len);
  if (pos >= n_live) return;
  const int group = a.q_heads / a.kv_heads;
  float s = 0.0f;
  for (int h = 0; h < group; ++h) {
    const size_t row = (size_t)b * a.q_heads + (size_t)kv * group + h;
    s += __builtin_amdgcn_exp2f(a.head_logits[row * a.max_len + pos] - a.stat_m[row]) / a.stat_l[row];
  }
  a.scores[((size_t)b * a.kv_heads + kv) * a.max_len + pos] = s;
}

}  // namespace

hipError_t launch_softmax_scores(const SoftmaxScoreArgs& a, hipStream_t stream) {
  if (a.batch <= 0 || a.max_len <= 0) return hipSuccess;
  if (a.kv_heads > 65535 || a.batch > 65535) return hipErrorInvalidValue;
  softmax_stats_kernel<<<dim3(a.batch * a.q_heads), dim3(kThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((a.max_len + kThreads - 1) / kThreads, a.kv_heads, a.batch);
  softmax_scores_kernel<<<grid, dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ppsa
