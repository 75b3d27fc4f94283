// Coverage budget (gfx950): how many positions a unit keeps when the
// lowest-mass tail is pruned until its mass exceeds a threshold tau, instead
// of keeping a fixed k. The page on token-sparse attention (its dynamic
// token coverage paragraph) describes this budget: sort the positions by
// importance ascending and prune from the bottom until the pruned mass
// passes tau. Here the importance is a position's mass m_n = (the group's
// softmax-weight sum at n) / group, so a unit's masses total about 1.
//
// One 1024-thread workgroup per (batch row, KV head). Masses become 24-bit
// fixed point (m * 2^24, rounded in float32; a position's mass is a function
// of its score alone) so that every sum is an exact integer and the result
// does not depend on the order of the atomic adds. The crossing
// point -- the smallest count p of lowest-mass positions whose mass sum
// exceeds T = floor(tau * total) -- is found by three radix digits of the
// order-preserving 32-bit key of the score (11/11/10 bits), each pass
// building per-bin counts and mass sums in LDS and walking the bins upward;
// equal keys carry equal masses, so the count taken among the crossing key's
// copies is arithmetic. unit_k = n - p (0 when the whole mass is at most T).
#include <math.h>

#include "device_common.h"
#include "ppsa_internal.h"

namespace ppsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kBins = 2048;
constexpr float kFix = 16777216.0f;  // 2^24
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t fixed_mass(float score, float fix_per_group) {
  const float m = score * fix_per_group;  // masses are at most 1, so this stays below 2^24 + rounding
  return m > 0.0f ? (uint32_t)(m + 0.5f) : 0u;
}

// Wave 0: with per-bin masses and counts complete, finds the bin at which the running mass (bins in
// ascending order, starting from `base`) first exceeds t, and the mass and count of the bins below it.
template <int BINS>
__device__ void find_crossing(const unsigned long long* mass, const uint32_t* cnt, unsigned long long base,
                              unsigned long long t, uint32_t* bin, unsigned long long* mass_below,
                              uint32_t* count_below) {
  constexpr int per = BINS / kWave;  // bins per lane, in order
  const int lane = threadIdx.x % kWave;
  unsigned long long msum = 0ull;
  uint32_t csum = 0u;
  for (int i = 0; i < per; ++i) {
    msum += mass[lane * per + i];
    csum += cnt[lane * per + i];
  }
  // Exclusive prefix of the lane totals.
  unsigned long long mpre = msum;
  uint32_t cpre = csum;
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned long long mo = __shfl_up(mpre, off);
    const uint32_t co = __shfl_up(cpre, off);
    if (lane >= off) {
      mpre += mo;
      cpre += co;
    }
  }
  unsigned long long m = base + mpre - msum;
  uint32_t c = cpre - csum;
  for (int i = 0; i < per; ++i) {
    const unsigned long long mi = mass[lane * per + i];
    if (m <= t && t < m + mi) {  // exactly one bin satisfies this when the crossing exists
      *bin = (uint32_t)(lane * per + i);
      *mass_below = m - base;
      *count_below = c;
    }
    m += mi;
    c += cnt[lane * per + i];
  }
}

__global__ __launch_bounds__(kThreads) void coverage_kernel(CoverageArgs a) {
  __shared__ unsigned long long hm[kBins];
  __shared__ uint32_t hc[kBins];
  __shared__ unsigned long long s_part[kWaves], s_mb;
  __shared__ uint32_t s_bin, s_cb;

  const int unit = blockIdx.x, tid = threadIdx.x;
  const int b = unit / a.kv_heads;
  const int n = min(max(a.seq_lens[b], 0), a.max_len);
  const float* s = a.scores + (size_t)unit * a.max_len;
  const float fix_per_group = kFix / (float)a.group;

  // Total mass: per-thread sums, then the waves' sums.
  unsigned long long part = 0ull;
  for (int i = tid; i < n; i += kThreads) part += fixed_mass(s[i], fix_per_group);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) part += __shfl_xor(part, off);
  if (tid % kWave == 0) s_part[tid / kWave] = part;
  __syncthreads();
  unsigned long long total = 0ull;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) total += s_part[w];
  const unsigned long long t = (unsigned long long)((double)a.tau * (double)total);
  if (n == 0 || t >= total) {  // nothing to prune past the threshold: every position goes
    if (tid == 0) a.unit_k[unit] = 0;
    return;
  }

  uint32_t prefix = 0u, mask = 0u, count_below = 0u;
  unsigned long long mass_below = 0ull;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int i = tid; i < kBins; i += kThreads) {
      hm[i] = 0ull;
      hc[i] = 0u;
    }
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const float v = s[i];
      const uint32_t key = order_key(v);
      if ((key & mask) == prefix) {
        const uint32_t d = (key >> shift) & dmask;
        atomicAdd(&hm[d], (unsigned long long)fixed_mass(v, fix_per_group));
        atomicAdd(&hc[d], 1u);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      if (pass < 2) find_crossing<2048>(hm, hc, mass_below, t, &s_bin, &s_mb, &s_cb);
      else find_crossing<1024>(hm, hc, mass_below, t, &s_bin, &s_mb, &s_cb);
    }
    __syncthreads();
    prefix |= s_bin << shift;
    mask |= dmask << shift;
    mass_below += s_mb;
    count_below += s_cb;
    __syncthreads();
  }
  if (tid == 0) {
    // prefix is the crossing key; its copies each carry mass m_star > 0.
    const unsigned long long m_star =
        fixed_mass(__uint_as_float((prefix & 0x80000000u) ? (prefix & 0x7FFFFFFFu) : ~prefix), fix_per_group);
    const unsigned long long e = m_star > 0ull ? (t - mass_below) / m_star + 1ull : 1ull;
    const long long p = (long long)count_below + (long long)e;
    a.unit_k[unit] = (int32_t)max(0ll, (long long)n - p);
  }
}

}  // namespace

hipError_t launch_coverage(const CoverageArgs& a, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  if (a.group < 1) return hipErrorInvalidValue;
  coverage_kernel<<<dim3(a.batch * a.kv_heads), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ppsa
