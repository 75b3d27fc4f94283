// Top-k token selection per (batch row, KV head) on gfx950.
//
// The selection step of the TidalDecode review page (section 2, solution
// overview; section 3 decode-step framework figure): keep the k positions
// with the highest attention score. Scores are float32; equal scores go to
// the lower position. Output is the selected positions in ascending order.
//
// Method: one 1024-thread workgroup per unit. Positions are read in rounds
// of 4096: in round r thread t holds positions 4096r + 4t .. 4096r + 4t + 3
// (one 16-byte load when the row is 16-byte aligned). Each score maps to an
// order-preserving 32-bit key (-0.0 folded onto +0.0), so ranking floats is
// ranking unsigned integers. An MSB-first radix select over digits of 11,
// 11 and 10 bits (histograms in LDS) finds the exact key T of the k-th
// largest score and how many keys equal to T are still needed. The output
// pass walks the rounds in position order; one workgroup prefix sum per
// round over packed (count > T, count == T) gives each thread its first
// output slot. Rows of up to kCachedRounds rounds keep their keys in
// registers; longer rows are re-read from memory on each pass.
#include <math.h>

#include "device_common.h"
#include "ppsa_internal.h"

namespace ppsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kPerRound = 4 * kThreads;
constexpr int kCachedRounds = 8;
constexpr int kMaxBins = 2048;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Pass {
  int shift, bins;
};
__device__ __forceinline__ Pass pass_of(int p) {
  return p == 0 ? Pass{21, 2048} : (p == 1 ? Pass{10, 2048} : Pass{0, 1024});
}

// Keys of positions p0..p0+3 (key 0 past n; callers mask with p < n).
__device__ __forceinline__ void load_keys(const float* s, int p0, int n, bool vec, uint32_t (&k)[4]) {
  if (vec && p0 + 3 < n) {
    const float4 f = *reinterpret_cast<const float4*>(s + p0);
    k[0] = order_key(f.x); k[1] = order_key(f.y); k[2] = order_key(f.z); k[3] = order_key(f.w);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) k[e] = p0 + e < n ? order_key(s[p0 + e]) : 0u;
  }
}

template <bool CACHED>
__global__ __launch_bounds__(kThreads) void select_topk_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kMaxBins];
  __shared__ uint32_t scan_lds[kThreads / kWave + 1];
  __shared__ uint32_t found_digit, found_above;

  const int unit = blockIdx.x, tid = threadIdx.x;
  const int b = unit / a.kv_heads;
  const int n = min(max(a.seq_lens[b], 0), a.max_len);
  const int k_eff = min(a.topk, n);
  const float* s = a.scores + (size_t)unit * a.max_len;
  int32_t* out = a.idx + (size_t)unit * a.topk;

  if (k_eff == n) {  // every live position is kept (includes n == 0)
    for (int i = tid; i < a.topk; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }

  // Every row starts 16-byte aligned when the base is and rows hold a multiple of 4 scores.
  const bool vec = (a.max_len % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) % 16) == 0;
  const int rounds = (n + kPerRound - 1) / kPerRound;
  uint32_t keys[CACHED ? kCachedRounds : 1][4];
  if constexpr (CACHED) {
#pragma unroll
    for (int r = 0; r < kCachedRounds; ++r)
      if (r < rounds) load_keys(s, r * kPerRound + 4 * tid, n, vec, keys[r]);
  }
  // Calls fn(round, keys of this thread's 4 positions in that round) for every
  // round in order; the round count is the same in every thread.
  auto for_each_round = [&](auto&& fn) {
    if constexpr (CACHED) {
#pragma unroll
      for (int rr = 0; rr < kCachedRounds; ++rr)
        if (rr < rounds) fn(rr, keys[rr]);
    } else {
      for (int rr = 0; rr < rounds; ++rr) {
        uint32_t kk[4];
        load_keys(s, rr * kPerRound + 4 * tid, n, vec, kk);
        fn(rr, kk);
      }
    }
  };

  uint32_t prefix = 0u, mask = 0u;
  uint32_t remaining = (uint32_t)k_eff;  // still to take among keys matching the prefix
#pragma unroll 1
  for (int p = 0; p < 3; ++p) {
    const Pass ps = pass_of(p);
    for (int i = tid; i < ps.bins; i += kThreads) hist[i] = 0u;
    __syncthreads();
    for_each_round([&](int rr, const uint32_t(&kk)[4]) {
      const int p0 = rr * kPerRound + 4 * tid;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (p0 + e < n && (kk[e] & mask) == prefix) atomicAdd(&hist[(kk[e] >> ps.shift) & (ps.bins - 1)], 1u);
    });
    __syncthreads();
    // Bins in descending digit order, bins/kThreads per thread; the exclusive
    // scan gives the number of keys with a larger digit.
    const int per_bin = ps.bins / kThreads;  // 2 or 1
    const int top = ps.bins - 1 - tid * per_bin;
    const uint32_t c[2] = {hist[top], per_bin == 2 ? hist[top - 1] : 0u};
    uint32_t total;
    uint32_t above = block_exclusive_scan<kThreads>(c[0] + c[1], scan_lds, &total);
    for (int j = 0; j < per_bin; ++j) {
      if (above < remaining && remaining <= above + c[j]) {
        found_digit = (uint32_t)(top - j);
        found_above = above;
      }
      above += c[j];
    }
    __syncthreads();
    prefix |= found_digit << ps.shift;
    mask |= (uint32_t)(ps.bins - 1) << ps.shift;
    remaining -= found_above;
    __syncthreads();
  }
  const uint32_t thresh = prefix;
  const uint32_t needed_eq = remaining;  // >= 1 keys equal to thresh, lowest positions first

  uint32_t written = 0u, eq_seen = 0u;
  for_each_round([&](int rr, const uint32_t(&kk)[4]) {
    const int p0 = rr * kPerRound + 4 * tid;
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (p0 + e < n) {
        gt += kk[e] > thresh;
        eq += kk[e] == thresh;
      }
    uint32_t total;
    const uint32_t before = block_exclusive_scan<kThreads>(gt | (eq << 16), scan_lds, &total);
    const uint32_t room = needed_eq > eq_seen ? needed_eq - eq_seen : 0u;  // equal keys still to take
    uint32_t eq_before = before >> 16;
    uint32_t slot = written + (before & 0xffffu) + min(eq_before, room);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (p0 + e < n) {
        const bool take = kk[e] > thresh || (kk[e] == thresh && eq_before < room);
        if (kk[e] == thresh) ++eq_before;
        if (take) out[slot++] = p0 + e;
      }
    written += (total & 0xffffu) + min(total >> 16, room);
    eq_seen += total >> 16;
  });
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  const dim3 grid(a.batch * a.kv_heads), block(kThreads);
  if (a.max_len <= kCachedRounds * kPerRound) select_topk_kernel<true><<<grid, block, 0, stream>>>(a);
  else select_topk_kernel<false><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ppsa
