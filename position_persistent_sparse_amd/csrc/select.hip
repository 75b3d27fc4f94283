// Top-k token selection per (batch row, KV head) on gfx950.
//
// The selection step of the TidalDecode review page (section 2, solution
// overview; section 3 decode-step framework figure): keep the k positions
// with the highest attention score. Scores are float32; equal scores go to
// the lower position. Output is the selected positions in ascending order.
//
// Method: one 1024-thread workgroup per unit. Each score maps to an
// order-preserving 32-bit key (-0.0 folded onto +0.0), so ranking floats is
// ranking unsigned integers. An MSB-first radix select (four 8-bit digits,
// histograms in LDS) finds the exact key T of the k-th largest score and how
// many keys equal to T are still needed. A final ordered pass keeps every
// key > T plus the first `needed` keys == T in position order; a workgroup
// prefix sum over (greater, equal) flags gives each kept position its slot.
#include <math.h>

#include "device_common.h"
#include "ppsa_internal.h"

namespace ppsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kBins = 256;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kThreads) void select_topk_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scan_lds[kThreads / kWave + 1];
  __shared__ uint32_t found_digit, found_above;

  const int unit = blockIdx.x, tid = threadIdx.x;
  const int b = unit / a.kv_heads;
  const int n = min(max(a.seq_lens[b], 0), a.max_len);
  const int k_eff = min(a.topk, n);
  const float* s = a.scores + (size_t)unit * a.max_len;
  int32_t* out = a.idx + (size_t)unit * a.topk;

  if (k_eff == n) {  // everything live is selected (includes n == 0)
    for (int i = tid; i < a.topk; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }

  uint32_t prefix = 0u, mask = 0u;
  uint32_t remaining = (uint32_t)k_eff;  // how many still to take at or below the current prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t key = order_key(s[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (kBins - 1)], 1u);
    }
    __syncthreads();
    // Thread t looks at digit 255 - t; an inclusive scan gives the count of
    // keys whose digit is >= that digit.
    const uint32_t c = tid < kBins ? hist[kBins - 1 - tid] : 0u;
    uint32_t total;
    const uint32_t above = block_exclusive_scan<kThreads>(c, scan_lds, &total);
    if (tid < kBins && above < remaining && remaining <= above + c) {
      found_digit = (uint32_t)(kBins - 1 - tid);
      found_above = above;
    }
    __syncthreads();
    prefix |= found_digit << shift;
    mask |= (uint32_t)(kBins - 1) << shift;
    remaining -= found_above;
    __syncthreads();
  }
  const uint32_t thresh = prefix;
  const uint32_t needed_eq = remaining;  // >= 1

  uint32_t written = 0u, eq_seen = 0u;
  for (int c0 = 0; c0 < n; c0 += kThreads) {
    const int i = c0 + tid;
    uint32_t gt = 0u, eq = 0u;
    if (i < n) {
      const uint32_t key = order_key(s[i]);
      gt = key > thresh;
      eq = key == thresh;
    }
    uint32_t total;
    const uint32_t before = block_exclusive_scan<kThreads>(gt | (eq << 16), scan_lds, &total);
    const uint32_t gt_before = before & 0xffffu, eq_before = before >> 16;
    const uint32_t eq_room = needed_eq > eq_seen ? needed_eq - eq_seen : 0u;
    if (gt || (eq && eq_before < eq_room)) {
      const uint32_t slot = written + gt_before + min(eq_before, eq_room);
      out[slot] = i;
    }
    written += (total & 0xffffu) + min(total >> 16, eq_room);
    eq_seen += total >> 16;
  }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  select_topk_kernel<<<dim3(a.batch * a.kv_heads), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ppsa
