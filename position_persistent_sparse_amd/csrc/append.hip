// Append of one decode token's K and V rows to the cache (gfx950).
//
// Decoding produces one token at a time and its K and V rows join the cache
// before the next attention (TidalDecode review page, section 2, problem
// definition). Two launches on one stream:
//  1. one workgroup per (batch row b, layer): reads n = seq_lens[b] and
//     copies the token's rows of every KV head to position n, in 16-byte
//     pieces (a layer's rows of one batch row are a few KiB, so the copy
//     spreads over B x L workgroups rather than a few CUs);
//  2. one workgroup stores the new lengths, after every copy has read the
//     old ones (the kernel boundary orders the two), and adds the number of
//     full batch rows to the caller's overflow counter when one is given.
// A full row (n = Nmax) takes nothing.
#include "device_common.h"
#include "ppsa_internal.h"

namespace ppsa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void append_rows_kernel(AppendArgs a) {
  const int b = blockIdx.x, layer = blockIdx.y, tid = threadIdx.x;
  const int n = min(max(a.seq_lens[b], 0), a.max_len);
  if (n >= a.max_len) return;
  const int pieces = a.row_bytes / 16;  // 16-byte pieces per row
  const uint4* __restrict__ kn = reinterpret_cast<const uint4*>(a.k_new);
  const uint4* __restrict__ vn = reinterpret_cast<const uint4*>(a.v_new);
  uint4* __restrict__ kc = reinterpret_cast<uint4*>(a.k_cache);
  uint4* __restrict__ vc = reinterpret_cast<uint4*>(a.v_cache);
  for (int i = tid; i < a.kv_heads * pieces; i += kThreads) {
    const int h = i / pieces, c = i % pieces;
    const size_t src_row = ((size_t)layer * a.batch + b) * a.kv_heads + h;
    const size_t dst = (src_row * (size_t)a.max_len + n) * pieces + c;
    const uint4 kv = kn[src_row * pieces + c];
    const uint4 vv = vn[src_row * pieces + c];
    kc[dst] = kv;
    vc[dst] = vv;
  }
}

__global__ __launch_bounds__(kThreads) void append_lengths_kernel(AppendArgs a) {
  __shared__ int sm_full;
  if (threadIdx.x == 0) sm_full = 0;
  __syncthreads();
  int full = 0;
  for (int b = threadIdx.x; b < a.batch; b += kThreads) {
    const int n = max(a.seq_lens[b], 0);
    full += n >= a.max_len;
    a.seq_lens[b] = min(n + 1, a.max_len);
  }
  if (full) atomicAdd(&sm_full, full);
  __syncthreads();
  if (threadIdx.x == 0 && a.overflow != nullptr && sm_full != 0) *a.overflow += sm_full;
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.batch <= 0 || a.layers <= 0) return hipSuccess;
  if (a.row_bytes % 16 != 0 || a.layers > 65535) return hipErrorInvalidValue;
  append_rows_kernel<<<dim3(a.batch, a.layers), dim3(kThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  append_lengths_kernel<<<dim3(1), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ppsa
