// Measurement probes (gfx950): instrumentation that measures what this GPU allows, so that the
// attention kernels' times can be read against a floor measured here rather than only against the
// published 8 TB/s. Not part of the method; nothing on the decode path calls them.
//
//   read_probe_kernel    a plain read of a buffer: every workgroup streams one contiguous chunk
//                        with 16-byte loads, eight in flight per lane (the best shape found for a
//                        bandwidth-bound read), optionally with the nontemporal hint. The rate it
//                        reaches over a buffer much larger than the last-level cache is the
//                        achievable HBM read bandwidth.
//   empty_probe_kernel   a launch that does nothing: back-to-back launches of it give the fixed cost
//                        of one kernel on the stream.
//   gather_twin_kernel   the sparse layer's gather with its arithmetic removed: the same grid, waves,
//                        split plan, slot-entry reads and K/V row loads as attn_sparse_kernel
//                        (sparse_gather.h), the loaded words folded with XOR so that no load is
//                        dropped. The sparse kernel cannot be faster than this twin.
#include "device_common.h"
#include "ppsa_internal.h"
#include "sparse_gather.h"

namespace ppsa {
namespace {

using namespace mt;

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr uint32_t kNeverMatch = 0x9e3779b9u;  // a fold that equals this writes it out (keeps the loads)

template <bool NT>
__global__ __launch_bounds__(kReadThreads) void read_probe_kernel(const char* __restrict__ base, uint32_t chunk,
                                                                  int32_t* sink) {
  const char* p = base + (size_t)blockIdx.x * chunk + threadIdx.x * 16;
  uint32_t acc = 0;
  for (uint32_t off = 0; off < chunk; off += kReadThreads * 16 * kReadUnroll) {
    uint4 w[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) w[u] = load16<NT>(p, off + kReadThreads * 16 * u);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  if (acc == kNeverMatch) sink[0] = (int32_t)acc;
}

__global__ void empty_probe_kernel(int32_t* sink) {
  if (threadIdx.x == 0xFFFFFFFFu) sink[0] = 0;
}

template <int WAVES, bool STREAM>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(2))) void gather_twin_kernel(
    AttnArgs a, int32_t* sink) {
  const int S = a.splits;
  const int unit = blockIdx.x / S, split = blockIdx.x - unit * S;
  const int b = unit / a.kv_heads;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane / 16, n = lane % 16;
  const int32_t* ip = a.idx + (size_t)unit * a.kslots;
  const int slot0 = split * a.rows_per_split;
  const int nrows = max(min(a.rows_per_split, a.kslots - slot0), 0);
  const __amdgpu_buffer_rsrc_t r_idx = rsrc(ip + slot0, (uint32_t)nrows * 4u);
  const bool vec = a.idx_vec != 0;
  const int ntiles = (nrows + kTile - 1) / kTile;
  int raw[2][4];
  if (wave < ntiles) fetch_positions(raw, r_idx, wave * kTile, vec, g);
  const int n_live = min(max(a.seq_lens[b], 0), a.max_len);
  const char* kb = reinterpret_cast<const char*>(a.k) + (size_t)unit * a.max_len * kRowBytes;
  const char* vb = reinterpret_cast<const char*>(a.v) + (size_t)unit * a.max_len * kRowBytes;
  const int ntiles_live = n_live > 0 ? ntiles : 0;
  uint32_t acc = 0;
  for (int ti = wave; ti < ntiles_live; ti += WAVES) {
    Tile t;
    load_gathered<STREAM>(t, kb, vb, raw, ti * kTile, nrows, n_live, g, n);
    if (ti + WAVES < ntiles_live) fetch_positions(raw, r_idx, (ti + WAVES) * kTile, vec, g);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc ^= t.k[blk][i].x ^ t.k[blk][i].y ^ t.k[blk][i].z ^ t.k[blk][i].w ^ t.v[blk][i].x ^ t.v[blk][i].y ^
               t.v[blk][i].z ^ t.v[blk][i].w ^ t.valid;
  }
  if (acc == kNeverMatch) sink[0] = (int32_t)acc;
}

size_t read_probe_chunk(size_t bytes) {
  // Bytes per workgroup: 512 KiB for large reads (a 512 MiB to 4 GiB read streams fastest so), fewer for
  // small ones so that the grid still has 2048 workgroups; a power-of-two multiple of one loop trip
  // (kReadThreads x 16 bytes x kReadUnroll = 32 KiB) that divides the size.
  constexpr size_t kTrip = (size_t)kReadThreads * 16 * kReadUnroll;
  size_t chunk = kTrip;
  while (chunk * 2 <= ((size_t)512 << 10) && chunk * 2 * 2048 <= bytes && bytes % (chunk * 2) == 0) chunk *= 2;
  return chunk;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, bool nontemporal, int32_t* sink, hipStream_t stream) {
  constexpr size_t kTrip = (size_t)kReadThreads * 16 * kReadUnroll;
  if (bytes == 0 || bytes % kTrip != 0) return hipErrorInvalidValue;
  const size_t chunk = read_probe_chunk(bytes);
  const size_t groups = bytes / chunk;
  if (groups > 0x7fffffff) return hipErrorInvalidValue;
  const char* p = static_cast<const char*>(buf);
  if (nontemporal)
    read_probe_kernel<true><<<dim3((unsigned)groups), dim3(kReadThreads), 0, stream>>>(p, (uint32_t)chunk, sink);
  else
    read_probe_kernel<false><<<dim3((unsigned)groups), dim3(kReadThreads), 0, stream>>>(p, (uint32_t)chunk, sink);
  return hipGetLastError();
}

hipError_t launch_empty_probe(int groups, int threads, int32_t* sink, hipStream_t stream) {
  if (groups < 1 || threads < 1 || threads > 1024) return hipErrorInvalidValue;
  empty_probe_kernel<<<dim3(groups), dim3(threads), 0, stream>>>(sink);
  return hipGetLastError();
}

hipError_t launch_gather_twin(const AttnArgs& a, int32_t* sink, hipStream_t stream) {
  if (a.splits <= 0 || a.batch <= 0 || a.kv_heads <= 0) return hipSuccess;
  const dim3 grid(a.batch * a.kv_heads * a.splits);
  // The sparse kernel's launch shape (attn_sparse.hip): one split per unit runs eight waves with
  // ordinary loads, several splits run four waves with the nontemporal hint.
  if (a.splits == 1 && attn_sparse_waves(a) == 8)
    gather_twin_kernel<8, false><<<grid, dim3(8 * kWave), 0, stream>>>(a, sink);
  else if (a.splits == 1)
    gather_twin_kernel<4, false><<<grid, dim3(4 * kWave), 0, stream>>>(a, sink);
  else
    gather_twin_kernel<4, true><<<grid, dim3(4 * kWave), 0, stream>>>(a, sink);
  return hipGetLastError();
}

}  // namespace ppsa
