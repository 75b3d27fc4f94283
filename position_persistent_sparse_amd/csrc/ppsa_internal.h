// Internal interfaces between the C-ABI front end (ppsa_api.hip) and the
// kernel translation units. Host and device code; gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ppsa {

enum AttnMode : int { MODE_FULL = 0, MODE_FULL_SCORES = 1, MODE_SPARSE = 2 };

// One launch of the split attention pass. Every pointer is a device pointer.
// The grid is (splits, Hkv, B); split s of unit (b, kv) covers slots
// [s*rows_per_split, (s+1)*rows_per_split) -- cache rows in full mode,
// entries of idx[b, kv, :] in sparse mode -- and writes one partial
// (m, l, o) per query head of the group:
//   m = max over its rows of the logit in log2 units (-inf if none),
//   l = sum 2^(logit - m), o[:] = sum 2^(logit - m) V[row, :].
struct AttnArgs {
  const void* q;            // [B, Hq, D]
  const void* k;            // [B, Hkv, Nmax, D]
  const void* v;            // [B, Hkv, Nmax, D]
  const int32_t* seq_lens;  // [B]
  const int32_t* idx;       // sparse: [B, Hkv, kslots]
  float* scores;            // full+scores: [B, Hkv, Nmax]
  float* part_m;            // [B, Hq, splits]
  float* part_l;            // [B, Hq, splits]
  float* part_o;            // [B, Hq, splits, D]
  int32_t batch, q_heads, kv_heads, group, max_len;
  int32_t kslots;           // sparse: entries per unit
  int32_t splits, rows_per_split;
  float scale;              // logit scale (natural units)
  float scale_log2;         // scale * log2(e)
};

// Merge the partials of every (b, hq) into out[b, hq, :] (dtype of the cache).
struct CombineArgs {
  const float* part_m;
  const float* part_l;
  const float* part_o;
  void* out;                // [B, Hq, D]
  int32_t rows;             // B * Hq
  int32_t splits;
};

struct SelectArgs {
  const float* scores;      // [B, Hkv, Nmax]
  const int32_t* seq_lens;  // [B]
  int32_t* idx;             // [B, Hkv, topk]
  int32_t batch, kv_heads, max_len, topk;
};

// Rows one attention workgroup covers per loop trip (split sizes are multiples).
int attn_rows_granule(int dtype, int head_dim);
// Largest split (in idx entries) the sparse mode stages in LDS.
int attn_max_sparse_rows();
// Largest group size the attention kernels take.
constexpr int kMaxGroup = 16;

hipError_t launch_attn(const AttnArgs& a, int mode, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

}  // namespace ppsa
