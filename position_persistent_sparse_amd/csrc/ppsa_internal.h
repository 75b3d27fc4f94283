// Internal interfaces between the C-ABI front end (ppsa_api.hip) and the
// kernel translation units. Host and device code; gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ppsa {

// MODE_FULL_HEADS: full attention writing the group-summed scores and also every query head's
// logit (log2 units) of every live row, for the softmax-weight selection variant.
enum AttnMode : int { MODE_FULL = 0, MODE_FULL_SCORES = 1, MODE_SPARSE = 2, MODE_FULL_HEADS = 3 };

// One launch of the split attention pass. Every pointer is a device pointer.
// The grid is (splits, Hkv, B); split s of unit (b, kv) covers slots
// [s*rows_per_split, (s+1)*rows_per_split) -- cache rows in full mode,
// entries of idx[b, kv, :] in sparse mode. With one split the workgroup
// writes out[b, hq, :] itself; otherwise each split leaves a partial
// (m, l, o) per query head of the group:
//   m = max over its rows of the logit in log2 units (-inf if none),
//   l = sum 2^(logit - m), o[:] = sum 2^(logit - m) V[row, :],
// and the merge pass (launch_combine) turns them into out.
struct AttnArgs {
  const void* q;            // [B, Hq, D]
  const void* k;            // [B, Hkv, Nmax, D]
  const void* v;            // [B, Hkv, Nmax, D]
  const int32_t* seq_lens;  // [B]
  const int32_t* idx;       // sparse: [B, Hkv, kslots]
  float* scores;            // full+scores: [B, Hkv, Nmax]
  void* out;                // [B, Hq, D], dtype of the cache
  float* part_m;            // [B, Hq, splits]
  float* part_l;            // [B, Hq, splits]
  float* part_o;            // [B, Hq, splits, D]
  float* head_logits;       // MODE_FULL_HEADS: [B, Hq, max_len], logit * scale * log2(e) per live row
  int32_t batch, q_heads, kv_heads, group, max_len;
  int32_t kslots;           // sparse: entries per unit
  int32_t splits, rows_per_split;
  float scale;              // logit scale (natural units)
  float scale_log2;         // scale * log2(e)
  int32_t idx_vec;          // sparse: 1 when idx rows may be read 16 bytes at a time (kslots % 4 == 0, 16-byte aligned)
};

// Merge the partials of every (b, hq) into out[b, hq, :] (dtype of the cache).
struct CombineArgs {
  const float* part_m;      // [rows, splits]
  const float* part_l;      // [rows, splits]
  const float* part_o;      // [rows, splits, D]
  void* out;                // [rows, D]
  int32_t rows;             // B * Hq
  int32_t splits;           // 1 .. kMaxSplitsPerUnit
  int32_t bf16;             // output format when merged inside the selection launch: 1 bf16, 0 float32
  int32_t head_dim;         // 64 or 128 (same)
};

// Softmax-weight selection scores (scores.hip): per (b, hq), M = max over live n of head_logits and
// L = sum 2^(x - M) (stats pass); then scores[b, kv, n] = sum over the group's heads of 2^(x - M) / L.
struct SoftmaxScoreArgs {
  const float* head_logits;  // [B, Hq, max_len]
  float* stat_m;             // [B, Hq] workspace
  float* stat_l;             // [B, Hq] workspace
  const int32_t* seq_lens;   // [B]
  float* scores;             // [B, Hkv, max_len]
  int32_t batch, q_heads, kv_heads, max_len;
};
hipError_t launch_softmax_scores(const SoftmaxScoreArgs& a, hipStream_t stream);

// Stages of a selection (per (batch row, KV head) sets only; 0 for the others):
//   0  one launch: each unit's whole row;
//   1  each unit's row cut into `nchunks` chunks of `chunk` positions, one workgroup each: the top
//      min(topk, live positions of the chunk) of the chunk go, as (score, position) in position
//      order, to the unit's candidate row at the offset of the chunk (the kept counts of the chunks
//      before it, a closed form of the live length);
//   2  each unit's candidate row (its live length is the sum of the chunks' kept counts): top-k,
//      the positions read back from the candidate row.
// Every position of the global top-k is in its chunk's top-k (fewer than k positions of the whole
// row rank above it, hence fewer than k of its chunk), and candidates sit in position order, so
// stage 2 over the candidates picks exactly the set stage 0 picks over the row, ties included.
struct SelectArgs {
  const float* scores;      // [B, Hkv, Nmax]
  const int32_t* seq_lens;  // [B]
  int32_t* idx;             // [B, Hkv, topk]
  int32_t batch, kv_heads, max_len, topk;
  int32_t shared;           // 1: one set per batch row over the sum of its KV heads' scores
  const int32_t* unit_k;    // optional [units]: per-unit budget (capped by topk)
  int32_t stage;            // 0, 1 or 2 (above)
  int32_t chunk, nchunks;   // stages 1 and 2: chunk length (a multiple of 4) and chunks per row
  int32_t cand_stride;      // stages 1 and 2: candidate row length per unit (>= nchunks * topk, multiple of 4)
  float* cand_score;        // stages 1 and 2: [B * Hkv, cand_stride]
  int32_t* cand_pos;        // stages 1 and 2: [B * Hkv, cand_stride]
};
// Two-stage plan for rows of max_len positions and top-k (per-KV-head sets): chunk length and count,
// or false when one launch is used (rows of at most two super-rounds of 32768 positions, or a
// candidate row longer than one).
bool select_two_stage(int max_len, int topk, int* chunk, int* nchunks);

// Coverage budget (coverage.hip): per (b, kv) unit, with masses m_n = scores[unit, n] / group (the
// group's softmax-weight sums, total ~1), the number of positions kept once the lowest-mass tail is
// pruned until its mass exceeds tau: unit_k = n_live - p, p the smallest count of lowest-mass
// positions (ascending mass, equal masses from the higher position) whose mass sum exceeds tau.
struct CoverageArgs {
  const float* scores;      // [B, Hkv, max_len]
  const int32_t* seq_lens;  // [B]
  int32_t* unit_k;          // [B * Hkv]
  int32_t batch, kv_heads, max_len, group;
  float tau;
};
hipError_t launch_coverage(const CoverageArgs& a, hipStream_t stream);

// Vector-ALU attention pass (any supported dtype / head_dim / group).
// Rows one workgroup covers per loop trip, and the largest sparse split
// (idx entries staged in LDS).
int attn_rows_granule(int dtype, int head_dim);
int attn_max_sparse_rows();

// Matrix-core full-attention pass (bf16, head_dim 128, group <= 16); sparse layers use launch_attn_sparse.
bool attn_mfma_supported(int dtype, int head_dim, int group);
int attn_mfma_rows_granule();
int attn_mfma_max_score_rows(int group);  // rows of one full-layer split (its scores are staged in LDS)
hipError_t launch_attn_mfma(const AttnArgs& a, int mode, hipStream_t stream);
// Sparse layer on the matrix cores (attn_sparse.hip, same contract as MODE_SPARSE): partials for
// launch_combine, or the output itself when the unit has one split.
hipError_t launch_attn_sparse(const AttnArgs& a, hipStream_t stream);
// Waves per workgroup of that launch.
int attn_sparse_waves(const AttnArgs& a);

// Measurement probes (probe.hip; instrumentation, not the method): a plain read of `bytes` (a
// multiple of 32 KiB), an empty kernel, and the sparse launch's load-only twin.
hipError_t launch_read_probe(const void* buf, size_t bytes, bool nontemporal, int32_t* sink, hipStream_t stream);
hipError_t launch_empty_probe(int groups, int threads, int32_t* sink, hipStream_t stream);
hipError_t launch_gather_twin(const AttnArgs& a, int32_t* sink, hipStream_t stream);
// Largest group size the attention kernels take.
constexpr int kMaxGroup = 16;
// Most splits one unit may be cut into.
constexpr int kMaxSplitsPerUnit = 256;

// Append of one token's K/V rows (append.hip): rows [L, B, Hkv] of row_bytes each go to position
// seq_lens[b] of the caches [L, B, Hkv, max_len]; seq_lens[b] then grows by one (capped at max_len).
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  int32_t* seq_lens;
  int32_t* overflow;        // or null: incremented by the number of full rows (tokens not stored)
  int32_t layers, batch, kv_heads, max_len, row_bytes;
};

hipError_t launch_attn(const AttnArgs& a, int mode, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);
// One launch for a selection layer's top-k (a) and its merge pass (c).
hipError_t launch_select_merge(const SelectArgs& a, const CombineArgs& c, hipStream_t stream);

// Launch timing (timing.hip). Kinds match the public PPSA_KERNEL_* values.
enum KernelKind : int {
  KERNEL_ATTN_FULL = 0,
  KERNEL_ATTN_FULL_SCORES = 1,
  KERNEL_ATTN_SPARSE = 2,
  KERNEL_COMBINE = 3,
  KERNEL_SELECT = 4,
  KERNEL_APPEND = 5,
  KERNEL_SOFTMAX_SCORES = 6,
  KERNEL_COVERAGE = 7,
  KERNEL_KINDS = 8
};
// Records a begin event on `stream` when timing is on; returns a token (-1: untimed) and the end event.
int timing_begin(hipStream_t stream, hipEvent_t* end);
// Records the end event of a timed launch of `kind`.
void timing_end(int token, int kind, hipEvent_t end, hipStream_t stream);

}  // namespace ppsa
