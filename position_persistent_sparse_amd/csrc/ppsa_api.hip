// C-ABI front end of the PPSA decode-step library: argument checks, split
// planning, workspace carving and the per-layer dispatch of the decode step
// (the three layer kinds of the TidalDecode review page, section 2 solution
// overview and section 3 decode-step framework figure). Host code only;
// it never allocates, frees or synchronises.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "ppsa_internal.h"
#include "ppsa.h"

// Device memory of ppsa_decode_step_static: a fixed array in the library's code object (one copy
// per GPU the library runs on, held until the process ends), for callers that cannot allocate.
// Host code never names it directly: its device address comes from hipGetSymbolAddress, per device.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace ppsa {
namespace {

constexpr size_t kAlign = 256;
// Workgroups a layer is cut into, about (MI355X: 256 CUs). Measured on the LLaMA-3-8B GQA
// 32K shape: one long run per CU is fastest for full layers (fewest partials, fewest
// concurrent DRAM streams); gathered sparse layers want two workgroups per CU.
constexpr int kFullTargetGroups = 256;
constexpr int kSparseTargetGroups = 512;
// A unit whose K+V rows total at most this many bytes runs as one split: the merge pass then
// disappears, which saves more than the extra rows cost one workgroup (measured: LLaMA-2-7B at
// k = 512 and LLaMA-3-70B at k = 256, 32 and 64 units, sparse layers 25-40 % faster).
constexpr int64_t kSingleSplitBytes = 256 * 1024;
constexpr int kMaxGridYZ = 65535;


// Attention implementation: the matrix-core pass wherever it applies, unless
// PPSA_ATTN_IMPL=valu selects the vector-ALU pass (both compute the same
// result; the switch exists to compare them).
bool use_mfma(const ppsa_dims& d) {
  static const bool force_valu = [] {
    const char* e = getenv("PPSA_ATTN_IMPL");
    return e && strcmp(e, "valu") == 0;
  }();
  // The matrix-core pass addresses rows by 32-bit byte offsets within a (batch row, KV head).
  const bool offsets_fit = (int64_t)d.max_seq_len * d.head_dim * 2 < (int64_t(1) << 32);
  return !force_valu && offsets_fit && attn_mfma_supported(d.dtype, d.head_dim, d.num_q_heads / d.num_kv_heads);
}

// Planner override (ppsa_set_split_rows): rows per split of full and sparse layers, 0 = automatic.
std::atomic<int> g_full_rows_override{0};
std::atomic<int> g_sparse_rows_override{0};

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int round_up(int64_t x, int g) { return (int)(ceil_div(x, g) * g); }

struct Plan {
  int full_rows = 0, full_splits = 0;
  int sparse_rows = 0, sparse_splits = 0;
  int max_splits = 0;
  size_t off_m = 0, off_l = 0, off_o = 0, off_scores = 0, total = 0;
  size_t off_heads = 0, off_fm = 0, off_fl = 0;  // softmax-weight selection: head logits, final max / sum
  size_t off_unitk = 0;                           // coverage budget per unit
  size_t off_cand_score = 0, off_cand_pos = 0;    // two-stage selection: candidate rows
  int sel_chunk = 0, sel_nchunks = 0, sel_stride = 0;  // two-stage selection geometry (0: one launch)
  bool full_ok = true;    // false: full layers would need more splits than one unit may have
  bool sparse_ok = true;  // false: the budget needs more splits than one unit may have
  bool mfma = false;
};

size_t elem_bytes(int dtype) { return dtype == PPSA_BF16 ? 2 : 4; }

// Scalar checks of the dims (no pointers).
int check_dims(const ppsa_dims* d) {
  if (!d) return PPSA_ERR_INVALID_ARG;
  if (d->batch < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->max_seq_len < 1 || d->head_dim < 1)
    return PPSA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return PPSA_ERR_INVALID_ARG;
  if (!isfinite(d->scale)) return PPSA_ERR_INVALID_ARG;
  if (d->dtype != PPSA_F32 && d->dtype != PPSA_BF16) return PPSA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return PPSA_ERR_UNSUPPORTED;
  if (d->num_q_heads / d->num_kv_heads > kMaxGroup) return PPSA_ERR_UNSUPPORTED;
  if (d->batch > kMaxGridYZ || d->num_kv_heads > kMaxGridYZ) return PPSA_ERR_UNSUPPORTED;
  return PPSA_OK;
}

// `variants`: also carve the regions the selection variants need (softmax-weight and coverage
// selection); the default per-KV-head selection does without them. `score_buffer`: a score array
// for selection layers whose caller passes none.
Plan make_plan(const ppsa_dims& d, int topk, bool variants = true, bool score_buffer = true) {
  Plan p;
  p.mfma = use_mfma(d);
  const int granule = p.mfma ? attn_mfma_rows_granule() : attn_rows_granule(d.dtype, d.head_dim);
  const int64_t units = (int64_t)std::max(d.batch, 1) * d.num_kv_heads;
  const int64_t kv_row_bytes = 2 * (int64_t)d.head_dim * (int64_t)elem_bytes(d.dtype);
  int64_t rows = ceil_div(units * d.max_seq_len, kFullTargetGroups);
  rows = std::max<int64_t>(rows, ceil_div(d.max_seq_len, kMaxSplitsPerUnit));
  if ((int64_t)d.max_seq_len * kv_row_bytes <= kSingleSplitBytes) rows = d.max_seq_len;
  if (const int o = g_full_rows_override.load(std::memory_order_relaxed)) rows = std::max<int64_t>(o, ceil_div(d.max_seq_len, kMaxSplitsPerUnit));
  p.full_rows = std::max(round_up(rows, granule), granule);
  if (p.mfma) p.full_rows = std::min(p.full_rows, attn_mfma_max_score_rows(d.num_q_heads / d.num_kv_heads));
  p.full_splits = (int)ceil_div(d.max_seq_len, p.full_rows);
  if (p.full_splits > kMaxSplitsPerUnit) p.full_ok = false;  // only with the score-staging cap, N > 2M rows
  if (topk > 0) {
    rows = ceil_div(units * topk, kSparseTargetGroups);
    rows = std::max<int64_t>(rows, ceil_div(topk, kMaxSplitsPerUnit));
    if ((int64_t)topk * kv_row_bytes <= kSingleSplitBytes) rows = topk;
    if (const int o = g_sparse_rows_override.load(std::memory_order_relaxed)) rows = std::max<int64_t>(o, ceil_div(topk, kMaxSplitsPerUnit));
    const int cap = p.mfma ? (1 << 20) : attn_max_sparse_rows() / granule * granule;
    p.sparse_rows = std::max(round_up(rows, granule), granule);
    if (p.sparse_rows > cap) {
      p.sparse_ok = false;
      p.sparse_rows = cap;
    }
    p.sparse_splits = (int)ceil_div(topk, p.sparse_rows);
  }
  p.max_splits = std::max(p.full_splits, p.sparse_splits);
  const size_t heads = (size_t)std::max(d.batch, 0) * d.num_q_heads;
  size_t off = 0;
  p.off_m = off; off = align_up(off + heads * p.max_splits * sizeof(float));
  p.off_l = off; off = align_up(off + heads * p.max_splits * sizeof(float));
  p.off_o = off; off = align_up(off + heads * p.max_splits * d.head_dim * sizeof(float));
  p.off_scores = off;
  if (score_buffer) off = align_up(off + (size_t)std::max(d.batch, 0) * d.num_kv_heads * d.max_seq_len * sizeof(float));
  if (topk > 0 && variants) {  // regions of the softmax-weight selection variant
    p.off_heads = off; off = align_up(off + heads * d.max_seq_len * sizeof(float));
    p.off_fm = off; off = align_up(off + heads * sizeof(float));
    p.off_fl = off; off = align_up(off + heads * sizeof(float));
    p.off_unitk = off; off = align_up(off + (size_t)std::max(d.batch, 0) * d.num_kv_heads * sizeof(int32_t));
  }
  if (topk > 0 && select_two_stage(d.max_seq_len, topk, &p.sel_chunk, &p.sel_nchunks)) {
    p.sel_stride = (int)round_up((int64_t)p.sel_nchunks * topk, 4);
    const size_t cand = (size_t)std::max(d.batch, 0) * d.num_kv_heads * p.sel_stride;
    p.off_cand_score = off; off = align_up(off + cand * sizeof(float));
    p.off_cand_pos = off; off = align_up(off + cand * sizeof(int32_t));
  }
  p.total = off;
  return p;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

float eff_scale(const ppsa_dims& d) { return d.scale != 0.0f ? d.scale : 1.0f / sqrtf((float)d.head_dim); }

struct Ctx {
  const ppsa_dims* d;
  Plan plan;
  char* ws;
  hipStream_t stream;
};

AttnArgs base_args(const Ctx& c, const void* q, const void* k, const void* v, const int32_t* seq_lens,
                   void* out) {
  AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k = k;
  a.v = v;
  a.seq_lens = seq_lens;
  a.part_m = reinterpret_cast<float*>(c.ws + c.plan.off_m);
  a.part_l = reinterpret_cast<float*>(c.ws + c.plan.off_l);
  a.part_o = reinterpret_cast<float*>(c.ws + c.plan.off_o);
  a.batch = c.d->batch;
  a.q_heads = c.d->num_q_heads;
  a.kv_heads = c.d->num_kv_heads;
  a.group = c.d->num_q_heads / c.d->num_kv_heads;
  a.max_len = c.d->max_seq_len;
  a.scale = eff_scale(*c.d);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  return a;
}

int finish(hipError_t e) { return e == hipSuccess ? PPSA_OK : PPSA_ERR_HIP; }

// Runs launch() between the two events of a timed launch when timing is on.
template <typename F>
hipError_t timed(int kind, hipStream_t stream, F&& launch) {
  hipEvent_t end = nullptr;
  const int token = timing_begin(stream, &end);
  const hipError_t e = launch();
  timing_end(token, e == hipSuccess ? kind : -1, end, stream);
  return e;
}

CombineArgs combine_args(const Ctx& c, int splits, void* out) {
  CombineArgs cb{};
  cb.part_m = reinterpret_cast<const float*>(c.ws + c.plan.off_m);
  cb.part_l = reinterpret_cast<const float*>(c.ws + c.plan.off_l);
  cb.part_o = reinterpret_cast<const float*>(c.ws + c.plan.off_o);
  cb.out = out;
  cb.rows = c.d->batch * c.d->num_q_heads;
  cb.splits = splits;
  cb.bf16 = c.d->dtype == PPSA_BF16 ? 1 : 0;
  cb.head_dim = c.d->head_dim;
  return cb;
}

// Merge pass after a multi-split attention launch (a single split writes out itself).
int run_combine(const Ctx& c, int splits, void* out) {
  if (splits <= 1) return PPSA_OK;
  const CombineArgs cb = combine_args(c, splits, out);
  return finish(timed(KERNEL_COMBINE, c.stream, [&] { return launch_combine(cb, c.d->dtype, c.d->head_dim, c.stream); }));
}

// Top-k selection; with `merge`, the same launch also merges the layer's split partials.
int run_select(const Ctx& c, const float* scores, const int32_t* seq_lens, int topk, int32_t* idx, int mode,
               const int32_t* unit_k = nullptr, const CombineArgs* merge = nullptr) {
  SelectArgs s{};
  s.unit_k = unit_k;
  s.shared = mode == PPSA_SELECT_SHARED ? 1 : 0;
  s.scores = scores;
  s.seq_lens = seq_lens;
  s.idx = idx;
  s.batch = c.d->batch;
  s.kv_heads = c.d->num_kv_heads;
  s.max_len = c.d->max_seq_len;
  s.topk = topk;
  // Long rows of per-KV-head sets: top-k per chunk of the row, then over the chunks' winners (two
  // launches, the first spread over chunks x units workgroups). Needs the workspace's candidate rows.
  if (mode == PPSA_SELECT_PER_KV_HEAD && !unit_k && c.ws && c.plan.sel_nchunks > 0) {
    s.chunk = c.plan.sel_chunk;
    s.nchunks = c.plan.sel_nchunks;
    s.cand_stride = c.plan.sel_stride;
    s.cand_score = reinterpret_cast<float*>(c.ws + c.plan.off_cand_score);
    s.cand_pos = reinterpret_cast<int32_t*>(c.ws + c.plan.off_cand_pos);
    s.stage = 1;
    int rc = finish(timed(KERNEL_SELECT, c.stream, [&] {
      return merge ? launch_select_merge(s, *merge, c.stream) : launch_select(s, c.stream);
    }));
    if (rc != PPSA_OK) return rc;
    s.stage = 2;
    return finish(timed(KERNEL_SELECT, c.stream, [&] { return launch_select(s, c.stream); }));
  }
  return finish(timed(KERNEL_SELECT, c.stream, [&] {
    return merge ? launch_select_merge(s, *merge, c.stream) : launch_select(s, c.stream);
  }));
}

int run_full(const Ctx& c, const void* q, const void* k, const void* v, const int32_t* seq_lens, void* out,
             int topk, float* scores, int32_t* idx, int select_mode, float tau = 0.0f) {
  AttnArgs a = base_args(c, q, k, v, seq_lens, out);
  a.splits = c.plan.full_splits;
  a.rows_per_split = c.plan.full_rows;
  const bool select = idx != nullptr;
  const bool coverage = select && select_mode == PPSA_SELECT_COVERAGE;
  const bool softmax = select && (select_mode == PPSA_SELECT_SOFTMAX || coverage);
  if (select) a.scores = scores ? scores : reinterpret_cast<float*>(c.ws + c.plan.off_scores);
  if (softmax) a.head_logits = reinterpret_cast<float*>(c.ws + c.plan.off_heads);
  const int mode = softmax ? MODE_FULL_HEADS : (select ? MODE_FULL_SCORES : MODE_FULL);
  int rc = finish(timed(select ? KERNEL_ATTN_FULL_SCORES : KERNEL_ATTN_FULL, c.stream, [&] {
    return c.plan.mfma ? launch_attn_mfma(a, mode, c.stream) : launch_attn(a, mode, c.d->dtype, c.d->head_dim, c.stream);
  }));
  // A selection layer ranked by the logit sums merges its partials inside the selection launch: the
  // two read disjoint inputs, and the merge then runs beside the top-k work on CUs it leaves idle
  // instead of as a launch of its own.
  const bool merge_in_select = select && !softmax && a.splits > 1;
  if (rc == PPSA_OK && !merge_in_select) rc = run_combine(c, a.splits, out);
  if (rc != PPSA_OK || !select) return rc;
  if (softmax) {
    // The scores the selection ranks become the group's softmax-weight sums (written over the logit sums).
    SoftmaxScoreArgs sa{};
    sa.head_logits = a.head_logits;
    sa.stat_m = reinterpret_cast<float*>(c.ws + c.plan.off_fm);
    sa.stat_l = reinterpret_cast<float*>(c.ws + c.plan.off_fl);
    sa.seq_lens = seq_lens;
    sa.scores = a.scores;
    sa.batch = c.d->batch;
    sa.q_heads = c.d->num_q_heads;
    sa.kv_heads = c.d->num_kv_heads;
    sa.max_len = c.d->max_seq_len;
    rc = finish(timed(KERNEL_SOFTMAX_SCORES, c.stream, [&] { return launch_softmax_scores(sa, c.stream); }));
    if (rc != PPSA_OK) return rc;
  }
  int32_t* unit_k = nullptr;
  if (coverage) {
    CoverageArgs ca{};
    ca.scores = a.scores;
    ca.seq_lens = seq_lens;
    ca.unit_k = unit_k = reinterpret_cast<int32_t*>(c.ws + c.plan.off_unitk);
    ca.batch = c.d->batch;
    ca.kv_heads = c.d->num_kv_heads;
    ca.max_len = c.d->max_seq_len;
    ca.group = c.d->num_q_heads / c.d->num_kv_heads;
    ca.tau = tau;
    rc = finish(timed(KERNEL_COVERAGE, c.stream, [&] { return launch_coverage(ca, c.stream); }));
    if (rc != PPSA_OK) return rc;
  }
  const CombineArgs cb = combine_args(c, a.splits, out);
  return run_select(c, a.scores, seq_lens, topk, idx, softmax ? PPSA_SELECT_PER_KV_HEAD : select_mode, unit_k,
                    merge_in_select ? &cb : nullptr);
}

int run_sparse(const Ctx& c, const void* q, const void* k, const void* v, const int32_t* seq_lens,
               const int32_t* idx, int topk, void* out, int phases = PPSA_PHASE_ATTN | PPSA_PHASE_MERGE) {
  AttnArgs a = base_args(c, q, k, v, seq_lens, out);
  a.idx = idx;
  a.kslots = topk;
  a.splits = c.plan.sparse_splits;
  a.rows_per_split = c.plan.sparse_rows;
  a.idx_vec = (topk % 4 == 0 && aligned(idx, 16)) ? 1 : 0;
  int rc = PPSA_OK;
  if (phases & PPSA_PHASE_ATTN)
    rc = finish(timed(KERNEL_ATTN_SPARSE, c.stream, [&] {
      return c.plan.mfma ? launch_attn_sparse(a, c.stream) : launch_attn(a, MODE_SPARSE, c.d->dtype, c.d->head_dim, c.stream);
    }));
  return rc == PPSA_OK && (phases & PPSA_PHASE_MERGE) ? run_combine(c, a.splits, out) : rc;
}

// Pointer and workspace checks common to the attention entry points.
int check_io(const void* q, const void* k, const void* v, const int32_t* seq_lens, const void* out) {
  if (!q || !k || !v || !seq_lens || !out) return PPSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(seq_lens, 4))
    return PPSA_ERR_INVALID_ARG;
  return PPSA_OK;
}

int check_tensors(const ppsa_dims* d, const void* q, const void* k, const void* v, const int32_t* seq_lens,
                  const void* out, const void* ws) {
  (void)d;
  if (!ws || !aligned(ws, 16)) return PPSA_ERR_INVALID_ARG;
  return check_io(q, k, v, seq_lens, out);
}

int check_topk(const ppsa_dims* d, int topk) {
  return (topk >= 1 && topk <= d->max_seq_len) ? PPSA_OK : PPSA_ERR_INVALID_ARG;
}

// Device address of `scratch` on the current device, looked up once per device (under a lock) with
// that device current; the stored address is what kernels get, never the host-side symbol.
constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxScratchDevices];

int static_scratch(char** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return PPSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PPSA_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *addr = static_cast<char*>(g_scratch_addr[dev]);
  return PPSA_OK;
}

}  // namespace
}  // namespace ppsa

using namespace ppsa;

extern "C" {

int ppsa_abi_version(void) { return PPSA_ABI_VERSION; }

const char* ppsa_status_string(int status) {
  switch (status) {
    case PPSA_OK: return "ok";
    case PPSA_ERR_INVALID_ARG: return "invalid argument";
    case PPSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PPSA_ERR_WORKSPACE: return "workspace too small";
    case PPSA_ERR_SCHEDULE: return "invalid decode schedule";
    case PPSA_ERR_HIP: return "HIP runtime call failed";
    case PPSA_ERR_SCRATCH: return "needs more device memory than the static scratch holds";
    default: return "unknown status";
  }
}

size_t ppsa_workspace_bytes(const ppsa_dims* dims, int32_t topk) {
  if (check_dims(dims) != PPSA_OK || topk < 0) return 0;
  return make_plan(*dims, topk).total;
}

int ppsa_full_attn(const ppsa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* seq_lens, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != PPSA_OK) return rc;
  if (dims->batch == 0) return PPSA_OK;
  if ((rc = check_tensors(dims, q, k_cache, v_cache, seq_lens, out, workspace)) != PPSA_OK) return rc;
  Ctx c{dims, make_plan(*dims, 0), static_cast<char*>(workspace), static_cast<hipStream_t>(stream)};
  if (!c.plan.full_ok) return PPSA_ERR_UNSUPPORTED;
  if (workspace_bytes < c.plan.total) return PPSA_ERR_WORKSPACE;
  (void)hipGetLastError();
  return run_full(c, q, k_cache, v_cache, seq_lens, out, 0, nullptr, nullptr, PPSA_SELECT_PER_KV_HEAD);
}

int ppsa_full_attn_select(const ppsa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, int32_t topk, void* out, float* scores, int32_t* idx,
                          void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != PPSA_OK) return rc;
  if ((rc = check_topk(dims, topk)) != PPSA_OK) return rc;
  if (dims->batch == 0) return PPSA_OK;
  if ((rc = check_tensors(dims, q, k_cache, v_cache, seq_lens, out, workspace)) != PPSA_OK) return rc;
  if (!idx || !aligned(idx, 4) || (scores && !aligned(scores, 4))) return PPSA_ERR_INVALID_ARG;
  Ctx c{dims, make_plan(*dims, topk), static_cast<char*>(workspace), static_cast<hipStream_t>(stream)};
  if (!c.plan.full_ok) return PPSA_ERR_UNSUPPORTED;
  if (workspace_bytes < c.plan.total) return PPSA_ERR_WORKSPACE;
  (void)hipGetLastError();
  return run_full(c, q, k_cache, v_cache, seq_lens, out, topk, scores, idx, PPSA_SELECT_PER_KV_HEAD);
}

int ppsa_select_topk(const ppsa_dims* dims, const float* scores, const int32_t* seq_lens, int32_t topk,
                     int32_t* idx, void* workspace, size_t workspace_bytes, void* stream) {
  return ppsa_select_topk_ex(dims, scores, seq_lens, topk, PPSA_SELECT_PER_KV_HEAD, idx, workspace, workspace_bytes,
                             stream);
}

int ppsa_select_topk_ex(const ppsa_dims* dims, const float* scores, const int32_t* seq_lens, int32_t topk,
                        int32_t select_mode, int32_t* idx, void* workspace, size_t workspace_bytes, void* stream) {
  // PPSA_SELECT_SOFTMAX needs each head's logits, which a score array does not hold.
  if (select_mode != PPSA_SELECT_PER_KV_HEAD && select_mode != PPSA_SELECT_SHARED) return PPSA_ERR_INVALID_ARG;
  int rc = check_dims(dims);
  if (rc != PPSA_OK) return rc;
  if ((rc = check_topk(dims, topk)) != PPSA_OK) return rc;
  if (dims->batch == 0) return PPSA_OK;
  if (!scores || !seq_lens || !idx || !aligned(scores, 4) || !aligned(seq_lens, 4) || !aligned(idx, 4))
    return PPSA_ERR_INVALID_ARG;
  if (workspace_bytes > 0 && !workspace) return PPSA_ERR_INVALID_ARG;
  if (workspace && !aligned(workspace, 16)) return PPSA_ERR_INVALID_ARG;
  Ctx c{dims, make_plan(*dims, topk), static_cast<char*>(workspace), static_cast<hipStream_t>(stream)};
  if (workspace_bytes < c.plan.total) c.ws = nullptr;  // one launch: no room for the candidate rows
  (void)hipGetLastError();
  return run_select(c, scores, seq_lens, topk, idx, select_mode);
}

int ppsa_sparse_attn(const ppsa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* seq_lens, const int32_t* idx, int32_t topk, void* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return ppsa_sparse_attn_phases(dims, q, k_cache, v_cache, seq_lens, idx, topk, PPSA_PHASE_ATTN | PPSA_PHASE_MERGE,
                                 out, workspace, workspace_bytes, stream);
}

int ppsa_sparse_attn_phases(const ppsa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, const int32_t* idx, int32_t topk, int32_t phases, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (phases < 1 || phases > (PPSA_PHASE_ATTN | PPSA_PHASE_MERGE)) return PPSA_ERR_INVALID_ARG;
  int rc = check_dims(dims);
  if (rc != PPSA_OK) return rc;
  if ((rc = check_topk(dims, topk)) != PPSA_OK) return rc;
  if (dims->batch == 0) return PPSA_OK;
  if ((rc = check_tensors(dims, q, k_cache, v_cache, seq_lens, out, workspace)) != PPSA_OK) return rc;
  if (!idx || !aligned(idx, 4)) return PPSA_ERR_INVALID_ARG;
  Ctx c{dims, make_plan(*dims, topk), static_cast<char*>(workspace), static_cast<hipStream_t>(stream)};
  if (!c.plan.sparse_ok) return PPSA_ERR_UNSUPPORTED;
  if (workspace_bytes < c.plan.total) return PPSA_ERR_WORKSPACE;
  (void)hipGetLastError();
  return run_sparse(c, q, k_cache, v_cache, seq_lens, idx, topk, out, phases);
}

int ppsa_append_kv(const ppsa_dims* dims, int32_t num_layers, const void* k_new, const void* v_new,
                   void* k_cache, void* v_cache, int32_t* seq_lens, int32_t* overflow, void* stream) {
  int rc = check_dims(dims);
  if (rc != PPSA_OK) return rc;
  if (num_layers < 0) return PPSA_ERR_INVALID_ARG;
  if (dims->batch == 0 || num_layers == 0) return PPSA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !seq_lens) return PPSA_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(seq_lens, 4) || (overflow && !aligned(overflow, 4)))
    return PPSA_ERR_INVALID_ARG;
  AppendArgs a{};
  a.overflow = overflow;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.seq_lens = seq_lens;
  a.layers = num_layers;
  a.batch = dims->batch;
  a.kv_heads = dims->num_kv_heads;
  a.max_len = dims->max_seq_len;
  a.row_bytes = dims->head_dim * (int)elem_bytes(dims->dtype);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  return finish(timed(KERNEL_APPEND, st, [&] { return launch_append(a, st); }));
}

int ppsa_set_split_rows(int32_t full_rows, int32_t sparse_rows) {
  if (full_rows < 0 || sparse_rows < 0) return PPSA_ERR_INVALID_ARG;
  g_full_rows_override.store(full_rows, std::memory_order_relaxed);
  g_sparse_rows_override.store(sparse_rows, std::memory_order_relaxed);
  return PPSA_OK;
}

int ppsa_probe_read(const void* buf, size_t bytes, int32_t nontemporal, int32_t* sink, void* stream) {
  constexpr size_t kUnit = (size_t)32 << 10;
  if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4) || bytes == 0 || bytes % kUnit != 0 ||
      bytes / kUnit > 0x7fffffff)
    return PPSA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return finish(launch_read_probe(buf, bytes, nontemporal != 0, sink, static_cast<hipStream_t>(stream)));
}

int ppsa_probe_empty(int32_t groups, int32_t threads, int32_t* sink, void* stream) {
  if (groups < 1 || threads < 1 || threads > 1024 || !sink || !aligned(sink, 4)) return PPSA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return finish(launch_empty_probe(groups, threads, sink, static_cast<hipStream_t>(stream)));
}

int ppsa_probe_gather(const ppsa_dims* dims, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                      const int32_t* idx, int32_t topk, int32_t repeats, int32_t* sink, void* stream) {
  int rc = check_dims(dims);
  if (rc != PPSA_OK) return rc;
  if ((rc = check_topk(dims, topk)) != PPSA_OK) return rc;
  if (repeats < 1) return PPSA_ERR_INVALID_ARG;
  if (dims->batch == 0) return PPSA_OK;
  if (!k_cache || !v_cache || !seq_lens || !idx || !sink || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(seq_lens, 4) || !aligned(idx, 4) || !aligned(sink, 4))
    return PPSA_ERR_INVALID_ARG;
  Ctx c{dims, make_plan(*dims, topk), nullptr, static_cast<hipStream_t>(stream)};
  if (!c.plan.mfma) return PPSA_ERR_UNSUPPORTED;  // the twin mirrors the matrix-core sparse launch
  if (!c.plan.sparse_ok) return PPSA_ERR_UNSUPPORTED;
  AttnArgs a{};
  a.k = k_cache;
  a.v = v_cache;
  a.seq_lens = seq_lens;
  a.idx = idx;
  a.batch = dims->batch;
  a.q_heads = dims->num_q_heads;
  a.kv_heads = dims->num_kv_heads;
  a.group = dims->num_q_heads / dims->num_kv_heads;
  a.max_len = dims->max_seq_len;
  a.kslots = topk;
  a.splits = c.plan.sparse_splits;
  a.rows_per_split = c.plan.sparse_rows;
  a.idx_vec = (topk % 4 == 0 && aligned(idx, 16)) ? 1 : 0;
  (void)hipGetLastError();
  for (int r = 0; r < repeats; ++r)
    if ((rc = finish(launch_gather_twin(a, sink, c.stream))) != PPSA_OK) return rc;
  return PPSA_OK;
}

int ppsa_decode_step(const ppsa_dims* dims, int32_t num_layers, const int32_t* schedule, const void* q,
                     const void* k_cache, const void* v_cache, const int32_t* seq_lens, int32_t topk, void* out,
                     int32_t* idx, float* scores, void* workspace, size_t workspace_bytes, void* stream) {
  return ppsa_decode_step_ex(dims, num_layers, schedule, q, k_cache, v_cache, seq_lens, topk, PPSA_SELECT_PER_KV_HEAD,
                             0.0f, out, idx, scores, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace ppsa {
namespace {

// Argument checks of a decode step (no HIP call). On success sets the numbers of selection and
// sparse layers.
int check_step(const ppsa_dims* dims, int32_t num_layers, const int32_t* schedule, const void* q,
               const void* k_cache, const void* v_cache, const int32_t* seq_lens, int32_t topk,
               int32_t select_mode, float coverage_tau, const void* out, const int32_t* idx, const float* scores,
               int* n_sel_out, int* n_sparse_out) {
  if (select_mode < PPSA_SELECT_PER_KV_HEAD || select_mode > PPSA_SELECT_COVERAGE) return PPSA_ERR_INVALID_ARG;
  if (select_mode == PPSA_SELECT_COVERAGE && !(coverage_tau >= 0.0f && coverage_tau < 1.0f))
    return PPSA_ERR_INVALID_ARG;  // also rejects NaN
  int rc = check_dims(dims);
  if (rc != PPSA_OK) return rc;
  if (num_layers < 0 || (num_layers > 0 && !schedule)) return PPSA_ERR_INVALID_ARG;
  int n_sel = 0, n_sparse = 0;
  for (int l = 0; l < num_layers; ++l) {
    const int kind = schedule[l];
    if (kind == PPSA_FULL_SELECT) ++n_sel;
    else if (kind == PPSA_SPARSE) {
      if (n_sel == 0) return PPSA_ERR_SCHEDULE;
      ++n_sparse;
    } else if (kind != PPSA_FULL) {
      return PPSA_ERR_SCHEDULE;
    }
  }
  if (n_sel > 0 && (rc = check_topk(dims, topk)) != PPSA_OK) return rc;
  *n_sel_out = n_sel;
  *n_sparse_out = n_sparse;
  if (dims->batch == 0 || num_layers == 0) return PPSA_OK;
  if ((rc = check_io(q, k_cache, v_cache, seq_lens, out)) != PPSA_OK) return rc;
  if (n_sel > 0 && (!idx || !aligned(idx, 4))) return PPSA_ERR_INVALID_ARG;
  if (scores && !aligned(scores, 4)) return PPSA_ERR_INVALID_ARG;
  return PPSA_OK;
}

// The layers of a checked decode step, in order, on the workspace of plan `c`.
int run_step(const Ctx& c, int32_t num_layers, const int32_t* schedule, const void* q, const void* k_cache,
             const void* v_cache, const int32_t* seq_lens, int32_t topk, int32_t select_mode, float coverage_tau,
             void* out, int32_t* idx, float* scores) {
  const ppsa_dims* dims = c.d;
  const size_t eb = elem_bytes(dims->dtype);
  const size_t q_layer = (size_t)dims->batch * dims->num_q_heads * dims->head_dim * eb;
  const size_t kv_layer = (size_t)dims->batch * dims->num_kv_heads * dims->max_seq_len * dims->head_dim * eb;
  const size_t idx_slot = (size_t)dims->batch * dims->num_kv_heads * (size_t)std::max(topk, 0);
  const size_t score_slot = (size_t)dims->batch * dims->num_kv_heads * dims->max_seq_len;
  (void)hipGetLastError();
  int sel = -1, rc = PPSA_OK;
  for (int l = 0; l < num_layers; ++l) {
    const char* ql = static_cast<const char*>(q) + l * q_layer;
    const char* kl = static_cast<const char*>(k_cache) + l * kv_layer;
    const char* vl = static_cast<const char*>(v_cache) + l * kv_layer;
    char* ol = static_cast<char*>(out) + l * q_layer;
    switch (schedule[l]) {
      case PPSA_FULL:
        rc = run_full(c, ql, kl, vl, seq_lens, ol, 0, nullptr, nullptr, select_mode);
        break;
      case PPSA_FULL_SELECT:
        ++sel;
        rc = run_full(c, ql, kl, vl, seq_lens, ol, topk, scores ? scores + sel * score_slot : nullptr,
                      idx + sel * idx_slot, select_mode, coverage_tau);
        break;
      default:
        rc = run_sparse(c, ql, kl, vl, seq_lens, idx + sel * idx_slot, topk, ol);
        break;
    }
    if (rc != PPSA_OK) return rc;
  }
  return PPSA_OK;
}

}  // namespace
}  // namespace ppsa

extern "C" {

int ppsa_decode_step_ex(const ppsa_dims* dims, int32_t num_layers, const int32_t* schedule, const void* q,
                        const void* k_cache, const void* v_cache, const int32_t* seq_lens, int32_t topk,
                        int32_t select_mode, float coverage_tau, void* out, int32_t* idx, float* scores,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int n_sel = 0, n_sparse = 0;
  int rc = check_step(dims, num_layers, schedule, q, k_cache, v_cache, seq_lens, topk, select_mode, coverage_tau,
                      out, idx, scores, &n_sel, &n_sparse);
  if (rc != PPSA_OK || dims->batch == 0 || num_layers == 0) return rc;
  if (!workspace || !aligned(workspace, 16)) return PPSA_ERR_INVALID_ARG;
  Ctx c{dims, make_plan(*dims, n_sel > 0 ? topk : 0), static_cast<char*>(workspace),
        static_cast<hipStream_t>(stream)};
  if (num_layers > n_sparse && !c.plan.full_ok) return PPSA_ERR_UNSUPPORTED;
  if (n_sparse > 0 && !c.plan.sparse_ok) return PPSA_ERR_UNSUPPORTED;
  if (workspace_bytes < c.plan.total) return PPSA_ERR_WORKSPACE;
  return run_step(c, num_layers, schedule, q, k_cache, v_cache, seq_lens, topk, select_mode, coverage_tau, out, idx,
                  scores);
}

int ppsa_decode_step_static(const ppsa_dims* dims, int32_t num_layers, const int32_t* schedule, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* seq_lens, int32_t topk,
                            void* out, int32_t* idx, float* scores, void* stream) {
  int n_sel = 0, n_sparse = 0;
  int rc = check_step(dims, num_layers, schedule, q, k_cache, v_cache, seq_lens, topk, PPSA_SELECT_PER_KV_HEAD, 0.0f,
                      out, idx, scores, &n_sel, &n_sparse);
  if (rc != PPSA_OK || dims->batch == 0 || num_layers == 0) return rc;
  // The default selection only: no regions for the selection variants.
  Ctx c{dims, make_plan(*dims, n_sel > 0 ? topk : 0, false, n_sel > 0 && scores == nullptr), nullptr,
        static_cast<hipStream_t>(stream)};
  if (num_layers > n_sparse && !c.plan.full_ok) return PPSA_ERR_UNSUPPORTED;
  if (n_sparse > 0 && !c.plan.sparse_ok) return PPSA_ERR_UNSUPPORTED;
  if (c.plan.total > kStaticScratchBytes) return PPSA_ERR_SCRATCH;
  if ((rc = static_scratch(&c.ws)) != PPSA_OK) return rc;
  return run_step(c, num_layers, schedule, q, k_cache, v_cache, seq_lens, topk, PPSA_SELECT_PER_KV_HEAD, 0.0f, out,
                  idx, scores);
}

}  // extern "C"
