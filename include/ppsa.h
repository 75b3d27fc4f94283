/*
 * ppsa.h -- C ABI of the PPSA (position persistent sparse attention) decode
 * step for AMD Instinct MI355X (gfx950).
 *
 * The method is TidalDecode's, as described on the paper-review page
 * "TidalDecode: Fast and Accurate LLM Decoding with Position Persistent Sparse
 * Attention" (arXiv 2410.05076):
 *   - section 3, PPSA paragraph, attention equation: per query head,
 *     A = q K^T * scale and H = softmax(A) V, scale = 1/sqrt(head_dim);
 *   - section 2, solution overview, and section 3, decode-step framework
 *     figure: each decode step runs full attention in its first layers, full
 *     attention plus top-k token selection at two layers, and sparse
 *     attention over the most recently selected positions everywhere else;
 *   - section 3, PPSA paragraph: a sparse layer reuses the positions of the
 *     preceding selection layer.
 * Readings where the page is silent: the selection score of a position is
 * the float32 sum, over the query heads sharing a KV head, of its raw logit
 * q.k*scale; one set is selected per (batch row, KV head); equal scores go to
 * the lower position; a sparse layer renormalises over its positions.
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless marked (host). The caller owns all
 *     memory; the library never allocates, frees or synchronises. Every call
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns before they finish.
 *   - Layouts are dense row-major: q and out [B, Hq, d]; K and V caches
 *     [B, Hkv, Nmax, d] (one row of d elements per position); seq_lens [B]
 *     int32; scores [B, Hkv, Nmax] float32; idx [B, Hkv, topk] int32. q, K,
 *     V and out share the element type `dtype`. Query head hq uses KV head
 *     hq / (Hq / Hkv).
 *   - q, K, V, out and the workspace must be 16-byte aligned.
 *   - Device-side lengths: seq_lens[b] is clamped into [0, Nmax]. Rows at or
 *     past it are never read. A unit with no live rows outputs zeros and
 *     selects nothing.
 *   - Errors: every argument is checked on the host before any HIP call. A
 *     failing check returns a negative ppsa_status and enqueues nothing. A
 *     failed launch returns PPSA_ERR_HIP. The library never aborts or throws.
 *   - Method calls keep no state between calls (the instruments at the end --
 *     launch timing, the split-planner override -- are process-wide
 *     settings). Concurrent calls must use distinct workspaces.
 */
#ifndef PPSA_H
#define PPSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PPSA_ABI_VERSION 2

typedef enum ppsa_status {
  PPSA_OK = 0,
  PPSA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or count */
  PPSA_ERR_UNSUPPORTED = -2, /* valid but not implemented: head_dim, group size, dtype */
  PPSA_ERR_WORKSPACE = -3,   /* workspace smaller than ppsa_workspace_bytes() */
  PPSA_ERR_SCHEDULE = -4,    /* decode schedule: unknown kind, or sparse before any selection */
  PPSA_ERR_HIP = -5,         /* a HIP runtime call failed (kernel launch, event) */
  PPSA_ERR_SCRATCH = -6      /* ppsa_decode_step_static: the step needs more than its static scratch */
} ppsa_status;

typedef enum ppsa_dtype { PPSA_F32 = 0, PPSA_BF16 = 1 } ppsa_dtype;

typedef enum ppsa_layer_kind { PPSA_FULL = 0, PPSA_FULL_SELECT = 1, PPSA_SPARSE = 2 } ppsa_layer_kind;

typedef struct ppsa_dims {
  int32_t batch;        /* B >= 0; B == 0 makes every call a no-op returning PPSA_OK */
  int32_t num_q_heads;  /* Hq >= 1, a multiple of num_kv_heads, Hq/Hkv <= 16 */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t max_seq_len;  /* Nmax >= 1: cache rows per (batch row, KV head) */
  int32_t dtype;        /* ppsa_dtype of q, K, V and out */
  float scale;          /* logit scale; 0 means 1/sqrt(head_dim) */
} ppsa_dims;

/* Library ABI version (PPSA_ABI_VERSION). 2: ppsa_append_kv takes the dropped-token counter;
 * ppsa_sparse_attn_phases, ppsa_decode_step_static, ppsa_set_split_rows and the probes added. */
int ppsa_abi_version(void);

/* Static text for a status code. */
const char* ppsa_status_string(int status);

/*
 * Workspace bytes any single call below needs for these dims and token
 * budget (topk), including ppsa_decode_step. Pure host function; returns 0
 * for invalid dims.
 */
size_t ppsa_workspace_bytes(const ppsa_dims* dims, int32_t topk);

/*
 * Full attention (section 3 attention equation; the "full attention" layer
 * kind of the section 3 framework figure): for every (b, hq),
 *   out[b,hq,:] = sum_n softmax_n(q[b,hq].K[b,kv,n] * scale) V[b,kv,n,:]
 * over the live rows n in [0, seq_lens[b]), kv = hq / (Hq/Hkv).
 */
int ppsa_full_attn(const ppsa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* seq_lens, void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Full attention plus token selection (the selection layer kind of the
 * section 3 framework figure; top-k by attention score, section 2 solution
 * overview). Writes `out` as ppsa_full_attn, and for every (b, kv):
 *   scores[b,kv,n] = sum over the group's query heads of q.K[n]*scale (float32)
 *                    for live n; entries past seq_lens[b] are left untouched;
 *   idx[b,kv,:]    = the k_eff = min(topk, seq_lens[b]) live positions with
 *                    the highest score, equal scores to the lower position,
 *                    in ascending position order, slots k_eff..topk-1 = -1.
 * `scores` may be NULL (the workspace then holds them). 1 <= topk <= Nmax.
 */
int ppsa_full_attn_select(const ppsa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, int32_t topk, void* out, float* scores, int32_t* idx,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Token selection alone, on given scores [B, Hkv, Nmax] (float32, only the
 * live entries are read): writes idx exactly as ppsa_full_attn_select does.
 * Scores must not be NaN. -0.0 ranks equal to +0.0. The workspace is
 * optional (NULL with workspace_bytes 0): given one of at least
 * ppsa_workspace_bytes(dims, topk) bytes, 16-byte aligned, per-KV-head sets
 * of rows longer than 65536 positions are chosen in two launches (top-k of
 * each chunk of the row, then top-k of the chunks' winners: the same set)
 * when the chunks' winners fit 32768 entries; otherwise in one.
 */
int ppsa_select_topk(const ppsa_dims* dims, const float* scores, const int32_t* seq_lens, int32_t topk,
                     int32_t* idx, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Selection semantics (the page does not fix them; see the header note).
 * PPSA_SELECT_PER_KV_HEAD (the default everywhere): one set per (batch row,
 * KV head), ranked by that KV head's scores. PPSA_SELECT_SHARED: one set per
 * batch row, ranked by the float32 sum over its KV heads of their scores (so
 * by the sum of the raw logits of every query head), and written to every KV
 * head's row of idx -- the reading of the section 3 PPSA paragraph in which
 * the set is shared by all heads rather than chosen per head.
 * PPSA_SELECT_SOFTMAX (decode steps only): one set per (batch row, KV head),
 * ranked by the float32 sum over the group's query heads of the softmax
 * weight each gives the position (2^(x - M) / L with the head's final max M
 * and normaliser L of the same full-attention pass); `scores`, when given,
 * receives these sums. The workspace from ppsa_workspace_bytes(dims, topk)
 * with topk > 0 covers the head logits this needs.
 * PPSA_SELECT_COVERAGE (decode steps only): the softmax-weight sums again,
 * but the number kept per (batch row, KV head) is a coverage budget instead
 * of topk: with masses m_n = sum / group (about 1 in total), the positions
 * are pruned from the lowest mass upward (equal masses from the higher
 * position) until the pruned mass exceeds coverage_tau; the rest are kept,
 * at most topk of them (the token-sparse page's dynamic token coverage
 * paragraph). Masses are summed in 24-bit fixed point, so the budget does
 * not depend on summation order (masses below 2^-25 count as zero).
 */
typedef enum ppsa_select_mode {
  PPSA_SELECT_PER_KV_HEAD = 0,
  PPSA_SELECT_SHARED = 1,
  PPSA_SELECT_SOFTMAX = 2,
  PPSA_SELECT_COVERAGE = 3
} ppsa_select_mode;

/* ppsa_select_topk with a selection mode (PPSA_SELECT_PER_KV_HEAD or PPSA_SELECT_SHARED; any other
 * mode returns PPSA_ERR_INVALID_ARG). */
int ppsa_select_topk_ex(const ppsa_dims* dims, const float* scores, const int32_t* seq_lens, int32_t topk,
                        int32_t select_mode, int32_t* idx, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse attention over pre-selected positions (the PPSA layer kind, section
 * 3 PPSA paragraph): attention of every query head of KV group kv over the
 * rows idx[b,kv,0..topk) only, renormalised over them. Entries outside
 * [0, seq_lens[b]) are skipped; a repeated entry counts once per occurrence;
 * a unit with no valid entry outputs zeros.
 */
int ppsa_sparse_attn(const ppsa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* seq_lens, const int32_t* idx, int32_t topk, void* out, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * ppsa_sparse_attn as its two launches, for callers that place or time them
 * apart. `phases` is a bitwise OR of:
 *   PPSA_PHASE_ATTN   the attention launch: with one split per (b, kv) unit it
 *                     writes out itself; otherwise it leaves each split's
 *                     partial (max, normaliser, weighted V sum) in workspace;
 *   PPSA_PHASE_MERGE  the merge launch: turns the partials in workspace into
 *                     out (nothing to do, and no launch, with one split).
 * PPSA_PHASE_ATTN | PPSA_PHASE_MERGE is ppsa_sparse_attn. A merge-only call
 * takes the same arguments as the attention call it completes (same dims,
 * topk and workspace; the plan, hence the partial layout, follows from them)
 * and merges whatever that workspace holds. Errors as ppsa_sparse_attn, plus
 * PPSA_ERR_INVALID_ARG for phases outside 1..3.
 */
enum { PPSA_PHASE_ATTN = 1, PPSA_PHASE_MERGE = 2 };
int ppsa_sparse_attn_phases(const ppsa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, const int32_t* idx, int32_t topk, int32_t phases, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step over `num_layers` layers (section 3 framework figure):
 * layer l runs the kind schedule[l] (host array of ppsa_layer_kind values)
 * on q[l], K[l], V[l] and writes out[l]. A PPSA_FULL_SELECT layer writes the
 * next slot of `idx`; a PPSA_SPARSE layer reads the most recently written
 * slot. A sparse layer before any selection returns PPSA_ERR_SCHEDULE.
 *   q, out:        [L, B, Hq, d]
 *   k/v_cache:     [L, B, Hkv, Nmax, d]
 *   idx:           [S, B, Hkv, topk], S = number of PPSA_FULL_SELECT layers
 *                  (may be NULL when S == 0)
 *   scores:        [S, B, Hkv, Nmax] float32, or NULL
 * seq_lens is shared by all layers. 1 <= topk <= Nmax when S > 0.
 */
int ppsa_decode_step(const ppsa_dims* dims, int32_t num_layers, const int32_t* schedule, const void* q,
                     const void* k_cache, const void* v_cache, const int32_t* seq_lens, int32_t topk, void* out,
                     int32_t* idx, float* scores, void* workspace, size_t workspace_bytes, void* stream);

/* ppsa_decode_step with a selection mode for its PPSA_FULL_SELECT layers and, for
 * PPSA_SELECT_COVERAGE, the threshold coverage_tau in [0, 1) (ignored otherwise). scores, when given,
 * receives the quantity ranked per KV head (logit sums, or softmax-weight sums in the softmax and
 * coverage modes). An unknown mode or a tau outside [0, 1) returns PPSA_ERR_INVALID_ARG. */
int ppsa_decode_step_ex(const ppsa_dims* dims, int32_t num_layers, const int32_t* schedule, const void* q,
                        const void* k_cache, const void* v_cache, const int32_t* seq_lens, int32_t topk,
                        int32_t select_mode, float coverage_tau, void* out, int32_t* idx, float* scores,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * ppsa_decode_step (default selection: per KV head, logit sums) without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The call allocates nothing; its split partials and, when
 * `scores` is NULL, its score array live in a static device array of 16 MiB
 * built into the library (one per GPU the library runs on, held until the
 * process ends; its device address is looked up once per device, with that
 * device current, on the first call there). Arguments, layouts and results
 * are those of ppsa_decode_step with the same plan, so outputs and indices
 * are identical to it.
 * The step needs 256-byte aligned regions of B*Hq*S*4 bytes (twice) and
 * B*Hq*S*d*4 bytes for the partials (S <= 256 splits per unit), plus
 * B*Hkv*Nmax*4 bytes for the scores when `scores` is NULL; a step that does
 * not fit returns PPSA_ERR_SCRATCH before any HIP call (pass `scores`, or use
 * ppsa_decode_step with a workspace). Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other threads)
 * race and must not be issued; calls in one stream's order are safe. Nothing
 * in the array needs clearing between calls. The stream must belong to the
 * current device.
 */
int ppsa_decode_step_static(const ppsa_dims* dims, int32_t num_layers, const int32_t* schedule, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* seq_lens, int32_t topk,
                            void* out, int32_t* idx, float* scores, void* stream);

/*
 * Append one decode token to the caches (section 2, problem definition:
 * decoding produces one token at a time and each token's K and V rows join
 * the cache before the next attention). For every batch row b with
 * n = seq_lens[b] clamped into [0, Nmax]: when n < Nmax, k_new[l,b,h,:] and
 * v_new[l,b,h,:] are stored at row n of k_cache[l,b,h] and v_cache[l,b,h]
 * for every layer l < num_layers and KV head h, and seq_lens[b] becomes
 * n + 1; when n = Nmax (full) nothing is stored and seq_lens[b] becomes
 * Nmax.
 *   k_new, v_new:  [L, B, Hkv, d], element type `dtype`
 *   k/v_cache:     [L, B, Hkv, Nmax, d], written at one row per (l, b, h)
 *   seq_lens:      [B] int32, read and written on the device
 *   overflow:      device int32 or NULL; when given, the number of batch rows
 *                  that were full (whose token was not stored) is added to it,
 *                  so a caller running past the cache's capacity can see it
 * Two launches on `stream`, in order: the row copy, then the length update
 * (which reads and counts the lengths the copy used). A ppsa_decode_step
 * enqueued after them on the same stream sees the new rows and lengths. A
 * multi-token decode calls this, then ppsa_decode_step, once per token.
 * Pointers must be 16-byte aligned (seq_lens and overflow 4-byte); errors as
 * for the other entry points.
 */
int ppsa_append_kv(const ppsa_dims* dims, int32_t num_layers, const void* k_new, const void* v_new,
                   void* k_cache, void* v_cache, int32_t* seq_lens, int32_t* overflow, void* stream);

/*
 * Launch timing (instrumentation; not part of the method). While timing is
 * on, every kernel the entry points above enqueue is bracketed by two HIP
 * events recorded on the same stream, and ppsa_timing_read() returns, per
 * kernel kind, how many launches completed and their summed elapsed time
 * (begin event to end event) since the previous read.
 *
 * ppsa_timing_enable(capacity): capacity > 0 switches timing on with a pool
 * of events for `capacity` launches between reads (created here, the only
 * allocation); a launch that finds the pool empty is not timed and counts as
 * dropped. capacity == 0 switches timing off and destroys the pool. Either
 * call first waits for launches still pending. Returns PPSA_OK,
 * PPSA_ERR_INVALID_ARG (capacity < 0) or PPSA_ERR_HIP.
 *
 * ppsa_timing_read(counts, total_ms, num_kinds, dropped): host arrays of
 * num_kinds >= PPSA_KERNEL_KINDS entries, indexed by ppsa_kernel_kind;
 * dropped (host, may be NULL) receives the number of untimed launches. Waits
 * for the recorded events (this call synchronises). Returns PPSA_OK,
 * PPSA_ERR_INVALID_ARG or PPSA_ERR_HIP.
 *
 * Timing state is process-wide. Do not read while another thread enqueues.
 */
typedef enum ppsa_kernel_kind {
  PPSA_KERNEL_ATTN_FULL = 0,        /* split attention pass of a full layer */
  PPSA_KERNEL_ATTN_FULL_SCORES = 1, /* the same pass writing selection scores */
  PPSA_KERNEL_ATTN_SPARSE = 2,      /* split attention pass over selected rows */
  PPSA_KERNEL_COMBINE = 3,          /* merge of split partials */
  PPSA_KERNEL_SELECT = 4,           /* top-k selection */
  PPSA_KERNEL_APPEND = 5,           /* append of a token's K/V rows */
  PPSA_KERNEL_SOFTMAX_SCORES = 6,   /* softmax-weight selection scores */
  PPSA_KERNEL_COVERAGE = 7,         /* coverage budget per unit */
  PPSA_KERNEL_KINDS = 8
} ppsa_kernel_kind;

int ppsa_timing_enable(int32_t capacity);
int ppsa_timing_read(int32_t* counts, double* total_ms, int32_t num_kinds, int64_t* dropped);
/* Static description of a kernel kind ("unknown" outside the enum). */
const char* ppsa_timing_kernel_name(int32_t kind);

/*
 * Split-planner override (tuning and testing; not part of the method). Each
 * attention layer is cut into splits of rows per (batch row, KV head), merged
 * afterwards; the library sizes them for this GPU. full_rows / sparse_rows > 0
 * set the rows of one split of full / sparse layers (rounded up to the
 * kernels' granule, capped as the automatic plan is); 0 restores the
 * automatic choice. Process-wide; affects ppsa_workspace_bytes and every
 * later call. Results do not depend on the plan beyond float32 rounding.
 * Returns PPSA_OK, or PPSA_ERR_INVALID_ARG for a negative value.
 */
int ppsa_set_split_rows(int32_t full_rows, int32_t sparse_rows);

/*
 * Measurement probes (instrumentation; not part of the method, never called
 * by the entry points above). Each enqueues one kernel on `stream` and
 * returns without waiting; time them with events on that stream. `sink` is a
 * device int32 the kernels may write (so that no load is optimised away).
 * Errors: PPSA_ERR_INVALID_ARG for bad arguments (before any HIP call),
 * PPSA_ERR_HIP for a failed launch.
 *
 * ppsa_probe_read: reads `bytes` of device memory at `buf` once (16-byte
 *   loads, each workgroup one contiguous chunk of 32 to 512 KiB, at least
 *   2048 workgroups when the size allows); bytes must be a positive multiple
 *   of 32 KiB and buf 16-byte aligned. nontemporal != 0
 *   loads with the nontemporal hint, as the streaming attention launches do.
 *   bytes / time is the achievable HBM read bandwidth when buf is much larger
 *   than the last-level cache (256 MB).
 * ppsa_probe_empty: an empty kernel of `groups` workgroups of `threads`
 *   (1..1024) work-items; back-to-back launches give the per-launch floor.
 * ppsa_probe_gather: `repeats` (>= 1) back-to-back launches of the load-only
 *   twin of ppsa_sparse_attn's kernel for these dims and idx (same plan,
 *   grid, waves, slot-entry reads and K/V row loads; no attention arithmetic,
 *   no merge, no output). The sparse kernel's time over the twin's is what
 *   its arithmetic, LDS traffic and epilogue cost on top of the gather. bf16,
 *   head_dim 128 only (the matrix-core path), else PPSA_ERR_UNSUPPORTED.
 */
int ppsa_probe_read(const void* buf, size_t bytes, int32_t nontemporal, int32_t* sink, void* stream);
int ppsa_probe_empty(int32_t groups, int32_t threads, int32_t* sink, void* stream);
int ppsa_probe_gather(const ppsa_dims* dims, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                      const int32_t* idx, int32_t topk, int32_t repeats, int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PPSA_H */
