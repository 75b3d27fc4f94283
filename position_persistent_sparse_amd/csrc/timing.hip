// Opt-in launch timing: two HIP events around every kernel the library
// enqueues, read back per kernel kind. Host code only.
//
// The events come from a pool created when timing is switched on, so the
// timed calls still allocate nothing; a launch that finds the pool empty is
// left untimed and counted as dropped.
#include <mutex>
#include <vector>

#include "ppsa_internal.h"
#include "ppsa.h"

namespace ppsa {

static_assert(KERNEL_ATTN_FULL == PPSA_KERNEL_ATTN_FULL && KERNEL_ATTN_FULL_SCORES == PPSA_KERNEL_ATTN_FULL_SCORES &&
                  KERNEL_ATTN_SPARSE == PPSA_KERNEL_ATTN_SPARSE && KERNEL_COMBINE == PPSA_KERNEL_COMBINE &&
                  KERNEL_SELECT == PPSA_KERNEL_SELECT && KERNEL_APPEND == PPSA_KERNEL_APPEND &&
                  KERNEL_SOFTMAX_SCORES == PPSA_KERNEL_SOFTMAX_SCORES && KERNEL_COVERAGE == PPSA_KERNEL_COVERAGE &&
                  KERNEL_KINDS == PPSA_KERNEL_KINDS,
              "internal kernel kinds must match ppsa_kernel_kind");

namespace {

struct Pending {
  hipEvent_t begin, end;
  int kind;
};

struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;     // free events
  std::vector<hipEvent_t> created;  // every event of the current pool
  std::vector<Pending> pending;     // recorded, not yet read
  int64_t dropped = 0;
};

TimingState& state() {
  static TimingState s;
  return s;
}

// Waits for every pending pair, returns its events to the pool and, when counts != NULL, adds its
// elapsed time to its kind.
hipError_t drain(TimingState& s, int32_t* counts, double* ms) {
  hipError_t err = hipSuccess;
  for (const Pending& p : s.pending) {
    float t = 0.0f;
    if (p.kind < -1) {  // end event never recorded
      s.pool.push_back(p.begin);
      s.pool.push_back(p.end);
      continue;
    }
    hipError_t e = hipEventSynchronize(p.end);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, p.begin, p.end);
    if (e != hipSuccess && err == hipSuccess) err = e;
    if (e == hipSuccess && counts && p.kind >= 0 && p.kind < KERNEL_KINDS) {
      counts[p.kind] += 1;
      ms[p.kind] += t;
    }
    s.pool.push_back(p.begin);
    s.pool.push_back(p.end);
  }
  s.pending.clear();
  return err;
}

hipError_t destroy_pool(TimingState& s) {
  hipError_t err = drain(s, nullptr, nullptr);
  for (hipEvent_t e : s.created) {
    const hipError_t r = hipEventDestroy(e);
    if (r != hipSuccess && err == hipSuccess) err = r;
  }
  s.created.clear();
  s.pool.clear();
  return err;
}

}  // namespace

int timing_begin(hipStream_t stream, hipEvent_t* end_out) {
  TimingState& s = state();
  std::lock_guard<std::mutex> lock(s.mu);
  if (!s.on) return -1;
  if (s.pool.size() < 2) {
    ++s.dropped;
    return -1;
  }
  hipEvent_t b = s.pool.back();
  s.pool.pop_back();
  hipEvent_t e = s.pool.back();
  s.pool.pop_back();
  if (hipEventRecord(b, stream) != hipSuccess) {
    s.pool.push_back(e);
    s.pool.push_back(b);
    ++s.dropped;
    return -1;
  }
  s.pending.push_back(Pending{b, e, -1});
  *end_out = e;
  return (int)s.pending.size() - 1;
}

void timing_end(int token, int kind, hipEvent_t end, hipStream_t stream) {
  if (token < 0) return;
  TimingState& s = state();
  std::lock_guard<std::mutex> lock(s.mu);
  if (token >= (int)s.pending.size() || s.pending[token].end != end) return;  // drained meanwhile
  // The end event is recorded even for a failed launch (kind -1), so reading never waits on an
  // event that was not recorded; such pairs are not counted.
  if (hipEventRecord(end, stream) != hipSuccess) {
    s.pending[token].kind = -2;  // end never recorded: skipped when read
    ++s.dropped;
    return;
  }
  s.pending[token].kind = kind;
}

}  // namespace ppsa

using namespace ppsa;

extern "C" {

int ppsa_timing_enable(int32_t capacity) {
  if (capacity < 0) return PPSA_ERR_INVALID_ARG;
  TimingState& s = state();
  std::lock_guard<std::mutex> lock(s.mu);
  hipError_t err = destroy_pool(s);
  s.on = false;
  s.dropped = 0;
  if (err != hipSuccess) return PPSA_ERR_HIP;
  if (capacity == 0) return PPSA_OK;
  for (int32_t i = 0; i < 2 * capacity; ++i) {
    hipEvent_t e;
    // Timing only: no system-scope fence (cache writeback and invalidate) when the event is recorded,
    // which would otherwise sit between the timed kernels and lengthen every bracket.
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
      (void)destroy_pool(s);
      return PPSA_ERR_HIP;
    }
    s.created.push_back(e);
    s.pool.push_back(e);
  }
  s.on = true;
  return PPSA_OK;
}

int ppsa_timing_read(int32_t* counts, double* total_ms, int32_t num_kinds, int64_t* dropped) {
  if (!counts || !total_ms || num_kinds < KERNEL_KINDS) return PPSA_ERR_INVALID_ARG;
  TimingState& s = state();
  std::lock_guard<std::mutex> lock(s.mu);
  for (int32_t i = 0; i < num_kinds; ++i) {
    counts[i] = 0;
    total_ms[i] = 0.0;
  }
  const hipError_t err = drain(s, counts, total_ms);
  if (dropped) *dropped = s.dropped;
  s.dropped = 0;
  return err == hipSuccess ? PPSA_OK : PPSA_ERR_HIP;
}

const char* ppsa_timing_kernel_name(int32_t kind) {
  switch (kind) {
    case KERNEL_ATTN_FULL: return "attention, full layer";
    case KERNEL_ATTN_FULL_SCORES: return "attention + score write, selection layer";
    case KERNEL_ATTN_SPARSE: return "attention, sparse layer";
    case KERNEL_COMBINE: return "merge of split partials";
    case KERNEL_SELECT: return "top-k selection";
    case KERNEL_APPEND: return "append of a token's K/V rows";
    case KERNEL_SOFTMAX_SCORES: return "softmax-weight selection scores";
    case KERNEL_COVERAGE: return "coverage budget per unit";
    default: return "unknown";
  }
}

}  // extern "C"
