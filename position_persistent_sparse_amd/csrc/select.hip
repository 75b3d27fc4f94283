// Top-k token selection per (batch row, KV head) on gfx950.
//
// The selection step of the TidalDecode review page (section 2, solution
// overview; section 3 decode-step framework figure): keep the k positions
// with the highest attention score. Scores are float32; equal scores go to
// the lower position. Output is the selected positions in ascending order.
//
// One 1024-thread workgroup per unit; the work is bound by latency, barriers
// and instruction issue on that one CU, so every step keeps the per-score
// work to a few instructions and avoids per-score branches. Positions are taken in
// super-rounds of up to 32768: in super-round r thread t owns per_r
// contiguous positions (per_r = ceil(n_r / 1024) rounded up to a multiple of
// 4, <= 32, loaded 16 bytes at a time when aligned), so position order is
// (super-round, thread, bit). Each score maps to an
// order-preserving 32-bit key (-0.0 folded onto +0.0): ranking floats is
// ranking unsigned integers.
//  1. Radix digit 1 (key bits 31..21) over all keys: an LDS histogram (in
//     four lane-interleaved copies, folded) and a workgroup scan of the bins
//     from the top give the bin holding the k-th largest key and how many
//     keys lie above it.
//  2. The keys of that bin (the candidates) are copied to LDS (each thread's
//     share placed by a workgroup scan of the per-thread counts); digits 2
//     (bits 20..10) and 3 (bits 9..0) are resolved over the candidates only,
//     giving the exact key T of the k-th largest score and how many keys
//     equal to T are still to take (lowest positions first). If the bin does
//     not fit in LDS (heavily tied scores), digits 2 and 3 run over all keys.
//  3. Each thread builds bit masks of its keys > T and == T; one workgroup
//     prefix sum of the packed counts gives its first output slot, and it
//     writes its kept positions in order by walking the set bits.
// Rows of one super-round keep their keys in registers through all steps;
// longer rows reload their super-rounds in each step. When the threshold bin
// fits in LDS, step 3 works from the masks step 2 kept (in registers for one
// super-round, in LDS for up to four) and the candidates' keys, so no step
// after 2 passes over every key again. The work is bound by instruction issue
// on the one CU (16 waves on 4 SIMDs), so the per-key steps carry no per-key
// branch or test beyond their arithmetic.
//
// Rows of more than two super-rounds may instead be taken in two launches
// (SelectArgs::stage): the same kernel first runs on chunks of the row, one
// workgroup per (unit, chunk), each keeping its chunk's top-k as (score,
// position) in a candidate row, then on each unit's candidate row. Each
// launch costs its serial phases once; from three chunks up the parallel
// first stage more than pays for the second launch.
#include <math.h>

#include "combine_row.h"
#include "device_common.h"
#include "ppsa_internal.h"

namespace ppsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kCached = 32;                    // positions per thread and super-round
constexpr int kPerSuper = kCached * kThreads;  // positions per super-round
constexpr int kBins = 2048;
constexpr int kMaxCand = 8192;
// Digit 1 counts into kCopies interleaved histograms (lane % kCopies picks the copy; the copies of a
// bin sit in adjacent banks), folded afterwards: scores pile into a few hot bins, and lanes of one
// instruction hitting the same bin serialise.
constexpr int kCopies = 4;
constexpr int kMaskSR = 4;  // super-rounds whose key masks the candidate pass keeps (rows <= 131072)

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// With the histogram of one digit complete: finds the digit (walking bins
// from the top) at which the running count reaches `remaining`, and
// publishes it with the count of keys above it. Barriers inside.
template <int BINS>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t remaining, uint32_t* scan_lds, int& parity,
                                           uint32_t* digit, uint32_t* above_out) {
  constexpr int per = BINS / kThreads;  // 2 or 1
  const int tid = threadIdx.x;
  const int top = BINS - 1 - tid * per;
  const uint32_t c0 = hist[top], c1 = per == 2 ? hist[top - 1] : 0u;
  uint32_t total;
  const uint32_t above = block_exclusive_scan<kThreads>(c0 + c1, scan_lds, parity, &total);
  if (above < remaining && remaining <= above + c0) {
    *digit = (uint32_t)top;
    *above_out = above;
  } else if (per == 2 && above + c0 < remaining && remaining <= above + c0 + c1) {
    *digit = (uint32_t)(top - 1);
    *above_out = above + c0;
  }
  __syncthreads();
}

// The lowest `count` set bits of m.
__device__ __forceinline__ uint32_t lowest_bits(uint32_t m, uint32_t count) {
  uint32_t r = 0u;
  for (uint32_t i = 0; i < count && m; ++i) {
    const uint32_t low = m & (0u - m);
    r |= low;
    m ^= low;
  }
  return r;
}

// SHARED: one set per batch row, ranked by the sum of its KV heads' scores and written to every KV
// head's row of idx (the head-shared selection variant); otherwise one set per (batch row, KV head).
// MERGE: workgroups past the selection units merge the layer's split partials, one (batch row, query
// head) per wave; the merge and the selection read disjoint inputs and write disjoint outputs, so they
// share the launch and the merge runs on CUs the selection leaves idle.
template <bool CACHED, bool SHARED, bool MERGE>
__global__ __launch_bounds__(kThreads) void select_topk_kernel(SelectArgs a, CombineArgs c) {
  if constexpr (MERGE) {
    const int units = (SHARED ? a.batch : a.batch * a.kv_heads) * (!SHARED && a.stage == 1 ? a.nchunks : 1);
    if ((int)blockIdx.x >= units) {
      const int row = ((int)blockIdx.x - units) * kWaves + (int)threadIdx.x / kWave;
      const int ln = (int)threadIdx.x % kWave;
      if (row < c.rows) {  // the output format is uniform across the launch
        if (c.bf16) {
          if (c.head_dim == 128) merge::combine_row<uint16_t, 128>(c, row, ln);
          else merge::combine_row<uint16_t, 64>(c, row, ln);
        } else {
          if (c.head_dim == 128) merge::combine_row<float, 128>(c, row, ln);
          else merge::combine_row<float, 64>(c, row, ln);
        }
      }
      return;
    }
  }
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t histc[kBins * kCopies];
  __shared__ uint32_t scan_lds[2 * kWaves];
  int parity = 0;  // scan buffer (block_exclusive_scan alternates two)
  __shared__ uint32_t cand[kMaxCand];
  __shared__ uint32_t s_digit, s_above;

  const int stage = SHARED ? 0 : a.stage;
  const int nch = stage == 1 ? a.nchunks : 1;
  const int unit = (int)blockIdx.x / nch, chunk_i = (int)blockIdx.x - unit * nch;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int b = SHARED ? unit : unit / a.kv_heads;
  const int n_live = min(max(a.seq_lens[b], 0), a.max_len);
  // Kept count of chunk c (stages 1 and 2).
  auto chunk_keep = [&](int c) { return min(a.topk, min(max(n_live - c * a.chunk, 0), a.chunk)); };
  // The row this workgroup ranks: `n` live scores from `s` (summed over all KV heads of the batch row
  // when SHARED), `pitch` apart between rows, and where the kept positions go.
  const int rows = SHARED ? a.kv_heads : 1;
  const float* s;
  int n, pitch, pos0 = 0;
  float* cand_score = nullptr;
  int32_t* cand_pos = nullptr;
  const int32_t* pos_map = nullptr;
  if (stage == 1) {
    pos0 = chunk_i * a.chunk;
    n = min(max(n_live - pos0, 0), a.chunk);
    s = a.scores + (size_t)unit * a.max_len + pos0;
    pitch = a.max_len;
    int off = 0;
    for (int c = 0; c < chunk_i; ++c) off += chunk_keep(c);
    cand_score = a.cand_score + (size_t)unit * a.cand_stride + off;
    cand_pos = a.cand_pos + (size_t)unit * a.cand_stride + off;
  } else if (stage == 2) {
    n = 0;
    for (int c = 0; c < a.nchunks; ++c) n += chunk_keep(c);
    s = a.cand_score + (size_t)unit * a.cand_stride;
    pitch = a.cand_stride;
    pos_map = a.cand_pos + (size_t)unit * a.cand_stride;
  } else {
    n = n_live;
    s = a.scores + (size_t)unit * rows * a.max_len;
    pitch = a.max_len;
  }
  int k_eff = min(a.topk, n);
  if (stage == 0 && a.unit_k) k_eff = min(k_eff, max(a.unit_k[unit], 0));  // per-unit budget (coverage variant)
  int32_t* out = a.idx + (size_t)unit * rows * a.topk;
  // Kept position `pos` of the row to output slot `slot`.
  auto emit = [&](uint32_t slot, int32_t pos) {
    if (stage == 1) {
      cand_score[slot] = s[pos];
      cand_pos[slot] = pos0 + pos;
    } else {
      const int32_t p = stage == 2 ? pos_map[pos] : pos;
      for (int r = 0; r < rows; ++r) out[(size_t)r * a.topk + slot] = p;
    }
  };
  // Output slots left empty (a chunk's candidate row has no such slots).
  auto emit_empty = [&](uint32_t slot) {
    if (stage != 1)
      for (int r = 0; r < rows; ++r) out[(size_t)r * a.topk + slot] = -1;
  };

  if (k_eff == n || k_eff == 0) {  // every live position is kept, or none (includes n == 0)
    for (int i = tid; i < a.topk; i += kThreads) {
      if (i < k_eff) emit(i, i);
      else emit_empty(i);
    }
    return;
  }
  for (int i = k_eff + tid; i < a.topk; i += kThreads) emit_empty(i);  // slots past a per-unit budget

  // Rows start 16-byte aligned when their first score is and rows hold a multiple of 4 scores.
  const bool aligned = (pitch % 4) == 0 && (reinterpret_cast<uintptr_t>(s) % 16) == 0;
  const int n_sr = (n + kPerSuper - 1) / kPerSuper;
  // Super-round r spans n_r positions; thread t owns per_r of them from p0(r, t) = 32768 r + t per_r,
  // per_r = ceil(n_r / 1024) rounded up to a multiple of 4 (so that full spans load 16 bytes at a
  // time; the last threads may own fewer or none). Loads this thread's keys (0 past its live ones)
  // and the mask of the live ones. per_r is the same for every thread: the steps below skip keys
  // past it four at a time on a scalar branch and mask the rest with `live`, with no per-key test.
  struct Span {
    int p0, per;
    uint32_t live;
  };
  auto span_of = [&](int r) -> Span {
    const int n_r = min(kPerSuper, n - r * kPerSuper);
    const int per = __builtin_amdgcn_readfirstlane(((n_r + kThreads - 1) / kThreads + 3) & ~3);
    const int p0 = r * kPerSuper + tid * per;
    const int cnt = max(0, min(per, r * kPerSuper + n_r - p0));
    return Span{p0, per, cnt >= kCached ? 0xFFFFFFFFu : ((1u << cnt) - 1u)};
  };
  auto load_sr = [&](int r, auto& k) -> Span {
    const Span sp0 = span_of(r);
    const int p0 = sp0.p0, per = sp0.per;
    const int cnt = __popc(sp0.live);
    const uint32_t live = sp0.live;
    if (aligned && (per % 4) == 0 && cnt == per) {
#pragma unroll
      for (int j = 0; j < kCached / 4; ++j)
        if (4 * j < per) {
          float4 f = *reinterpret_cast<const float4*>(s + p0 + 4 * j);
          for (int r = 1; r < rows; ++r) {  // heads in order: the same float32 sum every time
            const float4 g = *reinterpret_cast<const float4*>(s + (size_t)r * pitch + p0 + 4 * j);
            f.x += g.x;
            f.y += g.y;
            f.z += g.z;
            f.w += g.w;
          }
          k[4 * j] = order_key(f.x);
          k[4 * j + 1] = order_key(f.y);
          k[4 * j + 2] = order_key(f.z);
          k[4 * j + 3] = order_key(f.w);
        } else {
          k[4 * j] = k[4 * j + 1] = k[4 * j + 2] = k[4 * j + 3] = 0u;
        }
    } else {
#pragma unroll
      for (int i = 0; i < kCached; ++i) {
        float f = 0.0f;
        if (i < cnt) {
          f = s[p0 + i];
          for (int r = 1; r < rows; ++r) f += s[(size_t)r * pitch + p0 + i];
        }
        k[i] = i < cnt ? order_key(f) : 0u;
      }
    }
    return Span{p0, per, live};
  };
  // fn(i) for this thread's keys i < per_r, four at a time on a scalar branch (per_r is a multiple
  // of 4 and the same for every thread).
  auto for_keys = [&](const Span& sp, auto&& fn) {
#pragma unroll
    for (int j = 0; j < kCached / 4; ++j)
      if (4 * j < sp.per) {
        fn(4 * j);
        fn(4 * j + 1);
        fn(4 * j + 2);
        fn(4 * j + 3);
      }
  };
  uint32_t keys[CACHED ? kCached : 1];
  Span span{0, 0, 0u};
  if constexpr (CACHED) span = load_sr(0, keys);
  // fn(keys, span) for every super-round in order.
  auto for_sr = [&](auto&& fn) {
    if constexpr (CACHED) {
      fn(keys, span);
    } else {
      for (int r = 0; r < n_sr; ++r) {
        uint32_t kk[kCached];  // per trip, so it stays in registers
        const Span sp = load_sr(r, kk);
        fn(kk, sp);
      }
    }
  };

  // 1. Digit 1 over all live keys.
  for (int i = tid; i < kBins * kCopies; i += kThreads) histc[i] = 0u;
  __syncthreads();
  const uint32_t copy = (uint32_t)(lane % kCopies);
  for_sr([&](const uint32_t(&k)[kCached], const Span& sp) {
    // Each key adds its live bit (a dead key adds 0 to bin 0): no branch per key.
    for_keys(sp, [&](int i) { atomicAdd(&histc[(k[i] >> 21) * kCopies + copy], (sp.live >> i) & 1u); });
  });
  __syncthreads();
  for (int i = tid; i < kBins; i += kThreads) {
    uint32_t c = 0u;
#pragma unroll
    for (int j = 0; j < kCopies; ++j) c += histc[i * kCopies + j];
    hist[i] = c;
  }
  __syncthreads();
  uint32_t remaining = (uint32_t)k_eff;
  find_digit<kBins>(hist, remaining, scan_lds, parity, &s_digit, &s_above);
  uint32_t prefix = s_digit << 21;
  uint32_t mask = 0xFFE00000u;
  remaining -= s_above;
  const uint32_t n_cand = hist[s_digit];
  const bool use_cand = n_cand <= (uint32_t)kMaxCand;
  __syncthreads();

  // 2. Digits 2 and 3, over the candidates (or over all keys if they do not fit).
  // The candidate pass also keeps, per super-round, the bit masks of this thread's keys above the
  // threshold bin and in it, and where its candidates went in `cand` (in registers for rows of one
  // super-round; in LDS for rows of up to kMaskSR, which are re-read from memory in every pass); the
  // output step then needs only those and the candidates, not another pass over every key.
  const bool keep_masks = use_cand && (CACHED || n_sr <= kMaskSR);
  // [super-round][above, cand, first cand slot][thread], in LDS: registers are at their limit here.
  __shared__ uint32_t sm_marks[CACHED ? 1 : kMaskSR * 3 * kThreads];
  auto mark = [&](int r, int f) -> uint32_t& { return sm_marks[(r * 3 + f) * kThreads + tid]; };
  struct Marks {
    uint32_t above, cand, at;
  };
  Marks reg_marks{0u, 0u, 0u};  // rows of one super-round
  if (use_cand) {
    // Each thread marks its candidates in a bit mask; one workgroup scan of the counts gives its
    // first slot in `cand` (candidates taken in position order, no atomics on a shared counter).
    uint32_t base = 0u;
    auto collect = [&](const uint32_t(&k)[kCached], const Span& sp) -> Marks {
      uint32_t cm = 0u, abv = 0u;
      for_keys(sp, [&](int i) {
        cm |= (uint32_t)((k[i] & mask) == prefix) << i;
        abv |= (uint32_t)((k[i] & mask) > prefix) << i;
      });
      cm &= sp.live;
      uint32_t total;
      uint32_t slot = base + block_exclusive_scan<kThreads>(__popc(cm), scan_lds, parity, &total);
      const Marks marks{abv & sp.live, cm, slot};
      for_keys(sp, [&](int i) {
        if ((cm >> i) & 1u) cand[slot++] = k[i];
      });
      base += total;
      return marks;
    };
    if constexpr (CACHED) {
      reg_marks = collect(keys, span);
    } else if (keep_masks) {
#pragma unroll
      for (int r = 0; r < kMaskSR; ++r)
        if (r < n_sr) {  // the same for every thread
          uint32_t kk[kCached];
          const Span sp = load_sr(r, kk);
          const Marks mk = collect(kk, sp);
          mark(r, 0) = mk.above;
          mark(r, 1) = mk.cand;
          mark(r, 2) = mk.at;
        }
    } else {
      for_sr([&](const uint32_t(&k)[kCached], const Span& sp) { (void)collect(k, sp); });
    }
  }
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const uint32_t dmask = pass == 0 ? 0x7FFu : 0x3FFu;
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
    __syncthreads();
    if (use_cand) {
      for (uint32_t i = tid; i < n_cand; i += kThreads) {
        const uint32_t key = cand[i];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      }
    } else {
      for_sr([&](const uint32_t(&k)[kCached], const Span& sp) {
        for_keys(sp, [&](int i) {
          if (((sp.live >> i) & 1u) && (k[i] & mask) == prefix) atomicAdd(&hist[(k[i] >> shift) & dmask], 1u);
        });
      });
    }
    __syncthreads();
    if (pass == 0) find_digit<2048>(hist, remaining, scan_lds, parity, &s_digit, &s_above);
    else find_digit<1024>(hist, remaining, scan_lds, parity, &s_digit, &s_above);
    // s_digit and s_above are next written by the next find_digit, after the next pass's barriers,
    // which every thread reaches only after reading them here; hist is read inside find_digit
    // before its scan's barrier, so the next pass may clear it.
    prefix |= s_digit << shift;
    mask |= dmask << shift;
    remaining -= s_above;
  }
  const uint32_t thresh = prefix;
  const uint32_t needed_eq = remaining;  // >= 1 keys equal to thresh, lowest positions first

  // 3. Output in position order (super-round, thread, bit), from each thread's masks of keys > T
  //    and == T.
  // Writes the positions p0 + (set bits of `take`, lowest first) to slots slot, slot + 1, ...
  // Stage 0 stores positions only; stages 1 and 2 also load a value per position (its score, its
  // original position): eight loads in flight before their stores, not one round trip each.
  auto emit_bits = [&](uint32_t take, uint32_t slot, int p0) {
    if (stage == 0) {
      for (; take != 0u; take &= take - 1u, ++slot) {
        const int32_t p = p0 + __ffs(take) - 1;
        for (int r = 0; r < rows; ++r) out[(size_t)r * a.topk + slot] = p;
      }
      return;
    }
    constexpr int kBatch = 8;
    while (take != 0u) {
      int pos[kBatch];
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        pos[j] = take != 0u ? p0 + __ffs(take) - 1 : p0;
        cnt += take != 0u ? 1 : 0;
        take &= take - 1u;
      }
      if (stage == 1) {
        float v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) v[j] = j < cnt ? s[pos[j]] : 0.0f;
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          if (j < cnt) {
            cand_score[slot + j] = v[j];
            cand_pos[slot + j] = pos0 + pos[j];
          }
      } else {
        int32_t v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) v[j] = j < cnt ? pos_map[pos[j]] : 0;
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          if (j < cnt) out[slot + j] = v[j];
      }
      slot += (uint32_t)cnt;
    }
  };
  uint32_t gt_seen = 0u, eq_seen = 0u;  // over earlier super-rounds
  auto emit_sr = [&](uint32_t gtm, uint32_t eqm, const Span& sp) {
    const uint32_t n_gt = __popc(gtm), n_eq = __popc(eqm);
    // One scan of both counts: per super-round each total is at most 32768, so the counts of keys
    // == T (low 16 bits) never carry into those of keys > T (high 16 bits).
    uint32_t tot;
    const uint32_t before = block_exclusive_scan<kThreads>((n_gt << 16) | n_eq, scan_lds, parity, &tot);
    const uint32_t gt_before = gt_seen + (before >> 16), eq_before = eq_seen + (before & 0xFFFFu);
    const uint32_t tot_gt = tot >> 16, tot_eq = tot & 0xFFFFu;
    // Saturating forms only: hipcc 7.2 turned a guarded `needed - before` feeding min() into an
    // unconditional one assumed not to wrap, which dropped the clamp on the slot below.
    const uint32_t room = max(needed_eq, eq_before) - eq_before;  // keys == T this thread may take
    emit_bits(gtm | lowest_bits(eqm, min(room, n_eq)), gt_before + (needed_eq - room), sp.p0);
    gt_seen += tot_gt;
    eq_seen += tot_eq;
  };
  // From the candidate pass's masks: keys above the threshold bin are kept, and candidates are
  // compared with T as `cand` holds them (this thread's, in bit order from its first slot).
  auto emit_marks = [&](uint32_t above, uint32_t cm, uint32_t at, const Span& sp) {
    uint32_t gtm = above, eqm = 0u;
    for (; cm != 0u; cm &= cm - 1u) {
      const uint32_t key = cand[at++], bit = cm & (0u - cm);
      if (key > thresh) gtm |= bit;
      else if (key == thresh) eqm |= bit;
    }
    emit_sr(gtm, eqm, sp);
  };
  if (keep_masks) {
    if constexpr (CACHED) {
      emit_marks(reg_marks.above, reg_marks.cand, reg_marks.at, span);
    } else {
#pragma unroll
      for (int r = 0; r < kMaskSR; ++r)
        if (r < n_sr) emit_marks(mark(r, 0), mark(r, 1), mark(r, 2), span_of(r));
    }
  } else {
    for_sr([&](const uint32_t(&k)[kCached], const Span& sp) {
      uint32_t gtm = 0u, eqm = 0u;
      for_keys(sp, [&](int i) {
        gtm |= (uint32_t)(k[i] > thresh) << i;
        eqm |= (uint32_t)(k[i] == thresh) << i;
      });
      emit_sr(gtm & sp.live, eqm & sp.live, sp);
    });
  }
}

}  // namespace

namespace {

template <bool MERGE>
void launch_select_kernel(const SelectArgs& a, const CombineArgs& c, int extra_blocks, hipStream_t stream) {
  const int groups = a.shared ? a.batch : a.batch * a.kv_heads * (a.stage == 1 ? a.nchunks : 1);
  const dim3 grid(groups + extra_blocks), block(kThreads);
  const int row_len = a.shared || a.stage == 0 ? a.max_len : (a.stage == 1 ? a.chunk : a.cand_stride);
  const bool cached = row_len <= kPerSuper;
  if (a.shared) {
    if (cached) select_topk_kernel<true, true, MERGE><<<grid, block, 0, stream>>>(a, c);
    else select_topk_kernel<false, true, MERGE><<<grid, block, 0, stream>>>(a, c);
  } else {
    if (cached) select_topk_kernel<true, false, MERGE><<<grid, block, 0, stream>>>(a, c);
    else select_topk_kernel<false, false, MERGE><<<grid, block, 0, stream>>>(a, c);
  }
}

}  // namespace

bool select_two_stage(int max_len, int topk, int* chunk, int* nchunks) {
  // From three chunks up: each launch has a fixed cost (its serial phases on one CU), which two
  // chunks' parallel first stage barely wins back (36000 to 65536 positions: 2-10 % faster in two
  // launches for k <= 2048, 10-20 % slower for k = 4096); at 102400 positions two launches take
  // 29 us against 47 us in one.
  if (max_len <= 2 * kPerSuper || topk < 1) return false;
  const int nc = (max_len + kPerSuper - 1) / kPerSuper;
  // Equal chunks, each a multiple of 4 positions (16-byte aligned loads) and at most one super-round.
  int c = (max_len + nc - 1) / nc;
  c = (c + 3) / 4 * 4;
  if (c > kPerSuper) return false;
  const int n = (max_len + c - 1) / c;
  if ((int64_t)n * topk > kPerSuper) return false;  // candidate row longer than one super-round
  *chunk = c;
  *nchunks = n;
  return true;
}

// Stage arguments that the kernel's indexing relies on.
bool stage_args_ok(const SelectArgs& a) {
  if (a.stage == 0) return true;
  if (a.stage != 1 && a.stage != 2) return false;
  if (a.shared || a.unit_k || !a.cand_score || !a.cand_pos) return false;
  if (a.chunk < 4 || a.chunk % 4 != 0 || a.chunk > kPerSuper || a.nchunks < 1) return false;
  if ((int64_t)a.chunk * a.nchunks < a.max_len) return false;
  if (a.cand_stride % 4 != 0 || a.cand_stride > kPerSuper || (int64_t)a.nchunks * a.topk > a.cand_stride) return false;
  return (int64_t)a.batch * a.kv_heads * a.nchunks <= 0x7fffffff;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  if (!stage_args_ok(a)) return hipErrorInvalidValue;
  launch_select_kernel<false>(a, CombineArgs{}, 0, stream);
  return hipGetLastError();
}

hipError_t launch_select_merge(const SelectArgs& a, const CombineArgs& c, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  if (c.rows <= 0) return launch_select(a, stream);
  if (!stage_args_ok(a)) return hipErrorInvalidValue;
  if (c.splits < 1 || c.splits > kMaxSplitsPerUnit) return hipErrorInvalidValue;
  if (c.head_dim != 64 && c.head_dim != 128) return hipErrorInvalidValue;
  launch_select_kernel<true>(a, c, (c.rows + kWaves - 1) / kWaves, stream);
  return hipGetLastError();
}

}  // namespace ppsa
