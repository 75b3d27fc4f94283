// PPSA sparse attention layer on the matrix cores (gfx950, bf16, head_dim 128).
//
// A sparse layer attends, for each (batch row, KV head) unit and each query head of its group, to
// the cache rows the unit's most recent selection layer chose: softmax(q K[idx]^T * scale) V[idx],
// renormalised over the selected rows (TidalDecode review page, section 3, PPSA paragraph: later
// layers reuse the positions chosen at the selection layer and load only those tokens; the
// attention equation of the same paragraph). Slots past the live length, or holding -1, are
// skipped.
//
// Work split: a unit's slots are cut into `splits` runs of rows_per_split slots, one workgroup
// each; each wave walks 32-slot tiles (mfma_tile.h). Slot positions are read straight into
// registers (no LDS staging, no barrier before the first K/V request) and the next tile's
// positions are requested while the current tile's rows are in flight. K and V rows are loaded
// whole (four 256-byte rows per load instruction); K reaches the operand layout through a
// wave-private LDS block.
//
// A unit with one split writes its output directly; with several splits each workgroup leaves a
// partial (max m, normaliser l, weighted sum o per query head of the group) for the merge pass
// (combine.hip). (A merge inside this kernel by the last-arriving workgroup of a unit was measured
// slower than the separate pass at every workload shape: that workgroup's partial stores, arrival
// count and partial loads form a chain of memory round trips while the gather still saturates the
// memory system.)
#include <math.h>

#include "attn_epilogue.h"
#include "device_common.h"
#include "mfma_tile.h"
#include "sparse_gather.h"
#include "ppsa_internal.h"
#include "ppsa.h"

namespace ppsa {
namespace {

using namespace mt;

constexpr int kWaves = 4;          // multi-split launches: two workgroups per CU
constexpr int kWavesSingle = 8;    // one split per unit: one long workgroup per unit
constexpr int kORow = kD + 4;      // floats per head row of a wave's partial output in LDS (bank spread)
constexpr int kMaxRowsPerSplit = 1 << 20;

__host__ __device__ constexpr int wave_floats(int group) {
  return kKBlockBytes / 4 > group * kORow ? kKBlockBytes / 4 : group * kORow;
}

__device__ __forceinline__ void store_out4(uint16_t* p, float4_t o, float inv) {
  *reinterpret_cast<uint2*>(p) = make_uint2(bf16_pair(o[0] * inv, o[1] * inv), bf16_pair(o[2] * inv, o[3] * inv));
}

template <int WAVES, bool STREAM>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(2))) void attn_sparse_kernel(AttnArgs a) {
  constexpr int kThreads = WAVES * kWave;
  extern __shared__ __attribute__((aligned(16))) float dyn[];  // [WAVES] wave regions: K block during the tile loop, then the wave's O
  __shared__ float sm_m[WAVES][kMaxGroup];
  __shared__ float sm_l[WAVES][kMaxGroup];
  const int group = a.group, S = a.splits;
  const int unit = blockIdx.x / S, split = blockIdx.x - unit * S;
  const int b = unit / a.kv_heads, kv = unit - b * a.kv_heads;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: branches on it stay scalar
  const int g = lane / 16, n = lane % 16;
  const int wstride = wave_floats(group);

  // Slot entries and q first: with the live length they are all the first K/V requests wait for.
  const int32_t* ip = a.idx + (size_t)unit * a.kslots;
  const int slot0 = split * a.rows_per_split;
  const int nrows = max(min(a.rows_per_split, a.kslots - slot0), 0);
  const __amdgpu_buffer_rsrc_t r_idx = rsrc(ip + slot0, (uint32_t)nrows * 4u);
  const bool vec = a.idx_vec != 0;
  const int ntiles = (nrows + kTile - 1) / kTile;
  int raw[2][4];
  if (wave < ntiles) fetch_positions(raw, r_idx, wave * kTile, vec, g);
  // q fragments of head n (heads past the group read the group's first head: their columns of the
  // products are never combined with real heads and never written).
  bf16x8_t qf[4];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((size_t)b * a.q_heads + (size_t)kv * group + (n < group ? n : 0)) * kD;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + 32 * c + 8 * g));
  }
  const int n_live = min(max(a.seq_lens[b], 0), a.max_len);
  const char* kb = reinterpret_cast<const char*>(a.k) + (size_t)unit * a.max_len * kRowBytes;
  const char* vb = reinterpret_cast<const char*>(a.v) + (size_t)unit * a.max_len * kRowBytes;

  Online st;
  online_init(st);
  char* kbuf = reinterpret_cast<char*>(dyn + wave * wstride);
  // A unit with no live row has nothing to gather (its invalid slots would read padding rows, which
  // may hold anything: even a zero weight times a NaN is NaN).
  const int ntiles_live = n_live > 0 ? ntiles : 0;
  auto compute = [&](Tile& t) {
    k_to_operand(t, kbuf, g, n);
    float4_t s[2];
    qk_logits(t, qf, s);
    float x[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[blk][j] = ((t.valid >> (4 * blk + j)) & 1u) ? s[blk][j] * a.scale_log2 : -INFINITY;
    softmax_pv(t, x, st, g);
  };
  // One tile in flight per wave; occupancy (several waves per SIMD) hides the latency. The next
  // tile's slot entries are requested right behind this tile's rows. (Two tiles in flight per wave
  // measured slower: 8 % at the LLaMA-3-8B 32K shape, 13 % for one-split launches of 512 slots.)
  for (int ti = wave; ti < ntiles_live; ti += WAVES) {
    Tile t;
    load_gathered<STREAM>(t, kb, vb, raw, ti * kTile, nrows, n_live, g, n);
    if (ti + WAVES < ntiles_live) fetch_positions(raw, r_idx, (ti + WAVES) * kTile, vec, g);
    compute(t);
  }

  // Wave result to LDS: head n's max and normaliser; O rows (heads 4g + j, dims 8n + t) as two
  // 16-byte pieces per head, rows padded to kORow floats.
  const float l_tot = sum_rows4(st.l_run);
  if (g == 0 && n < group) {
    sm_m[wave][n] = st.m_run;
    sm_l[wave][n] = l_tot;
  }
  float* wo = dyn + wave * wstride;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * g + j;
    if (h < group) {
      *reinterpret_cast<float4_t*>(wo + h * kORow + 8 * n) =
          float4_t{st.acc[0][j], st.acc[1][j], st.acc[2][j], st.acc[3][j]};
      *reinterpret_cast<float4_t*>(wo + h * kORow + 8 * n + 4) =
          float4_t{st.acc[4][j], st.acc[5][j], st.acc[6][j], st.acc[7][j]};
    }
  }
  __syncthreads();

  // Workgroup result: thread i < group * 32 takes head i / 32, dims 4 (i % 32) .. +3, and combines
  // the waves with their weights 2^(m_w - M). group * 32 <= 512 items: at most two per thread.
  const int nq = group * (kD / 4);
  const size_t row0 = (size_t)b * a.q_heads + (size_t)kv * group;  // (b, first head of the group)
  auto combine = [&](int i) {
    const int h = i >> 5, d = (i & 31) * 4;
    float mw[WAVES], mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      mw[w] = sm_m[w][h];
      mx = fmaxf(mx, mw[w]);
    }
    float4_t ow[WAVES];
#pragma unroll
    for (int w = 0; w < WAVES; ++w) ow[w] = *reinterpret_cast<const float4_t*>(dyn + w * wstride + h * kORow + d);
    const float ms = mx == -INFINITY ? 0.0f : mx;
    float l = 0.0f;
    float4_t o = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float c = exp2_fast(mw[w] - ms);
      l += sm_l[w][h] * c;
      o += ow[w] * c;
    }
    if (S == 1) {
      store_out4(reinterpret_cast<uint16_t*>(a.out) + (row0 + h) * kD + d, o, l > 0.0f ? 1.0f / l : 0.0f);
      return;
    }
    const size_t row = part_row(a, b, kv, h, split);
    *reinterpret_cast<float4_t*>(a.part_o + row * kD + d) = o;
    if (d == 0) {
      a.part_m[row] = mx;
      a.part_l[row] = l;
    }
  };
  if (tid < nq) combine(tid);
  if (kThreads < kMaxGroup * (kD / 4) && tid + kThreads < nq) combine(tid + kThreads);
}

template <int WAVES, bool STREAM>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)WAVES * wave_floats(a.group) * sizeof(float);
  attn_sparse_kernel<WAVES, STREAM><<<dim3(a.batch * a.kv_heads * a.splits), dim3(WAVES * kWave), lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

int attn_sparse_waves(const AttnArgs& a) {
  // One split per unit means one workgroup per unit: twice the waves keep more rows in flight per
  // CU while the LDS stays within 64 KiB.
  return a.splits == 1 && (size_t)kWavesSingle * wave_floats(a.group) * sizeof(float) <= 65536 ? kWavesSingle
                                                                                               : kWaves;
}

hipError_t launch_attn_sparse(const AttnArgs& a, hipStream_t stream) {
  if (a.splits <= 0 || a.batch <= 0 || a.kv_heads <= 0) return hipSuccess;
  if (a.group < 1 || a.group > kMaxGroup || a.rows_per_split <= 0 || a.rows_per_split > kMaxRowsPerSplit)
    return hipErrorInvalidValue;
  if ((int64_t)a.splits * a.rows_per_split < a.kslots) return hipErrorInvalidValue;
  if ((int64_t)a.batch * a.kv_heads * a.splits > 0x7fffffff) return hipErrorInvalidValue;
  // Several splits per unit stream (nontemporal loads: bandwidth-bound); one split is bound by
  // latency and loads plainly.
  if (a.splits == 1)
    return attn_sparse_waves(a) == kWavesSingle ? launch_cfg<kWavesSingle, false>(a, stream)
                                                : launch_cfg<kWaves, false>(a, stream);
  return launch_cfg<kWaves, true>(a, stream);
}

}  // namespace ppsa
