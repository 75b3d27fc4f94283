// Full-attention split pass on the matrix cores (gfx950, bf16, head_dim 128): the full and
// full + selection layers of the decode step.
//
// Same contract as the vector-ALU pass (attn_valu.hip): per query head of a KV group,
// softmax(q K^T * scale) V (TidalDecode review page, section 3, PPSA paragraph, attention
// equation) over one split of cache rows, in order, as a partial for the merge pass (combine.hip),
// or as the output when the unit has a single split. Selection layers also write each live
// position's score, the group-summed raw logit (section 2: tokens ranked by attention score; the
// sum over the group is this library's reading for grouped heads), staged in LDS and written once
// per split; the softmax-weight variant additionally writes every head's logit.
//
// The tile math (two matrix-core products per 32 rows, lazy-rescaled online softmax) is in
// mfma_tile.h. Full launches load K straight into the A-operand layout (the four lanes of a row
// group read 64 contiguous bytes) and V as whole rows.
#include <math.h>

#include "attn_epilogue.h"
#include "device_common.h"
#include "mfma_tile.h"
#include "ppsa_internal.h"
#include "ppsa.h"

namespace ppsa {
namespace {

using namespace mt;

constexpr int kWaves = 4;                      // waves per workgroup, multi-split launches
constexpr int kWavesSingle = 8;                // one split per unit: fewer, longer workgroups
constexpr int kRowsTrip = kTile * kWaves;
// Scores of a full+scores split are gathered in LDS and written once the split is done (one
// coalesced pass instead of a few bytes per tile amid the K/V stream, which cost 10-15 % of the
// layer); a split's LDS (wave outputs + scores) stays within 64 KiB.
constexpr size_t kMaxLdsBytes = 65536;

// Floats of LDS per wave: its partial output (group heads x kD).
__host__ __device__ constexpr int wave_region_floats(int group) { return group * kD; }

// Full launches: cache rows in order, K straight into the operand layout (lane (g, n): row
// 16 blk + n, bytes 16g + 64c), V as whole rows (lane (g, n): rows 16 blk + 4g + i, bytes 16n).
// Slots past the live rows repeat the last live row and stay invalid.
template <bool STREAM>
__device__ __forceinline__ void load_tile_rows(Tile& t, const char* kb, const char* vb, int tslot, int slot_end,
                                               int g, int n) {
  t.valid = 0u;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    {
      const int slot = tslot + 16 * blk + n;
      const int row = slot < slot_end ? slot : slot_end - 1;
      const uint32_t off = (uint32_t)row * (kD * 2) + 16u * g;
#pragma unroll
      for (int c = 0; c < 4; ++c) t.k[blk][c] = load16<STREAM>(kb, off + 64u * c);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = tslot + 16 * blk + 4 * g + i;
      const bool ok = slot < slot_end;
      const int row = ok ? slot : slot_end - 1;
      t.valid |= (uint32_t)ok << (4 * blk + i);
      t.v[blk][i] = load16<STREAM>(vb, (uint32_t)row * (kD * 2) + 16u * n);
    }
  }
}

template <int MODE, int WAVES, bool STREAM>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(2))) void attn_mfma_kernel(AttnArgs a) {
  constexpr int kThreads = WAVES * kWave;
  constexpr bool kScores = MODE == MODE_FULL_SCORES || MODE == MODE_FULL_HEADS;
  // [WAVES] x (wave region) wave outputs, then the staged scores (selection layers).
  extern __shared__ __attribute__((aligned(16))) float dyn[];  // 16-byte aligned: read and written as float4
  __shared__ float sm_m[WAVES][kMaxGroup];
  __shared__ float sm_l[WAVES][kMaxGroup];
  const int group = a.group;
  const int wstride = wave_region_floats(group);
  float* sm_o = dyn;
  float* sm_sc = dyn + WAVES * wstride;

  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = lane / 16, n = lane % 16;

  const int n_live = min(max(a.seq_lens[b], 0), a.max_len);
  const size_t unit = (size_t)b * a.kv_heads + kv;
  // Unit bases; rows are addressed by 32-bit byte offsets (Nmax * 256 bytes < 4 GiB).
  const char* kb = reinterpret_cast<const char*>(a.k) + unit * (size_t)a.max_len * kD * 2;
  const char* vb = reinterpret_cast<const char*>(a.v) + unit * (size_t)a.max_len * kD * 2;
  const int slot0 = split * a.rows_per_split;
  const int slot_end = n_live == 0 ? slot0 : min(slot0 + a.rows_per_split, n_live);

  // q fragments: head n, dims 32c + 8g .. +8, zero for heads past the group (the score sum over
  // the sixteen head columns relies on those zeros).
  bf16x8_t qf[4];
  load_q(qf, reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.q_heads + (size_t)kv * group) * kD, group, g, n);

  Online st;
  online_init(st);

  const int rows = slot_end - slot0;
  const int ntiles = (rows + kTile - 1) / kTile;
  auto process = [&](const Tile& cur, int ti) {
    float4_t s[2];
    qk_logits(cur, qf, s);  // logits of rows 16*blk + 4g + j for head n
    if constexpr (kScores) {
      // Lane (g, 0) holds the sums of rows 16 blk + 4g .. +3: one 16-byte LDS write per block (four
      // single-float writes per block cost 5 % of a selection layer at the LLaMA-2-7B 100K shape).
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        float tot[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) tot[j] = group_sum<16>(s[blk][j]) * a.scale;  // heads past the group add exact zeros
        if (n == 0)
          *reinterpret_cast<float4*>(sm_sc + ti * kTile + 16 * blk + 4 * g) = make_float4(tot[0], tot[1], tot[2], tot[3]);
      }
    }
    float x[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[blk][j] = ((cur.valid >> (4 * blk + j)) & 1u) ? s[blk][j] * a.scale_log2 : -INFINITY;
    if constexpr (MODE == MODE_FULL_HEADS) {
      // Every query head's logit of the tile's live rows: lane (g, n < group) holds rows 16 blk + 4g + j,
      // four consecutive rows: one 16-byte store when all four are live and the row start allows it.
      if (n < group) {
        float* hl = a.head_logits + ((size_t)b * a.q_heads + (size_t)kv * group + n) * a.max_len + slot0 + ti * kTile;
        const bool vec = (a.max_len % 4) == 0 && (reinterpret_cast<uintptr_t>(a.head_logits) % 16) == 0;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          float* p = hl + 16 * blk + 4 * g;
          if (vec && ((cur.valid >> (4 * blk)) & 0xFu) == 0xFu) {
            *reinterpret_cast<float4*>(p) = make_float4(x[blk][0], x[blk][1], x[blk][2], x[blk][3]);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if ((cur.valid >> (4 * blk + j)) & 1u) p[j] = x[blk][j];
          }
        }
      }
    }
    softmax_pv(cur, x, st, g);
  };

  // One tile in flight per wave; occupancy (several waves per SIMD) hides the latency. Two
  // tiles per wave at two waves per SIMD, and a software-pipelined loop, measured slower.
  for (int ti = wave; ti < ntiles; ti += WAVES) {
    Tile t;
    load_tile_rows<STREAM>(t, kb, vb, slot0 + ti * kTile, slot_end, g, n);
    process(t, ti);
  }

  // Wave result: head n's max and normaliser; O rows are heads 4g + j, dims 8n + t.
  const float l_tot = sum_rows4(st.l_run);
  if (g == 0 && n < group) {
    sm_m[wave][n] = st.m_run;
    sm_l[wave][n] = l_tot;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * g + j;
    if (h < group) {
      float* dst = sm_o + wave * wstride + h * kD + 8 * n;
#pragma unroll
      for (int t = 0; t < 8; ++t) dst[t] = st.acc[t][j];
    }
  }
  __syncthreads();
  if constexpr (kScores) {
    // 16 bytes per thread and instruction when the row start allows it (a multiple of 4 positions
    // from a 16-byte aligned base), then the tail.
    float* dst = a.scores + unit * (size_t)a.max_len + slot0;
    const int nrow = slot_end - slot0;
    const bool vec = (a.max_len % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) % 16) == 0;
    const int nvec = vec ? nrow / 4 : 0;
    for (int i = tid; i < nvec; i += kThreads)
      reinterpret_cast<float4*>(dst)[i] = reinterpret_cast<const float4*>(sm_sc)[i];
    for (int i = 4 * nvec + tid; i < nrow; i += kThreads) dst[i] = sm_sc[i];
  }

  // Per head, once: the largest wave max M, each wave's weight 2^(m_w - M) (written over m_w) and
  // the merged normaliser, so that each output element is a plain weighted sum over the waves.
  __shared__ float sm_hm[kMaxGroup], sm_hl[kMaxGroup];
  if (tid < group) {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) mx = fmaxf(mx, sm_m[w][tid]);
    const float ms = mx == -INFINITY ? 0.0f : mx;
    float lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float c = exp2_fast(sm_m[w][tid] - ms);
      sm_m[w][tid] = c;
      lsum += sm_l[w][tid] * c;
    }
    sm_hm[tid] = mx;
    sm_hl[tid] = lsum;
  }
  __syncthreads();

  const bool single = a.splits == 1;
  for (int i = tid; i < group * kD; i += kThreads) {
    const int h = i / kD, d = i % kD;
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) o += sm_o[w * wstride + h * kD + d] * sm_m[w][h];
    const float lsum = sm_hl[h];
    if (single) {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((size_t)b * a.q_heads + (size_t)kv * group + h) * kD + d;
      store_elem(op, lsum > 0.0f ? o / lsum : 0.0f);
      continue;
    }
    const size_t row = part_row(a, b, kv, h, split);
    a.part_o[row * kD + d] = o;
    if (d == 0) {
      a.part_m[row] = sm_hm[h];
      a.part_l[row] = lsum;
    }
  }
}

}  // namespace

int attn_mfma_rows_granule() { return kRowsTrip; }
int attn_mfma_max_score_rows(int group) {
  return (int)((kMaxLdsBytes - (size_t)kWaves * group * kD * sizeof(float)) / sizeof(float)) / kRowsTrip * kRowsTrip;
}

bool attn_mfma_supported(int dtype, int head_dim, int group) {
  return dtype == PPSA_BF16 && head_dim == kD && group >= 1 && group <= kMaxGroup;
}

namespace {

template <int WAVES, bool STREAM>
hipError_t launch_waves(const AttnArgs& a, int mode, size_t lds, hipStream_t stream) {
  const dim3 grid(a.splits, a.kv_heads, a.batch), block(WAVES * kWave);
  switch (mode) {
    case MODE_FULL: attn_mfma_kernel<MODE_FULL, WAVES, STREAM><<<grid, block, lds, stream>>>(a); break;
    case MODE_FULL_SCORES: attn_mfma_kernel<MODE_FULL_SCORES, WAVES, STREAM><<<grid, block, lds, stream>>>(a); break;
    case MODE_FULL_HEADS: attn_mfma_kernel<MODE_FULL_HEADS, WAVES, STREAM><<<grid, block, lds, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Dynamic LDS of a launch: wave partial outputs, then the staged sparse positions or scores.
size_t lds_bytes(const AttnArgs& a, int mode, int waves) {
  size_t lds = (size_t)waves * wave_region_floats(a.group) * sizeof(float);
  if (mode == MODE_FULL_SCORES || mode == MODE_FULL_HEADS) lds += (size_t)a.rows_per_split * 4;
  return lds;
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, int mode, hipStream_t stream) {
  if (a.splits <= 0 || a.batch <= 0) return hipSuccess;
  if (mode != MODE_FULL && mode != MODE_FULL_SCORES && mode != MODE_FULL_HEADS) return hipErrorInvalidValue;
  if ((mode == MODE_FULL_SCORES || mode == MODE_FULL_HEADS) && lds_bytes(a, mode, kWaves) > kMaxLdsBytes)
    return hipErrorInvalidValue;
  // One split per unit means one workgroup per unit: twice the waves keep more rows in flight per CU
  // (measured 8-10 % faster there), while LDS stays within 64 KiB.
  if (a.splits == 1) {
    if (lds_bytes(a, mode, kWavesSingle) <= kMaxLdsBytes)
      return launch_waves<kWavesSingle, false>(a, mode, lds_bytes(a, mode, kWavesSingle), stream);
    return launch_waves<kWaves, false>(a, mode, lds_bytes(a, mode, kWaves), stream);
  }
  return launch_waves<kWaves, true>(a, mode, lds_bytes(a, mode, kWaves), stream);
}

}  // namespace ppsa
