// Split attention pass on the matrix cores (gfx950, bf16, head_dim 128).
//
// Same contract as the vector-ALU pass (attn_valu.hip): per query head of a
// KV group, softmax(q K^T * scale) V (TidalDecode review page, section 3,
// PPSA paragraph, attention equation) over one split of rows -- cache rows
// in order (full, full+scores) or the rows listed in idx (sparse) -- as a
// partial for the merge pass (combine.hip), or as the output when the unit
// has a single split.
//
// All query heads of a KV group share every K and V row, so the group's
// logits for 16 rows are one 16x16 matrix product and the weighted V sum is
// another; both go to the MFMA units, with up to 16 heads per group (heads
// past the group size are zero columns). Each wave walks tiles of 32 rows
// (two blocks of 16):
//   S^T[row, head] = K[row, :] . q[head, :]
//       v_mfma_f32_16x16x32_bf16, A = K (lane%16 = row, lane/16 picks 8 of
//       each 32 dims), B = q (lane%16 = head); four products cover d = 128.
//       Full launches load K straight into that layout (the four lanes of a
//       row group read 64 contiguous bytes); sparse launches load gathered K
//       rows whole, like V below, and regroup them through LDS.
//   The result leaves lane (g = lane/16, n = lane%16) holding the logits of
//   rows 4g..4g+3 for head n, which is exactly the A operand layout of
//   v_mfma_f32_16x16x16_bf16 for P[head, row] over those 16 rows, so the
//   softmax weights never leave the lane.
//   O[head, dim] += P[head, :] . V[:, dim]
//       B = V needs rows along the operand elements: lane (g, n) loads rows
//       4g..4g+3 at dims 8n..8n+7 (16 lanes read whole 256-byte rows) and
//       product t uses dim 8n+t of each, regrouped with v_perm_b32. The
//       output column n of product t is dim 8n+t.
// The running max is shared by the four lanes holding a head (two xor
// shuffles per tile) and only moved when a tile exceeds it by more than
// 2^8 ("lazy" rescaling: weights may reach 256, still exact in the float32
// sums); the merge uses each partial's own max, so the result is the same
// softmax. Weights are rounded to bf16 for the product and the normaliser
// sums the rounded weights, so numerator and denominator match.
#include <math.h>

#include "attn_epilogue.h"
#include "device_common.h"
#include "ppsa_internal.h"
#include "ppsa.h"

namespace ppsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;                      // waves per workgroup, multi-split launches
constexpr int kWavesSingle = 8;                // one split per unit: fewer, longer workgroups
constexpr int kD = 128;
constexpr int kTile = 32;
constexpr int kRowsTrip = kTile * kWaves;
constexpr int kMaxSparseRowsMfma = 2048;
// Scores of a full+scores split are gathered in LDS and written once the split is done (one
// coalesced pass instead of a few bytes per tile amid the K/V stream, which cost 10-15 % of the
// layer); a split's LDS (wave outputs + scores) stays within 64 KiB.
constexpr size_t kMaxLdsBytes = 65536;
constexpr float kLazyLog2 = 8.0f;
// Sparse launches load K rows whole (four 256-byte rows per load instruction, the V pattern) and
// move them into the matrix-core operand layout through a wave-private LDS buffer of one 16-row
// block, padded to 272 bytes per row so that the sixteen rows one read instruction touches fall on
// distinct banks. A gathered row read as sixteen quarter rows per instruction (the direct operand
// layout) measured 1.1 us slower per 64 MiB layer in a load-only probe.
constexpr int kKRowPitch = kD * 2 + 16;
constexpr int kKBlockBytes = 16 * kKRowPitch;  // 4352 bytes per wave

// Floats of LDS per wave: its output (group heads x kD), or its K block when that is larger.
__host__ __device__ constexpr int wave_region_floats(bool kt, int group) {
  return kt && kKBlockBytes / 4 > group * kD ? kKBlockBytes / 4 : group * kD;
}

struct Tile {
  uint4 k[2][4];    // [block][c]: K[row 16*blk + n][32c + 8g .. +8] (sparse: once k_to_operand has run)
  uint4 v[2][4];    // [block][i]: V[row 16*blk + 4g + i][8n .. +8]
  uint32_t valid;   // bit 4*blk + i: row 16*blk + 4g + i is live
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return (uint32_t)bf16_round(lo) | ((uint32_t)bf16_round(hi) << 16);
}

// 16 bytes of a K or V row at a byte offset from a base every lane shares: 32-bit offsets let
// the loads use a scalar base plus one vector register per address. Rows are read once per
// layer; launches that stream (several splits per unit, bandwidth-bound) load with the
// nontemporal hint (measured on MI355X: a 512 MiB stream reads at 6.9 TB/s with it, 6.1 TB/s
// without), while one-split launches, bound by latency, were slower with it and load plainly.
template <bool STREAM>
__device__ __forceinline__ uint4 load16(const char* base, uint32_t off) {
  if constexpr (STREAM) {
    const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + off));
    return make_uint4(w.x, w.y, w.z, w.w);
  } else {
    return *reinterpret_cast<const uint4*>(base + off);
  }
}

// Sparse launches: K and V rows alike, whole rows per load instruction; lane (g, n) loads bytes
// 16n .. 16n+15 of rows 16 blk + 4g + i (the slots' positions, staged in LDS; -1 marks a slot
// with nothing to read, which loads row 0 and stays invalid). k_to_operand then moves K into the
// operand layout.
template <bool STREAM>
__device__ __forceinline__ void load_tile_gathered(Tile& t, const char* kb, const char* vb, int tslot, int slot0,
                                                   int slot_end, const int32_t* rows, int g, int n) {
  t.valid = 0u;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = tslot + 16 * blk + 4 * g + i;
      const int p = slot < slot_end ? rows[slot - slot0] : -1;
      const bool ok = p >= 0;
      const uint32_t off = (uint32_t)(ok ? p : 0) * (kD * 2) + 16u * n;
      t.valid |= (uint32_t)ok << (4 * blk + i);
      t.k[blk][i] = load16<STREAM>(kb, off);
      t.v[blk][i] = load16<STREAM>(vb, off);
    }
}

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

__device__ __forceinline__ uint32_t word(const uint4& u, int w) {
  return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

// Whole-row K pieces (lane (g, n): rows 16 blk + 4g + i, bytes 16n ..) to the operand layout
// (lane (g, n): row 16 blk + n, bytes 16g + 64c ..) through the wave's own 16-row LDS buffer, one
// block after the other. LDS instructions of one wave execute in order, so each read sees the
// writes before it and each write comes after the reads of the previous block.
__device__ __forceinline__ void k_to_operand(Tile& t, char* kbuf, int g, int n) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(kbuf + (4 * g + i) * kKRowPitch + 16 * n) = t.k[blk][i];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < 4; ++c)
      t.k[blk][c] = *reinterpret_cast<const uint4*>(kbuf + n * kKRowPitch + 16 * g + 64 * c);
    __builtin_amdgcn_wave_barrier();
  }
}

template <int MODE, int WAVES, bool STREAM>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(2))) void attn_mfma_kernel(AttnArgs a) {
  constexpr int kThreads = WAVES * kWave;
  constexpr bool kScores = MODE == MODE_FULL_SCORES || MODE == MODE_FULL_HEADS;
  constexpr bool KT = MODE == MODE_SPARSE;  // K rows through the per-wave LDS buffer
  // [WAVES] x (wave region) wave outputs -- with KT each wave's region is also its K block buffer,
  // reused for the output once the tile loop is done -- then the staged sparse positions or scores.
  extern __shared__ float dyn[];
  __shared__ float sm_m[WAVES][kMaxGroup];
  __shared__ float sm_l[WAVES][kMaxGroup];
  const int group = a.group;
  const int wstride = wave_region_floats(KT, group);
  float* sm_o = dyn;
  int32_t* sm_rows = reinterpret_cast<int32_t*>(dyn + WAVES * wstride);  // sparse mode
  float* sm_sc = dyn + WAVES * wstride;                                        // full+scores mode

  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = lane / 16, n = lane % 16;

  const int n_live = min(max(a.seq_lens[b], 0), a.max_len);
  const size_t unit = (size_t)b * a.kv_heads + kv;
  // Unit bases; rows are addressed by 32-bit byte offsets (Nmax * 256 bytes < 4 GiB).
  const char* kb = reinterpret_cast<const char*>(a.k) + unit * (size_t)a.max_len * kD * 2;
  const char* vb = reinterpret_cast<const char*>(a.v) + unit * (size_t)a.max_len * kD * 2;
  const int slot0 = split * a.rows_per_split;
  int slot_end = MODE == MODE_SPARSE ? min(slot0 + a.rows_per_split, a.kslots)
                                     : min(slot0 + a.rows_per_split, n_live);
  if (n_live == 0) slot_end = slot0;

  if constexpr (MODE == MODE_SPARSE) {
    const int32_t* ip = a.idx + unit * (size_t)a.kslots;
    for (int i = tid; i < slot_end - slot0; i += kThreads) {
      const int p = ip[slot0 + i];
      sm_rows[i] = (p >= 0 && p < n_live) ? p : -1;
    }
    __syncthreads();
  }

  // q fragments: head n, dims 32c + 8g .. +8 (zero for heads past the group).
  bf16x8_t qf[4];
  {
    const int hn = n < group ? n : 0;  // address a real head; zero the padding heads after the load
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.q_heads + (size_t)kv * group + hn) * kD;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 w = *reinterpret_cast<const uint4*>(qp + 32 * c + 8 * g);
      if (n >= group) w = make_uint4(0u, 0u, 0u, 0u);
      qf[c] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  float4_t acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY;  // per head n, shared by the four lanes of that head
  float l_run = 0.0f;       // this lane's rows only

  const int rows = slot_end - slot0;
  const int ntiles = (rows + kTile - 1) / kTile;
  auto process = [&](const Tile& cur, int ti) {
    // Logits of rows 16*blk + 4g + j for head n.
    float4_t s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[blk][c]), qf[c],
                                                         s[blk], 0, 0, 0);
    }
    if constexpr (kScores) {
      const int tslot = slot0 + ti * kTile;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float tot = group_sum<16>(s[blk][j]);  // heads past the group contribute exact zeros
          if (n == 0) sm_sc[tslot - slot0 + 16 * blk + 4 * g + j] = tot * a.scale;
        }
    }
    float x[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[blk][j] = ((cur.valid >> (4 * blk + j)) & 1u) ? s[blk][j] * a.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, x[blk][j]);
      }
    if constexpr (MODE == MODE_FULL_HEADS) {
      // Every query head's logit of the tile's live rows: lane (g, n < group) holds rows 16 blk + 4g + j.
      if (n < group) {
        float* hl = a.head_logits + ((size_t)b * a.q_heads + (size_t)kv * group + n) * a.max_len + slot0 + ti * kTile;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if ((cur.valid >> (4 * blk + j)) & 1u) hl[16 * blk + 4 * g + j] = x[blk][j];
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const bool need = tmax > m_run + kLazyLog2;
    if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
      const float m_new = need ? fmaxf(m_run, tmax) : m_run;
      const float alpha = m_new == m_run ? 1.0f : exp2_fast(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float aj = __shfl(alpha, 4 * g + j);  // lane 4g+j holds head 4g+j
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t][j] *= aj;
      }
      m_run = m_new;
    }
    const float ms = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      uint32_t p01 = bf16_pair(exp2_fast(x[blk][0] - ms), exp2_fast(x[blk][1] - ms));
      uint32_t p23 = bf16_pair(exp2_fast(x[blk][2] - ms), exp2_fast(x[blk][3] - ms));
      l_run += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
      const short4_t pa = __builtin_bit_cast(short4_t, make_uint2(p01, p23));
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t d0 = __builtin_amdgcn_perm(word(cur.v[blk][1], t >> 1), word(cur.v[blk][0], t >> 1), sel);
        const uint32_t d1 = __builtin_amdgcn_perm(word(cur.v[blk][3], t >> 1), word(cur.v[blk][2], t >> 1), sel);
        const short4_t vbv = __builtin_bit_cast(short4_t, make_uint2(d0, d1));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vbv, acc[t], 0, 0, 0);
      }
    }
  };

  // One tile in flight per wave; occupancy (several waves per SIMD) hides the latency. Two
  // tiles per wave at two waves per SIMD, and a software-pipelined loop, measured slower.
  for (int ti = wave; ti < ntiles; ti += WAVES) {
    Tile t;
    if constexpr (KT) {
      load_tile_gathered<STREAM>(t, kb, vb, slot0 + ti * kTile, slot0, slot_end, sm_rows, g, n);
      k_to_operand(t, reinterpret_cast<char*>(sm_o + wave * wstride), g, n);
    } else {
      load_tile_rows<STREAM>(t, kb, vb, slot0 + ti * kTile, slot_end, g, n);
    }
    process(t, ti);
  }

  // Wave result: head n's max and normaliser; O rows are heads 4g + j, dims 8n + t.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (g == 0 && n < group) {
    sm_m[wave][n] = m_run;
    sm_l[wave][n] = l_tot;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * g + j;
    if (h < group) {
      float* dst = sm_o + wave * wstride + h * kD + 8 * n;
#pragma unroll
      for (int t = 0; t < 8; ++t) dst[t] = acc[t][j];
    }
  }
  __syncthreads();
  if constexpr (kScores) {
    float* dst = a.scores + unit * (size_t)a.max_len + slot0;
    for (int i = tid; i < slot_end - slot0; i += kThreads) dst[i] = sm_sc[i];
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
int attn_mfma_max_sparse_rows() { return kMaxSparseRowsMfma; }
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
    case MODE_SPARSE: attn_mfma_kernel<MODE_SPARSE, WAVES, STREAM><<<grid, block, lds, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Dynamic LDS of a launch: wave partial outputs, then the staged sparse positions or scores.
size_t lds_bytes(const AttnArgs& a, int mode, int waves) {
  size_t lds = (size_t)waves * wave_region_floats(mode == MODE_SPARSE, a.group) * sizeof(float);
  if (mode == MODE_SPARSE || mode == MODE_FULL_SCORES || mode == MODE_FULL_HEADS) lds += (size_t)a.rows_per_split * 4;
  return lds;
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, int mode, hipStream_t stream) {
  if (a.splits <= 0 || a.batch <= 0) return hipSuccess;
  if (mode == MODE_SPARSE && a.rows_per_split > kMaxSparseRowsMfma) return hipErrorInvalidValue;
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
