// Split-N attention pass on the vector ALUs (gfx950, wave64).
//
// Computes, per query head of a KV group, the attention of the TidalDecode
// review page (section 3, PPSA paragraph, attention equation:
// softmax(q K^T * scale) V) over one split of rows, as an online-softmax
// partial (m, l, o) in log2 units. Full mode walks cache rows in order;
// sparse mode walks the positions listed in idx (the PPSA layer kind);
// full-with-scores mode also writes the group-summed logit of every row,
// which the selection kernel ranks.
//
// Memory layout and access: a K or V row is D elements. A lane owns 16
// bytes of a row (EPL elements), LPR = D/EPL lanes cover a row, so each
// wave-wide 16-byte load reads RPI = 64/LPR consecutive rows -- one
// contiguous 1 KiB block when rows are consecutive. Each lane keeps an
// independent softmax state per query head for its row slot; the slots of a
// wave and then the four waves of the workgroup are merged at the end; the
// splits of a unit are merged by the merge pass (combine.hip).
// Every row's logit is reduced over its LPR lanes with DPP, so all lanes of
// a row see the same bits.
#include <math.h>

#include "attn_epilogue.h"
#include "device_common.h"
#include "ppsa_internal.h"
#include "ppsa.h"

namespace ppsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;
constexpr int kMaxSparseRows = 2048;

template <typename T, int D>
struct Layout {
  static constexpr int EPL = 16 / (int)sizeof(T);
  static constexpr int LPR = D / EPL;
  static constexpr int RPI = kWave / LPR;
  static constexpr int ROWS_WAVE = RPI * kUnroll;
  static constexpr int ROWS_TRIP = ROWS_WAVE * kWaves;
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes of a K or V row; rows are read once per layer, so the load carries the nontemporal hint.
template <typename P>
__device__ __forceinline__ uint4 load_row16(const P* p) {
  const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}

__device__ __forceinline__ void widen16(const uint4& w, float (&x)[8]) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
  x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
  x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

__device__ __forceinline__ void widen16(const uint4& w, float (&x)[4]) {
  x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
  x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T, int D, int G, int MODE>
__global__ __launch_bounds__(kThreads) void attn_valu_kernel(AttnArgs a) {
  using Lay = Layout<T, D>;
  constexpr int EPL = Lay::EPL, LPR = Lay::LPR, RPI = Lay::RPI;
  constexpr float NEG_INF = -INFINITY;

  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ float sm_o[kWaves][G][D];
  __shared__ int32_t sm_rows[MODE == MODE_SPARSE ? kMaxSparseRows : 1];

  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r = lane / LPR, part = lane % LPR;
  const int group = a.group;

  const int n_live = min(max(a.seq_lens[b], 0), a.max_len);
  const size_t unit = (size_t)b * a.kv_heads + kv;
  const T* kbase = reinterpret_cast<const T*>(a.k) + unit * (size_t)a.max_len * D + part * EPL;
  const T* vbase = reinterpret_cast<const T*>(a.v) + unit * (size_t)a.max_len * D + part * EPL;
  const int slot0 = split * a.rows_per_split;
  int slot_end = MODE == MODE_SPARSE ? min(slot0 + a.rows_per_split, a.kslots)
                                     : min(slot0 + a.rows_per_split, n_live);
  if (n_live == 0) slot_end = slot0;

  if constexpr (MODE == MODE_SPARSE) {
    // Stage this split's positions; anything outside [0, n_live) becomes -1.
    const int32_t* ip = a.idx + unit * (size_t)a.kslots;
    for (int i = tid; i < slot_end - slot0; i += kThreads) {
      int p = ip[slot0 + i];
      sm_rows[i] = (p >= 0 && p < n_live) ? p : -1;
    }
    __syncthreads();
  }

  float qf[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (h < group) {
      const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.q_heads + (size_t)kv * group + h) * D + part * EPL;
      widen16(*reinterpret_cast<const uint4*>(qp), qf[h]);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[h][e] = 0.0f;
    }
  }

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = NEG_INF;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
  }

  for (int base = slot0 + wave * Lay::ROWS_WAVE; base < slot_end; base += Lay::ROWS_TRIP) {
    uint4 kr[kUnroll], vr[kUnroll];
    bool valid[kUnroll];
    int pos[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int slot = base + u * RPI + r;
      int row;
      if constexpr (MODE == MODE_SPARSE) {
        const int p = slot < slot_end ? sm_rows[slot - slot0] : -1;
        valid[u] = p >= 0;
        row = valid[u] ? p : 0;  // row 0 is live whenever this loop runs
      } else {
        valid[u] = slot < slot_end;
        row = valid[u] ? slot : slot_end - 1;
      }
      pos[u] = row;
      kr[u] = load_row16(kbase + (size_t)row * D);
      vr[u] = load_row16(vbase + (size_t)row * D);
    }

    float x[kUnroll][G];  // logits in log2 units, -inf for invalid rows
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kx[EPL];
      widen16(kr[u], kx);
      float score = 0.0f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(qf[h][e], kx[e], dot);
        dot = group_sum<LPR>(dot);
        if constexpr (MODE == MODE_FULL_SCORES) {
          if (h < group) score += dot * a.scale;
        }
        x[u][h] = valid[u] ? dot * a.scale_log2 : NEG_INF;
        if constexpr (MODE == MODE_FULL_SCORES) {  // softmax-weight variant: every head's logit too
          if (a.head_logits && valid[u] && part == 0 && h < group)
            a.head_logits[((size_t)b * a.q_heads + (size_t)kv * group + h) * a.max_len + pos[u]] = x[u][h];
        }
      }
      if constexpr (MODE == MODE_FULL_SCORES) {
        if (valid[u] && part == 0) a.scores[unit * (size_t)a.max_len + pos[u]] = score;
      }
    }

    float vx[kUnroll][EPL];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) widen16(vr[u], vx[u]);

#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mt = x[0][h];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u) mt = fmaxf(mt, x[u][h]);
      if (mt > m[h]) {
        const float alpha = exp2_fast(m[h] - mt);  // m = -inf gives 0
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
        m[h] = mt;
      }
      const float ms = m[h] == NEG_INF ? 0.0f : m[h];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float p = exp2_fast(x[u][h] - ms);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(p, vx[u][e], o[h][e]);
      }
    }
  }

  // Merge the row slots of this wave (lanes r*LPR + part, r = 0..RPI-1).
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float ms = mn == NEG_INF ? 0.0f : mn;
      const float ca = exp2_fast(m[h] - ms), cb = exp2_fast(mo - ms);
      l[h] = l[h] * ca + lo * cb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float oo = __shfl_xor(o[h][e], off);
        o[h][e] = o[h][e] * ca + oo * cb;
      }
      m[h] = mn;
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave][h][part * EPL + e] = o[h][e];
      if (lane == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // Merge the waves: this split's result for each query head of the group.
  const bool single = a.splits == 1;
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    if (h >= group) continue;
    float mx = NEG_INF;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm_m[w][h]);
    const float ms = mx == NEG_INF ? 0.0f : mx;
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float c = exp2_fast(sm_m[w][h] - ms);
      acc += sm_o[w][h][d] * c;
      lsum += sm_l[w][h] * c;
    }
    if (single) {
      T* o = reinterpret_cast<T*>(a.out) + ((size_t)b * a.q_heads + (size_t)kv * group + h) * D + d;
      store_elem(o, lsum > 0.0f ? acc / lsum : 0.0f);
      continue;
    }
    const size_t row = part_row(a, b, kv, h, split);
    a.part_o[row * D + d] = acc;
    if (d == 0) {
      a.part_m[row] = mx;
      a.part_l[row] = lsum;
    }
  }
}

template <typename T, int D, int G>
hipError_t launch_mode(const AttnArgs& a, int mode, hipStream_t stream) {
  dim3 grid(a.splits, a.kv_heads, a.batch), block(kThreads);
  switch (mode) {
    case MODE_FULL: attn_valu_kernel<T, D, G, MODE_FULL><<<grid, block, 0, stream>>>(a); break;
    case MODE_FULL_SCORES: attn_valu_kernel<T, D, G, MODE_FULL_SCORES><<<grid, block, 0, stream>>>(a); break;
    case MODE_SPARSE: attn_valu_kernel<T, D, G, MODE_SPARSE><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_group(const AttnArgs& a, int mode, hipStream_t stream) {
  if (a.group <= 1) return launch_mode<T, D, 1>(a, mode, stream);
  if (a.group <= 2) return launch_mode<T, D, 2>(a, mode, stream);
  if (a.group <= 4) return launch_mode<T, D, 4>(a, mode, stream);
  if (a.group <= 8) return launch_mode<T, D, 8>(a, mode, stream);
  if (a.group <= 16) return launch_mode<T, D, 16>(a, mode, stream);
  return hipErrorInvalidValue;
}

}  // namespace

int attn_rows_granule(int dtype, int head_dim) {
  if (dtype == PPSA_BF16) return head_dim == 64 ? Layout<uint16_t, 64>::ROWS_TRIP : Layout<uint16_t, 128>::ROWS_TRIP;
  return head_dim == 64 ? Layout<float, 64>::ROWS_TRIP : Layout<float, 128>::ROWS_TRIP;
}

int attn_max_sparse_rows() { return kMaxSparseRows; }

hipError_t launch_attn(const AttnArgs& a, int mode, int dtype, int head_dim, hipStream_t stream) {
  if (a.splits <= 0 || a.batch <= 0) return hipSuccess;
  if (mode == MODE_SPARSE && a.rows_per_split > kMaxSparseRows) return hipErrorInvalidValue;
  if (mode == MODE_FULL_HEADS) mode = MODE_FULL_SCORES;  // the head logits go out when a.head_logits is set
  if (dtype == PPSA_BF16) {
    if (head_dim == 128) return launch_group<uint16_t, 128>(a, mode, stream);
    if (head_dim == 64) return launch_group<uint16_t, 64>(a, mode, stream);
  } else if (dtype == PPSA_F32) {
    if (head_dim == 128) return launch_group<float, 128>(a, mode, stream);
    if (head_dim == 64) return launch_group<float, 64>(a, mode, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ppsa
