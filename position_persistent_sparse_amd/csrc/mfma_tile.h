// Matrix-core building blocks of the attention kernels (gfx950, bf16, head_dim 128): one wave
// processes tiles of 32 K/V rows for all query heads of a KV group.
//
// All query heads of a KV group share every K and V row, so the group's logits for 16 rows are
// one 16x16 matrix product and the weighted V sum is another; both go to the MFMA units, with up
// to 16 heads per group (heads past the group size are zero columns). A tile is two blocks of 16
// rows:
//   S^T[row, head] = K[row, :] . q[head, :]
//       v_mfma_f32_16x16x32_bf16, A = K (lane%16 = row, lane/16 picks 8 of each 32 dims), B = q
//       (lane%16 = head); four products cover d = 128.
//   The result leaves lane (g = lane/16, n = lane%16) holding the logits of rows 4g..4g+3 of each
//   block for head n: eight rows of the tile, 4g..4g+3 and 16+4g..16+4g+3. The contraction index
//   of a product may be numbered in any order both operands share, so those eight rows are the
//   lane's eight k slots of one v_mfma_f32_16x16x32_bf16 over the whole 32-row tile, with
//   A = P[head, row]: the softmax weights never leave the lane.
//   O[head, dim] += P[head, :] . V[:, dim]
//       B = V needs the same eight rows along the operand elements: lane (g, n) holds them at dims
//       8n..8n+7 (16 lanes cover a whole 256-byte row) and product t uses dim 8n+t of each,
//       regrouped with v_perm_b32. The output column n of product t is dim 8n+t; eight products
//       per tile.
// The running max is shared by the four lanes holding a head (a max across the wave's four rows
// per tile) and only moved when a tile exceeds it by more than 2^8 ("lazy" rescaling: weights may reach 256, still
// exact in the float32 sums); a merge uses each partial's own max, so the result is the same
// softmax. Weights are rounded to bf16 for the product and the normaliser sums the rounded
// weights, so numerator and denominator match.
#pragma once

#include <math.h>

#include "device_common.h"

namespace ppsa {
namespace mt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;
constexpr int kTile = 32;
constexpr float kLazyLog2 = 8.0f;
// Gathered K rows reach the A-operand layout through a wave-private LDS block of 16 rows, padded
// to 272 bytes per row so that the sixteen rows one read instruction touches fall on distinct banks.
constexpr int kKRowPitch = kRowBytes + 16;
constexpr int kKBlockBytes = 16 * kKRowPitch;  // 4352 bytes per wave

struct Tile {
  uint4 k[2][4];    // [block][c]: K[row 16*blk + n][32c + 8g .. +8] (gathered rows: once k_to_operand has run)
  uint4 v[2][4];    // [block][i]: V[row 16*blk + 4g + i][8n .. +8]
  uint32_t valid;   // bit 4*blk + i: row 16*blk + 4g + i is live
};

// Softmax state of one wave for the heads of its group: O rows are heads 4g + j, dims 8n + t.
struct Online {
  float4_t acc[8];
  float m_run;  // per head n, shared by the four lanes of that head (log2 units)
  float l_run;  // this lane's rows only
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats to two bf16 (low half first), round to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
}

// Max and sum over the four lanes n, n+16, n+32, n+48 (the four 16-lane rows of a wave), every lane
// getting the result: v_permlane16_swap pairs rows 0-1 and 2-3, v_permlane32_swap the two halves (VALU
// instructions; no trip through the LDS crossbar). Each sum adds the lower row to the upper one, so
// all four lanes hold the bit-identical value.
__device__ __forceinline__ float max_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t word(const uint4& u, int w) {
  return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

// 16 bytes of a K or V row at a byte offset from a base every lane shares (32-bit offsets: a
// scalar base plus one vector register per address). Streaming launches load with the
// nontemporal hint: rows are read once per layer.
template <bool STREAM>
__device__ __forceinline__ uint4 load16(const char* base, uint32_t off) {
  if constexpr (STREAM) {
    const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + off));
    return make_uint4(w.x, w.y, w.z, w.w);
  } else {
    return *reinterpret_cast<const uint4*>(base + off);
  }
}

__device__ __forceinline__ void online_init(Online& st) {
#pragma unroll
  for (int t = 0; t < 8; ++t) st.acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
}

// q fragments of the group's heads: lane (g, n) holds head n, dims 32c + 8g .. +8 (zero for heads
// past the group). `qh` points at the group's first head.
__device__ __forceinline__ void load_q(bf16x8_t (&qf)[4], const uint16_t* qh, int group, int g, int n) {
  const uint16_t* qp = qh + (size_t)(n < group ? n : 0) * kD;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 w = *reinterpret_cast<const uint4*>(qp + 32 * c + 8 * g);
    if (n >= group) w = make_uint4(0u, 0u, 0u, 0u);
    qf[c] = __builtin_bit_cast(bf16x8_t, w);
  }
}

// Whole-row K pieces (lane (g, n): rows 16 blk + 4g + i, bytes 16n ..) to the operand layout (lane
// (g, n): row 16 blk + n, bytes 16g + 64c ..) through the wave's own 16-row LDS block. LDS
// instructions of one wave execute in order, so each read sees the writes before it and each
// write comes after the reads of the previous block.
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

// Raw logits of the tile's rows 16 blk + 4g + j for head n (K in the operand layout).
__device__ __forceinline__ void qk_logits(const Tile& t, const bf16x8_t (&qf)[4], float4_t (&s)[2]) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    s[blk] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[blk][c]), qf[c], s[blk], 0,
                                                       0, 0);
  }
}

// One tile's softmax update and weighted V sum. x[blk][j] is the logit of row 16 blk + 4g + j for
// head n in log2 units (-inf for rows that are not live).
__device__ __forceinline__ void softmax_pv(const Tile& t, const float (&x)[2][4], Online& st, int g) {
  float tmax = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int j = 0; j < 4; ++j) tmax = fmaxf(tmax, x[blk][j]);
  tmax = max_rows4(tmax);
  const bool need = tmax > st.m_run + kLazyLog2;
  if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
    const float m_new = need ? fmaxf(st.m_run, tmax) : st.m_run;
    if (__builtin_amdgcn_ballot_w64(st.m_run != -INFINITY) != 0ull) {
      const float alpha = m_new == st.m_run ? 1.0f : exp2_fast(st.m_run - m_new);
      st.l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float aj = __shfl(alpha, 4 * g + j);  // lane 4g+j holds head 4g+j
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) st.acc[tt][j] *= aj;
      }
    }  // else nothing is accumulated yet (every sum is still zero): no rescaling to do
    st.m_run = m_new;
  }
  const float ms = st.m_run == -INFINITY ? 0.0f : st.m_run;
  // k slots 0..3: rows 4g..4g+3 of block 0; slots 4..7: the same rows of block 1.
  uint32_t p[2][2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    p[blk][0] = bf16_pair(exp2_fast(x[blk][0] - ms), exp2_fast(x[blk][1] - ms));
    p[blk][1] = bf16_pair(exp2_fast(x[blk][2] - ms), exp2_fast(x[blk][3] - ms));
    st.l_run += (bf16_lo(p[blk][0]) + bf16_hi(p[blk][0])) + (bf16_lo(p[blk][1]) + bf16_hi(p[blk][1]));
  }
  const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, make_uint4(p[0][0], p[0][1], p[1][0], p[1][1]));
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const uint32_t sel = (tt & 1) ? 0x07060302u : 0x05040100u;
    const int w = tt >> 1;
    const uint32_t d0 = __builtin_amdgcn_perm(word(t.v[0][1], w), word(t.v[0][0], w), sel);
    const uint32_t d1 = __builtin_amdgcn_perm(word(t.v[0][3], w), word(t.v[0][2], w), sel);
    const uint32_t d2 = __builtin_amdgcn_perm(word(t.v[1][1], w), word(t.v[1][0], w), sel);
    const uint32_t d3 = __builtin_amdgcn_perm(word(t.v[1][3], w), word(t.v[1][2], w), sel);
    const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, make_uint4(d0, d1, d2, d3));
    st.acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, st.acc[tt], 0, 0, 0);
  }
}

}  // namespace mt
}  // namespace ppsa
