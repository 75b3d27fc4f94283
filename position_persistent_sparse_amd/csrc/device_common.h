// Device helpers for the gfx950 kernels: bf16 packing, DPP reductions,
// workgroup scans. Wave size is 64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ppsa {

constexpr int kWave = 64;

// bf16 held in the low / high half of a 32-bit word, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t bf16_round(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in 1..64, power of two). Every lane of
// a group ends with the bit-identical sum: each step adds a lane's value to
// its partner's, and float addition is commutative.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]: partner lane ^ 1
  if constexpr (N >= 4) x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]: partner lane ^ 2
  if constexpr (N >= 8) x += dpp_f32<0x141>(x);  // row_half_mirror: lane i <-> 7 - i within 8
  if constexpr (N >= 16) x += dpp_f32<0x140>(x); // row_mirror: lane i <-> 15 - i within 16
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32_or_zero(uint32_t x) {
  // Lanes whose source is outside the row, or whose row is masked off, read 0.
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave, on the VALU through DPP:
// shifts by 1, 2, 4, 8 within each row of 16 lanes, then the last lane of
// row 0 (2) is added to row 1 (3) and the last lane of row 1 to rows 2, 3.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += dpp_u32_or_zero<0x111, 0xF>(x);  // row_shr:1
  x += dpp_u32_or_zero<0x112, 0xF>(x);  // row_shr:2
  x += dpp_u32_or_zero<0x114, 0xF>(x);  // row_shr:4
  x += dpp_u32_or_zero<0x118, 0xF>(x);  // row_shr:8
  x += dpp_u32_or_zero<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_u32_or_zero<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Sum over the 64 lanes of a wave (every lane gets the total).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(x), kWave - 1);
}

// Exclusive prefix sum over a workgroup of NT threads (NT a multiple of 64,
// at most 64 waves). Returns the exclusive sum and sets *total to the sum over
// the workgroup. One barrier: each wave writes its total to one of two LDS
// buffers (`lds` holds 2 * NT/64 words; `parity` picks the buffer and is
// flipped, so consecutive calls alternate), and after the barrier every wave
// scans the wave totals itself. A buffer is written again two calls later, by
// which time every thread has passed the barrier of the call in between, so
// all reads of it are done. Every thread must call it, with the same parity.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* lds, int& parity, uint32_t* total) {
  constexpr int NW = NT / kWave;
  static_assert(NW >= 1 && NW <= kWave, "one to 64 waves");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  uint32_t* buf = lds + parity * NW;
  parity ^= 1;
  const uint32_t inc = wave_inclusive_scan(x);
  if (lane == kWave - 1) buf[wave] = inc;
  __syncthreads();
  const uint32_t w = lane < NW ? buf[lane] : 0u;
  const uint32_t wi = wave_inclusive_scan(w);  // lanes < NW: inclusive prefix of the wave totals
  *total = (uint32_t)__builtin_amdgcn_readlane((int)wi, NW - 1);
  const uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)(wi - w), wave);
  return before + inc - x;
}

}  // namespace ppsa
