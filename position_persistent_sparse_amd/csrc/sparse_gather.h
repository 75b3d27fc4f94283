// Row gather of the sparse attention layer (gfx950, bf16, head_dim 128), shared by the kernel
// (attn_sparse.hip) and its load-only twin (probe.hip): the slot entries of a 32-slot tile and the
// K/V rows they name, in the lane layout of mfma_tile.h (lane (g, n): rows 16 blk + 4g + i, bytes
// 16n .. 16n+15 of each).
#pragma once

#include "mfma_tile.h"

namespace ppsa {
namespace mt {

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource, gfx9 data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// Raw slot entries of the tile's rows 16 blk + 4g + i (i = 0..3), `rel` = the tile's first slot
// relative to the split, through a buffer resource over the split's slots: reads past the split
// return 0 (the slot index marks them invalid at use). Unconditional loads: nothing waits on them
// until the rows are requested.
__device__ __forceinline__ void fetch_positions(int (&raw)[2][4], __amdgpu_buffer_rsrc_t r, int rel, bool vec, int g) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const uint32_t off = (uint32_t)(rel + 16 * blk + 4 * g) * 4u;
    if (vec) {
      const u32x4v_t w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[blk][i] = (int)w[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[blk][i] = (int)__builtin_amdgcn_raw_buffer_load_b32(r, off + 4u * i, 0, 0);
    }
  }
}

// Lane (g, n) loads bytes 16n .. 16n+15 of the rows of slots rel + 16 blk + 4g + i of K and V. A
// slot past the split or an entry outside [0, n_live) loads row 0 and stays invalid.
template <bool STREAM>
__device__ __forceinline__ void load_gathered(Tile& t, const char* kb, const char* vb, const int (&raw)[2][4], int rel,
                                              int nrows, int n_live, int g, int n) {
  t.valid = 0u;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = raw[blk][i];
      const bool ok = rel + 16 * blk + 4 * g + i < nrows && (uint32_t)p < (uint32_t)n_live;
      const uint32_t off = (uint32_t)(ok ? p : 0) * kRowBytes + 16u * n;
      t.valid |= (uint32_t)ok << (4 * blk + i);
      t.k[blk][i] = load16<STREAM>(kb, off);
      t.v[blk][i] = load16<STREAM>(vb, off);
    }
}

}  // namespace mt
}  // namespace ppsa
