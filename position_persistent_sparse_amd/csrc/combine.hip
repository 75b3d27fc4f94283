// Merge of split attention partials (gfx950).
//
// Each split of a (batch row, query head) left m (max logit, log2 units),
// l = sum 2^(x - m) and o = sum 2^(x - m) V. The full softmax over the union
// of the splits is  out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),
// M = max_s m_s -- the attention equation of the TidalDecode review page
// (section 3, PPSA paragraph) evaluated in pieces. A row with no live
// position anywhere (M = -inf) outputs zeros.
#include <math.h>

#include "device_common.h"
#include "ppsa_internal.h"
#include "../../include/ppsa.h"

namespace ppsa {
namespace {

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = bf16_round(v); }

template <typename T, int D>
__global__ __launch_bounds__(D) void combine_kernel(CombineArgs a) {
  const int row = blockIdx.x, d = threadIdx.x;
  const float* pm = a.part_m + (size_t)row * a.splits;
  const float* pl = a.part_l + (size_t)row * a.splits;
  const float* po = a.part_o + (size_t)row * a.splits * D + d;
  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, pm[s]);
  float res = 0.0f;
  if (mx != -INFINITY) {
    float lsum = 0.0f, acc = 0.0f;
    for (int s = 0; s < a.splits; ++s) {
      const float c = __builtin_amdgcn_exp2f(pm[s] - mx);
      lsum += pl[s] * c;
      acc += po[(size_t)s * D] * c;
    }
    res = acc / lsum;
  }
  store_out(reinterpret_cast<T*>(a.out) + (size_t)row * D + d, res);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int dtype, int head_dim, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid(a.rows);
  if (dtype == PPSA_BF16) {
    if (head_dim == 128) combine_kernel<uint16_t, 128><<<grid, 128, 0, stream>>>(a);
    else if (head_dim == 64) combine_kernel<uint16_t, 64><<<grid, 64, 0, stream>>>(a);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 128) combine_kernel<float, 128><<<grid, 128, 0, stream>>>(a);
    else if (head_dim == 64) combine_kernel<float, 64><<<grid, 64, 0, stream>>>(a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ppsa
