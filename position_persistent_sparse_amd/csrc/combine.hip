// Merge pass of split attention partials (gfx950): one 64-lane wave per
// (batch row, query head), no LDS and no barrier, running
// merge::combine_row (combine_row.h). The pass moves about 0.5-1 % of a
// layer's bytes, so it is latency bound. (A 256-thread workgroup per row
// with the weights in LDS took about 0.8 us longer per launch.)
#include <math.h>

#include "combine_row.h"
#include "ppsa.h"
#include "ppsa_internal.h"

namespace ppsa {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(kWave) void combine_kernel(CombineArgs a) {
  merge::combine_row<T, D>(a, blockIdx.x, threadIdx.x);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int dtype, int head_dim, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.splits < 1 || a.splits > kMaxSplitsPerUnit) return hipErrorInvalidValue;
  const dim3 grid(a.rows), block(kWave);
  if (dtype == PPSA_BF16) {
    if (head_dim == 128) combine_kernel<uint16_t, 128><<<grid, block, 0, stream>>>(a);
    else if (head_dim == 64) combine_kernel<uint16_t, 64><<<grid, block, 0, stream>>>(a);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 128) combine_kernel<float, 128><<<grid, block, 0, stream>>>(a);
    else if (head_dim == 64) combine_kernel<float, 64><<<grid, block, 0, stream>>>(a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ppsa
