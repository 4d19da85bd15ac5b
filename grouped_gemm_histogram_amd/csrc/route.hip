// route.hip -- top-k routing, one wave64 per token (the per-token selection and
// softmax are in route_device.h).

#include "device_common.h"
#include "launch.h"
#include "route_device.h"

namespace moe {

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, long long valid_rows,
                                                         int renorm, int* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<EPL>(logits, t, E, k, valid_rows, renorm, ids, weights);
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, long long valid_rows,
                             int renorm, int* ids, float* weights, hipStream_t stream) {
  const dim3 grid((T + 3) / 4), block(256);
#define MOE_ROUTE_CASE(EPL)                                                                     \
  hipLaunchKernelGGL(route_topk_kernel<EPL>, grid, block, 0, stream, logits, T, E, k,         \
                     valid_rows, renorm, ids, weights);                                         \
  break;
  switch ((E + kWave - 1) / kWave) {
    case 1: MOE_ROUTE_CASE(1)
    case 2: MOE_ROUTE_CASE(2)
    case 3: case 4: MOE_ROUTE_CASE(4)
    case 5: case 6: case 7: case 8: MOE_ROUTE_CASE(8)
    default: MOE_ROUTE_CASE(16)
  }
#undef MOE_ROUTE_CASE
  return hipGetLastError();
}

}  // namespace moe
