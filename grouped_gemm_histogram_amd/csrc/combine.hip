// combine.hip -- back to token order, weighted by the router (the gather step of
// the LlamaFactory PR #10481 write-up, section 1).
//
//   out[t] = sum_{j ascending, row valid} w[t*k+j] * y[row_pos[t*k+j]]
//
// One wave per token; each lane owns 16 bytes of the output row per step and
// accumulates in fp32 in slot order (deterministic).  A row is valid iff its
// permuted position is below offsets[E]; sentinel rows are never read, so a
// token with no valid row stores exact zeros.

#include "device_common.h"
#include "launch.h"

namespace moe {

__device__ __forceinline__ void load16(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}

template <bool kBf16In, bool kBf16Out>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_,
                                                      const int* __restrict__ row_pos,
                                                      const float* __restrict__ weights,
                                                      const int* __restrict__ offsets, int E, int T,
                                                      int H, int k, void* __restrict__ out_) {
  // Elements per lane per step: 8 for bf16 input (one 16-B load), 4 for f32.
  constexpr int EL = kBf16In ? 8 : 4;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (t >= T) return;
  const int V = offsets[E];
  for (int c0 = lane * EL; c0 < H; c0 += kWave * EL) {
    float acc[EL];
#pragma unroll
    for (int i = 0; i < EL; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int p = row_pos[(size_t)t * k + j];
      if (p < 0 || p >= V || p >= T * k) continue;
      const float w = weights[(size_t)t * k + j];
      if constexpr (kBf16In) {
        const uint4 raw = *reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(y_) + (size_t)p * H + c0);
        const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(w, bf16_bits_to_f32(u[i] & 0xffffu), acc[2 * i]);
          acc[2 * i + 1] = fmaf(w, bf16_bits_to_f32(u[i] >> 16), acc[2 * i + 1]);
        }
      } else {
        float v[4];
        load16(static_cast<const float*>(y_) + (size_t)p * H + c0, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, v[i], acc[i]);
      }
    }
    if constexpr (kBf16Out) {
      uint16_t* o = static_cast<uint16_t*>(out_) + (size_t)t * H + c0;
      if constexpr (EL == 8) {
        *reinterpret_cast<uint4*>(o) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
      } else {
        *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      }
    } else {
      float* o = static_cast<float*>(out_) + (size_t)t * H + c0;
#pragma unroll
      for (int i = 0; i < EL; i += 4)
        *reinterpret_cast<float4*>(o + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    }
  }
}

hipError_t launch_combine(const void* y, bool y_bf16, const int* row_pos, const float* weights,
                          const int* offsets, int E, int T, int H, int k, void* out, bool out_bf16,
                          hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  if (y_bf16 && out_bf16)
    hipLaunchKernelGGL((combine_kernel<true, true>), grid, block, 0, stream, y, row_pos, weights,
                       offsets, E, T, H, k, out);
  else if (y_bf16)
    hipLaunchKernelGGL((combine_kernel<true, false>), grid, block, 0, stream, y, row_pos, weights,
                       offsets, E, T, H, k, out);
  else if (out_bf16)
    hipLaunchKernelGGL((combine_kernel<false, true>), grid, block, 0, stream, y, row_pos, weights,
                       offsets, E, T, H, k, out);
  else
    hipLaunchKernelGGL((combine_kernel<false, false>), grid, block, 0, stream, y, row_pos, weights,
                       offsets, E, T, H, k, out);
  return hipGetLastError();
}

}  // namespace moe
