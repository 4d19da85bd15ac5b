// combine.hip -- back to token order, weighted by the router (the gather step of
// the LlamaFactory PR #10481 write-up, section 1).
//
//   out[t] = sum_{j ascending, row valid} w[t*k+j] * y[row_pos[t*k+j]]
//
// One wave per token and column range (a token's row is split over several waves
// when there are few tokens, so that its loads are in flight at once); each lane
// owns 16 bytes of the output row per step and accumulates in fp32 in slot order
// (deterministic).  A row is valid iff its permuted position is below offsets[E];
// sentinel rows are never read, so a token with no valid row stores exact zeros.

#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "moe.h"

namespace moe {

__device__ __forceinline__ void load16(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}

template <bool kBf16In, bool kBf16Out, int kUnroll>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_,
                                                      const int* __restrict__ row_pos,
                                                      const float* __restrict__ weights,
                                                      const int* __restrict__ offsets, int E, int T,
                                                      int H, int k, int nsplit, int cols,
                                                      void* __restrict__ out_) {
  // Elements per lane per step: 8 for bf16 input (one 16-B load), 4 for f32.
  constexpr int EL = kBf16In ? 8 : 4;
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = wv / nsplit;
  const int lane = lane_id();
  if (t >= T) return;
  // columns [c_lo, c_hi) of the token (cols is a multiple of the 64-lane step)
  const int c_lo = (wv - t * nsplit) * cols;
  const int c_hi = min(H, c_lo + cols);
  const int V = offsets[E];
  // the token's k <= 16 slots, once: position (-1 if not a valid row) and weight of
  // slot j, made wave-uniform while every lane is still active
  int my_p = -1;
  float my_w = 0.0f;
  if (lane < k) {
    const int p = row_pos[(size_t)t * k + lane];
    if (p >= 0 && p < V && p < T * k) {
      my_p = p;
      my_w = weights[(size_t)t * k + lane];
    }
  }
  constexpr int kMaxK = MOE_MAX_TOPK;   // k is validated against it at the boundary
  int slot_p[kMaxK];
  float slot_w[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    slot_p[j] = __builtin_amdgcn_readlane(my_p, j);
    slot_w[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
  }
  auto load_row = [&](int p, int c0, float (&v)[EL]) {
    if constexpr (kBf16In) {
      const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(y_) + (size_t)p * H + c0);
      const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(u[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_f32(u[i] >> 16);
      }
    } else {
      load16(static_cast<const float*>(y_) + (size_t)p * H + c0, v);
    }
  };
  auto store_out = [&](int c0, const float (&acc)[EL]) {
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
  };
  constexpr int STEP = kWave * EL;
  for (int cb = c_lo + lane * EL; cb < c_hi; cb += kUnroll * STEP) {
    float acc[kUnroll][EL];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < EL; ++i) acc[u][i] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {   // slot order: the sum is deterministic
      const int p = slot_p[j];
      if (j >= k || p < 0) continue;
      const float w = slot_w[j];
      float v[kUnroll][EL];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (cb + u * STEP < c_hi) load_row(p, cb + u * STEP, v[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (cb + u * STEP < c_hi)
#pragma unroll
          for (int i = 0; i < EL; ++i) acc[u][i] = fmaf(w, v[u][i], acc[u][i]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (cb + u * STEP < c_hi) store_out(cb + u * STEP, acc[u]);
  }
}

hipError_t launch_combine(const void* y, bool y_bf16, const int* row_pos, const float* weights,
                          const int* offsets, int E, int T, int H, int k, void* out, bool out_bf16,
                          hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  // few tokens: split each row over up to ceil(1024 / T) waves of whole 64-lane steps
  const int step = kWave * (y_bf16 ? 8 : 4);
  const int steps = (H + step - 1) / step;
  int nsplit = T >= 1024 ? 1 : std::min(steps, (1024 + T - 1) / T);
  const int cols = (steps + nsplit - 1) / nsplit * step;
  nsplit = (H + cols - 1) / cols;
  const long long waves = (long long)T * nsplit;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  // column steps whose row loads are in flight together: four when y is larger than the
  // 256 MB MALL, so that its rows come from HBM (DeepSeek-V3-shaped combine, 940 MB:
  // 227 -> 214 us), else two (Mixtral-8x7B-shaped, 134 MB: 36 vs 39 us with four)
  const bool wide = (long long)T * k * H * (y_bf16 ? 2 : 4) > (256ll << 20);
#define MOE_COMBINE_LAUNCH(BI, BO)                                                                   \
  if (wide)                                                                                           \
    hipLaunchKernelGGL((combine_kernel<BI, BO, 4>), grid, block, 0, stream, y, row_pos, weights,     \
                       offsets, E, T, H, k, nsplit, cols, out);                                       \
  else                                                                                                \
    hipLaunchKernelGGL((combine_kernel<BI, BO, 2>), grid, block, 0, stream, y, row_pos, weights,     \
                       offsets, E, T, H, k, nsplit, cols, out);
  if (y_bf16 && out_bf16) {
    MOE_COMBINE_LAUNCH(true, true)
  } else if (y_bf16) {
    MOE_COMBINE_LAUNCH(true, false)
  } else if (out_bf16) {
    MOE_COMBINE_LAUNCH(false, true)
  } else {
    MOE_COMBINE_LAUNCH(false, false)
  }
#undef MOE_COMBINE_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
