// permute.hip -- token rows into expert-contiguous order (the scatter step of the
// LlamaFactory PR #10481 write-up, section 1), optionally quantising each row
// to OCP e4m3 per 128 channels (the per-token activation cast the
// transformers PR #45621 write-up, section 1, loads as fp8_act_quant /
// per_token_cast_to_fp8).
//
// One wave per permuted row (quantisation: per row and range of 512-channel
// steps, so that few rows still spread over many waves); 16-byte loads and
// stores, so each row moves as coalesced 1 KiB wave transactions.  Positions at
// or past offsets[E] (the sentinel tail) are skipped without touching memory.

#include "device_common.h"
#include "launch.h"

namespace moe {

// x [T, n16 x 16 B] -> xp [R, n16 x 16 B]
__global__ __launch_bounds__(256) void permute_copy_kernel(const uint4* __restrict__ x, int T,
                                                           int n16, int k, const int* __restrict__ sorted_rows,
                                                           const int* __restrict__ offsets, int E,
                                                           int R, uint4* __restrict__ xp) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (p >= R || p >= offsets[E]) return;
  const int src = sorted_rows[p] / k;
  if (src < 0 || src >= T) return;   // inconsistent permutation: leave the row unwritten
  const uint4* s = x + (size_t)src * n16;
  uint4* d = xp + (size_t)p * n16;
  int c = lane;
  for (; c + 3 * kWave < n16; c += 4 * kWave) {
    const uint4 a0 = s[c], a1 = s[c + kWave], a2 = s[c + 2 * kWave], a3 = s[c + 3 * kWave];
    d[c] = a0;
    d[c + kWave] = a1;
    d[c + 2 * kWave] = a2;
    d[c + 3 * kWave] = a3;
  }
  for (; c < n16; c += kWave) d[c] = s[c];
}

// bf16 (F32IN: f32) x [T, H] -> e4m3 codes xq [R, H] + scales xs [H/128, R]; H % 128 == 0.
// Each 16-lane group of the wave owns one 128-channel group per step; a wave
// covers units [u_lo, u_lo + units) of its row (8-channel units, a multiple of
// 64).  With sorted_rows and offsets null, row p is token row p and all R = T
// rows are written (the per-token quantisation alone, for a GEMM that gathers
// its rows).
template <bool F32IN>
__global__ __launch_bounds__(256) void permute_quant_kernel(const void* __restrict__ x_, int T,
                                                            int H, int k, const int* __restrict__ sorted_rows,
                                                            const int* __restrict__ offsets, int E,
                                                            int R, int nsplit, int units,
                                                            uint2* __restrict__ xq, float* __restrict__ xs,
                                                            const int* __restrict__ row_pos, int kslots,
                                                            float* __restrict__ xs_perm, int R_perm) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int p = wv / nsplit;
  const int lane = lane_id();
  if (p >= R || (offsets != nullptr && p >= offsets[E])) return;
  const int src = sorted_rows != nullptr ? sorted_rows[p] / k : p;
  if (src < 0 || src >= T) return;   // inconsistent permutation: leave the row unwritten
  const int n8 = H / 8;                       // 8-channel units per row
  const int u_lo = (wv - p * nsplit) * units;
  const int u_hi = min(n8, u_lo + units);
  const uint4* s = static_cast<const uint4*>(x_) + (size_t)src * n8 * (F32IN ? 2 : 1);
  uint2* d = xq + (size_t)p * n8;
  float* sc = xs + p;                         // scales are block-major: [H/128, R]
  // Token rows (no row map) with xs_perm: each scale is also stored at the permuted
  // positions of the token's kslots routed rows, xs_perm [H/128, R_perm], so that a
  // GEMM reading the token rows through the permutation finds a tile's scales in
  // consecutive words.  Lane j < kslots of each 16-lane group stores slot j's copy.
  int my_pos = -1;
  if (xs_perm != nullptr && (lane & 15) < kslots) {
    const int q = row_pos[(size_t)p * kslots + (lane & 15)];
    if (q >= 0 && q < R_perm) my_pos = q;
  }
  for (int base = u_lo; base < u_hi; base += kWave) {
    const int u = base + lane;
    const bool active = u < u_hi;             // whole 16-lane groups, as H % 128 == 0
    float v[8];
    float amax = 0.0f;
    if (active) {
      if constexpr (F32IN) {
        const float4 a = __builtin_bit_cast(float4, s[2 * u]), b = __builtin_bit_cast(float4, s[2 * u + 1]);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      } else {
        const uint4 raw = s[u];
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
          v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    if (active) {
      const float scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
      uint32_t lo = 0, hi = 0;
      lo = cvt_e4m3x2(clamp448(v[0] / scale), clamp448(v[1] / scale)) |
           (cvt_e4m3x2(clamp448(v[2] / scale), clamp448(v[3] / scale)) << 16);
      hi = cvt_e4m3x2(clamp448(v[4] / scale), clamp448(v[5] / scale)) |
           (cvt_e4m3x2(clamp448(v[6] / scale), clamp448(v[7] / scale)) << 16);
      d[u] = make_uint2(lo, hi);
      if ((lane & 15) == 0) sc[(size_t)(u / 16) * R] = scale;
      if (my_pos >= 0) xs_perm[(size_t)(u / 16) * R_perm + my_pos] = scale;
    }
  }
}

// One thread per routed position and a share of the scale groups: reads the
// position's token (one word), then that token's scale of each group it covers
// (the [G, T] table is a few MB and stays in L2) and writes them along p.
__global__ __launch_bounds__(256) void gather_scales_kernel(const float* __restrict__ xs, int T, int G,
                                                            const int* __restrict__ sorted_rows, int k,
                                                            const int* __restrict__ offsets, int E, int R,
                                                            float* __restrict__ xs_perm) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= R || p >= offsets[E]) return;
  const int t = sorted_rows[p] / k;
  if (t < 0 || t >= T) return;   // inconsistent permutation: leave the position unwritten
  for (int g = blockIdx.y; g < G; g += gridDim.y) xs_perm[(size_t)g * R + p] = xs[(size_t)g * T + t];
}

hipError_t launch_gather_scales(const float* xs, int T, int G, const int* sorted_rows, int k,
                                const int* offsets, int E, int R, float* xs_perm, hipStream_t stream) {
  if (R <= 0 || G <= 0) return hipSuccess;
  const dim3 grid((unsigned)((R + 255) / 256), (unsigned)(G < 8 ? G : 8));
  hipLaunchKernelGGL(gather_scales_kernel, grid, dim3(256), 0, stream, xs, T, G, sorted_rows, k, offsets, E, R,
                     xs_perm);
  return hipGetLastError();
}

hipError_t launch_permute_copy(const void* x, int T, int row_bytes, int k, const int* sorted_rows,
                               const int* offsets, int E, int R, void* xp, hipStream_t stream) {
  if (R > 0)
    hipLaunchKernelGGL(permute_copy_kernel, dim3((R + 3) / 4), dim3(256), 0, stream,
                       static_cast<const uint4*>(x), T, row_bytes / 16, k, sorted_rows, offsets, E, R,
                       static_cast<uint4*>(xp));
  return hipGetLastError();
}

hipError_t launch_permute_quant(const void* x, int T, int H, int k, const int* sorted_rows,
                                const int* offsets, int E, int R, void* xq, float* xs,
                                hipStream_t stream, bool f32_in, const int* row_pos, int kslots,
                                float* xs_perm, int R_perm) {
  if (R <= 0) return hipSuccess;
  // few rows: split each row over up to ceil(1024 / R) waves of whole 64-lane steps
  const int steps = (H / 8 + kWave - 1) / kWave;
  int nsplit = R >= 1024 ? 1 : (steps < (1024 + R - 1) / R ? steps : (1024 + R - 1) / R);
  const int units = (steps + nsplit - 1) / nsplit * kWave;
  nsplit = (H / 8 + units - 1) / units;
  const long long waves = (long long)R * nsplit;
  if (f32_in)
    hipLaunchKernelGGL(permute_quant_kernel<true>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, x,
                       T, H, k, sorted_rows, offsets, E, R, nsplit, units, static_cast<uint2*>(xq), xs,
                       row_pos, kslots, xs_perm, R_perm);
  else
    hipLaunchKernelGGL(permute_quant_kernel<false>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, x,
                       T, H, k, sorted_rows, offsets, E, R, nsplit, units, static_cast<uint2*>(xq), xs,
                       row_pos, kslots, xs_perm, R_perm);
  return hipGetLastError();
}

}  // namespace moe
