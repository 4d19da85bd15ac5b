// backward.hip -- the elementwise and data-movement steps of the layer's backward
// (bf16 layers).  The GEMMs of the backward run on grouped_gemm_kernel: the
// recomputed SiLU*up product (whose epilogue also keeps the f32 pre-activations
// gu), the two data-gradient products on transposed weights, and the two
// weight-gradient products in its K-grouped mode.
//
// The layer is the one of the LlamaFactory PR #10481 write-up (section 1):
// h = SiLU(gate) * up per permuted row, y = W2 h, out[t] = sum_j w[t,j] y.  Its
// backward, with the routing held fixed, is the chain rule through those steps;
// sentinel rows take no part in it, and no output that a sentinel row would
// own is left unwritten (the transformers PR #45621 write-up, section 3, traces
// a training NaN to exactly that).
//
//   data gradient: dh1[p] = dout[r / k] W2_e           (p < V; r = sorted_rows[p]; the
//                  unweighted product, a GEMM reading dout rows through the permutation)
//   silu_bwd:     dw[r]  = dh1[p] . h[p]                (0 for a sentinel slot), since
//                  dL/dw[r] = dout[r/k] . y[p] = dout[r/k] . (W2_e h[p]) = (dout[r/k] W2_e) . h[p];
//                  dh = w[r] dh1[p];  dgu[p] = [dh * u * silu'(g), dh * silu(g)]
//   weighted rows: dy[p] = w[r] * dout[r / k], formed while transposing for dW2
//   transposes:   weights [E, R, C] -> [E, C, R] (R, C multiples of 8); permuted
//                 activations [R, C] -> expert-major blocks [C, round_up(M_e, 64)]
//                 (rows of an expert contiguous, padding columns zero), so that every
//                 expert's K range is whole 64-element slices for the weight-gradient
//                 GEMM and each of its tiles reads a compact block.

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kMaxE = 1024;

__device__ __forceinline__ int clamp_off(const int* offsets, int e, int R) {
  return min(max(offsets[e], 0), R);
}

}  // namespace

// koff[e] = sum over e' < e of round_up(M_e', 64), e = 0..E.  One workgroup.
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int* __restrict__ offsets, int E, int R,
                                                           int* __restrict__ koff) {
  __shared__ int s[2][kMaxE + 1];
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    int m = 0;
    if (e > 0) m = max(clamp_off(offsets, e, R) - clamp_off(offsets, e - 1, R), 0);
    s[0][e] = (m + 63) & ~63;
  }
  __syncthreads();
  int src = 0;
  for (int d = 1; d <= E; d <<= 1) {   // inclusive scan over E+1 entries
    for (int e = threadIdx.x; e <= E; e += blockDim.x) s[src ^ 1][e] = s[src][e] + (e >= d ? s[src][e - d] : 0);
    __syncthreads();
    src ^= 1;
  }
  for (int e = threadIdx.x; e <= E; e += blockDim.x) koff[e] = s[src][e];
}

// The segment transposes move 64x64 element tiles through LDS with 16-byte global
// loads and stores (256 threads, two 8-element chunks each way).  In LDS, row r keeps its
// 16-byte chunk q at position q ^ ((r >> 3) & 7), so that the column reads of the
// second phase (lane = (column c, 8-row block b), eight rows 8b..8b+7 of one
// column) spread over the banks.
namespace {

__device__ __forceinline__ int tp_pos(int r, int q) { return r * 64 + ((q ^ ((r >> 3) & 7)) << 3); }

// Second phase: output chunk (c, b) = tile[8b .. 8b+7][c] as one 16-byte store.
__device__ __forceinline__ uint4 tp_column(const uint16_t* tile, int c, int b) {
  uint32_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * b + 2 * i;
    const uint32_t lo = tile[tp_pos(r, c >> 3) + (c & 7)];
    const uint32_t hi = tile[tp_pos(r + 1, c >> 3) + (c & 7)];
    v[i] = lo | (hi << 16);
  }
  return make_uint4(v[0], v[1], v[2], v[3]);
}

}  // namespace

// Permuted rows [R, C] -> expert-major transposed blocks: expert e's block is
// [C, kpad_e] (kpad_e = koff[e+1] - koff[e] = round_up(M_e, 64)) at element
// C * koff[e]; its column i holds row offsets[e] + i for i < M_e and zero
// after.  blockIdx.x walks 64-column blocks of the padded column range
// [0, koff[E]); a block lies inside one expert's range since every koff[e] is a
// multiple of 64.  C a multiple of 8; koff[E] <= ldd bounds the grid.  With
// src_rows set, row p is read from row src_rows[p] / src_div of src (token rows
// through the permutation; src has src_total rows, indices clamped into them),
// and with src_scale also set it is multiplied by src_scale[src_rows[p]] (one
// rounding to bf16 of the fp32 product).
__global__ __launch_bounds__(256) void transpose_segments_bf16_kernel(const uint16_t* __restrict__ src, int R,
                                                                      int C, const int* __restrict__ offsets,
                                                                      const int* __restrict__ koff, int E,
                                                                      const int* __restrict__ src_rows, int src_div,
                                                                      int src_total, const float* __restrict__ src_scale,
                                                                      uint16_t* __restrict__ dst, int ldd) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * 64];
  const int j0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int Vp = min(koff[E], ldd);
  if (j0 >= Vp) return;
  int lo = 0, hi = E;   // largest e with koff[e] <= j0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (koff[mid] <= j0) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int i0 = j0 - koff[e];                  // column of the expert's block
  const int kpad = koff[e + 1] - koff[e];
  const int p0 = clamp_off(offsets, e, R) + i0;
  const int pend = clamp_off(offsets, e + 1, R);
  uint16_t* blk = dst + (size_t)C * koff[e];    // the expert's [C, kpad] block
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = t + 256 * h;
    const int r = idx >> 3, q = idx & 7;
    const int p = p0 + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (p < pend && c0 + 8 * q < C) {
      if (src_rows != nullptr) {
        const int fr = min(max(src_rows[p], 0), src_total * src_div - 1);
        v = *reinterpret_cast<const uint4*>(src + (size_t)(fr / src_div) * C + c0 + 8 * q);
        if (src_scale != nullptr) {
          const float sc = src_scale[fr];
          const uint32_t in[4] = {v.x, v.y, v.z, v.w};
          uint32_t o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o[i] = pack_bf16x2(sc * bf16_bits_to_f32(in[i] & 0xffffu), sc * bf16_bits_to_f32(in[i] >> 16));
          v = make_uint4(o[0], o[1], o[2], o[3]);
        }
      } else {
        v = *reinterpret_cast<const uint4*>(src + (size_t)p * C + c0 + 8 * q);
      }
    }
    *reinterpret_cast<uint4*>(tile + tp_pos(r, q)) = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = t + 256 * h;
    const int c = idx >> 3, b = idx & 7;
    if (c0 + c < C) *reinterpret_cast<uint4*>(blk + (size_t)(c0 + c) * kpad + i0 + 8 * b) = tp_column(tile, c, b);
  }
}

// One wave per slot r, with p = row_pos[r] (valid when p < V):
//   dw[r]  = dh1[p] . h[p]   (fp32, lanes then a butterfly; 0 for a sentinel slot)
//   dgu[p] = [dh * u * silu'(g), dh * silu(g)] with dh = w[r] * dh1[p] (bf16 out)
// dw may be null (no routing-weight gradient wanted).
__global__ __launch_bounds__(256) void silu_bwd_route_kernel(const float* __restrict__ dh1, const float* __restrict__ gu,
                                                             const uint16_t* __restrict__ h, const float* __restrict__ w,
                                                             const int* __restrict__ row_pos,
                                                             const int* __restrict__ offsets, int E, int R, int I,
                                                             uint16_t* __restrict__ dgu, float* __restrict__ dw) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (r >= R) return;
  const int V = clamp_off(offsets, E, R);
  const int p = row_pos[r];
  float acc = 0.0f;
  if (p >= 0 && p < V) {
    const float wr = w[r];
    const float* d = dh1 + (size_t)p * I;
    const float* g = gu + (size_t)p * 2 * I;
    const float* u = g + I;
    const uint16_t* hp = h + (size_t)p * I;
    uint16_t* og = dgu + (size_t)p * 2 * I;
    uint16_t* ou = og + I;
    for (int c = lane * 4; c < I; c += kWave * 4) {
      const float4 d4 = *reinterpret_cast<const float4*>(d + c);
      const float4 g4 = *reinterpret_cast<const float4*>(g + c);
      const float4 u4 = *reinterpret_cast<const float4*>(u + c);
      const uint2 h4 = *reinterpret_cast<const uint2*>(hp + c);
      acc = fmaf(d4.x, bf16_bits_to_f32(h4.x & 0xffffu), acc);
      acc = fmaf(d4.y, bf16_bits_to_f32(h4.x >> 16), acc);
      acc = fmaf(d4.z, bf16_bits_to_f32(h4.y & 0xffffu), acc);
      acc = fmaf(d4.w, bf16_bits_to_f32(h4.y >> 16), acc);
      const float dd[4] = {wr * d4.x, wr * d4.y, wr * d4.z, wr * d4.w};
      const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
      const float uu[4] = {u4.x, u4.y, u4.z, u4.w};
      float dg[4], du[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dg[i] = dd[i] * uu[i] * dsilu(gg[i]);
        du[i] = dd[i] * silu_mul(gg[i], 1.0f);
      }
      *reinterpret_cast<uint2*>(og + c) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
      *reinterpret_cast<uint2*>(ou + c) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
    }
    acc = wave_sum(acc);
  }
  if (dw != nullptr && lane == 0) dw[r] = acc;
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ p, long long n, float v) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

namespace {
dim3 grid1d(long long n, int per_block) {
  long long b = (n + per_block - 1) / per_block;
  return dim3((unsigned)(b < 1 ? 1 : (b > 65535LL * 32 ? 65535LL * 32 : b)));
}
}  // namespace

// ---------------------------------------------------------------- fp8 layer
//
// The fp8 layer's backward runs the steps above on dequantised operands, straight
// through its quantisers: x-hat = dq(q(x)) per token and 128 channels, the weights'
// dequantised block values, and h-hat = dq(q(h)) per row and 128 channels in place of
// h (y and dW2 of the fp8 forward use the quantised h).  Codes are decided with the
// forward's arithmetic (scale = amax / 448, code = RNE(clamp(v / scale)), e4m3) and
// decoded exactly; the dequantised values are rounded once to bf16.

namespace {

// 8 values of one 128-channel group held by a lane of a 16-lane group -> their
// quantise-dequantise images, rounded to bf16 (4 packed pairs)
__device__ __forceinline__ uint4 fake_quant8(const float (&v)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  const float scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t c = cvt_e4m3x2(clamp448(v[2 * i] / scale), clamp448(v[2 * i + 1] / scale));
    out[i] = pack_bf16x2(__builtin_amdgcn_cvt_f32_fp8((int)c, 0) * scale,
                         __builtin_amdgcn_cvt_f32_fp8((int)c, 1) * scale);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

}  // namespace

// x-hat [T, H] from bf16 x [T, H] (H % 128 == 0): one 16-lane group per row and
// 128-channel group, 8 channels per lane.
__global__ __launch_bounds__(256) void fake_quant_rows_kernel(const uint4* __restrict__ x, long long groups,
                                                              uint4* __restrict__ xhat) {
  const long long gi = ((long long)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int li = threadIdx.x & 15;
  const bool ok = gi < groups;
  float v[8];
  const uint4 raw = ok ? x[gi * 16 + li] : make_uint4(0, 0, 0, 0);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
  const uint4 o = fake_quant8(v);
  if (ok) xhat[gi * 16 + li] = o;
}

// h-hat rows p < offsets[E] of h [R, I] from the f32 pre-activations gu = [g | u]
// [R, 2I]: h = silu(g) * u (the forward epilogue's function), then quantise-dequantise
// per 128 channels.  One 16-lane group per row and 128-channel group.
__global__ __launch_bounds__(256) void h_fake_quant_kernel(const float* __restrict__ gu, const int* __restrict__ offsets,
                                                           int E, int R, int I, uint4* __restrict__ h) {
  const long long gi = ((long long)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int li = threadIdx.x & 15;
  const int per_row = I / 128;
  const long long V = min(max(offsets[E], 0), R);
  const bool ok = gi < V * per_row;
  const long long p = ok ? gi / per_row : 0;
  const int c = (int)(ok ? gi - p * per_row : 0) * 128 + li * 8;
  float v[8];
  if (ok) {
    const float4* gp = reinterpret_cast<const float4*>(gu + p * 2 * I + c);
    const float4* up = reinterpret_cast<const float4*>(gu + p * 2 * I + I + c);
    const float4 g0 = gp[0], g1 = gp[1], u0 = up[0], u1 = up[1];
    v[0] = silu_mul(g0.x, u0.x); v[1] = silu_mul(g0.y, u0.y); v[2] = silu_mul(g0.z, u0.z); v[3] = silu_mul(g0.w, u0.w);
    v[4] = silu_mul(g1.x, u1.x); v[5] = silu_mul(g1.y, u1.y); v[6] = silu_mul(g1.z, u1.z); v[7] = silu_mul(g1.w, u1.w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  const uint4 o = fake_quant8(v);
  if (ok) h[(p * I + c) / 8] = o;
}

// bf16 [E, N, K] from e4m3 codes [E, N, K] and block scales [E, N/128, K/128]
// (N, K multiples of 128).  A workgroup takes kDqRows rows of the flattened [E*N, K] code
// matrix at a time (a row: one expert and output channel, so one row of scales), each
// thread 16 codes per row and column step; all of a step's loads are issued before any is
// converted, so that each thread keeps kDqRows 16-byte loads in flight.
constexpr int kDqRows = 8;
__global__ __launch_bounds__(256) void dequant_blocks_kernel(const uint4* __restrict__ q, const float* __restrict__ s,
                                                             long long rows, int N, int K, uint4* __restrict__ out) {
  const int k16 = K / 16, kb = K / 128, nb = N / 128;
  for (long long row0 = (long long)blockIdx.x * kDqRows; row0 < rows; row0 += (long long)gridDim.x * kDqRows) {
    for (int c = threadIdx.x; c < k16; c += 256) {
      uint4 v[kDqRows];
#pragma unroll
      for (int r = 0; r < kDqRows; ++r)
        if (row0 + r < rows) v[r] = q[(row0 + r) * k16 + c];
#pragma unroll
      for (int r = 0; r < kDqRows; ++r) {
        const long long row = row0 + r;
        if (row >= rows) break;
        const long long e = row / N;
        const int n = (int)(row - e * N);
        const float sc = s[(e * nb + n / 128) * kb + (c >> 3)];   // codes 16c.. lie in 128-block c / 8
        const uint32_t w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int wv = (int)w[j];
          o[2 * j] = pack_bf16x2(__builtin_amdgcn_cvt_f32_fp8(wv, 0) * sc, __builtin_amdgcn_cvt_f32_fp8(wv, 1) * sc);
          o[2 * j + 1] = pack_bf16x2(__builtin_amdgcn_cvt_f32_fp8(wv, 2) * sc, __builtin_amdgcn_cvt_f32_fp8(wv, 3) * sc);
        }
        uint4* orow = out + row * k16 * 2;
        orow[2 * c] = make_uint4(o[0], o[1], o[2], o[3]);
        orow[2 * c + 1] = make_uint4(o[4], o[5], o[6], o[7]);
      }
    }
  }
}

hipError_t launch_fake_quant_rows(const void* x, long long T, int H, void* xhat, hipStream_t stream) {
  const long long groups = T * (H / 128);
  if (groups == 0) return hipSuccess;
  const long long blocks = (groups * 16 + 255) / 256;
  hipLaunchKernelGGL(fake_quant_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(x), groups, static_cast<uint4*>(xhat));
  return hipGetLastError();
}

hipError_t launch_h_fake_quant(const float* gu, const int* offsets, int E, int R, int I, void* h, hipStream_t stream) {
  const long long groups = (long long)R * (I / 128);
  if (groups == 0) return hipSuccess;
  const long long blocks = (groups * 16 + 255) / 256;
  hipLaunchKernelGGL(h_fake_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, gu, offsets, E, R, I,
                     static_cast<uint4*>(h));
  return hipGetLastError();
}

hipError_t launch_dequant_blocks(const void* q, const float* s, int E, int N, int K, void* out, hipStream_t stream) {
  const long long rows = (long long)E * N;
  if (rows == 0 || K == 0) return hipSuccess;
  const long long blocks = std::min<long long>((rows + kDqRows - 1) / kDqRows, 16384);
  hipLaunchKernelGGL(dequant_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(q), s, rows, N, K, static_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_pad_offsets(const int* offsets, int E, int R, int* koff, hipStream_t stream) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(1024), 0, stream, offsets, E, R, koff);
  return hipGetLastError();
}

hipError_t launch_transpose_segments_bf16(const void* src, int R, int C, const int* offsets, const int* koff, int E,
                                          const int* src_rows, int src_div, int src_total, const float* src_scale,
                                          void* dst, int ldd, hipStream_t stream) {
  if (R > 0 && C > 0)
    hipLaunchKernelGGL(transpose_segments_bf16_kernel, dim3((ldd + 63) / 64, (C + 63) / 64), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(src), R, C, offsets, koff, E, src_rows, src_div > 0 ? src_div : 1,
                       src_total, src_scale, static_cast<uint16_t*>(dst), ldd);
  return hipGetLastError();
}

hipError_t launch_silu_bwd_route(const float* dh1, const float* gu, const void* h, const float* w,
                                 const int* row_pos, const int* offsets, int E, int R, int I, void* dgu, float* dw,
                                 hipStream_t stream) {
  if (R > 0)
    hipLaunchKernelGGL(silu_bwd_route_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, stream, dh1, gu,
                       static_cast<const uint16_t*>(h), w, row_pos, offsets, E, R, I, static_cast<uint16_t*>(dgu), dw);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, long long n, float v, hipStream_t stream) {
  if (n > 0) hipLaunchKernelGGL(fill_f32_kernel, grid1d(n, 256 * 4), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

}  // namespace moe
