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
//   expand:       dy[p]  = w[r] * dout[r / k]           (p < V; r = sorted_rows[p])
//   silu_bwd:     dgu[p] = [dh * u * silu'(g), dh * silu(g)]
//   route_grad:   dw[r]  = dout[r / k] . y[row_pos[r]]  (0 for a sentinel slot)
//   transposes:   weights [E, R, C] -> [E, C, R] (R, C multiples of 8); permuted
//                 activations [R, C] -> expert-major blocks [C, round_up(M_e, 64)]
//                 (rows of an expert contiguous, padding columns zero), so that every
//                 expert's K range is whole 64-element slices for the weight-gradient
//                 GEMM and each of its tiles reads a compact block.

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kMaxE = 1024;

__device__ __forceinline__ int clamp_off(const int* offsets, int e, int R) {
  return min(max(offsets[e], 0), R);
}

__device__ __forceinline__ float bf16_at(const uint16_t* p) { return bf16_bits_to_f32(*p); }

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

// Transposes move 64x64 element tiles through LDS with 16-byte global loads and
// stores (256 threads, two 8-element chunks each way).  In LDS, row r keeps its
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

// Batched: dst[b][c][r] = src[b][r][c]; R and C multiples of 8.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src, int R, int C,
                                                             uint16_t* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * 64];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const size_t bz = blockIdx.z;
  const uint16_t* s = src + bz * (size_t)R * C;
  uint16_t* d = dst + bz * (size_t)R * C;
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = t + 256 * h;            // chunk (row r, chunk q) of the source tile
    const int r = idx >> 3, q = idx & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + r < R && c0 + 8 * q < C) v = *reinterpret_cast<const uint4*>(s + (size_t)(r0 + r) * C + c0 + 8 * q);
    *reinterpret_cast<uint4*>(tile + tp_pos(r, q)) = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = t + 256 * h;            // output chunk (column c, row block b)
    const int c = idx >> 3, b = idx & 7;
    if (c0 + c < C && r0 + 8 * b < R)
      *reinterpret_cast<uint4*>(d + (size_t)(c0 + c) * R + r0 + 8 * b) = tp_column(tile, c, b);
  }
}

// Permuted rows [R, C] -> expert-major transposed blocks: expert e's block is
// [C, kpad_e] (kpad_e = koff[e+1] - koff[e] = round_up(M_e, 64)) at element
// C * koff[e]; its column i holds row offsets[e] + i for i < M_e and zero
// after.  blockIdx.x walks 64-column blocks of the padded column range
// [0, koff[E]); a block lies inside one expert's range since every koff[e] is a
// multiple of 64.  C a multiple of 8; koff[E] <= ldd bounds the grid.  With
// src_rows set, row p is read from row src_rows[p] / src_div of src (token rows
// through the permutation; src has src_total rows, indices clamped into them).
__global__ __launch_bounds__(256) void transpose_segments_bf16_kernel(const uint16_t* __restrict__ src, int R,
                                                                      int C, const int* __restrict__ offsets,
                                                                      const int* __restrict__ koff, int E,
                                                                      const int* __restrict__ src_rows, int src_div,
                                                                      int src_total, uint16_t* __restrict__ dst,
                                                                      int ldd) {
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
      const int sr = src_rows != nullptr ? min(max(src_rows[p] / src_div, 0), src_total - 1) : p;
      v = *reinterpret_cast<const uint4*>(src + (size_t)sr * C + c0 + 8 * q);
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

// dgu[p] = [dh * u * silu'(g), dh * silu(g)] for p < V; bf16 out.
__global__ __launch_bounds__(256) void silu_bwd_rows_kernel(const float* __restrict__ dh, const float* __restrict__ gu,
                                                            const int* __restrict__ offsets, int E, int R, int I,
                                                            uint16_t* __restrict__ dgu) {
  const int V = clamp_off(offsets, E, R);
  const long long n4 = (long long)V * (I / 4);
  for (long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += (long long)gridDim.x * blockDim.x) {
    const long long p = q / (I / 4);
    const int c = (int)(q - p * (I / 4)) * 4;
    const float4 d = *reinterpret_cast<const float4*>(dh + p * I + c);
    const float4 g = *reinterpret_cast<const float4*>(gu + p * 2 * I + c);
    const float4 u = *reinterpret_cast<const float4*>(gu + p * 2 * I + I + c);
    const float dg[4] = {d.x * u.x * dsilu(g.x), d.y * u.y * dsilu(g.y), d.z * u.z * dsilu(g.z), d.w * u.w * dsilu(g.w)};
    const float du[4] = {d.x * silu_mul(g.x, 1.0f), d.y * silu_mul(g.y, 1.0f), d.z * silu_mul(g.z, 1.0f),
                         d.w * silu_mul(g.w, 1.0f)};
    *reinterpret_cast<uint2*>(dgu + p * 2 * I + c) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
    *reinterpret_cast<uint2*>(dgu + p * 2 * I + I + c) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
  }
}

// dy[p] = w[r] * dout[r / k] (bf16) for p < V; one wave per row, 8 columns per lane step.
__global__ __launch_bounds__(256) void expand_rows_kernel(const uint16_t* __restrict__ dout, const float* __restrict__ w,
                                                          const int* __restrict__ sorted_rows, const int* __restrict__ offsets,
                                                          int E, int T, int k, int H, uint16_t* __restrict__ dy) {
  const int R = T * k;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (p >= clamp_off(offsets, E, R)) return;
  const int r = sorted_rows[p];
  if (r < 0 || r >= R) return;   // inconsistent permutation: leave the row unwritten
  const float wr = w[r];
  const uint4* s = reinterpret_cast<const uint4*>(dout + (size_t)(r / k) * H);
  uint4* d = reinterpret_cast<uint4*>(dy + (size_t)p * H);
  for (int c = lane; c < H / 8; c += kWave) {
    const uint4 v = s[c];
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_bf16x2(wr * bf16_bits_to_f32(in[i] & 0xffffu), wr * bf16_bits_to_f32(in[i] >> 16));
    d[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// dw[r] = dout[r / k] . y[row_pos[r]] over valid slots, 0 otherwise; one wave per slot.
__global__ __launch_bounds__(256) void route_grad_kernel(const uint16_t* __restrict__ dout, const float* __restrict__ y,
                                                         const int* __restrict__ row_pos, const int* __restrict__ offsets,
                                                         int E, int T, int k, int H, float* __restrict__ dw) {
  const int R = T * k;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (r >= R) return;
  const int V = clamp_off(offsets, E, R);
  const int p = row_pos[r];
  float acc = 0.0f;
  if (p >= 0 && p < V) {
    const uint16_t* dt = dout + (size_t)(r / k) * H;
    const float* yp = y + (size_t)p * H;
    for (int c = lane; c < H; c += kWave) acc = fmaf(bf16_at(dt + c), yp[c], acc);
    acc = wave_sum(acc);
  }
  if (lane == 0) dw[r] = acc;
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

hipError_t launch_pad_offsets(const int* offsets, int E, int R, int* koff, hipStream_t stream) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(1024), 0, stream, offsets, E, R, koff);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void* src, int batch, int R, int C, void* dst, hipStream_t stream) {
  if (batch > 0 && R > 0 && C > 0)
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((R + 63) / 64, (C + 63) / 64, batch), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(src), R, C, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_transpose_segments_bf16(const void* src, int R, int C, const int* offsets, const int* koff, int E,
                                          const int* src_rows, int src_div, int src_total, void* dst, int ldd,
                                          hipStream_t stream) {
  if (R > 0 && C > 0)
    hipLaunchKernelGGL(transpose_segments_bf16_kernel, dim3((ldd + 63) / 64, (C + 63) / 64), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(src), R, C, offsets, koff, E, src_rows, src_div > 0 ? src_div : 1,
                       src_total, static_cast<uint16_t*>(dst), ldd);
  return hipGetLastError();
}

hipError_t launch_silu_bwd_rows(const float* dh, const float* gu, const int* offsets, int E, int R, int I, void* dgu,
                                hipStream_t stream) {
  if (R > 0)
    hipLaunchKernelGGL(silu_bwd_rows_kernel, grid1d((long long)R * (I / 4), 256 * 8), dim3(256), 0, stream, dh, gu,
                       offsets, E, R, I, static_cast<uint16_t*>(dgu));
  return hipGetLastError();
}

hipError_t launch_expand_rows(const void* dout, const float* w, const int* sorted_rows, const int* offsets, int E,
                              int T, int k, int H, void* dy, hipStream_t stream) {
  const long long R = (long long)T * k;
  if (R > 0)
    hipLaunchKernelGGL(expand_rows_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(dout), w, sorted_rows, offsets, E, T, k, H,
                       static_cast<uint16_t*>(dy));
  return hipGetLastError();
}

hipError_t launch_route_grad(const void* dout, const float* y, const int* row_pos, const int* offsets, int E, int T,
                             int k, int H, float* dw, hipStream_t stream) {
  const long long R = (long long)T * k;
  if (R > 0)
    hipLaunchKernelGGL(route_grad_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(dout), y, row_pos, offsets, E, T, k, H, dw);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, long long n, float v, hipStream_t stream) {
  if (n > 0) hipLaunchKernelGGL(fill_f32_kernel, grid1d(n, 256 * 4), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

}  // namespace moe
