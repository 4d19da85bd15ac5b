// launch.h -- internal launchers behind the C ABI (not part of the public interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_route_topk(const float* logits, int T, int E, int k, long long valid_rows,
                             int renorm, int* ids, float* weights, hipStream_t stream);

// T*k <= 1024: routing and offsets in one launch (one workgroup of 16 waves, a wave per
// token at a time); same outputs as launch_route_topk followed by launch_build_offsets.
hipError_t launch_route_offsets_single(const float* logits, int T, int E, int k, long long valid_rows, int renorm,
                                       int* ids, float* weights, int* offsets, int* sorted_rows, int* row_pos,
                                       hipStream_t stream);
// T >= 1, k <= 16: routing with per-chunk histograms in one launch (launch_route_hist),
// then a per-bin scan over chunks and the scatter (launch_offsets_from_hist, on the same
// workspace): three launches instead of four, with the outputs of launch_route_topk
// followed by launch_build_offsets.  workspace: route_offsets_workspace_bytes(T, E) bytes,
// 4-byte aligned.
size_t route_offsets_workspace_bytes(long long T, int E);
hipError_t launch_route_hist(const float* logits, int T, int E, int k, long long valid_rows, int renorm,
                             int* ids, float* weights, void* workspace, hipStream_t stream);
hipError_t launch_offsets_from_hist(const int* ids, int T, int E, int k, int* offsets, int* sorted_rows,
                                    int* row_pos, void* workspace, hipStream_t stream);
size_t build_offsets_workspace_bytes(long long R, int E);
// the allocation-free variant's static scratch: its size, and this device's address of it
size_t build_offsets_noalloc_capacity();
hipError_t build_offsets_noalloc_scratch(void** out);
hipError_t launch_build_offsets(const int* ids, int R, int E, int* offsets, int* sorted_rows,
                                int* row_pos, void* workspace, hipStream_t stream);

hipError_t launch_permute_copy(const void* x, int T, int row_bytes, int k, const int* sorted_rows,
                               const int* offsets, int E, int R, void* xp, hipStream_t stream);
// sorted_rows and offsets null: row p of xq is token row p, R = T rows; f32_in: x is f32.
// Token rows with xs_perm set: each token's scales are also stored at the permuted
// positions row_pos[t*kslots + j] (j < kslots) of xs_perm [H/128, R_perm].
hipError_t launch_permute_quant(const void* x, int T, int H, int k, const int* sorted_rows,
                                const int* offsets, int E, int R, void* xq, float* xs,
                                hipStream_t stream, bool f32_in = false, const int* row_pos = nullptr,
                                int kslots = 0, float* xs_perm = nullptr, int R_perm = 0);
// xs_perm [G, R] at routed position p < offsets[E] = xs [G, T] of the row's token
// (sorted_rows[p] / k): the token scales copied to the permuted positions by a gather,
// coalesced along p, instead of the quantising kernel's per-slot stores.
hipError_t launch_gather_scales(const float* xs, int T, int G, const int* sorted_rows, int k,
                                const int* offsets, int E, int R, float* xs_perm, hipStream_t stream);

struct GemmLaunch {
  const void* A;
  const float* a_scales;
  const void* B;
  const float* b_scales;
  int ab_dtype;  // moe_dtype_t
  const int* offsets;
  int E;
  long long M_rows, N, K;
  bool silu;
  void* C;
  int c_dtype;   // moe_dtype_t
  float* c_scales;
  // K-grouped mode (bf16 operands, no SiLU, f32/bf16 C): when koff is set,
  // C[e] [M_rows, N] = A_e B_e^T for e < E, with A_e [M_rows, kpad_e] at element
  // M_rows * koff[e] of A and B_e [N, kpad_e] at element N * koff[e] of B
  // (kpad_e = koff[e+1] - koff[e], a multiple of 64); offsets is unused and
  // lda = ldb bound koff[E] (the padded column count).
  const int* koff = nullptr;
  long long lda = 0, ldb = 0;
  // Gathered A (M-grouped mode only): row p of the product reads row
  // a_rows[p] / a_div of A, which has a_total rows (a_scales [K/128, a_total]).
  const int* a_rows = nullptr;
  int a_div = 1;
  long long a_total = 0;
  // fp8 with a row map: a_scales indexed by product row ([K/128, M_rows]) instead of by A row
  bool a_scales_by_row = false;
  // bf16 operands and C, M-grouped mode: SiLU*up also stores the f32 pre-activations
  // [M_rows, 2 N_out] (pre_out)
  float* pre_out = nullptr;
  // rows the tile choice assumes (0: M_rows); a caller that knows on the host that only
  // the first tile_rows rows can be valid passes that count
  long long tile_rows = 0;
  // M-grouped bf16 without SiLU: B stored [E][K][N] (N contiguous) instead of [E][N][K]
  bool b_kn = false;
};
hipError_t launch_grouped_gemm(const GemmLaunch& p, hipStream_t stream);
bool grouped_gemm_tile_shape(int ab_dtype, bool silu, int c_dtype, long long M_rows, int E, int* tile_m,
                             int* tile_n, int* k_slice);
// launches of at most 8 rows per expert take the decode tiles (bf16; fp8 with bf16/f32 output)
bool use_decode_tiles(long long M_rows, int E);

// backward steps (backward.hip)
hipError_t launch_pad_offsets(const int* offsets, int E, int R, int* koff, hipStream_t stream);
// src_rows nullable: row p of the segments is src row src_rows[p] / src_div (of src_total),
// times src_scale[src_rows[p]] when src_scale is set
hipError_t launch_transpose_segments_bf16(const void* src, int R, int C, const int* offsets, const int* koff, int E,
                                          const int* src_rows, int src_div, int src_total, const float* src_scale,
                                          void* dst, int ldd, hipStream_t stream);
// per slot r (p = row_pos[r] < V): dw[r] = dh1[p] . h[p]; dgu[p] = SiLU*up backward of w[r] * dh1[p]
hipError_t launch_silu_bwd_route(const float* dh1, const float* gu, const void* h, const float* w,
                                 const int* row_pos, const int* offsets, int E, int R, int I, void* dgu, float* dw,
                                 hipStream_t stream);
hipError_t launch_fill_f32(float* p, long long n, float v, hipStream_t stream);
// fp8 layer backward: x-hat = dq(q(x)) per token and 128 channels (bf16 in and out);
// h-hat rows p < offsets[E] of h [R, I] (bf16) from the f32 pre-activations gu [R, 2I];
// bf16 [E, N, K] from e4m3 codes with [E, N/128, K/128] block scales
hipError_t launch_fake_quant_rows(const void* x, long long T, int H, void* xhat, hipStream_t stream);
hipError_t launch_h_fake_quant(const float* gu, const int* offsets, int E, int R, int I, void* h, hipStream_t stream);
hipError_t launch_dequant_blocks(const void* q, const float* s, int E, int N, int K, void* out, hipStream_t stream);

hipError_t launch_combine(const void* y, bool y_bf16, const int* row_pos, const float* weights,
                          const int* offsets, int E, int T, int H, int k, void* out, bool out_bf16,
                          hipStream_t stream);

}  // namespace moe
