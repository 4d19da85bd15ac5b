/*
 * moe.h -- C ABI of the MoE expert layer's grouped-GEMM path for MI355X (gfx950).
 *
 * The path: top-k routing -> per-expert histogram with sentinel rows counted
 * out -> exclusive-scan offsets -> stable permutation into expert-contiguous
 * order -> grouped GEMM gate/up with a fused SiLU(gate)*up -> grouped GEMM
 * down -> routing-weight-scaled combine back to token order.
 *
 * Sources (the three web write-ups the method is described in):
 *   [T45621]  "Hugging Face Transformers: MoE 및 FP8 커널 최적화를 통한 성능 향상"
 *             (transformers PR #45621 analysis); section 1 (kernel loading),
 *             section 2 (sentinel-token handling), section 3 (fp8 NaN fix).
 *   [LF10481] "LlamaFactory의 Triton 기반 Fused MoE 커널 도입"
 *             (LlamaFactory PR #10481 analysis); section 1 (fused MoE pipeline).
 *   [MoEs]    "트랜스포머에서 전문가 혼합 (MoEs)"; sections on MoE basics,
 *             WeightConverter, expert backends and expert parallelism.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major,
 *    densely packed (no padding between rows), 16-byte aligned.
 *  - Flat routed row r = t*k + j (token t, slot j).  R = T*k.
 *  - Expert id E is the sentinel: a row that is not computed (unrouted or
 *    padding).  Ids outside [0, E] are treated as sentinel as well.
 *  - offsets is int32[E+1]: offsets[0] = 0, offsets[e+1] - offsets[e] = rows
 *    routed to expert e, offsets[E] = V = number of valid (non-sentinel) rows.
 *    Permuted positions [offsets[e], offsets[e+1]) belong to expert e;
 *    positions [V, R) are sentinel.
 *  - Packed weights are expert-major (the stacked layout of [MoEs],
 *    WeightConverter / MergeModulelist): gate/up W13 [E, 2I, H] with rows
 *    [0, I) = gate and [I, 2I) = up; down W2 [E, H, I].  Both are [E, N, K]
 *    with K contiguous.
 *  - fp8 is OCP E4M3 ("e4m3fn", max 448).  fp8 weights carry one fp32 scale
 *    per 128x128 block ([E, N/128, K/128]); fp8 activations carry one fp32
 *    scale per row and 128 consecutive channels, stored channel-block-major
 *    ([K/128, rows]: the scales of one 128-channel block are contiguous over
 *    rows).  A value is code * scale.  Activation scales are amax/448 (1 for an all-zero group),
 *    codes are round-to-nearest-even of value/scale, saturating.
 *  - Every call validates its arguments on the host first and returns
 *    MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED / MOE_ERR_WORKSPACE without
 *    launching anything when they fail.  Otherwise it enqueues its kernels on
 *    `stream` (a hipStream_t; NULL = the default stream) and returns without
 *    synchronising; a launch failure returns MOE_ERR_LAUNCH.  No call
 *    allocates or frees memory or keeps a pointer after it returns.  No C++
 *    exception crosses this boundary.  moe_last_error() gives a thread-local
 *    message for the last non-OK status.
 *  - Limits: 1 <= E <= 1024, 1 <= k <= min(E, 16), R = T*k < 2^31.
 *  - Results are deterministic: repeated calls on the same inputs give
 *    bitwise-identical outputs (no floating-point atomics, no split-K).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_LAUNCH = 4
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype_t;

typedef enum { MOE_EPI_NONE = 0, MOE_EPI_SILU_MUL = 1 } moe_epilogue_t;

/*
 * moe_route_topk -- the router's choice of a small subset of experts per
 * token ([MoEs], MoE basics).
 *
 *   logits        f32 [T, E], finite values.
 *   topk_ids      out int32 [T, k]: slot j holds the expert with the j-th
 *                 largest logit; equal logits go to the lower expert id.
 *   topk_weights  out f32 [T, k]: renormalize = 1: softmax over the k
 *                 selected logits; renormalize = 0: softmax over all E logits
 *                 read at the selected experts.
 *   num_valid_rows  < 0: all R = T*k flat rows are valid; otherwise flat rows
 *                 r >= num_valid_rows are written as sentinel (id = E,
 *                 weight = 0).
 */
moe_status_t moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                            int64_t num_valid_rows, int32_t renormalize,
                            int32_t* topk_ids, float* topk_weights, void* stream);

/* Bytes of device workspace moe_build_offsets needs for R rows and E experts. */
size_t moe_build_offsets_workspace(int64_t R, int32_t E);

/*
 * moe_build_offsets -- per-expert histogram with the sentinel bin left out,
 * its exclusive scan, and the stable permutation ([T45621] section 2:
 * sentinel rows are excluded from the histogram, or sorted as the largest key
 * so that they fall to the end; offsets[-1] is the valid-row count; [MoEs]
 * expert backends: grouped_mm sorts tokens by expert id).
 *
 *   topk_ids     int32 [R], values in [0, E]; E (or anything outside
 *                [0, E]) = sentinel.
 *   offsets      out int32 [E+1] (see conventions).
 *   sorted_rows  out int32 [R]: flat row at each permuted position; rows of
 *                one expert in ascending flat order, sentinel rows last (also
 *                ascending).
 *   row_pos      out int32 [R]: inverse of sorted_rows.
 *   workspace    device scratch of >= moe_build_offsets_workspace(R, E)
 *                bytes (else MOE_ERR_WORKSPACE); contents need no
 *                initialisation and are garbage afterwards.
 */
moe_status_t moe_build_offsets(const int32_t* topk_ids, int64_t R, int32_t E,
                               int32_t* offsets, int32_t* sorted_rows, int32_t* row_pos,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_build_offsets_noalloc -- moe_build_offsets for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * results and errors as moe_build_offsets, without the workspace: the
 * kernels' per-chunk histograms live in a static device array inside the
 * library, 4 MiB per GPU, held from the first call on that GPU until the
 * process ends.  Calls whose moe_build_offsets_workspace(R, E) exceeds 4 MiB
 * (e.g. R > ~1M rows at E = 1024) return MOE_ERR_WORKSPACE before launching.
 * The first call on a GPU looks up that GPU's address of the array (the
 * stream must belong to the current device, as for every entry point).
 * Nothing is allocated and nothing in the array needs clearing, but every
 * call on one GPU uses the same array: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 */
moe_status_t moe_build_offsets_noalloc(const int32_t* topk_ids, int64_t R, int32_t E,
                                       int32_t* offsets, int32_t* sorted_rows, int32_t* row_pos,
                                       void* stream);

/*
 * moe_permute -- moves token rows into expert-contiguous order (the
 * scatter step of [LF10481] section 1): x_perm[p] = x[sorted_rows[p] / k]
 * for p < offsets[E].  Rows p >= offsets[E] of x_perm are not written.
 *
 *   x            [T, H] of x_dtype (MOE_F32 or MOE_BF16).
 *   perm_dtype   == x_dtype: exact copy.  MOE_FP8_E4M3 (x_dtype MOE_BF16,
 *                H % 128 == 0): each row is quantised per 128 channels
 *                (the per-token activation cast that [T45621] section 1
 *                loads as fp8_act_quant / per_token_cast_to_fp8) into
 *                x_perm codes [R, H] and x_perm_scales f32 [H/128, R].
 *   R            rows of x_perm (>= offsets[E]); T*k for the layer.
 */
moe_status_t moe_permute(const void* x, moe_dtype_t x_dtype, int64_t T, int64_t H, int32_t k,
                         const int32_t* sorted_rows, const int32_t* offsets, int32_t E,
                         int64_t R, void* x_perm, moe_dtype_t perm_dtype,
                         float* x_perm_scales, void* stream);

/*
 * moe_grouped_gemm -- one GEMM per expert over its row segment, same N and K
 * for every group (the group_gemm_same_nk step of [LF10481] section 1;
 * [MoEs] expert backends, grouped_mm):
 *
 *   for p in [offsets[e], offsets[e+1]):  acc[p, n] = sum_k A[p, k] * B[e, n, k]
 *
 *   A         [M_rows, K] of ab_dtype; a_scales f32 [K/128, M_rows] for fp8.
 *   B         [E, N, K] of ab_dtype;   b_scales f32 [E, N/128, K/128] for fp8.
 *   ab_dtype  MOE_F32, MOE_BF16 or MOE_FP8_E4M3 (K % 128 == 0 for fp8).
 *   offsets   device int32 [E+1]; read on the device (no host sync).
 *   epi       MOE_EPI_NONE: C = acc, N_out = N.
 *             MOE_EPI_SILU_MUL: N even, B rows [0, N/2) are gate and
 *             [N/2, N) up; C = silu(gate) * up, N_out = N/2 (the
 *             SiLU(fc1_1) * fc1_2 step of [LF10481] section 1).
 *   C         [M_rows, N_out] of c_dtype: MOE_F32, MOE_BF16, or MOE_FP8_E4M3
 *             (ab_dtype fp8 and N_out % 128 == 0: rows quantised per 128
 *             channels from the fp32 result, scales in c_scales
 *             f32 [N_out/128, M_rows]).
 *
 * Only rows below offsets[E] are computed: no tile is launched past the last
 * valid row.  Rows [offsets[E], M_rows) of C are written as exact zeros
 * (their fp8 scales as 1.0) -- never left uninitialised ([T45621] section 3
 * traces a NaN to sentinel outputs that a kernel left unwritten).
 * Accumulation is fp32; C is rounded once (RNE).  A must span under 4 GiB, and
 * so must one expert's B (MOE_ERR_INVALID_ARG otherwise).
 */
moe_status_t moe_grouped_gemm(const void* A, const float* a_scales, const void* B,
                              const float* b_scales, moe_dtype_t ab_dtype, const int32_t* offsets,
                              int32_t E, int64_t M_rows, int64_t N, int64_t K,
                              moe_epilogue_t epi, void* C, moe_dtype_t c_dtype, float* c_scales,
                              void* stream);

/*
 * moe_grouped_gemm_gather -- moe_grouped_gemm whose A rows are read through a
 * row map instead of from a permuted copy: the fusion of the scatter step into
 * the GEMM's operand load (the pipeline of [LF10481] section 1 without its
 * separate moe_scatter pass).
 *
 *   for p in [offsets[e], offsets[e+1]):
 *       acc[p, n] = sum_k A[gather_rows[p] / gather_div, k] * B[e, n, k]
 *
 *   A            [A_rows, K] of ab_dtype: token rows (x of the layer, or its
 *                per-token e4m3 codes from moe_quantize_rows).
 *   a_scales     f32 [K/128, A_rows] for fp8 (the scales of A's rows).
 *   gather_rows  device int32 [M_rows]: sorted_rows of moe_build_offsets.
 *   gather_div   k: a flat routed row r belongs to token r / k.
 *
 * Everything else (B, offsets, epi, C, rows past offsets[E] written as zeros,
 * errors) is as in moe_grouped_gemm; the results are bitwise identical to
 * moe_permute followed by moe_grouped_gemm on the same inputs.  A row index
 * outside [0, A_rows) (an inconsistent map) is clamped into it, so no read
 * leaves A.  A must span under 4 GiB, and so must one expert's B.
 */
moe_status_t moe_grouped_gemm_gather(const void* A, const float* a_scales, int64_t A_rows,
                                     const int32_t* gather_rows, int32_t gather_div, const void* B,
                                     const float* b_scales, moe_dtype_t ab_dtype,
                                     const int32_t* offsets, int32_t E, int64_t M_rows, int64_t N,
                                     int64_t K, moe_epilogue_t epi, void* C, moe_dtype_t c_dtype,
                                     float* c_scales, void* stream);

/*
 * moe_quantize_rows -- the per-token activation cast of [T45621] section 1
 * (fp8_act_quant / per_token_cast_to_fp8) on token rows, once per token: bf16
 * x [T, H] (H % 128 == 0) -> e4m3 codes xq [T, H] and scales xq_scales
 * f32 [H/128, T], per row and 128 channels as in moe_permute.  The fp8 layer
 * feeds it to moe_grouped_gemm_gather, so each token is quantised once rather
 * than once per routed copy.
 */
moe_status_t moe_quantize_rows(const void* x, int64_t T, int64_t H, void* xq, float* xq_scales,
                               void* stream);

/*
 * moe_grouped_gemm_tile_shape -- the tile moe_grouped_gemm (and _gather) uses
 * for an operand dtype, epilogue, output dtype and launch size (M_rows product
 * rows over E experts; launches with at most 8 rows per expert -- decode sizes --
 * take small tiles, except fp8 launches with e4m3 output):
 * *tile_m activation rows by *tile_n weight rows (SiLU*up tiles hold tile_n/2
 * gate and tile_n/2 up rows), *k_slice elements of K per step.  Lets a caller
 * predict the MFMA work from offsets: each expert segment of M_e rows is
 * covered by ceil(M_e / tile_m) tiles in M, each computing 16 * ceil(rows / 16)
 * rows.  Returns MOE_ERR_INVALID_ARG for bad enums, sizes or null outputs.
 */
moe_status_t moe_grouped_gemm_tile_shape(moe_dtype_t ab_dtype, moe_epilogue_t epi, moe_dtype_t c_dtype,
                                         int64_t M_rows, int32_t E, int32_t* tile_m, int32_t* tile_n,
                                         int32_t* k_slice);

/*
 * moe_unpermute_combine -- back to token order, scaled by the routing
 * weights (the gather step of [LF10481] section 1):
 *
 *   out[t] = sum over j = 0..k-1 (ascending) with row_pos[t*k+j] < offsets[E]
 *            of topk_weights[t*k+j] * y[row_pos[t*k+j]]
 *
 * accumulated in fp32 and rounded once to out_dtype.  Tokens with no valid
 * row get exact zeros.  Sentinel rows of y are never read.
 *
 *   y            [R, H] of y_dtype (MOE_F32 or MOE_BF16).
 *   out          [T, H] of out_dtype (MOE_F32 or MOE_BF16).
 */
moe_status_t moe_unpermute_combine(const void* y, moe_dtype_t y_dtype, const int32_t* row_pos,
                                   const float* topk_weights, const int32_t* offsets, int32_t E,
                                   int64_t T, int64_t H, int32_t k, void* out,
                                   moe_dtype_t out_dtype, void* stream);

/* Stages of moe_forward, in launch order. */
#define MOE_FORWARD_STAGES 6   /* route, offsets, activation staging, gate/up GEMM, down GEMM, combine */

/* Optional caller-owned storage for the routing intermediates of moe_forward.
 * Each non-NULL pointer is used instead of workspace storage, so the caller
 * can read the values after the stream completes.
 * stage_events, when non-NULL, points to MOE_FORWARD_STAGES + 1 hipEvent_t
 * handles created by the caller: event 0 is recorded on the stream before the
 * first stage and event i after stage i, so hipEventElapsedTime gives each
 * stage's device time. */
typedef struct {
  int32_t* topk_ids;      /* [T*k]  */
  float* topk_weights;    /* [T*k]  */
  int32_t* offsets;       /* [E+1]  */
  int32_t* sorted_rows;   /* [T*k]  */
  int32_t* row_pos;       /* [T*k]  */
  void** stage_events;    /* [MOE_FORWARD_STAGES + 1] hipEvent_t, or NULL */
} moe_aux_t;

/* Bytes of device workspace moe_forward needs (routing arrays, the fp8
 * layer's quantised token rows with their scales, by token and by routed row,
 * h, per-row expert outputs). */
size_t moe_forward_workspace(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                             moe_dtype_t w_dtype);

/*
 * moe_forward -- the whole layer on one stream: route, offsets, grouped GEMM
 * gate/up + SiLU*up reading token rows through the permutation
 * (moe_grouped_gemm_gather), grouped GEMM down, combine ([LF10481] section 1
 * pipeline with the scatter fused into the first GEMM's load; [T45621]
 * section 2 sentinel exclusion).  The activation-staging stage is empty for
 * f32 and bf16 layers and is moe_quantize_rows (once per token) for fp8.
 *
 *   x            [T, H]: MOE_F32 when w_dtype is MOE_F32, else MOE_BF16.
 *   router_logits f32 [T, E].
 *   w13, w2      packed weights of w_dtype (MOE_F32, MOE_BF16 or
 *                MOE_FP8_E4M3); w13_scales [E, 2I/128, H/128] and
 *                w2_scales [E, H/128, I/128] for fp8 (H, I % 128 == 0).
 *   num_valid_rows, renormalize: as for moe_route_topk.
 *   out          [T, H] of out_dtype (MOE_F32 for f32 weights, else MOE_BF16).
 *   aux          nullable; see moe_aux_t.
 *   workspace    >= moe_forward_workspace(...) bytes; no initialisation needed.
 *
 * Intermediates: f32 weights keep f32 throughout; bf16 weights round h and
 * the expert outputs to bf16; fp8 weights quantise the token rows and h per
 * row and 128 channels, and keep expert outputs in bf16.  Outputs are bitwise
 * those of the unfused sequence moe_permute -> moe_grouped_gemm -> ...
 */
moe_status_t moe_forward(const void* x, moe_dtype_t x_dtype, const float* router_logits,
                         const void* w13, const float* w13_scales, const void* w2,
                         const float* w2_scales, moe_dtype_t w_dtype, int64_t T, int64_t H,
                         int64_t I, int32_t E, int32_t k, int64_t num_valid_rows,
                         int32_t renormalize, void* out, moe_dtype_t out_dtype, moe_aux_t* aux,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace moe_backward needs (recomputed forward
 * intermediates, gradient intermediates, the expert-padded transposed
 * activations, and for w_dtype MOE_FP8_E4M3 the dequantised operands).  0 for
 * invalid arguments. */
size_t moe_backward_workspace(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k, moe_dtype_t w_dtype);

/*
 * moe_backward -- gradients of the layer computed by moe_forward, for the
 * routing that forward chose (held fixed).  The pages trace a training NaN to
 * sentinel outputs a kernel left uninitialised in the fp8 path's backward
 * ([T45621] section 3): here sentinel rows take no part and every gradient
 * element is written.  With p = row_pos[r] the permuted position of routed
 * slot r = t*k + j (valid iff p < offsets[E]) and e its expert:
 *
 *   dy_p   = w[r] * dout[t]                       (the weight is applied in the combine)
 *   dw[r]  = dout[t] . y_p,   y_p = W2[e] (silu(g) * u),   [g | u] = W13[e] x_t
 *   dh_p   = W2[e]^T dy_p,    dgu_p = [dh * u * silu'(g), dh * silu(g)]
 *   dx[t]  = sum over the token's valid slots (ascending j) of W13[e]^T dgu_p
 *   dW2[e] = sum over the expert's rows of dy_p h_p^T
 *   dW13[e] = sum over the expert's rows of dgu_p x_t^T
 *
 * dtype MOE_FP8_E4M3 (the fp8 layer of moe_forward: e4m3 weights with
 * [E, N/128, K/128] block scales, token rows and h quantised per row and 128
 * channels): the same chain rule on the values the forward used, straight
 * through its quantisers -- x_t is the token row quantised and dequantised,
 * W13 and W2 are the dequantised weights, and h_p in y_p and dW2 is the
 * quantised-dequantised h, while dh_p passes to h unchanged; dw13 and dw2 are
 * the gradients of the dequantised weight values.
 *
 * The forward's h and pre-activations [g | u] are recomputed here (its SiLU*up
 * grouped GEMM, pre-activations kept in f32); nothing of the forward's workspace
 * is needed.  y_p is not: dw[r] is evaluated as (W2[e]^T dout[t]) . h_p, the same
 * quantity, from the unweighted product W2[e]^T dout[t] that dh_p = w[r] times.
 *
 *   x, dout      bf16 [T, H]: the token rows given to moe_forward.
 *   w13, w2      [E, 2I, H] and [E, H, I] of dtype (MOE_BF16 or MOE_FP8_E4M3);
 *                w13_scales [E, 2I/128, H/128] and w2_scales [E, H/128, I/128]
 *                for fp8 (H, I % 128 == 0), else ignored.  H and I multiples of 8.
 *   topk_weights f32 [T, k], offsets [E+1], sorted_rows [T*k], row_pos [T*k]:
 *                the routing of the forward (moe_aux_t of moe_forward, or
 *                moe_route_topk + moe_build_offsets).
 *   dx [T, H], dw13 [E, 2I, H], dw2 [E, H, I] of grad_dtype (MOE_F32 or
 *                MOE_BF16): written in full (tokens with no valid slot and
 *                experts with no rows get exact zeros).
 *   dtopk_weights f32 [T, k]: dw; 0 for sentinel slots.  Nullable.
 *   workspace    >= moe_backward_workspace(T, H, I, E, k, dtype) bytes.
 * Accumulation is fp32.  MFMA operands are bf16: dout (the routing weight is
 * applied to the fp32 product), dy rounded once (for dW2), h, dgu and x (fp8:
 * the dequantised x, weights and h, each rounded once to bf16).
 */
moe_status_t moe_backward(const void* x, const void* w13, const float* w13_scales, const void* w2,
                          const float* w2_scales, moe_dtype_t dtype, int64_t T, int64_t H, int64_t I,
                          int32_t E, int32_t k, const float* topk_weights, const int32_t* offsets,
                          const int32_t* sorted_rows, const int32_t* row_pos, const void* dout,
                          void* dx, void* dw13, void* dw2, moe_dtype_t grad_dtype,
                          float* dtopk_weights, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Short name of a status code. */
const char* moe_status_string(moe_status_t status);

/* Thread-local message describing the last non-OK status returned on this
 * thread ("" if none). */
const char* moe_last_error(void);

/* MOE_ABI_VERSION of the loaded library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
