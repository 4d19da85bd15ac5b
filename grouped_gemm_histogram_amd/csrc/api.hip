// api.hip -- the extern "C" entry points declared in include/moe.h.
//
// Every entry point validates its arguments on the host before any launch,
// enqueues work on the caller's stream, never synchronises, allocates nothing
// and keeps no pointer.  Errors come back as moe_status_t plus a thread-local
// message; no C++ exception crosses the boundary.

#include <stdarg.h>
#include <stdio.h>

#include <algorithm>

#include "launch.h"
#include "moe.h"

namespace {

thread_local char g_err[512] = "";

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe_status_t ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

moe_status_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize(moe_dtype_t d) { return d == MOE_F32 ? 4 : (d == MOE_BF16 ? 2 : 1); }

bool valid_dtype(int d) { return d == MOE_F32 || d == MOE_BF16 || d == MOE_FP8_E4M3; }

constexpr long long kMaxRows = 0x7fffffffLL;
// fp8 layers of at least this many routed rows copy the token scales to the routed
// positions with a separate gather pass (see moe_forward)
constexpr long long kGatherScalesMinRows = 4096;

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

#define MOE_REQUIRE(cond, ...) \
  do {                         \
    if (!(cond)) return fail(MOE_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

moe_status_t check_experts(int32_t E, int32_t k) {
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  MOE_REQUIRE(k >= 1 && k <= MOE_MAX_TOPK && k <= E, "k=%d outside [1, min(E, %d)]", k, MOE_MAX_TOPK);
  return MOE_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct FwdLayout {
  size_t ids, w, offsets, sorted, rowpos, offws, xp, xps, xpsr, hf, h, hs, y, total;
};

FwdLayout fwd_layout(long long T, long long H, long long I, int E, int k, moe_dtype_t w_dtype) {
  const long long R = T * k;
  const bool fp8 = w_dtype == MOE_FP8_E4M3;
  const size_t e_act = w_dtype == MOE_F32 ? 4 : (fp8 ? 1 : 2);  // h
  const size_t e_y = w_dtype == MOE_F32 ? 4 : 2;
  FwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.ids = take(R * 4);
  L.w = take(R * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted = take(R * 4);
  L.rowpos = take(R * 4);
  L.offws = take(std::max(moe::build_offsets_workspace_bytes(R, E), moe::route_offsets_workspace_bytes(T, E)));
  L.xp = take(fp8 ? T * H : 0);                     // fp8: quantised token rows
  L.xps = take(fp8 ? T * (H / 128) * 4 : 0);
  L.xpsr = take(fp8 ? R * (H / 128) * 4 : 0);          // the same scales at the routed rows
  // fp8 at decode sizes: the gate/up GEMM's f32 h, quantised in a second pass
  L.hf = take(fp8 && moe::use_decode_tiles(R, E) ? R * I * 4 : 0);
  L.h = take(R * I * e_act);
  L.hs = take(fp8 ? R * (I / 128) * 4 : 0);
  L.y = take(R * H * e_y);
  L.total = off;
  return L;
}

// Shape rules of moe_forward that the per-argument checks do not cover: its GEMMs
// address operands with 32-bit byte offsets, so the gathered token rows, h, and one
// expert's W13 and W2 must each span under 4 GiB.  nullptr when the shape is accepted.
const char* forward_shape_error(long long T, long long H, long long I, int E, int k, moe_dtype_t w_dtype) {
  if (E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E) return "bad E or k";
  if (!valid_dtype(w_dtype)) return "bad w_dtype";
  if (T < 0 || H <= 0 || I <= 0 || H > kMaxRows || I > kMaxRows || T * k > kMaxRows) return "bad sizes";
  const bool fp8 = w_dtype == MOE_FP8_E4M3;
  if (fp8 && (H % 128 != 0 || I % 128 != 0)) return "fp8 layer needs H and I multiples of 128";
  if (!fp8 && ((H * esize(w_dtype)) % 16 != 0 || (I * esize(w_dtype)) % 16 != 0))
    return "H and I rows must be multiples of 16 bytes";
  const long long e_w = esize(w_dtype);
  const long long e_act = fp8 ? 1 : e_w;   // gathered token rows (fp8: their e4m3 codes) and h
  const long long R = T * k;
  if (T * H * e_act > (long long)UINT32_MAX) return "token rows must span under 4 GiB";
  if (R * I * e_act > (long long)UINT32_MAX) return "h (T*k rows of I) must span under 4 GiB";
  if (2 * I * H * e_w > (long long)UINT32_MAX || H * I * e_w > (long long)UINT32_MAX)
    return "one expert's W13 and W2 must each span under 4 GiB";
  return nullptr;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status_t moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                            int64_t num_valid_rows, int32_t renormalize, int32_t* topk_ids,
                            float* topk_weights, void* stream) {
  if (moe_status_t s = check_experts(E, k)) return s;
  MOE_REQUIRE(T >= 0 && T * k <= kMaxRows, "T=%lld out of range", (long long)T);
  if (T == 0) return ok();
  MOE_REQUIRE(logits && topk_ids && topk_weights, "null pointer argument");
  return launched(moe::launch_route_topk(logits, (int)T, E, k, num_valid_rows, renormalize ? 1 : 0,
                                         topk_ids, topk_weights, as_stream(stream)),
                  "route_topk");
}

size_t moe_build_offsets_workspace(int64_t R, int32_t E) {
  if (R < 0 || E < 1 || E > MOE_MAX_EXPERTS) return 0;
  return moe::build_offsets_workspace_bytes(R, E);
}

moe_status_t moe_build_offsets(const int32_t* topk_ids, int64_t R, int32_t E, int32_t* offsets,
                               int32_t* sorted_rows, int32_t* row_pos, void* workspace,
                               size_t workspace_bytes, void* stream) {
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  MOE_REQUIRE(R >= 0 && R <= kMaxRows, "R=%lld out of range", (long long)R);
  MOE_REQUIRE(offsets, "offsets is null");
  MOE_REQUIRE(R == 0 || (topk_ids && sorted_rows && row_pos), "null pointer argument");
  const size_t need = moe::build_offsets_workspace_bytes(R, E);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  return launched(moe::launch_build_offsets(topk_ids, (int)R, E, offsets, sorted_rows, row_pos,
                                            workspace, as_stream(stream)),
                  "build_offsets");
}

moe_status_t moe_build_offsets_noalloc(const int32_t* topk_ids, int64_t R, int32_t E, int32_t* offsets,
                                       int32_t* sorted_rows, int32_t* row_pos, void* stream) {
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  MOE_REQUIRE(R >= 0 && R <= kMaxRows, "R=%lld out of range", (long long)R);
  MOE_REQUIRE(offsets, "offsets is null");
  MOE_REQUIRE(R == 0 || (topk_ids && sorted_rows && row_pos), "null pointer argument");
  const size_t need = moe::build_offsets_workspace_bytes(R, E);
  const size_t cap = moe::build_offsets_noalloc_capacity();
  if (need > cap)
    return fail(MOE_ERR_WORKSPACE, "R=%lld, E=%d needs %zu bytes of scratch; the static scratch holds %zu",
                (long long)R, E, need, cap);
  void* scratch = nullptr;
  if (hipError_t e = moe::build_offsets_noalloc_scratch(&scratch))
    return fail(MOE_ERR_LAUNCH, "static scratch address: %s", hipGetErrorString(e));
  return launched(moe::launch_build_offsets(topk_ids, (int)R, E, offsets, sorted_rows, row_pos, scratch,
                                            as_stream(stream)),
                  "build_offsets_noalloc");
}

moe_status_t moe_permute(const void* x, moe_dtype_t x_dtype, int64_t T, int64_t H, int32_t k,
                         const int32_t* sorted_rows, const int32_t* offsets, int32_t E, int64_t R,
                         void* x_perm, moe_dtype_t perm_dtype, float* x_perm_scales,
                         void* stream) {
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  MOE_REQUIRE(k >= 1 && k <= MOE_MAX_TOPK, "k=%d outside [1, %d]", k, MOE_MAX_TOPK);
  MOE_REQUIRE(T >= 0 && R >= 0 && R <= kMaxRows && H > 0 && H <= kMaxRows, "bad sizes");
  MOE_REQUIRE(x_dtype == MOE_F32 || x_dtype == MOE_BF16, "x_dtype must be MOE_F32 or MOE_BF16");
  if (R == 0) return ok();
  MOE_REQUIRE(x && sorted_rows && offsets && x_perm, "null pointer argument");
  MOE_REQUIRE(aligned16(x) && aligned16(x_perm), "x and x_perm must be 16-byte aligned");
  MOE_REQUIRE((H * esize(x_dtype)) % 16 == 0, "rows of x must be a multiple of 16 bytes");
  if (perm_dtype == x_dtype)
    return launched(moe::launch_permute_copy(x, (int)T, (int)(H * esize(x_dtype)), k, sorted_rows, offsets,
                                             E, (int)R, x_perm, as_stream(stream)),
                    "permute");
  if (perm_dtype == MOE_FP8_E4M3 && x_dtype == MOE_BF16) {
    MOE_REQUIRE(H % 128 == 0, "fp8 permute needs H %% 128 == 0");
    MOE_REQUIRE(x_perm_scales, "x_perm_scales is null");
    return launched(moe::launch_permute_quant(x, (int)T, (int)H, k, sorted_rows, offsets, E, (int)R, x_perm,
                                              x_perm_scales, as_stream(stream)),
                    "permute_quant");
  }
  return fail(MOE_ERR_UNSUPPORTED, "permute from dtype %d to dtype %d", (int)x_dtype, (int)perm_dtype);
}

}  // extern "C"

namespace {

// The grouped GEMM with A read directly (a_rows null) or gathered through a_rows.
// a_scales_by_row (fp8 with a row map): a_scales is [K/128, M_rows], indexed by product row.
moe_status_t grouped_gemm_impl(const void* A, const float* a_scales, long long A_rows,
                               const int32_t* a_rows, int32_t a_div, const void* B,
                               const float* b_scales, moe_dtype_t ab_dtype, const int32_t* offsets,
                               int32_t E, int64_t M_rows, int64_t N, int64_t K, moe_epilogue_t epi,
                               void* C, moe_dtype_t c_dtype, float* c_scales, void* stream,
                               bool a_scales_by_row = false, long long tile_rows = 0) {
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  MOE_REQUIRE(valid_dtype(ab_dtype) && valid_dtype(c_dtype), "bad dtype");
  MOE_REQUIRE(epi == MOE_EPI_NONE || epi == MOE_EPI_SILU_MUL, "bad epilogue");
  MOE_REQUIRE(M_rows >= 0 && M_rows <= kMaxRows && N > 0 && N <= kMaxRows && K > 0 &&
                  K * esize(ab_dtype) <= kMaxRows,
              "bad sizes");
  const bool silu = epi == MOE_EPI_SILU_MUL;
  MOE_REQUIRE(!silu || N % 2 == 0, "SiLU*up needs an even N");
  const long long N_out = silu ? N / 2 : N;
  MOE_REQUIRE((K * esize(ab_dtype)) % 16 == 0, "rows of A and B must be a multiple of 16 bytes");
  MOE_REQUIRE((N_out * esize(c_dtype)) % 16 == 0, "rows of C must be a multiple of 16 bytes");
  if (ab_dtype == MOE_FP8_E4M3) {
    MOE_REQUIRE(K % 128 == 0 && N % 128 == 0, "fp8 GEMM needs N and K multiples of 128");
    MOE_REQUIRE(a_scales && b_scales, "fp8 GEMM needs a_scales and b_scales");
    MOE_REQUIRE(!silu || N_out % 128 == 0, "fp8 SiLU*up needs N/2 %% 128 == 0");
  }
  if (c_dtype == MOE_FP8_E4M3) {
    if (!(ab_dtype == MOE_FP8_E4M3 && silu))
      return fail(MOE_ERR_UNSUPPORTED, "fp8 output is supported for fp8 operands with SiLU*up");
    MOE_REQUIRE(N_out % 128 == 0 && c_scales, "fp8 output needs N_out %% 128 == 0 and c_scales");
  }
  if (a_rows) {
    MOE_REQUIRE(a_div >= 1 && a_div <= MOE_MAX_TOPK, "gather_div=%d outside [1, %d]", a_div, MOE_MAX_TOPK);
    MOE_REQUIRE(A_rows >= 0 && A_rows <= kMaxRows, "bad A_rows");
    MOE_REQUIRE(A_rows * (K * esize(ab_dtype)) <= (long long)UINT32_MAX,
                "gathered A must span under 4 GiB");
  } else {
    MOE_REQUIRE(M_rows * (K * esize(ab_dtype)) <= (long long)UINT32_MAX, "A must span under 4 GiB");
  }
  MOE_REQUIRE(N * (K * esize(ab_dtype)) <= (long long)UINT32_MAX, "one expert's B must span under 4 GiB");
  if (M_rows == 0) return ok();
  MOE_REQUIRE(A && B && offsets && C, "null pointer argument");
  MOE_REQUIRE(aligned16(A) && aligned16(B) && aligned16(C), "A, B and C must be 16-byte aligned");
  if (a_rows && A_rows == 0)
    return fail(MOE_ERR_INVALID_ARG, "gathered A has no rows but the product has %lld", (long long)M_rows);
  moe::GemmLaunch p{};
  p.a_rows = a_rows;
  p.a_div = a_div;
  p.a_total = A_rows;
  p.a_scales_by_row = a_scales_by_row;
  p.A = A;
  p.a_scales = a_scales;
  p.B = B;
  p.b_scales = b_scales;
  p.ab_dtype = ab_dtype;
  p.offsets = offsets;
  p.E = E;
  p.M_rows = M_rows;
  p.N = N;
  p.K = K;
  p.silu = silu;
  p.C = C;
  p.c_dtype = c_dtype;
  p.c_scales = c_scales;
  p.tile_rows = tile_rows;
  return launched(moe::launch_grouped_gemm(p, as_stream(stream)), "grouped_gemm");
}

}  // namespace

extern "C" {

moe_status_t moe_grouped_gemm(const void* A, const float* a_scales, const void* B,
                              const float* b_scales, moe_dtype_t ab_dtype, const int32_t* offsets,
                              int32_t E, int64_t M_rows, int64_t N, int64_t K, moe_epilogue_t epi,
                              void* C, moe_dtype_t c_dtype, float* c_scales, void* stream) {
  return grouped_gemm_impl(A, a_scales, M_rows, nullptr, 1, B, b_scales, ab_dtype, offsets, E, M_rows,
                           N, K, epi, C, c_dtype, c_scales, stream);
}

moe_status_t moe_grouped_gemm_gather(const void* A, const float* a_scales, int64_t A_rows,
                                     const int32_t* gather_rows, int32_t gather_div, const void* B,
                                     const float* b_scales, moe_dtype_t ab_dtype,
                                     const int32_t* offsets, int32_t E, int64_t M_rows, int64_t N,
                                     int64_t K, moe_epilogue_t epi, void* C, moe_dtype_t c_dtype,
                                     float* c_scales, void* stream) {
  MOE_REQUIRE(gather_rows || M_rows == 0, "gather_rows is null");
  return grouped_gemm_impl(A, a_scales, A_rows, gather_rows, gather_div, B, b_scales, ab_dtype, offsets, E,
                           M_rows, N, K, epi, C, c_dtype, c_scales, stream);
}

moe_status_t moe_quantize_rows(const void* x, int64_t T, int64_t H, void* xq, float* xq_scales,
                               void* stream) {
  MOE_REQUIRE(T >= 0 && T <= kMaxRows && H > 0 && H <= kMaxRows, "bad sizes");
  MOE_REQUIRE(H % 128 == 0, "fp8 quantisation needs H %% 128 == 0");
  if (T == 0) return ok();
  MOE_REQUIRE(x && xq && xq_scales, "null pointer argument");
  MOE_REQUIRE(aligned16(x) && aligned16(xq), "x and xq must be 16-byte aligned");
  return launched(moe::launch_permute_quant(x, (int)T, (int)H, 1, nullptr, nullptr, 0, (int)T, xq, xq_scales,
                                            as_stream(stream)),
                  "quantize_rows");
}

moe_status_t moe_grouped_gemm_tile_shape(moe_dtype_t ab_dtype, moe_epilogue_t epi, moe_dtype_t c_dtype,
                                         int64_t M_rows, int32_t E, int32_t* tile_m, int32_t* tile_n,
                                         int32_t* k_slice) {
  MOE_REQUIRE(tile_m && tile_n && k_slice, "null output pointer");
  MOE_REQUIRE(epi == MOE_EPI_NONE || epi == MOE_EPI_SILU_MUL, "bad epilogue");
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS && M_rows >= 0, "bad M_rows or E");
  int m = 0, n = 0, ks = 0;
  MOE_REQUIRE(valid_dtype(c_dtype), "bad c_dtype");
  if (!moe::grouped_gemm_tile_shape(ab_dtype, epi == MOE_EPI_SILU_MUL, c_dtype, M_rows, E, &m, &n, &ks))
    return fail(MOE_ERR_INVALID_ARG, "bad dtype %d", (int)ab_dtype);
  *tile_m = m;
  *tile_n = n;
  *k_slice = ks;
  return ok();
}

moe_status_t moe_unpermute_combine(const void* y, moe_dtype_t y_dtype, const int32_t* row_pos,
                                   const float* topk_weights, const int32_t* offsets, int32_t E,
                                   int64_t T, int64_t H, int32_t k, void* out,
                                   moe_dtype_t out_dtype, void* stream) {
  if (moe_status_t s = check_experts(E, k)) return s;
  MOE_REQUIRE(T >= 0 && T * k <= kMaxRows && H > 0 && H <= kMaxRows, "bad sizes");
  MOE_REQUIRE(y_dtype == MOE_F32 || y_dtype == MOE_BF16, "y_dtype must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(out_dtype == MOE_F32 || out_dtype == MOE_BF16, "out_dtype must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE((H * esize(y_dtype)) % 16 == 0 && H % 4 == 0, "rows of y must be a multiple of 16 bytes");
  if (T == 0) return ok();
  MOE_REQUIRE(y && row_pos && topk_weights && offsets && out, "null pointer argument");
  MOE_REQUIRE(aligned16(y) && aligned16(out), "y and out must be 16-byte aligned");
  return launched(moe::launch_combine(y, y_dtype == MOE_BF16, row_pos, topk_weights, offsets, E, (int)T,
                                      (int)H, k, out, out_dtype == MOE_BF16, as_stream(stream)),
                  "unpermute_combine");
}

size_t moe_forward_workspace(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                             moe_dtype_t w_dtype) {
  if (forward_shape_error(T, H, I, E, k, w_dtype) != nullptr) return 0;   // moe_forward rejects it
  return fwd_layout(T, H, I, E, k, w_dtype).total;
}

moe_status_t moe_forward(const void* x, moe_dtype_t x_dtype, const float* router_logits,
                         const void* w13, const float* w13_scales, const void* w2,
                         const float* w2_scales, moe_dtype_t w_dtype, int64_t T, int64_t H,
                         int64_t I, int32_t E, int32_t k, int64_t num_valid_rows,
                         int32_t renormalize, void* out, moe_dtype_t out_dtype, moe_aux_t* aux,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (moe_status_t s = check_experts(E, k)) return s;
  MOE_REQUIRE(valid_dtype(w_dtype), "bad w_dtype");
  MOE_REQUIRE(T >= 0 && T * k <= kMaxRows && H > 0 && I > 0 && H <= kMaxRows && I <= kMaxRows,
              "bad sizes");
  const bool fp8 = w_dtype == MOE_FP8_E4M3;
  MOE_REQUIRE(x_dtype == (w_dtype == MOE_F32 ? MOE_F32 : MOE_BF16),
              "x_dtype must be MOE_F32 for f32 weights and MOE_BF16 otherwise");
  MOE_REQUIRE(out_dtype == MOE_F32 || out_dtype == MOE_BF16, "out_dtype must be MOE_F32 or MOE_BF16");
  if (const char* why = forward_shape_error(T, H, I, E, k, w_dtype)) return fail(MOE_ERR_INVALID_ARG, "%s", why);
  if (fp8) MOE_REQUIRE(w13_scales && w2_scales, "fp8 layer needs weight scales");
  const FwdLayout L = fwd_layout(T, H, I, E, k, w_dtype);
  if (T > 0) {
    MOE_REQUIRE(x && router_logits && w13 && w2 && out, "null pointer argument");
    MOE_REQUIRE(aligned16(x) && aligned16(w13) && aligned16(w2) && aligned16(out),
                "x, weights and out must be 16-byte aligned");
  }
  if (!workspace || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, L.total);
  MOE_REQUIRE(aligned16(workspace), "workspace must be 16-byte aligned");

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* ids = (aux && aux->topk_ids) ? aux->topk_ids : reinterpret_cast<int32_t*>(ws + L.ids);
  float* wts = (aux && aux->topk_weights) ? aux->topk_weights : reinterpret_cast<float*>(ws + L.w);
  int32_t* offs = (aux && aux->offsets) ? aux->offsets : reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted = (aux && aux->sorted_rows) ? aux->sorted_rows : reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* rowpos = (aux && aux->row_pos) ? aux->row_pos : reinterpret_cast<int32_t*>(ws + L.rowpos);
  const long long R = T * k;
  void** ev = aux ? aux->stage_events : nullptr;
  auto mark = [&](int i) -> moe_status_t {
    if (ev && ev[i] && hipEventRecord(static_cast<hipEvent_t>(ev[i]), as_stream(stream)) != hipSuccess)
      return fail(MOE_ERR_LAUNCH, "hipEventRecord of stage event %d failed", i);
    return MOE_OK;
  };

  moe_status_t s;
  if ((s = mark(0))) return s;
  if (R > 0 && R <= 1024 && T <= 16) {
    // decode sizes: routing and offsets in one launch, a wave per token (the offsets
    // stage's events then enclose no work).  With more tokens than the workgroup's 16
    // waves the waves route several tokens one after another, which measured slower
    // than the separate routing launch (T = 64: +9 us; T = 1 and 8: -1 and -3 us).
    if ((s = launched(moe::launch_route_offsets_single(router_logits, (int)T, E, k, num_valid_rows,
                                                       renormalize ? 1 : 0, ids, wts, offs, sorted, rowpos,
                                                       as_stream(stream)),
                      "route_offsets_single")))
      return s;
    if ((s = mark(1))) return s;
  } else if (T > 0) {
    // routing with the per-chunk histograms (the routing stage), then the per-bin scan
    // over chunks and the scatter (the offsets stage)
    if ((s = launched(moe::launch_route_hist(router_logits, (int)T, E, k, num_valid_rows, renormalize ? 1 : 0,
                                             ids, wts, ws + L.offws, as_stream(stream)),
                      "route_hist")))
      return s;
    if ((s = mark(1))) return s;
    if ((s = launched(moe::launch_offsets_from_hist(ids, (int)T, E, k, offs, sorted, rowpos, ws + L.offws,
                                                    as_stream(stream)),
                      "offsets_from_hist")))
      return s;
  } else {
    if ((s = moe_route_topk(router_logits, T, E, k, num_valid_rows, renormalize, ids, wts, stream)))
      return s;
    if ((s = mark(1))) return s;
    if ((s = moe_build_offsets(ids, R, E, offs, sorted, rowpos, ws + L.offws,
                               moe::build_offsets_workspace_bytes(R, E), stream)))
      return s;
  }
  if ((s = mark(2))) return s;
  if (T == 0) {
    for (int i = 3; i <= MOE_FORWARD_STAGES; ++i)
      if ((s = mark(i))) return s;
    return ok();
  }
  const moe_dtype_t act = fp8 ? MOE_FP8_E4M3 : w_dtype;
  // bf16 GEMM tiles are chosen for the rows that can be valid (flat rows past
  // num_valid_rows are sentinel), known here without reading the offsets; the f32 and fp8
  // layers keep the choice by routed rows (the fp8 workspace depends on it)
  const long long V_host = (num_valid_rows >= 0 && num_valid_rows < R) ? num_valid_rows : R;
  const long long tile_rows = (w_dtype == MOE_BF16) ? (V_host > 0 ? V_host : 1) : R;
  const moe_dtype_t ydt = w_dtype == MOE_F32 ? MOE_F32 : MOE_BF16;
  float* xps = fp8 ? reinterpret_cast<float*>(ws + L.xps) : nullptr;
  float* xpsr = fp8 ? reinterpret_cast<float*>(ws + L.xpsr) : nullptr;
  float* hs = fp8 ? reinterpret_cast<float*>(ws + L.hs) : nullptr;
  // The gate/up GEMM reads token rows through the permutation.  The fp8 layer quantises
  // each token once first and also stores each scale at the token's routed rows
  // (xpsr [H/128, R]), so that a tile of routed rows finds its scales in consecutive
  // words instead of one cache line per row.  With many rows a second pass gathers them
  // along the routed positions (the quantising kernel's per-slot stores would touch one
  // cache line per scale); with few, the quantising kernel stores them through row_pos
  // and saves a launch.
  const bool gather_sc = fp8 && R >= kGatherScalesMinRows;
  if (fp8 && (s = launched(moe::launch_permute_quant(x, (int)T, (int)H, 1, nullptr, nullptr, 0, (int)T, ws + L.xp,
                                                     xps, as_stream(stream), false, gather_sc ? nullptr : rowpos,
                                                     gather_sc ? 0 : k, gather_sc ? nullptr : xpsr, (int)R),
                           "quantize_rows")))
    return s;
  if (gather_sc && (s = launched(moe::launch_gather_scales(xps, (int)T, (int)(H / 128), sorted, k, offs, E, (int)R,
                                                           xpsr, as_stream(stream)),
                                 "gather scales")))
    return s;
  if ((s = mark(3))) return s;
  if (fp8 && moe::use_decode_tiles(R, E)) {
    // decode sizes: the small tiles write f32 h (an e4m3 group spans several of them),
    // quantised per row and 128 channels after, with the fused epilogue's arithmetic
    float* hf = reinterpret_cast<float*>(ws + L.hf);
    if ((s = grouped_gemm_impl(ws + L.xp, xpsr, T, sorted, k, w13, w13_scales, w_dtype, offs, E, R, 2 * I, H,
                               MOE_EPI_SILU_MUL, hf, MOE_F32, nullptr, stream, true)))
      return s;
    if ((s = launched(moe::launch_permute_quant(hf, (int)R, (int)I, 1, nullptr, nullptr, 0, (int)R, ws + L.h, hs,
                                                as_stream(stream), true),
                      "quantize h")))
      return s;
  } else if ((s = grouped_gemm_impl(fp8 ? ws + L.xp : x, xpsr, T, sorted, k, w13, w13_scales, w_dtype, offs, E, R,
                                    2 * I, H, MOE_EPI_SILU_MUL, ws + L.h, act, hs, stream, fp8, tile_rows))) {
    return s;
  }
  if ((s = mark(4))) return s;
  if ((s = grouped_gemm_impl(ws + L.h, hs, R, nullptr, 1, w2, w2_scales, w_dtype, offs, E, R, H, I, MOE_EPI_NONE,
                             ws + L.y, ydt, nullptr, stream, false, tile_rows)))
    return s;
  if ((s = mark(5))) return s;
  if ((s = moe_unpermute_combine(ws + L.y, ydt, rowpos, wts, offs, E, T, H, k, out, out_dtype,
                                 stream)))
    return s;
  if ((s = mark(6))) return s;
  return ok();
}

// ---------------------------------------------------------------------------------- backward

}  // extern "C"

namespace {

struct BwdLayout {
  size_t koff, gu, h, dh, dgu, dxp, ones, ta, tb, xhat, xq, xs, w13hat, w2hat, total;
  long long ldd;   // row stride of the expert-padded transposes (elements)
};

BwdLayout bwd_layout(long long T, long long H, long long I, int E, int k, bool fp8) {
  BwdLayout L{};
  const long long R = T * k;
  L.ldd = ((R + 64LL * E) + 63) / 64 * 64;   // >= sum over experts of round_up(M_e, 64)
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.koff = take((size_t)(E + 1) * 4);
  L.gu = take((size_t)R * 2 * I * 4);
  L.h = take((size_t)R * I * 2);
  L.dh = take((size_t)R * I * 4);
  L.dgu = take((size_t)R * 2 * I * 2);
  L.dxp = take((size_t)R * H * 4);
  L.ones = take((size_t)R * 4);
  L.ta = take((size_t)(H > 2 * I ? H : 2 * I) * L.ldd * 2);
  L.tb = take((size_t)(H > I ? H : I) * L.ldd * 2);
  // fp8 layer: the dequantised operands (bf16) the backward runs on
  L.xhat = take(fp8 ? (size_t)T * H * 2 : 0);
  L.xq = take(fp8 ? (size_t)T * H : 0);
  L.xs = take(fp8 ? (size_t)T * (H / 128) * 4 : 0);
  L.w13hat = take(fp8 ? (size_t)E * 2 * I * H * 2 : 0);
  L.w2hat = take(fp8 ? (size_t)E * H * I * 2 : 0);
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

size_t moe_backward_workspace(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k, moe_dtype_t w_dtype) {
  if (T < 0 || H <= 0 || I <= 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK ||
      (w_dtype != MOE_BF16 && w_dtype != MOE_FP8_E4M3))
    return 0;
  return bwd_layout(T, H, I, E, k, w_dtype == MOE_FP8_E4M3).total;
}

moe_status_t moe_backward(const void* x, const void* w13, const float* w13_scales, const void* w2,
                          const float* w2_scales, moe_dtype_t dtype, int64_t T, int64_t H, int64_t I,
                          int32_t E, int32_t k, const float* topk_weights, const int32_t* offsets,
                          const int32_t* sorted_rows, const int32_t* row_pos, const void* dout,
                          void* dx, void* dw13, void* dw2, moe_dtype_t grad_dtype,
                          float* dtopk_weights, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (moe_status_t s = check_experts(E, k)) return s;
  MOE_REQUIRE(dtype == MOE_BF16 || dtype == MOE_FP8_E4M3, "dtype must be MOE_BF16 or MOE_FP8_E4M3");
  const bool fp8 = dtype == MOE_FP8_E4M3;
  MOE_REQUIRE(grad_dtype == MOE_F32 || grad_dtype == MOE_BF16, "grad_dtype must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(T >= 0 && H > 0 && I > 0 && H % 8 == 0 && I % 8 == 0, "bad sizes (H, I multiples of 8)");
  if (fp8) {
    MOE_REQUIRE(H % 128 == 0 && I % 128 == 0, "fp8 layer needs H and I multiples of 128");
    MOE_REQUIRE(w13_scales && w2_scales, "fp8 layer needs weight scales");
  }
  const BwdLayout L = bwd_layout(T, H, I, E, k, fp8);
  const long long R = T * k;
  // the segment transposes and the K-grouped GEMM address rows of ldd elements with 32-bit
  // offsets; the other GEMMs address one expert's weights and their A operands (x, dout, dgu)
  // with 32-bit byte offsets
  MOE_REQUIRE(R <= kMaxRows / 2 && (2 * I > H ? 2 * I : H) * L.ldd * 2 < 0xffffffffLL &&
                  2 * I * H * 2 <= 0xffffffffLL && T * H * 2 <= 0xffffffffLL && R * 2 * I * 2 <= 0xffffffffLL,
              "sizes exceed the backward's 32-bit addressing");
  MOE_REQUIRE(dx && dw13 && dw2 && w13 && w2, "null pointer argument");
  if (T > 0)
    MOE_REQUIRE(x && dout && topk_weights && offsets && sorted_rows && row_pos, "null pointer argument");
  MOE_REQUIRE(aligned16(dx) && aligned16(dw13) && aligned16(dw2) && aligned16(w13) && aligned16(w2) &&
                  (T == 0 || (aligned16(x) && aligned16(dout))),
              "tensors must be 16-byte aligned");
  if (!workspace || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, L.total);
  MOE_REQUIRE(aligned16(workspace), "workspace must be 16-byte aligned");

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t st = as_stream(stream);
  int* koff = reinterpret_cast<int*>(ws + L.koff);
  float* gu = reinterpret_cast<float*>(ws + L.gu);
  float* dh = reinterpret_cast<float*>(ws + L.dh);
  float* dxp = reinterpret_cast<float*>(ws + L.dxp);
  float* ones = reinterpret_cast<float*>(ws + L.ones);
  const int gdt = grad_dtype;
  auto gemm = [&](const void* A, const void* B, long long M, long long N, long long K, void* C, int cdt,
                  const int* kof, long long lda, long long ldb, int nE, const int* offs,
                  const int* a_rows = nullptr, bool silu = false, float* pre_out = nullptr, bool b_kn = false) {
    moe::GemmLaunch p{};
    p.b_kn = b_kn;
    p.a_rows = a_rows;
    p.a_div = k;
    p.a_total = T;
    p.pre_out = pre_out;
    p.A = A;
    p.B = B;
    p.ab_dtype = MOE_BF16;
    p.offsets = offs;
    p.E = nE;
    p.M_rows = M;
    p.N = N;
    p.K = K;
    p.silu = silu;
    p.C = C;
    p.c_dtype = cdt;
    p.koff = kof;
    p.lda = lda;
    p.ldb = ldb;
    return moe::launch_grouped_gemm(p, st);
  };
  hipError_t e = hipSuccess;
  auto step = [&](hipError_t r) {
    if (e == hipSuccess) e = r;
  };
  if (T == 0) {
    // no rows: every weight gradient is zero (a fill kernel, not a memset node)
    step(moe::launch_fill_f32(static_cast<float*>(dw13), (long long)E * 2 * I * H * esize(grad_dtype) / 4, 0.0f, st));
    step(moe::launch_fill_f32(static_cast<float*>(dw2), (long long)E * H * I * esize(grad_dtype) / 4, 0.0f, st));
    return launched(e, "backward");
  }
  step(moe::launch_pad_offsets(offsets, E, (int)R, koff, st));
  if (fp8) {
    // fp8 layer: the forward's pre-activations gu, recomputed as the forward computed them
    // (the fp8 grouped GEMM on the token codes and weight codes with fp32 block scaling:
    // per element the forward's own accumulation), then h-hat = dq(q(silu(g) * u)) with the
    // forward's arithmetic, so h-hat's codes are the forward's.  The remaining steps run on
    // the dequantised operands, straight through the quantisers: x-hat, the weights'
    // block values, and h-hat in place of h.
    step(moe::launch_permute_quant(x, (int)T, (int)H, 1, nullptr, nullptr, 0, (int)T, ws + L.xq,
                                   reinterpret_cast<float*>(ws + L.xs), st));
    moe::GemmLaunch p{};
    p.A = ws + L.xq;
    p.a_scales = reinterpret_cast<const float*>(ws + L.xs);
    p.a_rows = sorted_rows;
    p.a_div = k;
    p.a_total = T;
    p.B = w13;
    p.b_scales = w13_scales;
    p.ab_dtype = MOE_FP8_E4M3;
    p.offsets = offsets;
    p.E = E;
    p.M_rows = R;
    p.N = 2 * I;
    p.K = H;
    p.silu = false;
    p.C = gu;
    p.c_dtype = MOE_F32;
    step(moe::launch_grouped_gemm(p, st));
    step(moe::launch_h_fake_quant(gu, offsets, E, (int)R, (int)I, ws + L.h, st));
    step(moe::launch_fake_quant_rows(x, T, (int)H, ws + L.xhat, st));
    step(moe::launch_dequant_blocks(w13, w13_scales, E, (int)(2 * I), (int)H, ws + L.w13hat, st));
    step(moe::launch_dequant_blocks(w2, w2_scales, E, (int)H, (int)I, ws + L.w2hat, st));
    x = ws + L.xhat;
    w13 = ws + L.w13hat;
    w2 = ws + L.w2hat;
  } else {
    // forward intermediates, recomputed: h (bf16) and its pre-activations gu = [g | u]
    // (f32) from one SiLU*up GEMM reading token rows through the permutation
    step(gemm(x, w13, R, 2 * I, H, ws + L.h, MOE_BF16, nullptr, 0, 0, E, offsets, sorted_rows, true, gu));
  }
  // data gradients: dh1 = dout W2 per routed row (W2 [E, H, I] read as [K, N] rows, dout
  // rows read through the permutation, routing weight not yet applied); then per slot the
  // routing-weight gradient dw = dh1 . h (= dout . y, so y is never recomputed) and the
  // SiLU*up backward of dh = w dh1; dx_perm = dgu W13 (W13 [E, 2I, H] read as [K, N]
  // rows).  (The SiLU*up backward stays a kernel of its own: in the GEMM's epilogue its
  // gu loads stalled every tile.)
  step(gemm(dout, w2, R, I, H, dh, MOE_F32, nullptr, 0, 0, E, offsets, sorted_rows, false, nullptr, true));
  step(moe::launch_silu_bwd_route(dh, gu, ws + L.h, topk_weights, row_pos, offsets, E, (int)R, (int)I, ws + L.dgu,
                                  dtopk_weights, st));
  step(gemm(ws + L.dgu, w13, R, H, 2 * I, dxp, MOE_F32, nullptr, 0, 0, E, offsets, nullptr, false, nullptr, true));
  step(moe::launch_fill_f32(ones, R, 1.0f, st));
  step(moe::launch_combine(dxp, false, row_pos, ones, offsets, E, (int)T, (int)H, k, dx,
                           grad_dtype == MOE_BF16, st));
  // weight gradients: K-grouped GEMMs over each expert's rows, on expert-padded transposes
  const int ldd = (int)L.ldd;
  // dy = w dout per routed row, formed while transposing (dout rows through the permutation)
  step(moe::launch_transpose_segments_bf16(dout, (int)R, (int)H, offsets, koff, E, sorted_rows, k, (int)T,
                                           topk_weights, ws + L.ta, ldd, st));
  step(moe::launch_transpose_segments_bf16(ws + L.h, (int)R, (int)I, offsets, koff, E, nullptr, 1, (int)R, nullptr,
                                           ws + L.tb, ldd, st));
  step(gemm(ws + L.ta, ws + L.tb, H, I, ldd, dw2, gdt, koff, ldd, ldd, E, nullptr));
  step(moe::launch_transpose_segments_bf16(ws + L.dgu, (int)R, (int)(2 * I), offsets, koff, E, nullptr, 1, (int)R,
                                           nullptr, ws + L.ta, ldd, st));
  // x's rows of each expert, read through the permutation
  step(moe::launch_transpose_segments_bf16(x, (int)R, (int)H, offsets, koff, E, sorted_rows, k, (int)T, nullptr,
                                           ws + L.tb, ldd, st));
  step(gemm(ws + L.ta, ws + L.tb, 2 * I, H, ldd, dw13, gdt, koff, ldd, ldd, E, nullptr));
  return launched(e, "backward");
}

}  // extern "C\"
