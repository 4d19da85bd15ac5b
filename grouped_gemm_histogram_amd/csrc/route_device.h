// route_device.h -- top-k routing of one token by one wave64, shared by the routing
// kernel and the one-workgroup routing + offsets kernel of decode sizes.
//
// The router picks a small subset of experts for each token ("트랜스포머에서
// 전문가 혼합 (MoEs)", MoE basics).  Selection is k rounds of a wave-wide
// arg-max over the token's logits (each lane holds E/64 of them in registers),
// ordering pairs by (logit descending, expert id ascending); -0.0 and +0.0
// compare equal.  Weights are a softmax over the k selected logits (or over
// all E when not renormalising), in fp32.
#pragma once

#include "device_common.h"

namespace moe {

// (value, id) pairs ordered by value descending, then id ascending; -0.0 and +0.0 are
// equal values.  This is a total order, so any reduction tree picks the same pair.
__device__ __forceinline__ void keep_better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

// One step of the arg-max within each 16-lane row: the pair held by the lane that the
// DPP pattern names (lane ^ 1, lane ^ 2, the mirrored lane within 8, within 16).
template <int kDppCtrl>
__device__ __forceinline__ void argmax_dpp_step(float& bv, int& bi) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), kDppCtrl, 0xf, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(0, bi, kDppCtrl, 0xf, 0xf, false);
  keep_better(bv, bi, ov, oi);
}

// Wave-wide arg-max; every lane gets the best pair.  Within each row of 16 lanes by DPP
// moves (no LDS traffic), then across the four rows from their first lanes.
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  argmax_dpp_step<0xb1>(bv, bi);    // quad_perm [1, 0, 3, 2]: lane ^ 1
  argmax_dpp_step<0x4e>(bv, bi);    // quad_perm [2, 3, 0, 1]: lane ^ 2
  argmax_dpp_step<0x141>(bv, bi);   // row_half_mirror: the other quad of the 8
  argmax_dpp_step<0x140>(bv, bi);   // row_mirror: the other 8 of the row
  float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 16; r < kWave; r += 16)
    keep_better(v, i, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), r)),
                __builtin_amdgcn_readlane(bi, r));
  bv = v;
  bi = i;
}

// Token t's k ids and weights (flat rows t*k .. t*k+k-1; rows at or past valid_rows,
// when valid_rows >= 0, become sentinel id E with weight 0).  Called by a whole wave.
// Returns, on lane j < k, the id stored for slot j (E for a sentinel row); -1 on the
// other lanes.
template <int EPL>
__device__ __forceinline__ int route_token(const float* __restrict__ logits, int t, int E, int k,
                                            long long valid_rows, int renorm, int* __restrict__ ids,
                                            float* __restrict__ weights) {
  const int lane = lane_id();
  const float* row = logits + (size_t)t * E;

  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    v[i] = (e < E) ? row[e] : 0.0f;
  }

  uint32_t taken = 0;  // bit i: this lane's logit i already selected
  float my_val = 0.0f, top = 0.0f;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + kWave * i;
      // ids grow with i, so a strict '>' keeps the lower id on ties
      if (e < E && !((taken >> i) & 1u) && (bi == 0x7fffffff || v[i] > bv)) {
        bv = v[i];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if (j == 0) top = bv;
    if (lane == j) {
      my_val = bv;
      my_idx = bi;
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi >> 6);
  }

  const float ex = (lane < k) ? expf(my_val - top) : 0.0f;
  float denom;
  if (renorm) {
    denom = wave_sum(ex);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i < E) s += expf(v[i] - top);
    denom = wave_sum(s);
  }
  int stored = -1;
  if (lane < k) {
    const long long r = (long long)t * k + lane;
    const bool valid = valid_rows < 0 || r < valid_rows;
    stored = valid ? my_idx : E;
    ids[r] = stored;
    weights[r] = valid ? ex / denom : 0.0f;
  }
  return stored;
}

}  // namespace moe
