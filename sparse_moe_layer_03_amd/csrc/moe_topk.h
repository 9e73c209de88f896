// Wave-level top-k selection shared by the router kernels (prefill and decode).
//
// Selection rule: the k largest logits, ordered by (logit descending, expert
// index ascending) -- exact ties go to the lowest expert index; -0 and +0
// compare equal.  Weights: softmax over the k selected logits, which equals
// the full softmax renormalised over the selection (guanjiawei.ai "AIMA
// AMD395 Qwen3.6-35B-A3B", data path: only the selected experts run).
//
// Each logit becomes one exact 64-bit key: the high word is the float's bits
// mapped to an unsigned integer of the same order, the low word the bitwise
// complement of the expert index, so a larger key is a larger logit or, for
// equal logits, a lower index.  Keys are unique; a selection round is one
// wave-wide maximum, reduced with DPP row shifts and row broadcasts.
#pragma once

#include "moe_internal.h"

namespace moe {

// Order-preserving map of a float (not NaN, -0 already mapped to +0) to
// uint32: a larger float gives a larger integer.  Never 0 for a finite float.
__device__ __forceinline__ uint32_t float_order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float float_from_order_key(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// One DPP step of a 64-bit maximum: (hi, lo) = max((hi, lo), lane-moved (hi, lo)).
// Lanes without a source read 0, the smallest key.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t oh = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, CTRL, ROW_MASK, 0xf, false);
  const uint32_t ol = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, CTRL, ROW_MASK, 0xf, false);
  const bool take = (oh > hi) || (oh == hi && ol > lo);
  hi = take ? oh : hi;
  lo = take ? ol : lo;
}

// Top-k of up to 256 logits held 4 per lane (lane l: experts l, l+64, l+128,
// l+192; absent experts invalid), for NT tokens at once: their selection
// rounds are independent, so the DPP chains interleave.  Lane r < k ends
// with rank r's expert in sel_e[t] and logit in sel_v[t], and w[t] returns
// rank r's weight in lane r:
//   w_r = exp(l_r - l_0) / sum_{r' < k} exp(l_r' - l_0), the sum in rank order.
template <int NT>
__device__ __forceinline__ void wave_topk_weights_n(const float (&v)[NT][4], const bool (&valid)[NT][4], int k,
                                                    int lane, int (&sel_e)[NT], float (&sel_v)[NT], float (&w)[NT]) {
  uint32_t kh[NT][4], kl[NT][4];
  float m[NT], sum[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float x = v[t][q];
      if (x == 0.0f) x = 0.0f;  // -0 -> +0
      kh[t][q] = valid[t][q] ? float_order_key(x) : 0u;
      kl[t][q] = valid[t][q] ? ~(uint32_t)(lane + 64 * q) : 0u;
    }
    sel_e[t] = -1;
    sel_v[t] = 0.0f;
    m[t] = 0.0f;
    sum[t] = 0.0f;
  }
  for (int r = 0; r < k; ++r) {
    uint32_t bh[NT], bl[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {  // this lane's best remaining key
      bh[t] = kh[t][0];
      bl[t] = kl[t][0];
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        const bool take = (kh[t][q] > bh[t]) || (kh[t][q] == bh[t] && kl[t][q] > bl[t]);
        bh[t] = take ? kh[t][q] : bh[t];
        bl[t] = take ? kl[t][q] : bl[t];
      }
    }
    // wave maxima: inclusive maxima within rows of 16 lanes, then rows 1 and
    // 3 take the previous row's, then rows 2 and 3 take row 1's (lane 63)
#pragma unroll
    for (int t = 0; t < NT; ++t) dpp_max_step<0x111, 0xf>(bh[t], bl[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) dpp_max_step<0x112, 0xf>(bh[t], bl[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) dpp_max_step<0x114, 0xf>(bh[t], bl[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) dpp_max_step<0x118, 0xf>(bh[t], bl[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) dpp_max_step<0x142, 0xa>(bh[t], bl[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) dpp_max_step<0x143, 0xc>(bh[t], bl[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t mh = (uint32_t)__builtin_amdgcn_readlane((int)bh[t], 63);
      const uint32_t ml = (uint32_t)__builtin_amdgcn_readlane((int)bl[t], 63);
      // the winning key is a valid one (k <= number of valid experts); the
      // clamp only keeps an index in range should that ever not hold
      const int e = min(max((int)~ml, 0), 255);
      const float val = float_from_order_key(mh);
      if (lane == r) {
        sel_e[t] = e;
        sel_v[t] = val;
      }
      if ((e & 63) == lane) {  // the owner drops the selected key
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q == (e >> 6)) kh[t][q] = kl[t][q] = 0u;
      }
      if (r == 0) m[t] = val;
      sum[t] += expf(val - m[t]);  // uniform, rank order
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) w[t] = (lane < k) ? expf(sel_v[t] - m[t]) / sum[t] : 0.0f;
}

// One token.
__device__ __forceinline__ void wave_topk_weights(const float (&v)[4], const bool (&valid)[4], int k, int lane,
                                                  int& sel_e, float& sel_v, float& w) {
  float vv[1][4];
  bool ok[1][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    vv[0][q] = v[q];
    ok[0][q] = valid[q];
  }
  int e[1];
  float sv[1], ww[1];
  wave_topk_weights_n<1>(vv, ok, k, lane, e, sv, ww);
  sel_e = e[0];
  sel_v = sv[0];
  w = ww[0];
}

}  // namespace moe
