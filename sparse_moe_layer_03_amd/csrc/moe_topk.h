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

// Maximum 64-bit key over the wave, returned to every lane (uniform).
__device__ __forceinline__ void wave_max_key(uint32_t hi, uint32_t lo, uint32_t& mhi, uint32_t& mlo) {
  // inclusive maxima within rows of 16 lanes, then rows 1 and 3 take the
  // previous row's maximum, then rows 2 and 3 take row 1's: lane 63 holds it
  dpp_max_step<0x111, 0xf>(hi, lo);
  dpp_max_step<0x112, 0xf>(hi, lo);
  dpp_max_step<0x114, 0xf>(hi, lo);
  dpp_max_step<0x118, 0xf>(hi, lo);
  dpp_max_step<0x142, 0xa>(hi, lo);
  dpp_max_step<0x143, 0xc>(hi, lo);
  mhi = (uint32_t)__builtin_amdgcn_readlane((int)hi, 63);
  mlo = (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
}

// Top-k of up to 256 logits held 4 per lane (lane l: experts l, l+64, l+128,
// l+192; absent experts invalid).  Lane r < k ends with rank r's expert in
// sel_e and logit in sel_v; w returns rank r's weight in lane r:
//   w_r = exp(l_r - l_0) / sum_{r' < k} exp(l_r' - l_0), the sum in rank order.
__device__ __forceinline__ void wave_topk_weights(const float (&v)[4], const bool (&valid)[4], int k, int lane,
                                                  int& sel_e, float& sel_v, float& w) {
  uint32_t kh[4], kl[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x = v[q];
    if (x == 0.0f) x = 0.0f;  // -0 -> +0
    kh[q] = valid[q] ? float_order_key(x) : 0u;
    kl[q] = valid[q] ? ~(uint32_t)(lane + 64 * q) : 0u;
  }
  sel_e = -1;
  sel_v = 0.0f;
  float m = 0.0f, sum = 0.0f;
  for (int r = 0; r < k; ++r) {
    // this lane's best remaining key
    uint32_t bh = kh[0], bl = kl[0];
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      const bool take = (kh[q] > bh) || (kh[q] == bh && kl[q] > bl);
      bh = take ? kh[q] : bh;
      bl = take ? kl[q] : bl;
    }
    uint32_t mh, ml;
    wave_max_key(bh, bl, mh, ml);
    // the winning key is a valid one (k <= number of valid experts); the
    // clamp only keeps an index in range should that ever not hold
    const int e = min(max((int)~ml, 0), 255);
    const float val = float_from_order_key(mh);
    if (lane == r) {
      sel_e = e;
      sel_v = val;
    }
    // the owner drops the selected key
    if ((e & 63) == lane) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q == (e >> 6)) kh[q] = kl[q] = 0u;
    }
    if (r == 0) m = val;
    sum += expf(val - m);  // uniform, rank order
  }
  w = (lane < k) ? expf(sel_v - m) / sum : 0.0f;
}

}  // namespace moe
