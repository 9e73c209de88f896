// Wave-level top-k selection shared by the router kernels (prefill and decode).
//
// Selection rule: the k largest logits, ordered by (logit descending, expert
// index ascending) -- exact ties go to the lowest expert index; -0 and +0
// compare equal.  Weights: softmax over the k selected logits, which equals
// the full softmax renormalised over the selection (guanjiawei.ai "AIMA
// AMD395 Qwen3.6-35B-A3B", data path: only the selected experts run).
//
// Each logit becomes a 32-bit key: the float's bits mapped to an unsigned
// integer of the same order.  A selection round is one wave-wide maximum of
// the keys (DPP row shifts and row broadcasts) followed by ballots that find
// the lowest expert index holding it.
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

// Maximum over the 64 lanes of a 32-bit unsigned value: inclusive maxima
// within rows of 16 lanes by DPP row_shr 1, 2, 4, 8, then row_bcast:15 and
// row_bcast:31 carry them up; lane 63 holds the result, returned uniform.
// Lanes without a DPP source read 0, the smallest value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of up to 256 logits held 4 per lane (lane l: experts l, l+64, l+128,
// l+192; absent experts invalid), for NT tokens at once: their selection
// rounds are independent, so their instruction chains interleave.  A round
// takes the wave maximum of the 32-bit order keys, then the lowest expert
// index holding that key: slot q covers indices 64 q .. 64 q + 63, so the
// first slot whose ballot of "key == maximum" is not empty, and its lowest
// lane, give it.  Keys are equal exactly when the logits are, so the order is
// (logit desc, index asc) with no approximation.  Lane r < k ends with rank
// r's expert in sel_e[t] and logit in sel_v[t], and w[t] returns rank r's
// weight in lane r:
//   w_r = exp(l_r - l_0) / sum_{r' < k} exp(l_r' - l_0), the sum in rank order.
template <int NT>
__device__ __forceinline__ void wave_topk_weights_n(const float (&v)[NT][4], const bool (&valid)[NT][4], int k,
                                                    int lane, int (&sel_e)[NT], float (&sel_v)[NT], float (&w)[NT]) {
  uint32_t key[NT][4];
  float m[NT], sum[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float x = v[t][q];
      if (x == 0.0f) x = 0.0f;  // -0 -> +0
      key[t][q] = valid[t][q] ? float_order_key(x) : 0u;  // 0: below every finite logit
    }
    sel_e[t] = -1;
    sel_v[t] = 0.0f;
    m[t] = 0.0f;
    sum[t] = 0.0f;
  }
  for (int r = 0; r < k; ++r) {
    uint32_t mk[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) mk[t] = max(max(key[t][0], key[t][1]), max(key[t][2], key[t][3]));
#pragma unroll
    for (int t = 0; t < NT; ++t) mk[t] = wave_max_u32(mk[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint64_t b0 = __ballot(key[t][0] == mk[t]), b1 = __ballot(key[t][1] == mk[t]);
      const uint64_t b2 = __ballot(key[t][2] == mk[t]), b3 = __ballot(key[t][3] == mk[t]);
      // the maximum is held by a valid key (k <= number of valid experts), so
      // one ballot is not empty
      const int e = b0 ? __builtin_ctzll(b0)
                       : b1 ? 64 + __builtin_ctzll(b1) : b2 ? 128 + __builtin_ctzll(b2) : 192 + __builtin_ctzll(b3 | (1ull << 63));
      const float val = float_from_order_key(mk[t]);
      if (lane == r) {
        sel_e[t] = e;
        sel_v[t] = val;
      }
      if ((e & 63) == lane) {  // the owner drops the selected key
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q == (e >> 6)) key[t][q] = 0u;
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
