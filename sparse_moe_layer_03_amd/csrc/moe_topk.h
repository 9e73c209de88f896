// Wave-level top-k selection shared by the router kernels (prefill and decode).
//
// Selection rule: the k largest logits, ordered by (logit descending, expert
// index ascending) -- exact ties go to the lowest expert index; -0 and +0
// compare equal.  Weights: softmax over the k selected logits, which equals
// the full softmax renormalised over the selection.
#pragma once

#include "moe_internal.h"

namespace moe {

// Wave-wide selection of the k largest (value desc, index asc) for NT tokens
// at once (their reduction chains are independent, so they interleave).
// Lane l holds the values of experts l, l+64, l+128, l+192 of every token
// (absent experts are invalid).  Lane r < k ends with (sel_e[t], sel_v[t]) of
// rank r of token t.
template <int NT>
__device__ __forceinline__ void wave_topk(float (&v)[NT][4], bool (&valid)[NT][4], int k, int lane,
                                          int (&sel_e)[NT], float (&sel_v)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    sel_e[t] = -1;
    sel_v[t] = 0.0f;
  }
  for (int r = 0; r < k; ++r) {
    float bv[NT];
    int be[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bv[t] = -INFINITY;
      be[t] = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (valid[t][q] && (be[t] == 0x7fffffff || v[t][q] > bv[t])) {  // ascending e: strict > keeps the lower index
          bv[t] = v[t][q];
          be[t] = lane + 64 * q;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float ov = __shfl_xor(bv[t], off);
        int oe = __shfl_xor(be[t], off);
        bool take = (oe != 0x7fffffff) && (be[t] == 0x7fffffff || ov > bv[t] || (ov == bv[t] && oe < be[t]));
        if (take) {
          bv[t] = ov;
          be[t] = oe;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (lane == r) {
        sel_e[t] = be[t];
        sel_v[t] = bv[t];
      }
      if ((be[t] & 63) == lane) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q == (be[t] >> 6)) valid[t][q] = false;
      }
    }
  }
}

// Weights of the selected experts: lane r < k holds rank r's logit.
__device__ __forceinline__ float wave_renorm_weight(float sel_v, int k, int lane) {
  float m = __shfl(sel_v, 0);
  float ex = (lane < k) ? expf(sel_v - m) : 0.0f;
  float sum = 0.0f;
  for (int r = 0; r < k; ++r) sum += __shfl(ex, r);  // rank order
  return ex / sum;
}

}  // namespace moe
