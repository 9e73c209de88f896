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

// ---- Sixteen lanes per token ----
// The same selection for 4 tokens per wave, one per 16-lane DPP row: sub-lane
// s = lane % 16 of row i holds experts 16 s .. 16 s + 15 of token i.  Each
// candidate becomes a unique 64-bit key, (order key of the logit) << 8 |
// (255 - expert): a larger key is a larger logit, or the same logit at a
// lower index, so the selection order is the key order with no ties to
// break; absent experts have key 0, below every finite logit.  A lane sorts
// its 16 keys once (Batcher's odd-even merge network); then each round takes
// the row maximum of the lanes' heads (a 4-step DPP butterfly, the result in
// every lane of the row) and the lane whose head it is drops it.  All rows
// run the same instructions, so the 4 tokens cost what one does.

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}

// Maximum over the 16 lanes of a DPP row, in every lane of the row: lane
// exchanges xor 1 and xor 2 (quad permutations), then the half-row and the
// row mirrors.
__device__ __forceinline__ uint64_t row16_max_u64(uint64_t v) {
  uint64_t o = dpp_u64<0xB1>(v);  // quad_perm [1,0,3,2]
  v = v > o ? v : o;
  o = dpp_u64<0x4E>(v);  // quad_perm [2,3,0,1]
  v = v > o ? v : o;
  o = dpp_u64<0x141>(v);  // row_half_mirror
  v = v > o ? v : o;
  o = dpp_u64<0x140>(v);  // row_mirror
  return v > o ? v : o;
}

// Sorts N (a power of two) keys into descending order: Batcher's odd-even
// merge sort; every index is a compile-time constant after unrolling.
template <int N>
__device__ __forceinline__ void sort_desc_u64(uint64_t (&a)[N]) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1)
#pragma unroll
    for (int k = p; k >= 1; k >>= 1)
#pragma unroll
      for (int j = k % p; j + k < N; j += 2 * k)
#pragma unroll
        for (int i = 0; i < k; ++i)
          if (i + j + k < N && (i + j) / (2 * p) == (i + j + k) / (2 * p)) {
            const uint64_t x = a[i + j], y = a[i + j + k];
            a[i + j] = x > y ? x : y;
            a[i + j + k] = x > y ? y : x;
          }
}

// The 64-bit key of expert e's logit v (valid: e exists).
__device__ __forceinline__ uint64_t topk_key64(float v, int e, bool valid) {
  if (v == 0.0f) v = 0.0f;  // -0 -> +0
  return valid ? ((uint64_t)float_order_key(v) << 8) | (uint64_t)(255 - e) : 0ull;
}

// Selection and weights for the token of this lane's row from its 16 keys
// (topk_key64, any order; k <= 16 <= number of valid experts is not needed:
// k <= the valid experts of the token).  Sub-lane r < k ends with rank r's
// expert in sel_e and logit in sel_v, and returns rank r's weight (0 in the
// other sub-lanes); the weights are those of wave_topk_weights_n:
//   w_r = exp(l_r - l_0) / sum_{r' < k} exp(l_r' - l_0), the sum in rank order.
// KMAX: an upper bound of k (8 or 16).  A lane gives at most k winners, so
// only the first KMAX of its sorted keys are ever its head: the pops shift
// those alone.
template <int KMAX = 16>
__device__ __forceinline__ float row16_topk_weights(uint64_t (&key)[16], int k, int sub, int& sel_e, float& sel_v) {
  static_assert(KMAX == 8 || KMAX == 16, "KMAX");
  sort_desc_u64<16>(key);
  sel_e = -1;
  sel_v = 0.0f;
  float m = 0.0f, sum = 0.0f;
  for (int r = 0; r < k; ++r) {
    const uint64_t M = row16_max_u64(key[0]);
    const bool win = key[0] == M;  // keys are unique: one lane of the row
#pragma unroll
    for (int i = 0; i < KMAX - 1; ++i) key[i] = win ? key[i + 1] : key[i];
    key[KMAX - 1] = win ? 0ull : key[KMAX - 1];
    const float val = float_from_order_key((uint32_t)(M >> 8));
    if (sub == r) {
      sel_e = 255 - (int)(M & 255u);
      sel_v = val;
    }
    if (r == 0) m = val;
    sum += expf(val - m);  // rank order
  }
  return sub < k ? expf(sel_v - m) / sum : 0.0f;
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
