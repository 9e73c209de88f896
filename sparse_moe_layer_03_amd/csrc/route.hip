// Top-k routing on router logits.
//
// The router GEMM (grouped_gemm.hip, ROUTER launch) writes fp32 logits
// (+ bias) and the shared-expert gate; its split form (ROUTER_PART) writes
// per-slice partial logits that router_reduce_topk_kernel sums before it
// selects.  Here one wavefront per token selects
// the k largest logits by (logit desc, index asc) and computes the
// renormalised softmax weights (guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B",
// data path: only the selected experts run; kongchang.com "GFX1151 engine",
// MoE kernel section: a few experts are activated per token).
#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int32_t* __restrict__ ids, float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[4];
  bool valid[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    valid[q] = e < E;
    v[q] = valid[q] ? logits[(size_t)t * E + e] : 0.0f;
  }
  int sel_e;
  float sel_v, wt;
  wave_topk_weights(v, valid, k, lane, sel_e, sel_v, wt);
  if (lane < k) {
    ids[(size_t)t * k + lane] = sel_e;
    wout[(size_t)t * k + lane] = wt;
  }
}

// Split router, second launch: token t's logits are the slices' partial sums
// added in slice order, plus the bias (-0 -> +0); then the selection above.
// Partial rows are EP = E rounded up to 4 floats apart.  A wave takes 4
// tokens, one per 16-lane row (row16_topk_weights); sub-lane s loads experts
// 16 s .. 16 s + 15 of every slice as 16-byte loads, all issued at once.
// With gpart, s[t] = sigmoid(sum of the slices' x . w_sg).
template <int S>
__global__ __launch_bounds__(256) void router_reduce_topk_kernel(const float* __restrict__ part,
                                                                 const float* __restrict__ gpart, int T, int E,
                                                                 int k, const float* __restrict__ bias,
                                                                 int32_t* __restrict__ ids, float* __restrict__ wout,
                                                                 float* __restrict__ s, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const int tw = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4;  // the wave's first token
  if (tw >= T) return;
  const int tok = tw + (lane >> 4);
  const int t = min(tok, T - 1);  // rows past T repeat the last token and are not stored
  const int EP = (E + 3) & ~3;
  const int e0 = 16 * sub;
  float4 pv[S][4];
#pragma unroll
  for (int sl = 0; sl < S; ++sl)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = e0 + 4 * c;
      pv[sl][c] = *reinterpret_cast<const float4*>(part + ((size_t)sl * T + t) * EP + (e < E ? e : 0));
    }
  // bias of this lane's 16 experts, loaded with the partials: clamped, not
  // skipped (a load under a per-lane condition is waited for on its own)
  float bv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) bv[i] = bias ? bias[min(e0 + i, E - 1)] : 0.0f;
  float gs = 0.0f;
  if (gpart && sub == 0) {
#pragma unroll
    for (int sl = 0; sl < S; ++sl) gs += gpart[(size_t)sl * T + t];
  }
  uint64_t key[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float4 a = pv[0][c];
#pragma unroll
    for (int sl = 1; sl < S; ++sl) {
      a.x += pv[sl][c].x;
      a.y += pv[sl][c].y;
      a.z += pv[sl][c].z;
      a.w += pv[sl][c].w;
    }
    const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + 4 * c + q;
      const bool valid = e < E;
      float v = av[q] + (valid ? bv[4 * c + q] : 0.0f);
      if (v == 0.0f) v = 0.0f;  // -0 -> +0
      if (logits && valid && tok < T) logits[(size_t)tok * E + e] = v;
      key[4 * c + q] = topk_key64(v, e, valid);
    }
  }
  int sel_e;
  float sel_v;
  const float w = row16_topk_weights(key, k, sub, sel_e, sel_v);
  if (tok < T && sub < k) {
    ids[(size_t)tok * k + sub] = sel_e;
    wout[(size_t)tok * k + sub] = w;
  }
  if (gpart && sub == 0 && tok < T) s[tok] = 1.0f / (1.0f + expf(-gs));
}

}  // namespace

hipError_t launch_router_reduce_topk(const float* part, const float* gpart, int S, int T, int E, int k,
                                     const float* bias, int32_t* ids, float* w, float* s, float* logits,
                                     hipStream_t st) {
  constexpr int per_block = 16;  // 4 waves of 4 tokens
  dim3 grid((T + per_block - 1) / per_block);
  switch (S) {
    case 1: hipLaunchKernelGGL(router_reduce_topk_kernel<1>, grid, dim3(256), 0, st, part, gpart, T, E, k, bias, ids, w, s, logits); break;
    case 2: hipLaunchKernelGGL(router_reduce_topk_kernel<2>, grid, dim3(256), 0, st, part, gpart, T, E, k, bias, ids, w, s, logits); break;
    case 4: hipLaunchKernelGGL(router_reduce_topk_kernel<4>, grid, dim3(256), 0, st, part, gpart, T, E, k, bias, ids, w, s, logits); break;
    case 8: hipLaunchKernelGGL(router_reduce_topk_kernel<8>, grid, dim3(256), 0, st, part, gpart, T, E, k, bias, ids, w, s, logits); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st) {
  dim3 grid((T + 3) / 4);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(256), 0, st, logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
