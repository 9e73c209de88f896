// Top-k routing on router logits.
//
// The router GEMM (grouped_gemm.hip, ROUTER launch) writes fp32 logits
// (+ bias) and the shared-expert gate.  Here one wavefront per token selects
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

}  // namespace

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st) {
  dim3 grid((T + 3) / 4);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(256), 0, st, logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
