// Top-k routing on router logits, plus the shared-expert gate.
//
// The router GEMM runs as a column block of the dense (router + shared
// expert) grouped-GEMM launch, which writes fp32 logits (+ bias).  Here one
// wavefront per token selects the k largest logits by (logit desc, index asc)
// and computes the renormalised softmax weights (guanjiawei.ai "AIMA AMD395
// Qwen3.6-35B-A3B", data path: only the selected experts run; kongchang.com
// "GFX1151 engine", MoE kernel section: a few experts are activated per
// token), and, when a gate vector is given, s = sigmoid(x_t . w_sg) from the
// token's row of x.
#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void topk_gate_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                        const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w_sg, int H,
                                                        int32_t* __restrict__ ids, float* __restrict__ wout,
                                                        float* __restrict__ sout) {
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
  // gate loads after the logits: the selection waits only for the logits
  u32x4 xv[4], gv[4];
  const int nch = H / 8;
  const bool gate = x != nullptr && w_sg != nullptr;
  if (gate) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = lane + 64 * q;
      if (c < nch) {
        xv[q] = reinterpret_cast<const u32x4*>(x + (size_t)t * H)[c];
        gv[q] = reinterpret_cast<const u32x4*>(w_sg)[c];
      }
    }
  }
  int sel_e;
  float sel_v, wt;
  wave_topk_weights(v, valid, k, lane, sel_e, sel_v, wt);
  if (lane < k) {
    ids[(size_t)t * k + lane] = sel_e;
    wout[(size_t)t * k + lane] = wt;
  }
  if (gate) {
    float g = 0.0f;
    for (int q = 0; q < 4; ++q) {
      const int c = lane + 64 * q;
      if (c < nch) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          g += bf16_to_f32((uint16_t)(xv[q][i] & 0xffff)) * bf16_to_f32((uint16_t)(gv[q][i] & 0xffff));
          g += bf16_to_f32((uint16_t)(xv[q][i] >> 16)) * bf16_to_f32((uint16_t)(gv[q][i] >> 16));
        }
      }
    }
    for (int c = lane + 256; c < nch; c += 64) {  // H > 2048
      const u32x4 a = reinterpret_cast<const u32x4*>(x + (size_t)t * H)[c];
      const u32x4 b = reinterpret_cast<const u32x4*>(w_sg)[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g += bf16_to_f32((uint16_t)(a[i] & 0xffff)) * bf16_to_f32((uint16_t)(b[i] & 0xffff));
        g += bf16_to_f32((uint16_t)(a[i] >> 16)) * bf16_to_f32((uint16_t)(b[i] >> 16));
      }
    }
    g = wave_sum(g);
    if (lane == 0) sout[t] = 1.0f / (1.0f + expf(-g));
  }
}

}  // namespace

hipError_t launch_topk(const float* logits, int T, int E, int k, const uint16_t* x, const uint16_t* w_sg, int H,
                       int32_t* ids, float* w, float* s, hipStream_t st) {
  dim3 grid((T + 3) / 4);
  hipLaunchKernelGGL(topk_gate_kernel, grid, dim3(256), 0, st, logits, T, E, k, x, w_sg, H, ids, w, s);
  return hipGetLastError();
}

}  // namespace moe
