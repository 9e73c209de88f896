// Router stage of the sparse MoE layer on gfx950.
//
// What it computes (guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B", data path:
// only the selected experts run; kongchang.com "GFX1151 engine", MoE kernel
// section: a few experts are activated per token by sparse routing):
//   logits[t,e] = sum_h x[t,h] W_router[e,h] (+ bias[e])     fp32 accumulate
//   ids[t,:]    = top-k by (logit desc, index asc)
//   w[t,j]      = exp(l_j - l_0) / sum_j' exp(l_j' - l_0)      (renormalised softmax)
//   s[t]        = 1 / (1 + exp(-x_t . w_sg))
//
// One workgroup (4 wavefronts) owns 32 tokens and all experts.  The router
// GEMM runs on v_mfma_f32_32x32x16_bf16 with the token tile and the router
// rows staged through LDS 64 columns at a time (double buffered, register
// prefetch).  The gate dot runs on the vector ALUs from the same LDS tile.
// The logits of the 32 tokens then sit in LDS and each wavefront selects the
// top-k of 8 tokens with wave-wide arg-max reductions.
#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {
namespace {

constexpr int RT = 32;       // tokens per workgroup
constexpr int RBK = 64;      // K columns per LDS stage (128 bytes per row)
constexpr int RCH = RBK / 8; // 16-byte chunks per row per stage

// 16-byte chunk swizzle of a 128-byte LDS row: 8 consecutive rows read at one
// logical chunk hit 8 distinct bank groups of a 128-byte bank row, and 16
// consecutive rows 16 distinct groups of a 256-byte one.
__device__ __forceinline__ int swz8(int row, int chunk) { return chunk ^ (((row >> 1) ^ ((row & 1) << 2)) & 7); }

__global__ __launch_bounds__(256) void route_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                    const float* __restrict__ bias,
                                                    const uint16_t* __restrict__ w_sg, int T, int H, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ wout,
                                                    float* __restrict__ sout, float* __restrict__ logits_out) {
  // stage: x tile [32][8 chunks] + router rows [EP][8 chunks], two stages.
  extern __shared__ __align__(16) unsigned char smem[];
  const int EP = (E + 31) & ~31;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT;
  u32x4* sx = reinterpret_cast<u32x4*>(smem);               // [2][RT*RCH]
  u32x4* sw = sx + 2 * RT * RCH;                             // [2][EP*RCH]

  // global -> register assignment
  const int xr = tid >> 3, xc = tid & 7;                     // one x chunk per thread
  // Rows past T and router rows past E load row 0 and are zeroed when they
  // are written to LDS (a select right after a load would stall on it).
  const bool xok = t0 + xr < T;
  const uint16_t* xrow = x + (size_t)(xok ? t0 + xr : 0) * H;
  const int nwl = (EP * RCH + 255) / 256;                    // router chunks per thread (<= 8)
  u32x4 px, pw[8];
  const u32x4 zero = {0u, 0u, 0u, 0u};

  auto gload = [&](int kb) {
    px = *reinterpret_cast<const u32x4*>(xrow + kb * RBK + xc * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nwl) {
        int idx = tid + 256 * i;
        int r = idx >> 3, c = idx & 7;
        pw[i] = *reinterpret_cast<const u32x4*>(wr + (size_t)(r < E ? r : 0) * H + kb * RBK + c * 8);
      }
    }
  };
  auto sstore = [&](int st) {
    sx[st * RT * RCH + xr * RCH + swz8(xr, xc)] = xok ? px : zero;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nwl) {
        int idx = tid + 256 * i;
        int r = idx >> 3, c = idx & 7;
        if (r < EP) sw[st * EP * RCH + r * RCH + swz8(r, c)] = (r < E) ? pw[i] : zero;
      }
    }
  };

  // expert blocks of this wave: w, w+4 (32 experts each)
  const int EB = EP / 32;
  f32x16 acc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[b][j] = 0.0f;
  float gpart = 0.0f;  // gate dot partial: token xr, chunk xc

  const int nk = H / RBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < nk) gload(kb + 1);
    const u32x4* cx = sx + st * RT * RCH;
    const u32x4* cw = sw + st * EP * RCH;
#pragma unroll
    for (int s = 0; s < RBK / 16; ++s) {
      int r = lane & 31, c = 2 * s + (lane >> 5);
      u32x4 a = cx[r * RCH + swz8(r, c)];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        int blk = wave + 4 * b;
        if (blk < EB) {
          int rr = blk * 32 + (lane & 31);
          u32x4 bw = cw[rr * RCH + swz8(rr, c)];
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, bw), acc[b], 0, 0, 0);
        }
      }
    }
    if (w_sg) {
      u32x4 xv = cx[xr * RCH + swz8(xr, xc)];
      u32x4 gv = *reinterpret_cast<const u32x4*>(w_sg + kb * RBK + xc * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        gpart += bf16_to_f32((uint16_t)(xv[q] & 0xffff)) * bf16_to_f32((uint16_t)(gv[q] & 0xffff));
        gpart += bf16_to_f32((uint16_t)(xv[q] >> 16)) * bf16_to_f32((uint16_t)(gv[q] >> 16));
      }
    }
    if (kb + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

  // logits (+bias) -> LDS [RT][EP+1]
  float* sl = reinterpret_cast<float*>(smem);
  const int LS = EP + 1;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    int blk = wave + 4 * b;
    if (blk < EB) {
      int e = blk * 32 + (lane & 31);
      float be = (bias && e < E) ? bias[e] : 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        int row = 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
        float v = acc[b][j] + be;
        if (v == 0.0f) v = 0.0f;  // -0 -> +0
        sl[row * LS + e] = v;
      }
    }
  }
  // gate: reduce the 8 partials of each token (consecutive lanes)
  gpart += __shfl_xor(gpart, 1);
  gpart += __shfl_xor(gpart, 2);
  gpart += __shfl_xor(gpart, 4);
  if (w_sg && xc == 0 && t0 + xr < T) sout[t0 + xr] = 1.0f / (1.0f + expf(-gpart));
  __syncthreads();

  constexpr int NT = RT / 4;  // tokens per wave
  const int r0 = wave * NT;
  float v[NT][4];
  bool valid[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = lane + 64 * q;
      valid[t][q] = e < E && t0 + r0 + t < T;
      v[t][q] = valid[t][q] ? sl[(r0 + t) * LS + e] : 0.0f;
      if (logits_out && valid[t][q]) logits_out[(size_t)(t0 + r0 + t) * E + e] = v[t][q];
    }
  }
  int sel_e[NT];
  float sel_v[NT];
  wave_topk<NT>(v, valid, k, lane, sel_e, sel_v);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = t0 + r0 + t;
    float wt = wave_renorm_weight(sel_v[t], k, lane);
    if (tok < T && lane < k) {
      ids[(size_t)tok * k + lane] = sel_e[t];
      wout[(size_t)tok * k + lane] = wt;
    }
  }
}

__global__ __launch_bounds__(256) void topk_from_logits_kernel(const float* __restrict__ logits, int T, int E,
                                                               int k, int32_t* __restrict__ ids,
                                                               float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[1][4];
  bool valid[1][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int e = lane + 64 * q;
    valid[0][q] = e < E;
    float val = valid[0][q] ? logits[(size_t)t * E + e] : 0.0f;
    if (val == 0.0f) val = 0.0f;
    v[0][q] = val;
  }
  int sel_e[1];
  float sel_v[1];
  wave_topk<1>(v, valid, k, lane, sel_e, sel_v);
  float wt = wave_renorm_weight(sel_v[0], k, lane);
  if (lane < k) {
    ids[(size_t)t * k + lane] = sel_e[0];
    wout[(size_t)t * k + lane] = wt;
  }
}

}  // namespace

hipError_t launch_route(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg,
                        int T, int H, int E, int k, int32_t* ids, float* w, float* s, float* logits,
                        hipStream_t st) {
  const int EP = (E + 31) & ~31;
  size_t stage_bytes = 2 * (size_t)(RT + EP) * RCH * 16;
  size_t logit_bytes = (size_t)RT * (EP + 1) * 4;
  size_t lds = stage_bytes > logit_bytes ? stage_bytes : logit_bytes;
  dim3 grid((T + RT - 1) / RT);
  hipLaunchKernelGGL(route_kernel, grid, dim3(256), lds, st, x, w_router, bias, w_sg, T, H, E, k, ids, w, s,
                     logits);
  return hipGetLastError();
}

hipError_t launch_route_from_logits(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                                    hipStream_t st) {
  dim3 grid((T + 3) / 4);
  hipLaunchKernelGGL(topk_from_logits_kernel, grid, dim3(256), 0, st, logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
