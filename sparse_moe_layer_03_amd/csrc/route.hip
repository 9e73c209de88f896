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

namespace moe {
namespace {

constexpr int RT = 32;       // tokens per workgroup
constexpr int RBK = 64;      // K columns per LDS stage (128 bytes per row)
constexpr int RCH = RBK / 8; // 16-byte chunks per row per stage

__device__ __forceinline__ int swz8(int row, int chunk) { return chunk ^ (row & 7); }

// Wave-wide selection of the k largest (value desc, index asc).  Lane l holds
// the values of experts l, l+64, l+128, l+192 (absent ones are invalid).
// Lane r < k ends with (sel_e, sel_v) of rank r.
__device__ __forceinline__ void wave_topk(float v[4], bool valid[4], int k, int lane, int& sel_e, float& sel_v) {
  sel_e = -1;
  sel_v = 0.0f;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = lane + 64 * q;
      if (valid[q] && (be == 0x7fffffff || v[q] > bv)) {  // ascending e: strict > keeps the lower index
        bv = v[q];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oe = __shfl_xor(be, off);
      bool take = (oe != 0x7fffffff) && (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
      if (take) {
        bv = ov;
        be = oe;
      }
    }
    if (lane == r) {
      sel_e = be;
      sel_v = bv;
    }
    if ((be & 63) == lane) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q == (be >> 6)) valid[q] = false;
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
  const uint16_t* xrow = (t0 + xr < T) ? x + (size_t)(t0 + xr) * H : nullptr;
  const int nwl = (EP * RCH + 255) / 256;                    // router chunks per thread (<= 8)
  u32x4 px, pw[8];
  const u32x4 zero = {0u, 0u, 0u, 0u};

  auto gload = [&](int kb) {
    px = xrow ? *reinterpret_cast<const u32x4*>(xrow + kb * RBK + xc * 8) : zero;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nwl) {
        int idx = tid + 256 * i;
        int r = idx >> 3, c = idx & 7;
        pw[i] = (r < E) ? *reinterpret_cast<const u32x4*>(wr + (size_t)r * H + kb * RBK + c * 8) : zero;
      }
    }
  };
  auto sstore = [&](int st) {
    sx[st * RT * RCH + xr * RCH + swz8(xr, xc)] = px;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nwl) {
        int idx = tid + 256 * i;
        int r = idx >> 3, c = idx & 7;
        if (r < EP) sw[st * EP * RCH + r * RCH + swz8(r, c)] = pw[i];
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

  for (int r = wave * (RT / 4); r < (wave + 1) * (RT / 4); ++r) {
    int t = t0 + r;
    if (t >= T) break;
    float v[4];
    bool valid[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = lane + 64 * q;
      valid[q] = e < E;
      v[q] = valid[q] ? sl[r * LS + e] : 0.0f;
      if (logits_out && valid[q]) logits_out[(size_t)t * E + e] = v[q];
    }
    int sel_e;
    float sel_v;
    wave_topk(v, valid, k, lane, sel_e, sel_v);
    float wt = wave_renorm_weight(sel_v, k, lane);
    if (lane < k) {
      ids[(size_t)t * k + lane] = sel_e;
      wout[(size_t)t * k + lane] = wt;
    }
  }
}

__global__ __launch_bounds__(256) void topk_from_logits_kernel(const float* __restrict__ logits, int T, int E,
                                                               int k, int32_t* __restrict__ ids,
                                                               float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[4];
  bool valid[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int e = lane + 64 * q;
    valid[q] = e < E;
    float val = valid[q] ? logits[(size_t)t * E + e] : 0.0f;
    if (val == 0.0f) val = 0.0f;
    v[q] = val;
  }
  int sel_e;
  float sel_v;
  wave_topk(v, valid, k, lane, sel_e, sel_v);
  float wt = wave_renorm_weight(sel_v, k, lane);
  if (lane < k) {
    ids[(size_t)t * k + lane] = sel_e;
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
