// Single-token (T = 1) decode path of the sparse MoE layer on gfx950.
//
// At batch-1 decode the layer is a set of matrix-vector products and is bound
// by HBM bandwidth: the bytes to move are the router, the k selected experts'
// weights and the shared expert (guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B",
// data path: only the selected experts are computed; kongchang.com
// "GFX1151 engine", MoE kernel section: sparse routing changes the memory
// access pattern of token generation).  Every weight row is read once, by one
// wavefront, with 16-byte loads (64 lanes x 16 B = 1 KiB per instruction),
// and all loads of a wavefront are issued before its reductions.
//
//   D1 router: wave per router row (logit); one wave for the shared gate
//      s = sigmoid(x.w_sg)
//   D2 top-k + gate/up: in every workgroup, wave 0 selects the k experts from
//      the E logits (same rule and weights as prefill) while waves 1..3
//      compute the shared expert's gate/up rows; then a wave per (expert,
//      row) pair computes h = silu(g) * u in fp32; workgroup 0 also stores
//      ids and weights for D3
//   D3 down projection + combine: wave per output column, k + 1 rows of
//      W_down / Ws_down, y = sum_j w_j o_j + s o_s in fp32 -> bf16
// Wave sums use DPP row shifts and row broadcasts (no LDS round trips).
#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {
namespace {

struct DecodeWs {
  float* logits;  // [E]
  int32_t* ids;   // [k]
  float* w;       // [k]
  float* s;       // [1]
  float* hs;      // [I_s]
  float* h;       // [k * I]
};

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

DecodeWs carve(void* base, int H, int E, int k, int I, int I_s) {
  (void)H;
  char* p = static_cast<char*>(base);
  DecodeWs d;
  d.logits = reinterpret_cast<float*>(p);
  p += align256((size_t)E * 4);
  d.ids = reinterpret_cast<int32_t*>(p);  // 256-byte slot: 64 entries, read 16 at a time
  p += 256;
  d.w = reinterpret_cast<float*>(p);
  p += 256;
  d.s = reinterpret_cast<float*>(p);
  p += 256;
  d.hs = reinterpret_cast<float*>(p);
  p += align256((size_t)(I_s > 0 ? I_s : 1) * 4);
  d.h = reinterpret_cast<float*>(p);
  return d;
}

__device__ __forceinline__ float dot8(u32x4 a, u32x4 b) {
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s += bf16_to_f32((uint16_t)(a[q] & 0xffff)) * bf16_to_f32((uint16_t)(b[q] & 0xffff));
    s += bf16_to_f32((uint16_t)(a[q] >> 16)) * bf16_to_f32((uint16_t)(b[q] >> 16));
  }
  return s;
}

// Dot products of x with one or two bf16 rows of length H.  x comes from LDS
// (sx) when given, else straight from global memory; every load of a group
// of 4 chunks per lane (x's included) is issued before the arithmetic.
__device__ __forceinline__ void row_dots(const u32x4* sx, const uint16_t* xg, const uint16_t* r0, const uint16_t* r1,
                                         int H, int lane, float& d0, float& d1) {
  const int nch = H / 8;
  d0 = 0.0f;
  d1 = 0.0f;
  for (int base = 0; base < nch; base += 256) {
    u32x4 a[4], b[4], xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c = base + q * 64 + lane;
      if (c < nch) {
        a[q] = reinterpret_cast<const u32x4*>(r0)[c];
        if (r1) b[q] = reinterpret_cast<const u32x4*>(r1)[c];
        xv[q] = sx ? sx[c] : reinterpret_cast<const u32x4*>(xg)[c];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c = base + q * 64 + lane;
      if (c < nch) {
        d0 += dot8(xv[q], a[q]);
        if (r1) d1 += dot8(xv[q], b[q]);
      }
    }
  }
  d0 = wave_sum(d0);
  d1 = wave_sum(d1);
}

__global__ __launch_bounds__(256) void decode_router_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            const uint16_t* __restrict__ w_sg, int H, int E,
                                                            DecodeWs d) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  float d0, d1;
  if (row < E) {
    row_dots(nullptr, x, wr + (size_t)row * H, nullptr, H, lane, d0, d1);
    if (lane == 0) {
      float v = d0 + (bias ? bias[row] : 0.0f);
      if (v == 0.0f) v = 0.0f;
      d.logits[row] = v;
    }
  } else if (row == E && w_sg) {
    row_dots(nullptr, x, w_sg, nullptr, H, lane, d0, d1);
    if (lane == 0) d.s[0] = 1.0f / (1.0f + expf(-d0));
  }
}

// Top-k of the E logits by wave 0 of the workgroup, results in LDS (the
// caller synchronises the workgroup before reading them).
__device__ __forceinline__ void block_topk(const float* __restrict__ logits, int E, int k, int* sel_e,
                                           float* sel_w) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    float v[4];
    bool valid[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      valid[q] = e < E;
      v[q] = valid[q] ? logits[e] : 0.0f;
    }
    int se;
    float sv, w;
    wave_topk_weights(v, valid, k, lane, se, sv, w);
    if (lane < k) {
      sel_e[lane] = se;
      sel_w[lane] = w;
    }
  }
}

// While wave 0 selects the experts, waves 1..3 compute the shared expert's
// gate/up rows (they do not depend on the routing): row i = silu(g) * u -> h_s.
__global__ __launch_bounds__(256) void decode_topk_gate_up_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ w_gate,
                                                                  const uint16_t* __restrict__ w_up,
                                                                  const uint16_t* __restrict__ ws_gate,
                                                                  const uint16_t* __restrict__ ws_up, int H, int E,
                                                                  int k, int I, int I_s, DecodeWs d) {
  __shared__ u32x4 sx[1024];
  __shared__ int sel_e[kMaxK];
  __shared__ float sel_w[kMaxK];
  for (int c = threadIdx.x; c < H / 8; c += 256) sx[c] = reinterpret_cast<const u32x4*>(x)[c];
  const int wave = threadIdx.x >> 6;
  if (wave == 0) {
    block_topk(d.logits, E, k, sel_e, sel_w);
  } else {
    for (int i = blockIdx.x * 3 + wave - 1; i < I_s; i += 3 * gridDim.x) {
      float g, u;
      row_dots(nullptr, x, ws_gate + (size_t)i * H, ws_up + (size_t)i * H, H, threadIdx.x & 63, g, u);
      if ((threadIdx.x & 63) == 0) d.hs[i] = silu(g) * u;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x < k) {
    d.ids[threadIdx.x] = sel_e[threadIdx.x];
    d.w[threadIdx.x] = sel_w[threadIdx.x];
  }
  // wave w of workgroup b takes row pairs b*4 + w + q*(4*gridDim.x), q = 0..NR-1;
  // the NR pairs' loads are all issued before any reduction
  constexpr int NR = 1;
  const int lane = threadIdx.x & 63;
  const int stride = 4 * gridDim.x;
  const int row0 = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = H / 8;  // chunks per weight row; lane handles chunks lane + 64 c
  float g[NR], u[NR];
#pragma unroll
  for (int q = 0; q < NR; ++q) g[q] = u[q] = 0.0f;
  for (int c0 = 0; c0 < nch; c0 += 64 * 4) {
    u32x4 a[NR][4], b[NR][4];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int row = row0 + q * stride;
      const int rr = row < k * I ? row : 0;
      const size_t off = ((size_t)sel_e[rr / I] * I + rr % I) * H;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int ch = c0 + lane + 64 * c;
        if (ch < nch) {
          a[q][c] = reinterpret_cast<const u32x4*>(w_gate + off)[ch];
          b[q][c] = reinterpret_cast<const u32x4*>(w_up + off)[ch];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NR; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int ch = c0 + lane + 64 * c;
        if (ch < nch) {
          const u32x4 xv = sx[ch];
          g[q] += dot8(xv, a[q][c]);
          u[q] += dot8(xv, b[q][c]);
        }
      }
  }
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    const int row = row0 + q * stride;
    const float gs = wave_sum(g[q]), us = wave_sum(u[q]);
    if (row < k * I && lane == 0) d.h[row] = silu(gs) * us;
  }
}

// Wave per CPW output columns: the k + 1 weight rows of the columns are
// loaded together (I / 8 chunks each), and each h value read serves them all.
template <int KT>  // k <= KT
__global__ __launch_bounds__(256) void decode_down_kernel(const uint16_t* __restrict__ w_down,
                                                          const uint16_t* __restrict__ ws_down, int H, int k, int I,
                                                          int I_s, DecodeWs d, uint16_t* __restrict__ y) {
  constexpr int CPW = 1;
  const int lane = threadIdx.x & 63;
  const int c0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * CPW;
  if (c0 >= H) return;
  // ids and weights: KT entries read with 16-byte loads (their workspace
  // slots hold 64 entries), entries past k unused
  int ids[KT];
  float wsel[KT];
#pragma unroll
  for (int q = 0; q < KT / 4; ++q) {
    const int4 iv = reinterpret_cast<const int4*>(d.ids)[q];
    const float4 wv = reinterpret_cast<const float4*>(d.w)[q];
    ids[4 * q] = iv.x, ids[4 * q + 1] = iv.y, ids[4 * q + 2] = iv.z, ids[4 * q + 3] = iv.w;
    wsel[4 * q] = wv.x, wsel[4 * q + 1] = wv.y, wsel[4 * q + 2] = wv.z, wsel[4 * q + 3] = wv.w;
  }
#pragma unroll
  for (int j = 0; j < KT; ++j) ids[j] = j < k ? ids[j] : 0;  // keep unused rows in range
  float part[CPW][KT + 1];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int j = 0; j <= KT; ++j) part[c][j] = 0.0f;
  auto accum = [&](float& acc, const u32x4& wv, const float* hv) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc += hv[2 * q] * bf16_to_f32((uint16_t)(wv[q] & 0xffff));
      acc += hv[2 * q + 1] * bf16_to_f32((uint16_t)(wv[q] >> 16));
    }
  };
  // Per step of 64 chunks: the loads that do not depend on the routing (the
  // shared row, h_s and every h_j) are issued first, then the k routed rows.
  const int nI = I / 8, nS = I_s > 0 ? I_s / 8 : 0;
  const int nmax = nI > nS ? nI : nS;
  for (int base = 0; base < nmax; base += 64) {
    const int ch = base + lane;
    const bool okS = ch < nS, okI = ch < nI;
    u32x4 wsv[CPW];
    float4 hs0 = {}, hs1 = {};
    if (okS) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) wsv[c] = reinterpret_cast<const u32x4*>(ws_down + (size_t)(c0 + c) * I_s)[ch];
      const float4* hp = reinterpret_cast<const float4*>(d.hs + ch * 8);
      hs0 = hp[0];
      hs1 = hp[1];
    }
    float4 h0[KT], h1[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j)
      if (j < k && okI) {
        const float4* hp = reinterpret_cast<const float4*>(d.h + (size_t)j * I + ch * 8);
        h0[j] = hp[0];
        h1[j] = hp[1];
      }
    u32x4 wv[KT][CPW];
#pragma unroll
    for (int j = 0; j < KT; ++j)
      if (j < k && okI)
#pragma unroll
        for (int c = 0; c < CPW; ++c)
          wv[j][c] = reinterpret_cast<const u32x4*>(w_down + ((size_t)ids[j] * H + c0 + c) * I)[ch];
    if (okS) {
      const float hv[8] = {hs0.x, hs0.y, hs0.z, hs0.w, hs1.x, hs1.y, hs1.z, hs1.w};
#pragma unroll
      for (int c = 0; c < CPW; ++c) accum(part[c][KT], wsv[c], hv);
    }
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      if (j < k && okI) {
        const float hv[8] = {h0[j].x, h0[j].y, h0[j].z, h0[j].w, h1[j].x, h1[j].y, h1[j].z, h1[j].w};
#pragma unroll
        for (int c = 0; c < CPW; ++c) accum(part[c][j], wv[j][c], hv);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    float yv = 0.0f;
#pragma unroll
    for (int j = 0; j < KT; ++j)
      if (j < k) yv += wsel[j] * wave_sum(part[c][j]);  // rank order
    if (I_s > 0) yv += d.s[0] * wave_sum(part[c][KT]);
    if (lane == 0) y[c0 + c] = f32_to_bf16(yv);
  }
}

}  // namespace

size_t decode_ids_offset(int E) { return align256((size_t)E * 4); }  // after the logits, as carve() lays them out

size_t decode_workspace_size(int H, int E, int k, int I, int I_s) {
  (void)H;
  return align256((size_t)E * 4) + 2 * 256 + 256 + align256((size_t)(I_s > 0 ? I_s : 1) * 4) +
         align256((size_t)k * I * 4);
}

hipError_t launch_decode(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_gate,
                         const uint16_t* w_up, const uint16_t* w_down, const uint16_t* ws_gate,
                         const uint16_t* ws_up, const uint16_t* ws_down, const uint16_t* w_sg, int H, int E,
                         int k, int I, int I_s, uint16_t* y, void* ws, hipStream_t st) {
  DecodeWs d = carve(ws, H, E, k, I, I_s);
  const int rows1 = E + (I_s > 0 ? 1 : 0);
  hipLaunchKernelGGL(decode_router_kernel, dim3((rows1 + 3) / 4), dim3(256), 0, st, x, w_router, bias,
                     I_s > 0 ? w_sg : nullptr, H, E, d);
  // 4 waves per workgroup, one routed row pair per wave; waves 1..3 also take the shared rows
  hipLaunchKernelGGL(decode_topk_gate_up_kernel, dim3((k * I + 3) / 4), dim3(256), 0, st, x, w_gate, w_up, ws_gate,
                     ws_up, H, E, k, I, I_s, d);
  // 4 waves per workgroup, one output column per wave (H is a multiple of 256)
  if (k <= 8)
    hipLaunchKernelGGL(decode_down_kernel<8>, dim3((H + 3) / 4), dim3(256), 0, st, w_down, ws_down, H, k, I, I_s, d,
                       y);
  else
    hipLaunchKernelGGL(decode_down_kernel<kMaxK>, dim3((H + 3) / 4), dim3(256), 0, st, w_down, ws_down, H, k, I, I_s,
                       d, y);
  return hipGetLastError();
}

}  // namespace moe
