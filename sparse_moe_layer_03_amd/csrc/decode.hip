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
//
// The expert matrices may be FP8 E4M3 codes with one fp32 scale per output
// row, or 4-bit weights with an fp16 scale per group of 32 (kongchang.com
// "GFX1151 engine", section on the two weight formats: FP8-quantised and
// 4-bit GGUF weights): then every weight load moves 8 or 4 bytes for the same
// 8 values, the codes are converted to fp32 in registers, and the FP8 row's
// scale multiplies the row's dot product (a 4-bit group's scale multiplies
// its weights as they are converted).
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
  const WsSections w = decode_sections(H, E, k, I, I_s);
  char* p = static_cast<char*>(base);
  DecodeWs d;
  d.logits = reinterpret_cast<float*>(p + w.off[0]);
  d.ids = reinterpret_cast<int32_t*>(p + w.off[1]);  // 256-byte slot: 64 entries, read 16 at a time
  d.w = reinterpret_cast<float*>(p + w.off[2]);
  d.s = reinterpret_cast<float*>(p + w.off[3]);
  d.hs = reinterpret_cast<float*>(p + w.off[4]);
  d.h = reinterpret_cast<float*>(p + w.off[5]);
  return d;
}

// Dot product of 8 bf16 x values with 8 weights (bf16, E4M3 codes, or 4-bit
// weights times their group scale).
template <class W>
__device__ __forceinline__ float dot8(u32x4 a, const W& b) {
  float f[8];
  chunk_to_f32(b, f);
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s += bf16_to_f32((uint16_t)(a[q] & 0xffff)) * f[2 * q];
    s += bf16_to_f32((uint16_t)(a[q] >> 16)) * f[2 * q + 1];
  }
  return s;
}

// Dot products of x with one or two weight rows of length H (r1 used when
// two; FP8 rows unscaled).  x comes from LDS (sx) when given, else straight
// from global memory; every load of a group of 4 chunks per lane (x's
// included) is issued before the arithmetic.
template <int F>
__device__ __forceinline__ void row_dots(const u32x4* sx, const uint16_t* xg, const WRow<F>& r0, const WRow<F>& r1,
                                         bool two, int H, int lane, float& d0, float& d1) {
  typedef wchunk_t<F> WC;
  const int nch = H / 8;
  d0 = 0.0f;
  d1 = 0.0f;
  for (int base = 0; base < nch; base += 256) {
    WC a[4], b[4];
    u32x4 xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c = base + q * 64 + lane;
      if (c < nch) {
        a[q] = r0[c];
        if (two) b[q] = r1[c];
        xv[q] = sx ? sx[c] : reinterpret_cast<const u32x4*>(xg)[c];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c = base + q * 64 + lane;
      if (c < nch) {
        d0 += dot8(xv[q], a[q]);
        if (two) d1 += dot8(xv[q], b[q]);
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
  // the bias is loaded before the dot product, so its latency hides under it
  const float bv = (bias && row < E) ? bias[row] : 0.0f;
  float d0, d1;
  if (row < E) {
    const WRow<W_BF16> r = wrow<W_BF16>(wr, nullptr, (size_t)row, H);
    row_dots<W_BF16>(nullptr, x, r, r, false, H, lane, d0, d1);
    if (lane == 0) {
      float v = d0 + bv;
      if (v == 0.0f) v = 0.0f;
      d.logits[row] = v;
    }
  } else if (row == E && w_sg) {
    const WRow<W_BF16> r = wrow<W_BF16>(w_sg, nullptr, 0, H);
    row_dots<W_BF16>(nullptr, x, r, r, false, H, lane, d0, d1);
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
#ifndef MOE_DECODE_GU_WAVES
#define MOE_DECODE_GU_WAVES 4
#endif
constexpr int DGW = MOE_DECODE_GU_WAVES;  // waves per workgroup of the gate/up launch
template <int F>
__global__ __launch_bounds__(64 * DGW) void decode_topk_gate_up_kernel(const uint16_t* __restrict__ x,
                                                                       ExpertWeights W, int H, int E, int k, int I,
                                                                       int I_s, DecodeWs d) {
  typedef wchunk_t<F> WC;
  constexpr bool RS = F == W_FP8;  // one scale per row, applied to the row's dot product
  __shared__ u32x4 sx[1024];
  __shared__ int sel_e[kMaxK];
  __shared__ float sel_w[kMaxK];
  for (int c = threadIdx.x; c < H / 8; c += 64 * DGW) sx[c] = reinterpret_cast<const u32x4*>(x)[c];
  const int wave = threadIdx.x >> 6;
  if (wave == 0) {
    block_topk(d.logits, E, k, sel_e, sel_w);
  } else {
    for (int i = blockIdx.x * (DGW - 1) + wave - 1; i < I_s; i += (DGW - 1) * gridDim.x) {
      const float scg = RS ? W.ssc_gate[i] : 1.0f, scu = RS ? W.ssc_up[i] : 1.0f;  // issued with the row loads
      float g, u;
      row_dots<F>(nullptr, x, wrow<F>(W.s_gate, W.gss_gate, (size_t)i, H), wrow<F>(W.s_up, W.gss_up, (size_t)i, H),
                  true, H, threadIdx.x & 63, g, u);
      if (RS) {
        g *= scg;
        u *= scu;
      }
      if ((threadIdx.x & 63) == 0) d.hs[i] = silu(g) * u;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x < k) {
    d.ids[threadIdx.x] = sel_e[threadIdx.x];
    d.w[threadIdx.x] = sel_w[threadIdx.x];
  }
  // wave w of workgroup b takes row pair b*DGW + w; its loads are all issued
  // before any reduction
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * DGW + (threadIdx.x >> 6);
  const int nch = H / 8;  // chunks per weight row; lane handles chunks lane + 64 c
  const int rr = row < k * I ? row : 0;
  const size_t rix = (size_t)sel_e[rr / I] * I + rr % I;  // row of W_gate / W_up
  const WRow<F> gp = wrow<F>(W.gate, W.gs_gate, rix, H);
  const WRow<F> up = wrow<F>(W.up, W.gs_up, rix, H);
  const float scg = RS ? W.sc_gate[rix] : 1.0f, scu = RS ? W.sc_up[rix] : 1.0f;  // in flight with the rows
  float g = 0.0f, u = 0.0f;
  for (int c0 = 0; c0 < nch; c0 += 64 * 4) {
    WC a[4], b[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch = c0 + lane + 64 * c;
      if (ch < nch) {
        a[c] = gp[ch];
        b[c] = up[ch];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch = c0 + lane + 64 * c;
      if (ch < nch) {
        const u32x4 xv = sx[ch];
        g += dot8(xv, a[c]);
        u += dot8(xv, b[c]);
      }
    }
  }
  float gs = wave_sum(g), us = wave_sum(u);
  if (RS) {
    gs *= scg;
    us *= scu;
  }
  if (row < k * I && lane == 0) d.h[row] = silu(gs) * us;
}

// Wave per CPW output columns: the k + 1 weight rows of each column are
// loaded together (I / 8 chunks each), and each h value read serves them all.
#ifndef MOE_DECODE_DOWN_COLS
#define MOE_DECODE_DOWN_COLS 1
#endif
constexpr int CPW = MOE_DECODE_DOWN_COLS;
template <int KT, int F>  // k <= KT
__global__ __launch_bounds__(256) void decode_down_kernel(ExpertWeights W, int H, int k, int I, int I_s, DecodeWs d,
                                                          uint16_t* __restrict__ y) {
  typedef wchunk_t<F> WC;
  constexpr bool RS = F == W_FP8;
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
  // row scales, loaded with the first weight rows rather than after the sums
  float scd[CPW][KT], scs[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
#pragma unroll
    for (int j = 0; j < KT; ++j) scd[c][j] = RS ? W.sc_down[(size_t)ids[j] * H + c0 + c] : 1.0f;
    scs[c] = (RS && I_s > 0) ? W.ssc_down[c0 + c] : 1.0f;
  }
  WRow<F> rows[CPW][KT], srow[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
#pragma unroll
    for (int j = 0; j < KT; ++j) rows[c][j] = wrow<F>(W.down, W.gs_down, (size_t)ids[j] * H + c0 + c, I);
    srow[c] = wrow<F>(W.s_down, W.gss_down, (size_t)(c0 + c), I_s);
  }
  float part[CPW][KT + 1];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int j = 0; j <= KT; ++j) part[c][j] = 0.0f;
  auto accum = [&](float& acc, const WC& wv, const float* hv) {
    float f[8];
    chunk_to_f32(wv, f);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += hv[q] * f[q];
  };
  // Per step of 64 chunks: the loads that do not depend on the routing (the
  // shared rows, h_s and every h_j) are issued first, then the routed rows.
  const int nI = I / 8, nS = I_s > 0 ? I_s / 8 : 0;
  const int nmax = nI > nS ? nI : nS;
  for (int base = 0; base < nmax; base += 64) {
    const int ch = base + lane;
    const bool okS = ch < nS, okI = ch < nI;
    WC wsv[CPW];
    float4 hs0 = {}, hs1 = {};
    if (okS) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) wsv[c] = srow[c][ch];
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
    WC wv[KT][CPW];
#pragma unroll
    for (int j = 0; j < KT; ++j)
      if (j < k && okI)
#pragma unroll
        for (int c = 0; c < CPW; ++c) wv[j][c] = rows[c][j][ch];
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
      if (j < k) {
        float oj = wave_sum(part[c][j]);
        if (RS) oj *= scd[c][j];
        yv += wsel[j] * oj;  // rank order
      }
    if (I_s > 0) {
      float os = wave_sum(part[c][KT]);
      if (RS) os *= scs[c];
      yv += d.s[0] * os;
    }
    if (lane == 0) y[c0 + c] = f32_to_bf16(yv);
  }
}

// The same with one column per wave, I and I_s at most 512 (one chunk per
// lane) and k * I at most kDownStage floats: the k hidden rows are staged in
// LDS once per workgroup (after the wave's weight loads are issued) instead of
// being read from L2 by every wave.
constexpr int kDownStage = 4096;
template <int KT, int F>  // k <= KT
__global__ __launch_bounds__(256) void decode_down_staged_kernel(ExpertWeights W, int H, int k, int I, int I_s,
                                                                 DecodeWs d, uint16_t* __restrict__ y) {
  typedef wchunk_t<F> WC;
  constexpr bool RS = F == W_FP8;
  __shared__ float4 shh[kDownStage / 4];
  const int lane = threadIdx.x & 63;
  const int c0 = blockIdx.x * 4 + (threadIdx.x >> 6);  // < H: the grid covers H exactly
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
  float scd[KT], scs = 1.0f;
#pragma unroll
  for (int j = 0; j < KT; ++j) scd[j] = RS ? W.sc_down[(size_t)ids[j] * H + c0] : 1.0f;
  if (RS && I_s > 0) scs = W.ssc_down[c0];
  const int ch = lane;  // the lane's chunk of 8 reduction values
  const bool okS = ch < I_s / 8, okI = ch < I / 8;
  WC wsv, wv[KT];
  float4 hs0 = {}, hs1 = {};
  if (okS) {
    wsv = wrow<F>(W.s_down, W.gss_down, (size_t)c0, I_s)[ch];
    const float4* hp = reinterpret_cast<const float4*>(d.hs + ch * 8);
    hs0 = hp[0];
    hs1 = hp[1];
  }
#pragma unroll
  for (int j = 0; j < KT; ++j)
    if (j < k && okI) wv[j] = wrow<F>(W.down, W.gs_down, (size_t)ids[j] * H + c0, I)[ch];
  for (int i = threadIdx.x; i < k * I / 4; i += 256) shh[i] = reinterpret_cast<const float4*>(d.h)[i];
  __syncthreads();
  auto accum = [&](float& acc, const WC& w, const float* hv) {
    float f[8];
    chunk_to_f32(w, f);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += hv[q] * f[q];
  };
  float part[KT + 1];
#pragma unroll
  for (int j = 0; j <= KT; ++j) part[j] = 0.0f;
  if (okS) {
    const float hv[8] = {hs0.x, hs0.y, hs0.z, hs0.w, hs1.x, hs1.y, hs1.z, hs1.w};
    accum(part[KT], wsv, hv);
  }
#pragma unroll
  for (int j = 0; j < KT; ++j) {
    if (j < k && okI) {
      const float4 h0 = shh[(j * I + ch * 8) / 4], h1 = shh[(j * I + ch * 8) / 4 + 1];
      const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
      accum(part[j], wv[j], hv);
    }
  }
  float yv = 0.0f;
#pragma unroll
  for (int j = 0; j < KT; ++j)
    if (j < k) {
      float oj = wave_sum(part[j]);
      if (RS) oj *= scd[j];
      yv += wsel[j] * oj;  // rank order
    }
  if (I_s > 0) {
    float os = wave_sum(part[KT]);
    if (RS) os *= scs;
    yv += d.s[0] * os;
  }
  if (lane == 0) y[c0] = f32_to_bf16(yv);
}

__global__ __launch_bounds__(256) void e4m3_to_f32_kernel(const uint8_t* __restrict__ codes, float* __restrict__ out,
                                                          int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  if (i + 8 <= n) {
    float f[8];
    chunk_to_f32(*reinterpret_cast<const u32x2*>(codes + i), f);
#pragma unroll
    for (int q = 0; q < 8; ++q) out[i + q] = f[q];
  } else {
    for (int64_t j = i; j < n; ++j) {  // tail: one code at a time, in the low byte
      float f[8];
      chunk_to_f32(u32x2{(uint32_t)codes[j], 0u}, f);
      out[j] = f[0];
    }
  }
}

template <int F>
void launch_decode_t(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg,
                     const ExpertWeights& W, int H, int E, int k, int I, int I_s, uint16_t* y, DecodeWs d,
                     hipStream_t st) {
  const int rows1 = E + (I_s > 0 ? 1 : 0);
  hipLaunchKernelGGL(decode_router_kernel, dim3((rows1 + 3) / 4), dim3(256), 0, st, x, w_router, bias,
                     I_s > 0 ? w_sg : nullptr, H, E, d);
  // DGW waves per workgroup, one routed row pair per wave; waves 1.. also take the shared rows
  hipLaunchKernelGGL(decode_topk_gate_up_kernel<F>, dim3((k * I + DGW - 1) / DGW), dim3(64 * DGW), 0, st, x, W, H, E,
                     k, I, I_s, d);
  // 4 waves per workgroup, CPW output columns per wave (H is a multiple of 256)
  const dim3 g_dn((H / CPW + 3) / 4);
#ifndef MOE_DECODE_DOWN_STAGE_H
#define MOE_DECODE_DOWN_STAGE_H 1
#endif
  // (not for 4-bit weights: staged, their decode took 19.5 us against 17.4 us)
  if (MOE_DECODE_DOWN_STAGE_H && F != W_Q4 && CPW == 1 && I <= 512 && I_s <= 512 && k * I <= kDownStage) {
    if (k <= 8)
      hipLaunchKernelGGL((decode_down_staged_kernel<8, F>), g_dn, dim3(256), 0, st, W, H, k, I, I_s, d, y);
    else
      hipLaunchKernelGGL((decode_down_staged_kernel<kMaxK, F>), g_dn, dim3(256), 0, st, W, H, k, I, I_s, d, y);
    return;
  }
  if (k <= 8)
    hipLaunchKernelGGL((decode_down_kernel<8, F>), g_dn, dim3(256), 0, st, W, H, k, I, I_s, d, y);
  else
    hipLaunchKernelGGL((decode_down_kernel<kMaxK, F>), g_dn, dim3(256), 0, st, W, H, k, I, I_s, d, y);
}

}  // namespace

// logits [E], ids and w (256-byte slots: the down launch reads 16 entries at a time), s, h_s [I_s],
// h [k, I] (fp32)
WsSections decode_sections(int H, int E, int k, int I, int I_s) {
  (void)H;
  WsSections w;
  w.take((size_t)E * 4);
  w.take(256);
  w.take(256);
  w.take(4);
  w.take((size_t)(I_s > 0 ? I_s : 1) * 4);
  w.take((size_t)k * I * 4);
  return w;
}

size_t decode_ids_offset(int H, int E, int k, int I, int I_s) { return decode_sections(H, E, k, I, I_s).off[1]; }

size_t decode_workspace_size(int H, int E, int k, int I, int I_s) { return decode_sections(H, E, k, I, I_s).total; }

hipError_t launch_decode(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg,
                         const ExpertWeights& W, int H, int E, int k, int I, int I_s, uint16_t* y, void* ws,
                         hipStream_t st) {
  DecodeWs d = carve(ws, H, E, k, I, I_s);
  if (W.fmt == W_FP8)
    launch_decode_t<W_FP8>(x, w_router, bias, w_sg, W, H, E, k, I, I_s, y, d, st);
  else if (W.fmt == W_Q4)
    launch_decode_t<W_Q4>(x, w_router, bias, w_sg, W, H, E, k, I, I_s, y, d, st);
  else
    launch_decode_t<W_BF16>(x, w_router, bias, w_sg, W, H, E, k, I, I_s, y, d, st);
  return hipGetLastError();
}

hipError_t launch_e4m3_to_f32(const uint8_t* codes, float* out, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 2047) / 2048;
  hipLaunchKernelGGL(e4m3_to_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, codes, out, n);
  return hipGetLastError();
}

}  // namespace moe
