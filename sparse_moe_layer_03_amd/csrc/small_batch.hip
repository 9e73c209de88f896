// Small-batch path of the sparse MoE layer (2 <= T <= 32 tokens) on gfx950.
//
// With a few tokens per step (several requests decoded together, or a short
// verification chunk) most experts receive one or two rows, so the layer is
// bound by reading the touched experts' weights, as at T = 1 (guanjiawei.ai
// "AIMA AMD395 Qwen3.6-35B-A3B", data path: only the selected experts are
// computed; kongchang.com "GFX1151 engine", MoE kernel section: sparse routing
// changes the memory access pattern).  Each weight row of a touched expert is
// read once, by one wavefront, with 16-byte loads, and applied to every token
// routed to that expert:
//   S1 router: wave per router row (and the shared gate), all T tokens
//   S2 select: one workgroup: top-k and weights of every token (the prefill
//      rule), then the plan: the touched experts in ascending order and, per
//      expert, its assignments a = t*k + j in ascending order
//   S3 gate/up: (touched expert, block of 8 intermediate rows) per workgroup,
//      the shared expert as one more expert over all T tokens:
//      h[a][i] = silu(g) * u in fp32
//   S4 down: (touched expert, block of 64 output columns) per workgroup:
//      o[a][c] = h[a] . W_down[e][c] in fp32 (shared: o_s[t][c])
//   S5 combine: y[t][c] = sum_j w[t][j] o[t*k+j][c] (j ascending) + s[t] o_s[t][c]
// With FP8 E4M3 expert weights (one fp32 scale per output row) or 4-bit
// weights (an fp16 scale per group of 32) the weight loads move 8 or 4 bytes
// per 8 values and the codes are converted in registers; the FP8 row's scale
// multiplies each dot product, a 4-bit group's scale its converted weights.
#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {
namespace {

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Record of one touched expert (slot u, ascending expert order): expert,
// offset of its assignments in asg, their count, then its first TBR
// assignments, so that a workgroup learns its expert, its tokens and its
// rows in one load round trip.
constexpr int TBR = 16, kRec0 = 4, kRecInts = 4 + TBR;

struct SmallWs {
  float* logits;  // [T, E]
  float* s;       // [T]
  int32_t* ids;   // [T, k]
  float* w;       // [T, k]
  int32_t* plan;  // [0] touched experts n_u; from kRec0, a record of kRecInts ints per expert slot
  int32_t* asg;   // [T * k] assignments grouped by expert
  float* h;       // [T * k, I]
  float* hs;      // [T, I_s]
  float* o;       // [T * k, H]
  float* os;      // [T, H]
};

SmallWs carve_small(void* base, int T, int H, int E, int k, int I, int I_s) {
  const WsSections w = small_batch_sections(T, H, E, k, I, I_s);
  char* p = static_cast<char*>(base);
  SmallWs d;
  d.logits = reinterpret_cast<float*>(p + w.off[0]);
  d.s = reinterpret_cast<float*>(p + w.off[1]);
  d.ids = reinterpret_cast<int32_t*>(p + w.off[2]);
  d.w = reinterpret_cast<float*>(p + w.off[3]);
  d.plan = reinterpret_cast<int32_t*>(p + w.off[4]);
  d.asg = reinterpret_cast<int32_t*>(p + w.off[5]);
  d.h = reinterpret_cast<float*>(p + w.off[6]);
  d.hs = reinterpret_cast<float*>(p + w.off[7]);
  d.o = reinterpret_cast<float*>(p + w.off[8]);
  d.os = reinterpret_cast<float*>(p + w.off[9]);
  return d;
}

// 8 bf16 x values . 8 weights (bf16, or E4M3 codes), ascending.
template <class W>
__device__ __forceinline__ float sb_dot8(const u32x4& a, const W& b) {
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

// 8 fp32 h values . 8 weights (bf16, or E4M3 codes).
template <class W>
__device__ __forceinline__ float dot8_f32w(const float4& h0, const float4& h1, const W& wv) {
  float f[8];
  chunk_to_f32(wv, f);
  return h0.x * f[0] + h0.y * f[1] + h0.z * f[2] + h0.w * f[3] + h1.x * f[4] + h1.y * f[5] + h1.z * f[6] +
         h1.w * f[7];
}

constexpr int TB = 16;  // tokens (or assignments) staged in LDS at a time

// One direct-to-LDS load: 16 bytes per lane from src into LDS at
// lds_base + 16 * lane (lds_base wave-uniform, in M0).  Inline assembly so
// that the compiler does not order later LDS reads behind it; the callers
// wait for it (s_waitcnt vmcnt(0)) before the barrier that publishes the data.
__device__ __forceinline__ void sb_dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ void sb_wait_vm0() { __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8)); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Stage rows t < n (n <= NTOK) of x, chosen by row(t) (wave-uniform), chunks
// [base, base + 256) of H, into LDS sx[t][256]: one 1 KB load instruction per
// (token, quarter), all in flight together, then one wait and a barrier.
// Chunks past H read the row's last chunk (the weight side is zeroed there);
// rows t >= n are not loaded (their slots are never read).
template <int NTOK = TB, class RowOf>
__device__ __forceinline__ void stage_x(u32x4* sx, const uint16_t* __restrict__ x, int H, int base_ch, int n,
                                        RowOf row) {
  const int nch = H / 8, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t sbase = lds_addr(sx);
  for (int ins = wave; ins < NTOK * 4; ins += nw) {  // instruction ins: token ins / 4, quarter ins % 4
    const int t = ins >> 2;
    if (t < n) {
      const int c = min(base_ch + (ins & 3) * 64 + lane, nch - 1);
      sb_dma16(x + (size_t)row(t) * H + (size_t)c * 8, sbase + (uint32_t)ins * 1024u);
    }
  }
  sb_wait_vm0();
  __syncthreads();
}

// S1: workgroup (4 router rows, token chunk blockIdx.y of 16 tokens); a wave
// per row (row E is the shared gate, s = sigmoid(x . w_sg)), the tokens'
// x rows staged in LDS 2048 columns at a time.
__global__ __launch_bounds__(256) void sb_router_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                        const float* __restrict__ bias,
                                                        const uint16_t* __restrict__ w_sg, int T, int H, int E,
                                                        SmallWs d) {
  __shared__ u32x4 sx[TB * 256];
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool gate = (r == E);
  const bool live = r < E || (gate && w_sg);
  const uint16_t* row = gate ? w_sg : wr + (size_t)min(r, E - 1) * H;
  // the bias is loaded before the dot products, so its latency hides under them
  const float bv = (bias && r < E) ? bias[r] : 0.0f;
  const int nch = H / 8;
  const int t0 = blockIdx.y * TB;
  const int nt = min(TB, T - t0);
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.0f;
  for (int base = 0; base < nch; base += 256) {
    u32x4 wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wv[q] = reinterpret_cast<const u32x4*>(row)[min(base + q * 64 + lane, nch - 1)];
    __syncthreads();  // the previous block's LDS reads are done
    stage_x(sx, x, H, base, nt, [&](int t) { return t0 + t; });
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (base + q * 64 + lane >= nch) wv[q] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (t < nt) {  // uniform
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t] += sb_dot8(sx[t * 256 + q * 64 + lane], wv[q]);
      }
    }
  }
  if (live) {
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (t < nt) {
        const float v = wave_sum(acc[t]);
        if (lane == 0) {
          if (gate) {
            d.s[t0 + t] = 1.0f / (1.0f + expf(-v));
          } else {
            float lv = v + bv;
            if (lv == 0.0f) lv = 0.0f;
            d.logits[(size_t)(t0 + t) * E + r] = lv;
          }
        }
      }
    }
  }
}

// Exclusive prefix sum of v over all threads of the workgroup (every thread
// must call it: it holds two workgroup barriers); total returned in tot.
// Wave scans by shuffles, then the wave totals through LDS (sw: one int per
// wave).
__device__ __forceinline__ int block_scan(int v, int* sw, int& tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == 63) sw[wave] = incl;
  __syncthreads();
  int off = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    off += (w < wave) ? sw[w] : 0;
    all += sw[w];
  }
  tot = all;
  __syncthreads();
  return off + incl - v;
}

// S2: one workgroup of 1024 threads.  Waves select the top k of 4 tokens at a
// time; then the plan: per-expert counts, the touched experts in ascending
// order (a prefix scan over the experts), and every assignment placed at its
// expert's offset plus its rank among that expert's assignments (ascending a).
__global__ __launch_bounds__(1024) void sb_select_kernel(int T, int E, int k, SmallWs d) {
  __shared__ int sid[kSmallMaxT * kMaxK];
  __shared__ int scnt[kMaxE], soff[kMaxE], suid[kMaxE], sw[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int t = wave; t < T; t += 16) {  // a wave per token: short selection chains
    float v[4];
    bool valid[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      valid[q] = e < E;
      v[q] = d.logits[(size_t)t * E + min(e, E - 1)];
    }
    int se;
    float sv, w;
    wave_topk_weights(v, valid, k, lane, se, sv, w);
    if (lane < k) {
      sid[t * k + lane] = se;
      d.ids[t * k + lane] = se;
      d.w[t * k + lane] = w;
    }
  }
  if (tid < kMaxE) scnt[tid] = 0;
  __syncthreads();
  const int n = T * k;
  if (tid < n) atomicAdd(&scnt[sid[tid]], 1);  // integer counts in LDS: order-free
  __syncthreads();
  {
    // every thread takes part in the scans (threads past E count nothing)
    const int c = tid < E ? scnt[tid] : 0;
    int tot_a, tot_u;
    const int off = block_scan(c, sw, tot_a);
    const int uid = block_scan(c > 0 ? 1 : 0, sw, tot_u);
    if (tid < E) soff[tid] = off;
    if (tid < E) suid[tid] = uid;
    if (c > 0) {
      int32_t* rec = d.plan + kRec0 + uid * kRecInts;
      rec[0] = tid;
      rec[1] = off;
      rec[2] = c;
    }
    if (tid == 0) d.plan[0] = tot_u;
  }
  __syncthreads();
  if (tid < n) {
    const int e = sid[tid];
    int rank = 0;
    for (int a = 0; a < tid; ++a) rank += (sid[a] == e) ? 1 : 0;
    d.asg[soff[e] + rank] = tid;
    if (rank < TBR) d.plan[kRec0 + suid[e] * kRecInts + 4 + rank] = tid;
  }
}

// S3: workgroup (expert slot u = blockIdx.y, intermediate rows GR blockIdx.x ..
// +GR-1): a wave per GP gate/up row pairs (GP * 8 KB of weights in flight per
// wave), every token routed to the expert, GT at a time, with their x rows
// staged in LDS (2048 columns at a time).  Slot u == n_u is the shared expert
// over all T tokens when I_s > 0.
// Tokens staged per pass (8: 32 KB of LDS, so several workgroups share a CU
// and more weight loads are in flight; 16 was 11% slower with FP8 weights at
// 8 and 32 tokens and the same with BF16).
#ifndef SB_GATE_UP_TOKENS
#define SB_GATE_UP_TOKENS 8
#endif
// Gate/up row pairs per wave (1: 4 pairs, 32 KB of weights, per workgroup;
// 2 pairs per wave were 8% slower at 8..32 tokens: fewer, larger workgroups).
#ifndef SB_GATE_UP_ROW_PAIRS
#define SB_GATE_UP_ROW_PAIRS 1
#endif
constexpr int GP = SB_GATE_UP_ROW_PAIRS, GR = 4 * GP, GT = SB_GATE_UP_TOKENS;
template <int F>
__global__ __launch_bounds__(256) void sb_gate_up_kernel(const uint16_t* __restrict__ x, ExpertWeights W, int T,
                                                         int H, int E, int k, int I, int I_s, SmallWs d) {
  typedef wchunk_t<F> WC;
  constexpr bool Q = F == W_FP8;  // one scale per row, applied to the row's dot products
  __shared__ u32x4 sx[GT * 256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nu = d.plan[0];
  const int u = blockIdx.y;
  const bool shared = (u == nu);
  if (u > nu || (shared && I_s == 0)) return;  // uniform over the workgroup
  const int nrow = shared ? I_s : I;
  if (blockIdx.x * GR >= nrow) return;
  const int i0 = blockIdx.x * GR + wave * GP;  // < nrow: nrow is a multiple of GR
  const int32_t* rec = d.plan + kRec0 + (shared ? 0 : u) * kRecInts;
  const int e = shared ? 0 : rec[0], off = shared ? 0 : rec[1], cnt = shared ? T : rec[2];
  // assignment q of the expert (shared expert: token q)
  auto asg_at = [&](int q) { return shared ? q : (q < TBR ? rec[4 + q] : d.asg[off + q]); };
  const size_t r0 = shared ? (size_t)i0 : (size_t)e * I + i0;  // first of the wave's GP rows
  WRow<F> gr[GP], ur[GP];
#pragma unroll
  for (int p = 0; p < GP; ++p) {
    gr[p] = wrow<F>(shared ? W.s_gate : W.gate, shared ? W.gss_gate : W.gs_gate, r0 + p, H);
    ur[p] = wrow<F>(shared ? W.s_up : W.up, shared ? W.gss_up : W.gs_up, r0 + p, H);
  }
  float scg[GP], scu[GP];
#pragma unroll
  for (int p = 0; p < GP; ++p) {
    scg[p] = Q ? (shared ? W.ssc_gate : W.sc_gate)[r0 + p] : 1.0f;
    scu[p] = Q ? (shared ? W.ssc_up : W.sc_up)[r0 + p] : 1.0f;
  }
  const int nch = H / 8;
  for (int q0 = 0; q0 < cnt; q0 += GT) {
    const int nt = min(GT, cnt - q0);
    float ag[GP][GT], au[GP][GT];
#pragma unroll
    for (int p = 0; p < GP; ++p)
#pragma unroll
      for (int t = 0; t < GT; ++t) ag[p][t] = au[p][t] = 0.0f;
    for (int base = 0; base < nch; base += 256) {
      WC gv[GP][4], uv[GP][4];
#pragma unroll
      for (int p = 0; p < GP; ++p)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const int c = min(base + c4 * 64 + lane, nch - 1);
          gv[p][c4] = gr[p][c];
          uv[p][c4] = ur[p][c];
        }
      __syncthreads();
      stage_x<GT>(sx, x, H, base, nt, [&](int t) { return shared ? q0 + t : asg_at(q0 + t) / k; });
#pragma unroll
      for (int p = 0; p < GP; ++p)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
          if (base + c4 * 64 + lane >= nch) gv[p][c4] = uv[p][c4] = WC{};
#pragma unroll
      for (int t = 0; t < GT; ++t) {
        if (t < nt) {  // uniform
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const u32x4 xv = sx[t * 256 + c4 * 64 + lane];
#pragma unroll
            for (int p = 0; p < GP; ++p) {
              ag[p][t] += sb_dot8(xv, gv[p][c4]);
              au[p][t] += sb_dot8(xv, uv[p][c4]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < GT; ++t) {
      if (t < nt) {
#pragma unroll
        for (int p = 0; p < GP; ++p) {
          float gs = wave_sum(ag[p][t]), us = wave_sum(au[p][t]);
          if (Q) {
            gs *= scg[p];
            us *= scu[p];
          }
          if (lane == 0) {
            if (shared)
              d.hs[(size_t)(q0 + t) * I_s + i0 + p] = silu(gs) * us;
            else
              d.h[(size_t)asg_at(q0 + t) * I + i0 + p] = silu(gs) * us;
          }
        }
      }
    }
  }
}

// S4: workgroup (expert slot u = blockIdx.y, output columns 4*DCW blockIdx.x ..
// +4*DCW-1): a wave per DCW columns.  Lane l takes column c0 + l / LPC and
// the reduction chunks j * LPC + l % LPC (adjacent lanes read contiguous
// bytes of a row); the LPC partial sums of a column meet in DPP steps.
// h rows of the expert's assignments (fp32) are staged in LDS, DT at a time.
// h rows staged per pass (8: 16 KB of LDS), as for gate/up.
#ifndef SB_DOWN_TOKENS
#define SB_DOWN_TOKENS 8
#endif
constexpr int DT = SB_DOWN_TOKENS;  // h rows staged at a time
// Lanes per output column (4, 8 or 16): a wave takes 64 / LPC columns, a lane
// 64 / LPC of the 64 chunks of a 512-value reduction block.
#ifndef SB_DOWN_LANES_PER_COL
#define SB_DOWN_LANES_PER_COL 8
#endif
constexpr int LPC = SB_DOWN_LANES_PER_COL, DCW = 64 / LPC, DNCH = 64 / LPC;
static_assert(LPC == 4 || LPC == 8 || LPC == 16, "lanes per column");
template <int F>
__global__ __launch_bounds__(256) void sb_down_kernel(ExpertWeights W, int T, int H, int E, int k, int I, int I_s,
                                                      SmallWs d) {
  typedef wchunk_t<F> WC;
  constexpr bool Q = F == W_FP8;
  __shared__ float4 shh[DT * 128];  // DT rows of up to 512 fp32 reduction values
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nu = d.plan[0];
  const int u = blockIdx.y;
  const bool shared = (u == nu);
  if (u > nu || (shared && I_s == 0)) return;  // uniform over the workgroup
  const int K = shared ? I_s : I;
  const int col = blockIdx.x * (4 * DCW) + wave * DCW + lane / LPC;
  const int32_t* rec = d.plan + kRec0 + (shared ? 0 : u) * kRecInts;
  const int e = shared ? 0 : rec[0], off = shared ? 0 : rec[1], cnt = shared ? T : rec[2];
  auto asg_at = [&](int q) { return shared ? q : (q < TBR ? rec[4 + q] : d.asg[off + q]); };
  const size_t wr = shared ? (size_t)col : (size_t)e * H + col;  // row of W_down / Ws_down
  const WRow<F> wrw = wrow<F>(shared ? W.s_down : W.down, shared ? W.gss_down : W.gs_down, wr, K);
  const float sc = Q ? (shared ? W.ssc_down : W.sc_down)[wr] : 1.0f;
  const int nch = K / 8;
  for (int kb = 0; kb < nch; kb += 64) {  // reduction blocks of 512 values
    const int nb = min(64, nch - kb);        // chunks in this block (a multiple of 16)
    WC wv[DNCH];
#pragma unroll
    for (int j = 0; j < DNCH; ++j) wv[j] = wrw[kb + min(j * LPC + lane % LPC, nb - 1)];
    for (int q0 = 0; q0 < cnt; q0 += DT) {
      const int nt = min(DT, cnt - q0);
      __syncthreads();
      {
        // one 1 KB load instruction per (assignment, half of the block's 512
        // values); halves past the reduction length are not loaded (those
        // lanes' chunks are skipped below)
        const uint32_t hb = lds_addr(shh);
        for (int ins = __builtin_amdgcn_readfirstlane(wave); ins < DT * 2; ins += 4) {
          const int t = ins >> 1, half = ins & 1;
          if (t < nt && half * 64 < nb * 2) {
            const int a = asg_at(q0 + t);
            const float* hr = shared ? d.hs + (size_t)a * I_s : d.h + (size_t)a * I;
            const int c4 = min(half * 64 + lane, nb * 2 - 1);
            sb_dma16(hr + kb * 8 + c4 * 4, hb + (uint32_t)ins * 1024u);
          }
        }
        sb_wait_vm0();
        __syncthreads();
      }
      for (int t = 0; t < nt; ++t) {
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < DNCH; ++j) {
          const int ch = j * LPC + lane % LPC;
          if (ch < nb) part += dot8_f32w(shh[t * 128 + 2 * ch], shh[t * 128 + 2 * ch + 1], wv[j]);
        }
        // sum of the LPC lanes of this column: DPP quad permutes (every lane
        // of a quad holds the quad's total), then the two quads of 8 lanes
        part += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(part), 0xB1, 0xf, 0xf, false));  // [1,0,3,2]
        part += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(part), 0x4E, 0xf, 0xf, false));  // [2,3,0,1]
        if (LPC >= 8) part += __shfl_xor(part, 4);
        if (LPC >= 16) part += __shfl_xor(part, 8);
        if (Q) part *= sc;
        if (lane % LPC == 0) {
          const int a = asg_at(q0 + t);
          float* out = (shared ? d.os : d.o) + (size_t)a * H + col;
          if (kb == 0)
            *out = part;
          else
            *out += part;  // same thread, same element: reduction blocks in order
        }
      }
    }
  }
}

// S5: y[t][c] = sum_j w[t][j] o[t*k+j][c] (j ascending) + s[t] o_s[t][c], fp32 -> bf16.
__global__ __launch_bounds__(256) void sb_combine_kernel(int T, int H, int k, int I_s, SmallWs d, uint16_t* y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * H) return;
  const int t = i / H, c = i % H;
  float acc = 0.0f;
  for (int j = 0; j < k; ++j) acc += d.w[t * k + j] * d.o[(size_t)(t * k + j) * H + c];
  if (I_s > 0) acc += d.s[t] * d.os[(size_t)t * H + c];
  y[i] = f32_to_bf16(acc);
}

}  // namespace

// logits [T, E], s [T], ids [T, k], w [T, k], the plan, the assignments grouped by expert, h [T*k, I],
// h_s [T, I_s], o [T*k, H], o_s [T, H] (fp32)
WsSections small_batch_sections(int T, int H, int E, int k, int I, int I_s) {
  WsSections w;
  w.take((size_t)T * E * 4);
  w.take((size_t)T * 4);
  w.take((size_t)T * k * 4);
  w.take((size_t)T * k * 4);
  w.take((size_t)(kRec0 + kRecInts * E) * 4);
  w.take((size_t)T * k * 4);
  w.take((size_t)T * k * I * 4);
  w.take((size_t)T * (I_s > 0 ? I_s : 0) * 4);
  w.take((size_t)T * k * H * 4);
  w.take((size_t)T * H * 4);
  return w;
}

size_t small_batch_ids_offset(int T, int H, int E, int k, int I, int I_s) {
  return small_batch_sections(T, H, E, k, I, I_s).off[2];
}

size_t small_batch_workspace_size(int T, int H, int E, int k, int I, int I_s) {
  return small_batch_sections(T, H, E, k, I, I_s).total;
}

hipError_t launch_small_batch(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg,
                              const ExpertWeights& W, int T, int H, int E, int k, int I, int I_s, uint16_t* y,
                              void* ws, hipStream_t st) {
  if (T < 1 || T > kSmallMaxT) return hipErrorInvalidValue;
  SmallWs d = carve_small(ws, T, H, E, k, I, I_s);
  const int rows1 = E + (I_s > 0 ? 1 : 0);
  hipLaunchKernelGGL(sb_router_kernel, dim3((rows1 + 3) / 4, (T + TB - 1) / TB), dim3(256), 0, st, x, w_router, bias,
                     I_s > 0 ? w_sg : nullptr, T, H, E, d);
  hipLaunchKernelGGL(sb_select_kernel, dim3(1), dim3(1024), 0, st, T, E, k, d);
  // expert slots: at most min(E, T*k) touched experts, plus the shared expert
  const int max_u = (T * k < E ? T * k : E) + (I_s > 0 ? 1 : 0);
  const int nrow = I > I_s ? I : I_s;
  const dim3 g_gu((nrow + GR - 1) / GR, max_u), g_dn(H / (4 * DCW), max_u);
  if (W.fmt == W_FP8) {
    hipLaunchKernelGGL(sb_gate_up_kernel<W_FP8>, g_gu, dim3(256), 0, st, x, W, T, H, E, k, I, I_s, d);
    hipLaunchKernelGGL(sb_down_kernel<W_FP8>, g_dn, dim3(256), 0, st, W, T, H, E, k, I, I_s, d);
  } else if (W.fmt == W_Q4) {
    hipLaunchKernelGGL(sb_gate_up_kernel<W_Q4>, g_gu, dim3(256), 0, st, x, W, T, H, E, k, I, I_s, d);
    hipLaunchKernelGGL(sb_down_kernel<W_Q4>, g_dn, dim3(256), 0, st, W, T, H, E, k, I, I_s, d);
  } else {
    hipLaunchKernelGGL(sb_gate_up_kernel<W_BF16>, g_gu, dim3(256), 0, st, x, W, T, H, E, k, I, I_s, d);
    hipLaunchKernelGGL(sb_down_kernel<W_BF16>, g_dn, dim3(256), 0, st, W, T, H, E, k, I, I_s, d);
  }
  hipLaunchKernelGGL(sb_combine_kernel, dim3((T * H + 255) / 256), dim3(256), 0, st, T, H, k, I_s, d, y);
  return hipGetLastError();
}

}  // namespace moe
