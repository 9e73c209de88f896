// Grouped expert GEMMs of the sparse MoE layer on gfx950 (CDNA4).
//
// Each expert's SwiGLU FFN runs only on the rows routed to it
// (guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B", data path: selected-expert
// MoE; kongchang.com "GFX1151 engine", MoE kernel section: the prefill gain
// came from a rewritten MoE kernel).  After the align stage every expert owns
// a run of padded rows cut into tiles; a workgroup computes a (tile,
// 256-column block) item as a dense BF16 GEMM on v_mfma_f32_32x32x16_bf16
// with fp32 accumulation.  Every output element sums its K products in the
// same order (16-column MFMA steps, ascending) whatever the tile height, so
// results do not depend on the tiling.
//
// Two kernels: grouped_gemm_kernel for tiles of 32 to 128 rows (below) and
// the persistent 256-row grouped_gemm_dma_kernel for the routed gate/up and
// down GEMMs of large token counts (described where it is defined).
// grouped_gemm_kernel has four launch kinds:
//   GATE_UP         routed tiles.  A = gathered token rows of x, B = 128 rows
//                   of W_gate and the matching 128 rows of W_up; epilogue
//                   silu(g) * u -> h (bf16).  The shared expert's gate/up over
//                   all tokens rides in the same launch as extra token tiles
//                   (epilogue -> h_s).
//   DOWN            routed tiles.  A = h rows, B = 256 rows of W_down -> o,
//                   stored at the row of the assignment (t*k + j) it holds
//   ROUTER          token tiles.  B = W_router (experts past E zero);
//                   epilogue: logits + bias in LDS (and to the optional fp32
//                   logits output), then top-k and the renormalised weights
//                   per token from LDS; the shared-expert gate x . w_sg
//                   accumulates from the A tiles in LDS
//   SHARED_COMBINE  token tiles.  A = h_s rows, B = 256 rows of Ws_down;
//                   epilogue is the deterministic combine
//                   y = sum_j w_j o[t*k + j] + s * acc
//
// Data movement of the BM <= 128 kernel (256 threads, 4 wavefronts, BM x 256
// tile; the 256-row kernel is described where it is defined):
//   * per K step of BK columns the A tile (BM x 2BK bytes) and B tile
//     (256 x 2BK bytes) are loaded with 16-byte global loads into registers
//     two steps ahead (two register sets), then written to one of two LDS
//     buffers with an XOR swizzle of the 16-byte chunk index, so that the
//     16 rows that one 256-byte LDS cycle serves hit 16 distinct bank groups;
//   * every load is unconditional: rows without data read row 0 and are
//     zeroed when written to LDS, and loads past the last K step re-read it
//     (a select right after a load, or a load skipped on one path, would
//     make the compiler drain the prefetch before the next LDS write);
//   * MFMA fragments are read one 16-column sub-step ahead of the MFMAs that
//     use them, also across the barrier;
//   * work items are dealt so that each XCD gets one contiguous run (the
//     tiles of one expert share that XCD's L2).
#include <type_traits>

#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {
namespace {

constexpr int BNB = 256;  // B rows per tile

enum { GATE_UP = 0, DOWN = 1, ROUTER = 2, SHARED_COMBINE = 3 };

// Kind of one work item.
enum { K_GU = 0, K_ROUTER = 1, K_DOWN = 2, K_COMBINE = 3 };

// Wave layout of a BM x 256 tile: NT threads, WAVES_M x WAVES_N wavefronts of
// WTM x WTN outputs each (MI x NJ blocks of 32 x 32).
template <int BM>
struct Cfg;
template <>
struct Cfg<256> {
  static constexpr int NT = 512, WAVES_M = 4, WTM = 64, MI = 2, WAVES_N = 2, WTN = 128, NJ = 4;
};
template <>
struct Cfg<128> {
  static constexpr int NT = 256, WAVES_M = 2, WTM = 64, MI = 2, WAVES_N = 2, WTN = 128, NJ = 4;
};
template <>
struct Cfg<64> {
  static constexpr int NT = 256, WAVES_M = 1, WTM = 64, MI = 2, WAVES_N = 4, WTN = 64, NJ = 2;
};
template <>
struct Cfg<32> {
  static constexpr int NT = 256, WAVES_M = 1, WTM = 32, MI = 1, WAVES_N = 4, WTN = 64, NJ = 2;
};

struct GemmParams {
  const uint16_t* a;    // x (GATE_UP, ROUTER), h (DOWN) or h_s (SHARED_COMBINE)
  int lda;              // elements per A row
  int K;                // reduction length
  const uint16_t* b0;   // routed W_gate / W_down
  const uint16_t* b1;   // routed W_up
  const uint16_t* bs0;  // shared Ws_gate / Ws_down
  const uint16_t* bs1;  // shared Ws_up
  const uint16_t* br;   // ROUTER: W_router
  int N;                // routed output columns per expert
  int N_s;              // shared output columns (0: no shared blocks)
  int E;                // experts (router rows)
  const int32_t* sorted;
  const int32_t* tiles;    // (expert, first row) per tile of this launch
  const int32_t* n_tiles;  // number of tiles of this launch (device)
  int T, k;
  uint16_t* out;    // h or o
  uint16_t* out_s;  // h_s or y
  int ldo, ldo_s;
  const uint16_t* o;  // combine inputs: o rows in assignment order (t*k + j)
  const float* w;
  const float* s;
  const float* bias;     // ROUTER: bias [E] or NULL
  float* logits;         // ROUTER: logits [T, E]
  const uint16_t* w_sg;  // ROUTER: shared-expert gate vector [K] or NULL
  float* gate_s;         // ROUTER: s = sigmoid(x . w_sg) [T] (when w_sg is given)
  int32_t* ids;          // ROUTER: top-k experts [T, k]
  float* wts;            // ROUTER: their renormalised weights [T, k]
  // FP8 weights (kernels instantiated with Q): b0/b1/bs0/bs1 then point at
  // E4M3 codes (one byte per weight), and each weight row has an fp32 scale:
  // routed sc0/sc1 [E * N], shared ssc0/ssc1 [N_s]
  const float* sc0;
  const float* sc1;
  const float* ssc0;
  const float* ssc1;
  int b_stream;  // persistent kernel, BF16, three-stage ring: an expert's only tile loads its weight rows
                 // with the non-temporal hint
};

// 16-byte chunk swizzles of an LDS row of KCH chunks.  Any 16 consecutive rows
// read at one logical chunk hit 16 distinct 16-byte bank groups of a 256-byte
// bank row, and any 8 consecutive rows 8 distinct groups of a 128-byte one.
template <int KCH>
__device__ __forceinline__ int swz(int row, int chunk);
template <>
__device__ __forceinline__ int swz<4>(int row, int chunk) { return chunk ^ (((row >> 1) ^ (row >> 2)) & 3); }
template <>
__device__ __forceinline__ int swz<8>(int row, int chunk) { return chunk ^ (((row >> 1) ^ ((row & 1) << 2)) & 7); }

// One work item: a BM-row tile times one block of output columns.  Flags are
// ints: with bool members the persistent kernel kept its per-item copies in a
// private stack object (scratch memory), which cost 2-4% of the GEMM time.
struct Item {
  int kind;   // K_GU, K_ROUTER, K_DOWN, K_COMBINE
  int dense;  // rows are tokens row0.. (else padded rows of one expert)
  int expert;
  int row0;  // first padded row or first token; -1: no item
  int nb;    // column block
  int tile;  // routed launches: index in the tile table (-1: dense)
};

// Routed launches (GATE_UP, DOWN): item count and item by index.  Routed
// tiles come first, tile major (the column blocks of a tile run together and
// share its A rows in L2); a GATE_UP launch then appends the shared expert's
// token tiles (they fill the launch's last, partly idle round).
struct RoutedItems {
  int n_routed, nb_per, nb_sh, total;
};
template <int BM, int MODE>
__device__ __forceinline__ RoutedItems routed_items(const GemmParams& p) {
  RoutedItems r;
  r.nb_per = (MODE == GATE_UP) ? p.N / 128 : p.N / 256;
  r.n_routed = p.n_tiles[0] * r.nb_per;
  r.nb_sh = (MODE == GATE_UP && p.bs0) ? p.N_s / 128 : 0;
  r.total = r.n_routed + ((p.T + BM - 1) / BM) * r.nb_sh;
  return r;
}
template <int BM, int MODE>
__device__ __forceinline__ Item routed_item_at(const GemmParams& p, const RoutedItems& r, int item) {
  Item it;
  it.kind = (MODE == DOWN) ? K_DOWN : K_GU;
  it.expert = 0;
  it.tile = -1;
  if (item < r.n_routed) {
    const int tile = item / r.nb_per;
    it.tile = tile;
    it.dense = false;
    it.nb = item % r.nb_per;
    it.expert = p.tiles[2 * tile];
    it.row0 = p.tiles[2 * tile + 1];
  } else {
    it.dense = true;
    it.row0 = ((item - r.n_routed) / r.nb_sh) * BM;
    it.nb = (item - r.n_routed) % r.nb_sh;
  }
  return it;
}

template <int BM, int MODE>
__device__ __forceinline__ Item decode_item(const GemmParams& p) {
  Item it;
  it.kind = (MODE == DOWN) ? K_DOWN : (MODE == SHARED_COMBINE) ? K_COMBINE : K_GU;
  it.dense = (MODE == ROUTER || MODE == SHARED_COMBINE);
  it.expert = 0;
  it.row0 = -1;
  it.nb = 0;
  const int n_tok_tiles = (p.T + BM - 1) / BM;
  if (MODE == GATE_UP || MODE == DOWN) {
    const RoutedItems r = routed_items<BM, MODE>(p);
    const int item = xcd_item(blockIdx.x, r.total);
    if (item < 0) return it;
    return routed_item_at<BM, MODE>(p, r, item);
  }
  const int nb_per = (MODE == ROUTER) ? 1 : p.N_s / 256;
  const int item = xcd_item(blockIdx.x, n_tok_tiles * nb_per);
  if (item < 0) return it;
  it.row0 = (item / nb_per) * BM;
  it.nb = item % nb_per;
  if (MODE == ROUTER) it.kind = K_ROUTER;
  return it;
}

// Source row of tile row r (r < BM) and whether it carries data.  Rows
// without data (padding, tokens past T) point at row 0 of the source.
template <int MODE>
__device__ __forceinline__ const uint16_t* a_row(const GemmParams& p, const Item it, int r, bool& ok) {
  size_t src_row = 0;
  if (it.dense) {
    const int t = it.row0 + r;
    ok = t < p.T;
    src_row = ok ? (size_t)t : 0;
  } else {
    const int a = p.sorted[it.row0 + r];
    ok = a >= 0;
    src_row = !ok ? 0 : (MODE == GATE_UP) ? (size_t)(a / p.k) : (size_t)(it.row0 + r);
  }
  return p.a + src_row * p.lda;
}

// Weight row of tile B-row j (0..255) and whether it carries data.  For
// gate/up items rows 0..127 are gate rows and 128..255 the up rows of the
// same 128 intermediate columns; router rows past E point at row 0.
// With Q the matrices hold one byte per weight (E4M3 codes); the returned
// pointer is then a byte address in the same type.
template <int MODE, bool Q = false>
__device__ __forceinline__ const uint16_t* b_row(const GemmParams& p, const Item it, int j, bool& ok) {
  constexpr size_t EB = Q ? 1 : 2;  // bytes per weight
  ok = true;
  if (MODE == ROUTER && it.kind == K_ROUTER) {
    ok = j < p.E;
    return p.br + (size_t)(ok ? j : 0) * p.K;
  }
  size_t row;  // weight row within the matrix
  const uint16_t* m;
  if (it.kind == K_GU) {
    m = (j < 128) ? (it.dense ? p.bs0 : p.b0) : (it.dense ? p.bs1 : p.b1);
    row = (size_t)it.nb * 128 + (j & 127);
  } else {
    m = it.dense ? p.bs0 : p.b0;
    row = (size_t)it.nb * 256 + j;
  }
  if (!it.dense) row += (size_t)it.expert * p.N;
  return reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(m) + row * p.K * EB);
}

// Scale of weight row j of the item's B tile (FP8 weights), as b_row.
template <int MODE>
__device__ __forceinline__ float b_scale(const GemmParams& p, const Item it, int j) {
  if (it.kind == K_GU) {
    const float* sc = (j < 128) ? (it.dense ? p.ssc0 : p.sc0) : (it.dense ? p.ssc1 : p.sc1);
    return sc[(it.dense ? 0 : (size_t)it.expert * p.N) + (size_t)it.nb * 128 + (j & 127)];
  }
  return (it.dense ? p.ssc0 : p.sc0)[(it.dense ? 0 : (size_t)it.expert * p.N) + (size_t)it.nb * 256 + j];
}

// Eight E4M3 codes -> eight bf16 (exact: every E4M3 value is a bf16), by the
// gfx950 scaled conversion with scale 1.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(const u32x2& c) {
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    r[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[q], 1.0f, false));
    r[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[q], 1.0f, true));
  }
  return r;
}

// Weighted sum of token t's k expert outputs at columns ocol..ocol+7, in
// rank order j = 0..k-1, fp32: y = ((w_0 o_0 + w_1 o_1) + ...) + w_{k-1} o_{k-1}.
// o holds one row per assignment a = t*k + j, so a token's k rows are
// contiguous and every load address is known up front; the 8 row loads of a
// group are issued together (only the sum is ordered).
__device__ __forceinline__ void gather_combine8(const uint16_t* __restrict__ o, const float* __restrict__ w, int t,
                                                int k, int ldo, int ocol, float (&y)[8]) {
#pragma unroll
  for (int q = 0; q < 8; ++q) y[q] = 0.0f;
  const size_t base = (size_t)t * k;
  for (int j0 = 0; j0 < k; j0 += 8) {
    float wj[8];
    u32x4 ov[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = (j0 + q < k) ? j0 + q : k - 1;
      wj[q] = w[base + j];
      ov[q] = *reinterpret_cast<const u32x4*>(o + (base + j) * ldo + ocol);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (j0 + q < k) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          y[2 * c] += wj[q] * bf16_to_f32((uint16_t)(ov[q][c] & 0xffff));
          y[2 * c + 1] += wj[q] * bf16_to_f32((uint16_t)(ov[q][c] >> 16));
        }
      }
    }
  }
}

// Sum of the 8 bf16 products of two 16-byte chunks, fp32.
__device__ __forceinline__ float dot8_bf16(const u32x4& a, const u32x4& b) {
  float r = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r += bf16_to_f32((uint16_t)(a[q] & 0xffff)) * bf16_to_f32((uint16_t)(b[q] & 0xffff));
    r += bf16_to_f32((uint16_t)(a[q] >> 16)) * bf16_to_f32((uint16_t)(b[q] >> 16));
  }
  return r;
}

constexpr int EPW = 64;        // epilogue staging: columns per pass
constexpr int ESLD = EPW + 4;  // fp32 row stride of the staging tile

// Epilogue: accumulators -> fp32 LDS staging 64 columns at a time -> stores.
// Wave layout: rows wm*WTM + m*32 + (MFMA row), tile columns bb[j] + (lane&31).
// Gate/up items pair column block j (gate) with j + NJ/2 (up).
// Router gate: the partial dot products x . w_sg (one per thread, KCH threads
// per token row, consecutive lanes of one wave) are summed and
// s = sigmoid(sum) stored.
template <int BM, int KCH>
__device__ __forceinline__ void router_gate(const GemmParams& p, const Item it, float gacc) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int off = 1; off < KCH; off <<= 1) gacc += __shfl_xor(gacc, off);
  const int t = it.row0 + tid / KCH;
  if (tid % KCH == 0 && t < p.T) p.gate_s[t] = 1.0f / (1.0f + expf(-gacc));
}

// Router epilogue: the tile holds all E logits of its BM tokens.  They go to
// LDS ([BM][RLD] fp32, bias added, -0 -> +0), to the logits output when one
// is given, and each wave selects the top k of BM / waves tokens from LDS
// (the selection rule and weights of moe_topk.h), NTK tokens interleaved.
constexpr int RLD = 256 + 8;  // row stride: the two lane halves of an MFMA store hit disjoint banks
template <int BM, int NT, int MI, int NJ, int WTM>
__device__ __forceinline__ void router_epilogue(const GemmParams& p, const Item it, f32x16 (&acc)[MI][NJ], int wm,
                                                const int (&bb)[NJ], unsigned char* smem) {
  constexpr int NW = NT / 64, NTK = 4;
  static_assert(BM % (NW * NTK) == 0, "tokens per wave");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* sl = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int m = 0; m < MI; ++m)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = bb[j] + (lane & 31);
      // clamped, not skipped: a load under a per-lane condition would be
      // waited for on its own (columns past E are not selected)
      const float b = p.bias ? p.bias[min(col, p.E - 1)] : 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = wm * WTM + m * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        float v = acc[m][j][q] + b;
        if (v == 0.0f) v = 0.0f;  // -0 -> +0
        sl[row * RLD + col] = v;
      }
    }
  __syncthreads();
  const int nrow = min(BM, p.T - it.row0);
  if (p.logits) {
    // rows of E logits are contiguous in the output: element i of the tile is
    // at (row0 * E + i)
    float* out = p.logits + (size_t)it.row0 * p.E;
    for (int i = tid; i < nrow * p.E; i += NT) out[i] = sl[(i / p.E) * RLD + i % p.E];
  }
  for (int r0 = wave * NTK; r0 < BM; r0 += NW * NTK) {
    float v[NTK][4];
    bool valid[NTK][4];
#pragma unroll
    for (int t = 0; t < NTK; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        valid[t][q] = e < p.E;
        v[t][q] = sl[(r0 + t) * RLD + e];
      }
    int se[NTK];
    float sv[NTK], w[NTK];
    wave_topk_weights_n<NTK>(v, valid, p.k, lane, se, sv, w);
#pragma unroll
    for (int t = 0; t < NTK; ++t) {
      const int tok = it.row0 + r0 + t;
      if (r0 + t < nrow && lane < p.k) {
        p.ids[(size_t)tok * p.k + lane] = se[t];
        p.wts[(size_t)tok * p.k + lane] = w[t];
      }
    }
  }
}

template <int BM, int NT, int MODE, int MI, int NJ, int WTM>
__device__ __forceinline__ void epilogue(const GemmParams& p, const Item it, f32x16 (&acc)[MI][NJ], int wm,
                                         const int (&bb)[NJ], unsigned char* smem) {
  constexpr int RG = NT / 8;    // copy-out: rows per group
  constexpr int RPT = BM / RG;  // copy-out: rows per thread
  const int tid = threadIdx.x, lane = tid & 63;
  float* sc = reinterpret_cast<float*>(smem);  // [BM][ESLD]
  const bool gu = it.kind == K_GU;
  const int ncol = gu ? 128 : 256;
  const int cr = tid >> 3;       // copy-out: row within a group of RG rows
  const int cc = (tid & 7) * 8;  // copy-out: first of 8 columns
  // DOWN: the assignment held by each of this thread's copy-out rows, read
  // once for all column passes (-1: padding row, not stored)
  int arow_of[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) arow_of[i] = (MODE == DOWN) ? p.sorted[it.row0 + cr + RG * i] : 0;
  for (int pass = 0; pass < ncol / EPW; ++pass) {
#pragma unroll
    for (int m = 0; m < MI; ++m) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (gu && j >= NJ / 2) continue;
        const int col = bb[j] + (lane & 31) - pass * EPW;
        if (col >= 0 && col < EPW) {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int row = wm * WTM + m * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            sc[row * ESLD + col] = gu ? silu(acc[m][j][q]) * acc[m][(j + NJ / 2) % NJ][q] : acc[m][j][q];
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < (MODE == SHARED_COMBINE ? 0 : RPT); ++i) {
      const int r = cr + RG * i;
      const float4 v0 = *reinterpret_cast<const float4*>(sc + r * ESLD + cc);
      const float4 v1 = *reinterpret_cast<const float4*>(sc + r * ESLD + cc + 4);
      float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      const int col = pass * EPW + cc;  // within the item's output columns
      if (it.kind == K_GU) {
        const u32x4 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7])};
        if (it.dense) {
          const int t = it.row0 + r;
          if (t < p.T) *reinterpret_cast<u32x4*>(p.out_s + (size_t)t * p.ldo_s + it.nb * 128 + col) = pk;
        } else {
          *reinterpret_cast<u32x4*>(p.out + (size_t)(it.row0 + r) * p.ldo + it.nb * 128 + col) = pk;
        }
      } else if (MODE == DOWN) {
        const int a = arow_of[i];
        if (a >= 0) {
          const u32x4 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7])};
          *reinterpret_cast<u32x4*>(p.out + (size_t)a * p.ldo + it.nb * 256 + col) = pk;
        }
      }
    }
    if constexpr (MODE == SHARED_COMBINE) {
      // every row of this thread gathers its k expert rows, then adds s[t]
      // times the shared expert's output
      float yv[RPT][8];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int t = it.row0 + cr + RG * i;
        gather_combine8(p.o, p.w, t < p.T ? t : p.T - 1, p.k, p.ldo, it.nb * 256 + pass * EPW + cc, yv[i]);
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = cr + RG * i;
        const int t = it.row0 + r;
        if (t < p.T) {
          const float4 v0 = *reinterpret_cast<const float4*>(sc + r * ESLD + cc);
          const float4 v1 = *reinterpret_cast<const float4*>(sc + r * ESLD + cc + 4);
          const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          const float st = p.s[t];
          float* y = yv[i];
#pragma unroll
          for (int q = 0; q < 8; ++q) y[q] += st * v[q];
          const u32x4 pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                            pack_bf16x2(y[6], y[7])};
          *reinterpret_cast<u32x4*>(p.out_s + (size_t)t * p.ldo_s + it.nb * 256 + pass * EPW + cc) = pk;
        }
      }
    }
    __syncthreads();
  }
}

template <int BM, int BK, int MODE>
constexpr size_t lds_bytes() {
  size_t stages = 2 * (size_t)(BM + BNB) * (BK / 8) * 16;
  size_t epi = (size_t)BM * (MODE == ROUTER ? RLD : ESLD) * 4;
  return stages > epi ? stages : epi;
}

// BM x 256 tile, K steps of BK columns, OCC workgroups per CU (register budget).
// Q: the B matrices are E4M3 codes with one fp32 scale per weight row; the
// codes are loaded as 8 bytes per 8 weights, widened to bf16 (exactly) when
// written to LDS, and the row scales multiply the accumulators in the
// epilogue.
template <int BM, int BK, int OCC, int MODE, bool Q = false>
__global__ __launch_bounds__(Cfg<BM>::NT, OCC) void grouped_gemm_kernel(GemmParams p) {
  static_assert(!Q || MODE != ROUTER, "the router weights stay bf16");
  constexpr bool RT = MODE == ROUTER;
  using C = Cfg<BM>;
  constexpr int KCH = BK / 8;               // 16-byte chunks per row per K step
  constexpr int RPP = C::NT / KCH;          // rows covered by one pass of the NT threads
  constexpr int NA = (BM + RPP - 1) / RPP;  // A chunks per thread per K step
  constexpr int NB = BNB / RPP;             // B chunks per thread per K step
  constexpr int SUB = BK / 16;              // MFMA K sub-steps per K step
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const Item it = decode_item<BM, MODE>(p);
  if (it.row0 < 0) return;

  const int chunk = tid % KCH;
  const int trow = tid / KCH;
  const uint16_t* arow[NA];
  uint32_t amask = 0;  // bit i: A chunk i carries data
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = trow + RPP * i;
    bool ok = false;
    arow[i] = (r < BM) ? a_row<MODE>(p, it, r, ok) : p.a;
    amask |= ok ? (1u << i) : 0u;
  }
  const uint16_t* brow[NB];
  uint32_t bmask = 0;  // bit i: B chunk i carries data (router rows past E do not)
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    bool ok;
    brow[i] = b_row<MODE, Q>(p, it, trow + RPP * i, ok);
    bmask |= ok ? (1u << i) : 0u;
  }

  u32x4* sA = reinterpret_cast<u32x4*>(smem);  // [2][BM*KCH]
  u32x4* sB = sA + 2 * BM * KCH;               // [2][BNB*KCH]
  const u32x4 zero = {0u, 0u, 0u, 0u};
  typedef wchunk_t<Q ? W_FP8 : W_BF16> BC;  // B chunk as loaded: 8 bf16, or 8 E4M3 codes
  u32x4 pa0[NA], pa1[NA];
  BC pb0[NB], pb1[NB];
  auto gload = [&](u32x4 (&pa)[NA], BC (&pb)[NB], int kb) {
    const int koff = kb * BK + chunk * 8;
#pragma unroll
    for (int i = 0; i < NA; ++i) pa[i] = *reinterpret_cast<const u32x4*>(arow[i] + koff);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if constexpr (Q)
        pb[i] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(brow[i]) + koff);
      else
        pb[i] = *reinterpret_cast<const u32x4*>(brow[i] + koff);
    }
  };
  auto widen = [&](const BC& c) -> u32x4 {
    if constexpr (Q)
      return e4m3x8_to_bf16x8(c);
    else
      return c;
  };
  auto sstore = [&](const u32x4 (&pa)[NA], const BC (&pb)[NB], int st) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int r = trow + RPP * i;
      if (r < BM) sA[st * BM * KCH + r * KCH + swz<KCH>(r, chunk)] = ((amask >> i) & 1u) ? pa[i] : zero;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int r = trow + RPP * i;
      if constexpr (RT)
        sB[st * BNB * KCH + r * KCH + swz<KCH>(r, chunk)] = ((bmask >> i) & 1u) ? pb[i] : zero;
      else
        sB[st * BNB * KCH + r * KCH + swz<KCH>(r, chunk)] = widen(pb[i]);
    }
  };
  int bb[C::NJ];
  {
    constexpr int half = C::NJ / 2;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
      bb[j] = (it.kind == K_GU) ? (j < half ? wn * half * 32 + j * 32 : 128 + wn * half * 32 + (j - half) * 32)
                                : wn * C::WTN + j * 32;
  }

  f32x16 acc[C::MI][C::NJ];
#pragma unroll
  for (int m = 0; m < C::MI; ++m)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[m][j][q] = 0.0f;

  struct Frag {
    bf16x8 a[C::MI], b[C::NJ];
  };
  auto read_frags = [&](Frag& f, int st, int sub) {
    const u32x4* cA = sA + st * BM * KCH;
    const u32x4* cB = sB + st * BNB * KCH;
    const int c = 2 * sub + (lane >> 5);
#pragma unroll
    for (int m = 0; m < C::MI; ++m) {
      const int r = wm * C::WTM + m * 32 + (lane & 31);
      f.a[m] = __builtin_bit_cast(bf16x8, cA[r * KCH + swz<KCH>(r, c)]);
    }
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int r = bb[j] + (lane & 31);
      f.b[j] = __builtin_bit_cast(bf16x8, cB[r * KCH + swz<KCH>(r, c)]);
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int m = 0; m < C::MI; ++m)
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
        acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[m], f.b[j], acc[m][j], 0, 0, 0);
  };

  // K loop: two LDS buffers, two register sets of prefetched chunks (global
  // loads two K steps ahead), unrolled by two steps so every buffer has a
  // fixed role (the number of K steps is even).  Inside a step: the first
  // fragment reads, then the LDS writes of the next step (their buffer was
  // released by the barrier just passed) and the next global loads, then the
  // MFMAs with the remaining fragment reads one sub-step ahead.
  // A wave whose first row carries no data has only padding rows (padding
  // sits at the end of a tile): it still loads and writes its share of the
  // tiles but issues no fragment reads and no MFMAs, leaving the SIMD's
  // matrix core to the other workgroup on the CU.
  bool live;
  {
    const int r = wm * C::WTM;
    if (it.dense) {
      live = it.row0 + r < p.T;
    } else {
      live = p.sorted[it.row0 + r] >= 0;
    }
    live = __builtin_amdgcn_readfirstlane((int)live) != 0;
  }
  const int nk = p.K / BK;
  gload(pa0, pb0, 0);
  gload(pa1, pb1, 1);
  sstore(pa0, pb0, 0);
  gload(pa0, pb0, min(2, nk - 1));
  __syncthreads();
  Frag f0, f1;
  bool pending = false;  // f1 holds the last sub-step of the previous K step
  // Router launches: partial x . w_sg of the shared-expert gate from the A
  // tile in LDS: thread t takes rows t / KCH + g NT / KCH (g < NG), 16-byte
  // chunk t % KCH of every K step
  constexpr int NG = (BM * KCH) / C::NT;
  static_assert(!RT || (NG >= 1 && NG * C::NT == BM * KCH), "router gate: whole A chunks per thread");
  static_assert(MODE != ROUTER || NG == 1, "router gate: one A chunk per thread");
  float gacc[NG > 0 ? NG : 1];
#pragma unroll
  for (int g = 0; g < (NG > 0 ? NG : 1); ++g) gacc[g] = 0.0f;
  auto kloop = [&](auto LIVE) {
    constexpr bool L = decltype(LIVE)::value;
    auto stage = [&](int st, u32x4 (&pa)[NA], BC (&pb)[NB], int next_kb, int ks) {
      u32x4 gv = {0u, 0u, 0u, 0u};
      if constexpr (RT) {
        if (p.w_sg) gv = *reinterpret_cast<const u32x4*>(p.w_sg + ks * BK + (tid % KCH) * 8);
      }
      if constexpr (L) read_frags(f0, st, 0);
      __builtin_amdgcn_sched_barrier(0);
      sstore(pa, pb, st ^ 1);
      gload(pa, pb, next_kb);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (L) {
        if (pending) mma(f1);
#pragma unroll
        for (int sub = 1; sub < SUB; ++sub) {
          if (sub & 1) {
            read_frags(f1, st, sub);
            mma(f0);
          } else {
            read_frags(f0, st, sub);
            mma(f1);
          }
        }
        if (SUB % 2 == 0) {
          pending = true;
        } else {
          mma(f0);
          pending = false;
        }
      }
      if constexpr (RT) {
        if (p.w_sg) {
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const int r = tid / KCH + g * (C::NT / KCH), c = tid % KCH;
            gacc[g] += dot8_bf16(sA[st * BM * KCH + r * KCH + swz<KCH>(r, c)], gv);
          }
        }
      }
    };
    for (int kb = 0; kb < nk; kb += 2) {
      stage(0, pa1, pb1, min(kb + 3, nk - 1), kb);  // step kb from LDS[0]; writes step kb+1 -> LDS[1]
      __syncthreads();
      stage(1, pa0, pb0, min(kb + 4, nk - 1), kb + 1);  // step kb+1 from LDS[1]; writes step kb+2 -> LDS[0]
      __syncthreads();
    }
  };
  if (live)
    kloop(std::true_type{});
  else
    kloop(std::false_type{});
  if (pending) mma(f1);
  if constexpr (MODE == ROUTER) {
    if (p.w_sg) router_gate<BM, KCH>(p, it, gacc[0]);
    router_epilogue<BM, C::NT, C::MI, C::NJ, C::WTM>(p, it, acc, wm, bb, smem);
  } else {
    if constexpr (Q) {
      // row scales of this lane's B columns (one per column block j)
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        const float scl = b_scale<MODE>(p, it, bb[j] + (lane & 31));
#pragma unroll
        for (int m = 0; m < C::MI; ++m)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[m][j][q] *= scl;
      }
    }
    epilogue<BM, C::NT, MODE, C::MI, C::NJ, C::WTM>(p, it, acc, wm, bb, smem);
  }
}

// 256 x 256 tiles for the routed gate/up and down GEMMs.  512 threads (8
// wavefronts of 64 x 128 outputs), one workgroup per CU, persistent: the
// workgroups of an XCD walk that XCD's contiguous run of items together.
//   * A and B rows arrive by direct-to-LDS loads (global_load_lds_dwordx4):
//     no staging registers and no LDS stores; a K step is 64 columns, so
//     every row load is one whole 128-byte line;
//   * two 64 KB stages: the loads of step k + 1 are in flight while step k
//     is computed, and the last step of an item overlaps the first loads of
//     the next item, which also run under the epilogue; or (R3, BF16 weights:
//     every down launch, and gate/up launches below a mean of 192 rows per
//     expert) two A stages and three B stages, the weight rows loaded two
//     steps ahead (160 KB of LDS);
//   * the MFMAs produce transposed output blocks, so every lane holds runs
//     of 4 consecutive output columns of one row: the gate/up epilogue
//     stores them as 8-byte writes straight from the accumulators (no LDS
//     staging, no barrier); in down items (rows of o are 4 KB apart) each
//     wave writes its block as 8-byte bf16 runs into its own part of the
//     stage that the last K step used and stores 128-byte (BF16) or 64-byte
//     (FP8: smaller stages) row segments; either way the next item's first
//     loads are in flight;
//   * the rows the epilogue stores to are read at item setup, so the
//     epilogue issues no load that would wait behind those loads;
//   * a wave issues no MFMA for a 32-row block of only padding rows (the
//     rows of a tile are sorted with padding last);
//   * A row groups of only padding are not loaded: their LDS rows hold
//     finite values of earlier data and feed only output rows that are not
//     stored (a row of A reaches only the same row of the product).
//   * with FP8 weights (Q) the B rows arrive as E4M3 codes (half the bytes
//     of every B load), are widened exactly to bf16 as fragments are read,
//     and the item's 256 row scales arrive by one more direct load into a
//     small LDS area (two items' worth), from which the epilogue scales the
//     accumulators.
#ifndef MOE_DMA_WAVES
#define MOE_DMA_WAVES 8
#endif
#ifndef MOE_DMA_SKIP_PAD_BLOCKS
#define MOE_DMA_SKIP_PAD_BLOCKS 1
#endif
// Wave layout of the persistent kernel's 256 x 256 tile: NW wavefronts, two
// across the columns (128 each), NW / 2 down the rows.
struct DCfg {
  static constexpr int NW = MOE_DMA_WAVES, NT = NW * 64, WAVES_N = 2, WAVES_M = NW / 2;
  static constexpr int WTM = 256 / WAVES_M, MI = WTM / 32, WTN = 128, NJ = 4;
  static constexpr int RPW = 256 / NW;  // A rows (and B rows) each wave loads
};
constexpr int DBM = 256, DNT = DCfg::NT, DBK = 64, DKCH = DBK / 8;
constexpr int DRPI = 64 / DKCH;                    // A rows filled by one load instruction (64 lanes x 16 B)
constexpr int DNQ = DCfg::RPW / DRPI;              // A load instructions per wave per K step
template <bool Q>
struct DmaGeom {
  static constexpr int BKCH = Q ? DKCH / 2 : DKCH;         // 16-byte chunks per B row per K step
  static constexpr int BRPI = 64 / BKCH;                   // B rows filled by one load instruction
  static constexpr int BNQ = DCfg::RPW / BRPI;             // B load instructions per wave per K step
  static constexpr int STAGE = DBM * DKCH + BNB * BKCH;    // 16-byte chunks per stage (A rows, then B rows)
  static constexpr size_t SCALES = Q ? 2 * BNB * 4 : 0;    // LDS bytes of two items' B-row scales
  static constexpr size_t LDS = 2 * (size_t)STAGE * 16 + SCALES;  // 128 KB (bf16), 98 KB (FP8)
  static_assert((size_t)DNT / 64 * (Q ? 4096 : 8192) <= (size_t)STAGE * 16, "down epilogue staging fits in one stage");
};

// LDS layout of the persistent kernel, in 16-byte chunks: two stages of A
// and B ([A0 B0][A1 B1]; the down epilogue stages its outputs in one whole
// stage), or (R3) two A stages and three B stages ([A0 A1][B0 B1 B2]), the
// weight rows then loaded two K steps ahead.
template <bool Q, bool R3>
struct DmaLay {
  using G = DmaGeom<Q>;
  static constexpr int ASZ = DBM * DKCH, BSZ = BNB * G::BKCH;
  static constexpr int TOTAL = R3 ? 2 * ASZ + 3 * BSZ : 2 * (ASZ + BSZ);
  static constexpr size_t LDS = (size_t)TOTAL * 16 + G::SCALES;  // 160 KB (bf16, R3)
  __device__ static constexpr int a_off(int s) { return R3 ? s * ASZ : s * (ASZ + BSZ); }
  __device__ static constexpr int b_off(int s) { return R3 ? 2 * ASZ + s * BSZ : s * (ASZ + BSZ) + ASZ; }
  static_assert(LDS <= 160 * 1024, "LDS per workgroup");
};

// One direct-to-LDS load: 16 bytes per lane from src into LDS at
// lds_base + 16 * lane (lds_base wave-uniform, in M0).  Inline assembly, so
// that the compiler's wait-count pass does not order later LDS reads behind
// it; the K loop waits for it explicitly before the barrier that publishes
// the stage.  (The compiler's own waits for its loads only grow stronger
// from loads it does not see: vector-memory counts complete in issue order.)
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(src)
               : "memory", "m0");
}
// The same with the non-temporal hint: the bytes are not kept in the caches
// for later readers.
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds_base), "v"(src)
               : "memory", "m0");
}

// wait until every vector-memory access of this wave has completed
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8)); }

// Per-item state of the persistent kernel.
struct DmaItem {
  Item it;
  const uint16_t* asrc[DNQ];  // this lane's A source of load q (K step 0)
  const char* bbase;          // this wave's B rows: bbase + the item-independent lane byte offsets
  const float* ssrc;          // FP8: this lane's 16 bytes of the item's B-row scales
  int spar;                   // FP8: which of the two LDS scale areas the item uses
  uint32_t aon;               // bit q: A group q holds a data row
  int live;                   // this wave's 64 rows hold data
  int nm;                     // 32-row blocks of this wave that hold data (padding rows are last)
  int bnt;                    // B rows loaded with the non-temporal hint (no other item reads them)
  int orow[DCfg::MI];         // this lane's epilogue rows (block m): assignment (down), or >= 0 if stored
};

template <int MODE, bool Q, bool NT>
__device__ __forceinline__ DmaItem dma_item(const GemmParams& p, const Item it, int wave, int wm, int lane,
                                            int spar) {
  constexpr size_t EB = Q ? 1 : 2;  // bytes per weight
  DmaItem d;
  d.it = it;
  d.aon = 0;
  // load q of wave w fills rows w*32 + q*8 .. +7 of the A (or B) part of a
  // stage: lane l -> row w*32 + q*8 + l/8, LDS slot l%8, which holds logical
  // chunk swz(row, l%8) (the swizzle is its own inverse)
#pragma unroll
  for (int q = 0; q < DNQ; ++q) {
    const int r = wave * DCfg::RPW + q * DRPI + lane / DKCH;
    const int ch = swz<DKCH>(r, lane % DKCH);
    bool ok;
    d.asrc[q] = a_row<MODE>(p, it, r, ok) + ch * 8;
    d.aon |= (__builtin_amdgcn_readfirstlane(ok ? 1 : 0) ? 1u : 0u) << q;  // lane 0 holds the group's first row
  }
  // B rows w*32 .. w*32+31: gate/up items take gate rows in waves 0-3 and up
  // rows in waves 4-7 (the same 128 intermediate columns)
  const size_t erow = it.dense ? 0 : (size_t)it.expert * p.N;  // the expert's first weight row
  if (MODE == GATE_UP) {
    const char* m =
        reinterpret_cast<const char*>(wave < DCfg::NW / 2 ? (it.dense ? p.bs0 : p.b0) : (it.dense ? p.bs1 : p.b1));
    d.bbase = m + (erow + (size_t)it.nb * 128) * p.K * EB;
  } else {
    d.bbase = reinterpret_cast<const char*>(it.dense ? p.bs0 : p.b0) + (erow + (size_t)it.nb * 256) * p.K * EB;
  }
  // the scales of B rows 0..255, 16 bytes per lane: gate/up items take the
  // 128 gate rows' scales in lanes 0-31 and the up rows' in lanes 32-63
  d.spar = spar;
  d.ssrc = nullptr;
  if constexpr (Q) {
    if (MODE == GATE_UP)
      d.ssrc = (lane < 32 ? (it.dense ? p.ssc0 : p.sc0) : (it.dense ? p.ssc1 : p.sc1)) + erow + (size_t)it.nb * 128 +
               (lane & 31) * 4;
    else
      d.ssrc = (it.dense ? p.ssc0 : p.sc0) + erow + (size_t)it.nb * 256 + lane * 4;
  }
  const int r = wm * DCfg::WTM;
  d.nm = 0;
#pragma unroll
  for (int m = 0; m < DCfg::MI; ++m) {
    const int rm = it.row0 + r + m * 32;
    const bool lv = it.dense ? (rm < p.T) : (p.sorted[rm] >= 0);
    d.nm += __builtin_amdgcn_readfirstlane((int)lv);
  }
  d.live = d.nm > 0;
  // an expert's only tile: no other item of the launch reads these weight
  // rows, so they are loaded past the caches, which then keep the token
  // rows, h and o that this and the next launches read again
  d.bnt = 0;
  if (NT && !it.dense) {
    const int ntl = p.n_tiles[0];
    const bool shared_w = (it.tile > 0 && p.tiles[2 * (it.tile - 1)] == it.expert) ||
                          (it.tile + 1 < ntl && p.tiles[2 * (it.tile + 1)] == it.expert);
    d.bnt = __builtin_amdgcn_readfirstlane(shared_w ? 0 : 1);
  }
  // the epilogue's rows, read here so that the epilogue issues no load (a
  // load there would wait behind the next item's loads already in flight)
#pragma unroll
  for (int m = 0; m < DCfg::MI; ++m) {
    const int rr = r + m * 32 + (lane & 31);
    d.orow[m] = it.dense ? (it.row0 + rr < p.T ? it.row0 + rr : -1) : p.sorted[it.row0 + rr];
  }
  return d;
}

template <int MODE, bool Q = false, bool R3 = false, bool NT = false>
__global__ __launch_bounds__(DNT, 1) void grouped_gemm_dma_kernel(GemmParams p) {
  static_assert(MODE == GATE_UP || MODE == DOWN, "routed GEMMs only");
  static_assert(!NT || (R3 && !Q), "non-temporal weight loads only with the BF16 three-stage ring");
  using C = DCfg;
  using G = DmaGeom<Q>;
  using L = DmaLay<Q, R3>;  // R3: weight rows two K steps ahead
  constexpr size_t EB = Q ? 1 : 2;  // bytes per weight
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  // this workgroup's items: slot s of its XCD takes items first, first + nslot, ...
  const RoutedItems ri = routed_items<DBM, MODE>(p);
  const int per = (ri.total + kNumXcd - 1) / kNumXcd;
  const int nslot = (int)gridDim.x / kNumXcd;
  const int xcd = (int)blockIdx.x % kNumXcd;
  const int first = xcd * per + (int)blockIdx.x / kNumXcd;
  const int last = min(ri.total, (xcd + 1) * per);
  if (first >= last) return;

  u32x4* sm = reinterpret_cast<u32x4*>(smem);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  // A groups that are never loaded must not hold arbitrary bits on the first item
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int i = tid; i < L::TOTAL; i += DNT) sm[i] = zero;
  __syncthreads();
  const uint32_t lds_scales = lds0 + (uint32_t)(L::TOTAL * 16);
  const float* scales = reinterpret_cast<const float*>(smem + L::TOTAL * 16);  // [2][BNB]

  // byte offset of this lane's B source of load q from the wave's bbase:
  // lane l fills row w*32 + q*BRPI + l/BKCH, LDS slot l%BKCH, which holds
  // logical chunk swz(row, l%BKCH)
  uint32_t boff[G::BNQ];
#pragma unroll
  for (int q = 0; q < G::BNQ; ++q) {
    const int r = wave * DCfg::RPW + q * G::BRPI + lane / G::BKCH;
    boff[q] = (uint32_t)(((MODE == GATE_UP ? (r & 127) : r) * p.K) * EB + swz<G::BKCH>(r, lane % G::BKCH) * 16);
  }
  // A K step's loads go out in two groups (below): group 0 right after the
  // barrier, group 1 after the MFMAs of two sub-steps.  A wave's load
  // instructions wait in issue while the CU's load path drains the other
  // waves' loads (64 KB per step), and its MFMAs queue behind them; moving
  // one operand's loads behind some MFMAs overlaps the two.  With two
  // stages gate/up issues B (the expert rows, mostly L2 misses) first, down
  // issues A first: measured, gate/up 385.6 -> 369.3 us and down 234.3 ->
  // 225.3 us against all loads in group 0 (the other orders were slower).
  // With the R3 ring group 0 is A of the next step and group 1 B of the
  // step after, so a step waits for all but the latest B group.
  constexpr bool a_first = MODE == DOWN;
  auto issue_a = [&](const DmaItem& d, uint32_t base, int kb) {
#pragma unroll
    for (int q = 0; q < DNQ; ++q)
      if ((d.aon >> q) & 1u)
        dma16(d.asrc[q] + kb * DBK, base + (uint32_t)(wave * DCfg::RPW + q * DRPI) * DKCH * 16);
  };
  auto issue_b = [&](const DmaItem& d, uint32_t base, int kb) {
    if (NT && d.bnt) {
#pragma unroll
      for (int q = 0; q < G::BNQ; ++q)
        dma16_nt(d.bbase + boff[q] + (size_t)kb * DBK * EB,
                 base + (uint32_t)((wave * DCfg::RPW + q * G::BRPI) * G::BKCH) * 16);
    } else {
#pragma unroll
      for (int q = 0; q < G::BNQ; ++q)
        dma16(d.bbase + boff[q] + (size_t)kb * DBK * EB,
              base + (uint32_t)((wave * DCfg::RPW + q * G::BRPI) * G::BKCH) * 16);
    }
  };
  auto issue_scales = [&](const DmaItem& d) {
    if constexpr (Q) {
      if (wave == 0) dma16(d.ssrc, lds_scales + (uint32_t)d.spar * BNB * 4);
    }
  };
  auto issue_grp = [&](const DmaItem& d, int st, int kb, int g) {
    if ((g == 0) == a_first)
      issue_a(d, lds0 + (uint32_t)L::a_off(st) * 16, kb);
    else
      issue_b(d, lds0 + (uint32_t)L::b_off(st) * 16, kb);
    if (g == 0 && kb == 0) issue_scales(d);
  };
  auto issue = [&](const DmaItem& d, int st, int kb) {
    issue_grp(d, st, kb, 0);
    issue_grp(d, st, kb, 1);
  };
  int bb[C::NJ];
  {
    constexpr int half = C::NJ / 2;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
      bb[j] = (MODE == GATE_UP) ? (j < half ? wn * half * 32 + j * 32 : 128 + wn * half * 32 + (j - half) * 32)
                                : wn * C::WTN + j * 32;
  }
  struct Frag {
    bf16x8 a[C::MI], b[C::NJ];
  };
  auto read_frags = [&](Frag& f, int ast, int bst, int sub) {
    const u32x4* cA = sm + L::a_off(ast);
    const u32x4* cB = sm + L::b_off(bst);
    const int c = 2 * sub + (lane >> 5);
#pragma unroll
    for (int m = 0; m < C::MI; ++m) {
      const int r = wm * C::WTM + m * 32 + (lane & 31);
      f.a[m] = __builtin_bit_cast(bf16x8, cA[r * DKCH + swz<DKCH>(r, c)]);
    }
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int r = bb[j] + (lane & 31);
      if constexpr (Q) {
        // K values 8c .. 8c+7 of row r: half (c & 1) of logical 16-byte chunk c / 2
        const u32x2 codes = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(cB) +
                                                            (r * G::BKCH + swz<G::BKCH>(r, c >> 1)) * 16 + (c & 1) * 8);
        f.b[j] = __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8(codes));
      } else {
        f.b[j] = __builtin_bit_cast(bf16x8, cB[r * DKCH + swz<DKCH>(r, c)]);
      }
    }
  };
  // Items compute transposed blocks (the weight fragment is the MFMA's first
  // operand): lane l then holds output row (l & 31) and, for q = 4 g + i,
  // output column 8 g + 4 (l >> 5) + i -- four consecutive columns of one row
  // per group g, stored as one 8-byte write (or staged as one 8-byte run).
  f32x16 acc[C::MI][C::NJ];
  int live_blocks = C::MI;  // the item's 32-row blocks of this wave that hold data
  auto mma = [&](const Frag& f) {
    // 32-row blocks of only padding rows are skipped (a scalar branch)
#pragma unroll
    for (int m = 0; m < C::MI; ++m)
      if (!MOE_DMA_SKIP_PAD_BLOCKS || m == 0 || m < live_blocks)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
          acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[m], acc[m][j], 0, 0, 0);
  };

  constexpr int SUB = DBK / 16;
  static_assert(SUB == 4, "the K loop below is written out for four sub-steps");
  const int nk = p.K / DBK;  // even: K is a multiple of 128
  DmaItem cur = dma_item<MODE, Q, NT>(p, routed_item_at<DBM, MODE>(p, ri, first), wave, wm, lane, 0);
  int bs = 0;       // R3: B stage of the current K step (cycles 0, 1, 2 across items)
  int nb_pend = 0;  // R3: B loads of the latest group, which the next step need not wait for
  if constexpr (R3) {
    issue_a(cur, lds0 + (uint32_t)L::a_off(0) * 16, 0);
    issue_b(cur, lds0 + (uint32_t)L::b_off(0) * 16, 0);
    issue_scales(cur);
    issue_b(cur, lds0 + (uint32_t)L::b_off(1) * 16, 1);
    nb_pend = G::BNQ;
  } else {
    issue(cur, 0, 0);
  }
  for (int item = first; item < last; item += nslot) {
    const int nxt = item + nslot;
    const bool has_next = nxt < last;
    DmaItem next = cur;
    if (has_next) next = dma_item<MODE, Q, NT>(p, routed_item_at<DBM, MODE>(p, ri, nxt), wave, wm, lane, cur.spar ^ 1);
#pragma unroll
    for (int m = 0; m < C::MI; ++m)
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[m][j][q] = 0.0f;
    live_blocks = cur.nm;
    // K loop: wait for this wave's loads of step kb, barrier (everyone's have
    // landed and everyone has finished reading the other stage), then load
    // step kb + 1 (or the next item's step 0) into the other stage in two
    // groups and compute step kb.  The last sub-step's fragments are read
    // before the barrier and their MFMAs issued after it.  (The live-row
    // test is made twice, around the second group: with the group inside
    // one conditional block the compiler spilled the accumulators.)
    Frag f0, f1;
    bool pending = false;
    if constexpr (R3) {
      // Step kb: wait for A(kb) (issued one step earlier) and B(kb) (two
      // steps earlier); B(kb + 1), the latest group, may still be in flight.
      // Group 0 loads A(kb + 1), group 1 B(kb + 2) -- of the next item past
      // the end of this one.  A stages alternate with kb (nk is even), B
      // stages cycle through three.
      // (The partial waits are inline assembly: the compiler's wait-count
      // pass does not see the direct-to-LDS loads and may turn a builtin
      // partial wait into a full one.  launch_dma instantiates R3 for BF16
      // weights, BNQ = 4; the FP8 count, 2, is kept for completeness.)
      for (int kb = 0; kb < nk; ++kb) {
        const int as = kb & 1;
        if (nb_pend >= 4)
          asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else if (nb_pend >= 2)
          asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
        else
          wait_vm0();
        __syncthreads();
        if (kb + 1 < nk)
          issue_a(cur, lds0 + (uint32_t)L::a_off(as ^ 1) * 16, kb + 1);
        else if (has_next)
          issue_a(next, lds0 + (uint32_t)L::a_off(0) * 16, 0);
        if (cur.live) {
          read_frags(f0, as, bs, 0);
          if (pending) mma(f1);
          read_frags(f1, as, bs, 1);
          mma(f0);
        }
        const int bs2 = bs == 0 ? 2 : bs - 1;  // (bs + 2) % 3
        nb_pend = 0;
        if (kb + 2 < nk) {
          issue_b(cur, lds0 + (uint32_t)L::b_off(bs2) * 16, kb + 2);
          nb_pend = G::BNQ;
        } else if (has_next) {
          issue_b(next, lds0 + (uint32_t)L::b_off(bs2) * 16, kb + 2 - nk);
          if (kb + 2 == nk) issue_scales(next);
          nb_pend = G::BNQ;
        }
        asm volatile("" : "+s"(nb_pend));  // opaque: the compiler then does not peel the first step
        if (cur.live) {
          read_frags(f0, as, bs, 2);
          mma(f1);
          read_frags(f1, as, bs, 3);
          mma(f0);
          pending = true;
        }
        bs = bs == 2 ? 0 : bs + 1;
      }
    } else {
      for (int kb = 0; kb < nk; ++kb) {
        const int st = kb & 1;
        wait_vm0();
        __syncthreads();
        // nk is even, so the next item's step 0 goes to stage 0 = st ^ 1 too
        auto group = [&](int g) {
          if (kb + 1 < nk)
            issue_grp(cur, st ^ 1, kb + 1, g);
          else if (has_next)
            issue_grp(next, 0, 0, g);
        };
        group(0);
        if (cur.live) {
          read_frags(f0, st, st, 0);
          if (pending) mma(f1);
          read_frags(f1, st, st, 1);
          mma(f0);
        }
        group(1);
        if (cur.live) {
          read_frags(f0, st, st, 2);
          mma(f1);
          read_frags(f1, st, st, 3);
          mma(f0);
          pending = true;
        }
      }
    }
    if (pending) mma(f1);

    const Item& it = cur.it;
    if constexpr (MODE == GATE_UP) {
      // Epilogue straight from the accumulators: per (m, j) block and group
      // g each lane stores 4 bf16 (8 bytes) of its row, silu(g) * u -> h (or
      // h_s for the shared expert's token tiles); the two lane halves cover
      // 16 contiguous bytes of a row.  Padding rows are not stored: a row of
      // A reaches only the same row of the product, so whatever a padding
      // row of h holds stays in padding rows of o.
      const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
      for (int m = 0; m < C::MI; ++m) {
        const int r = wm * C::WTM + m * 32 + lr;  // tile row
        const int o = cur.orow[m];                // token (shared tiles) or assignment; < 0: padding
        if (o >= 0) {
          uint16_t* orow = it.dense ? p.out_s + (size_t)o * p.ldo_s + it.nb * 128
                                    : p.out + (size_t)(it.row0 + r) * p.ldo + it.nb * 128;
#pragma unroll
          for (int j = 0; j < C::NJ / 2; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              float v[4];
              if constexpr (Q) {
                // B rows bb[j] + 8 g + 4 lh + i (gate) and the same of the up half
                const float* S = scales + cur.spar * BNB;
                const float4 sg = *reinterpret_cast<const float4*>(S + bb[j] + 8 * g + 4 * lh);
                const float4 su = *reinterpret_cast<const float4*>(S + bb[j + C::NJ / 2] + 8 * g + 4 * lh);
                const float fg[4] = {sg.x, sg.y, sg.z, sg.w}, fu[4] = {su.x, su.y, su.z, su.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  v[i] = silu(acc[m][j][4 * g + i] * fg[i]) * (acc[m][j + C::NJ / 2][4 * g + i] * fu[i]);
              } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = silu(acc[m][j][4 * g + i]) * acc[m][j + C::NJ / 2][4 * g + i];
              }
              const uint2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
              *reinterpret_cast<uint2*>(orow + bb[j] + 8 * g + 4 * lh) = pk;
            }
          }
        }
      }
    } else if constexpr (Q) {
      // Down, FP8: as the BF16 epilogue below, in 4 KB per
      // wave (an FP8 stage holds 48 KB), 32 columns a pass and 64-byte row
      // segments; each lane scales its 4 consecutive columns by their weight
      // rows' scales (in LDS since the item's first K step)
      __syncthreads();
      // the last step's A stage (R3: the next item's loads go to the other one and to other B stages)
      char* ew = reinterpret_cast<char*>(smem) + (size_t)L::a_off((nk - 1) & 1) * 16 + (size_t)wave * 4096;
      const float* S = scales + cur.spar * BNB;
      int arow[4];  // the assignment of this lane's copy-out rows lane / 4 + 16 i (block m = i / 2)
#pragma unroll
      for (int i = 0; i < 4; ++i) arow[i] = __shfl(cur.orow[i / 2], (lane / 4 + 16 * i) & 31);
#pragma unroll
      for (int pass = 0; pass < C::NJ; ++pass) {
#pragma unroll
        for (int m = 0; m < C::MI; ++m) {
          const int row = m * 32 + (lane & 31);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 sc = *reinterpret_cast<const float4*>(S + bb[pass] + 8 * g + 4 * (lane >> 5));
            const uint2 pk = {pack_bf16x2(acc[m][pass][4 * g] * sc.x, acc[m][pass][4 * g + 1] * sc.y),
                              pack_bf16x2(acc[m][pass][4 * g + 2] * sc.z, acc[m][pass][4 * g + 3] * sc.w)};
            *reinterpret_cast<uint2*>(ew + row * 64 + (g ^ (row & 3)) * 16 + (lane >> 5) * 8) = pk;
          }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = lane / 4 + 16 * i, c = lane & 3;
          const u32x4 v = *reinterpret_cast<const u32x4*>(ew + r * 64 + (c ^ (r & 3)) * 16);
          if (arow[i] >= 0)
            *reinterpret_cast<u32x4*>(p.out + (size_t)arow[i] * p.ldo + it.nb * 256 + wn * 128 + pass * 32 + c * 8) =
                v;
        }
        __builtin_amdgcn_wave_barrier();
      }
    } else {
      // Down, BF16: rows of o are 4 KB apart, so each wave
      // stages its own 64 x 128 block in its own 8 KB of the stage the last K
      // step used and stores 128-byte row segments, 64 columns a pass.  Only
      // the first barrier (every wave's fragment reads of that stage are done)
      // involves the workgroup; a wave's LDS operations complete in order, so
      // the rest needs none.  16-byte slots are XOR-swizzled by the row.
      __syncthreads();
      // the last step's stages: its A stage (waves 0-3) and B stage (waves 4-7), which no load in flight writes
      const int blast = bs == 0 ? 2 : bs - 1;  // R3: the B stage of step nk - 1
      char* ew = reinterpret_cast<char*>(smem) +
                 (R3 ? (wave < 4 ? (size_t)L::a_off(1) * 16 + (size_t)wave * 8192
                                 : (size_t)L::b_off(blast) * 16 + (size_t)(wave - 4) * 8192)
                     : (size_t)((nk - 1) & 1) * G::STAGE * 16 + (size_t)wave * 8192);
      // the assignment of this lane's copy-out rows lane / 8 + 8 i (block m = i / 4)
      int arow[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) arow[i] = __shfl(cur.orow[i / 4], (lane / 8 + 8 * i) & 31);
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int m = 0; m < C::MI; ++m) {
          const int row = m * 32 + (lane & 31);  // within the wave's 64 rows
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * pass + jj;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const uint2 pk = {pack_bf16x2(acc[m][j][4 * g], acc[m][j][4 * g + 1]),
                                pack_bf16x2(acc[m][j][4 * g + 2], acc[m][j][4 * g + 3])};
              const int slot = (jj * 4 + g) ^ (row & 7);
              *reinterpret_cast<uint2*>(ew + row * 128 + slot * 16 + (lane >> 5) * 8) = pk;
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = lane / 8 + 8 * i, c = lane & 7;
          const u32x4 v = *reinterpret_cast<const u32x4*>(ew + r * 128 + (c ^ (r & 7)) * 16);
          if (arow[i] >= 0)
            *reinterpret_cast<u32x4*>(p.out + (size_t)arow[i] * p.ldo + it.nb * 256 + wn * 128 + pass * 64 + c * 8) =
                v;
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    cur = next;
  }
}

// Combine without a shared expert: y[t,c] = sum_j w[t,j] o[t*k+j, c].
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o, const float* __restrict__ w,
                                                      int T, int H, int k, uint16_t* __restrict__ y) {
  const int per_tok = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)T * per_tok) return;
  const int t = (int)(idx / per_tok);
  const int col = (int)(idx % per_tok) * 8;
  float acc[8];
  gather_combine8(o, w, t, k, H, col, acc);
  u32x4 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
              pack_bf16x2(acc[6], acc[7])};
  *reinterpret_cast<u32x4*>(y + (size_t)t * H + col) = pk;
}

template <int BM, int BK, int OCC, int MODE, bool Q = false>
hipError_t launch_mode(const GemmParams& p, int64_t max_items, hipStream_t st) {
  const int64_t grid = ((max_items + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (grid <= 0) return hipSuccess;
  constexpr size_t lds = lds_bytes<BM, BK, MODE>();
  hipError_t e = hipFuncSetAttribute((const void*)grouped_gemm_kernel<BM, BK, OCC, MODE, Q>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((grouped_gemm_kernel<BM, BK, OCC, MODE, Q>), dim3((unsigned)grid), dim3(Cfg<BM>::NT), lds, st,
                     p);
  return hipGetLastError();
}

// Persistent launch: one workgroup per CU (at most one per item).  ring3:
// the three-stage weight ring (BF16 weights only); p.b_stream: with it, the
// non-temporal weight loads of single-tile experts (ignored without ring3).
template <int MODE, bool Q = false>
hipError_t launch_dma(const GemmParams& p, int64_t max_items, hipStream_t st, bool ring3) {
  if (max_items <= 0) return hipSuccess;
  if (p.K % (2 * DBK) != 0) return hipErrorInvalidValue;
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int64_t grid = n_cu < max_items ? n_cu : max_items;
  grid = ((grid + kNumXcd - 1) / kNumXcd) * kNumXcd;
  auto go = [&](auto R3, auto NT) -> hipError_t {
    constexpr bool r3 = decltype(R3)::value, nt = decltype(NT)::value;
    constexpr size_t lds = DmaLay<Q, r3>::LDS;
    hipError_t e2 = hipFuncSetAttribute((const void*)grouped_gemm_dma_kernel<MODE, Q, r3, nt>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e2 != hipSuccess) return e2;
    hipLaunchKernelGGL((grouped_gemm_dma_kernel<MODE, Q, r3, nt>), dim3((unsigned)grid), dim3(DNT), lds, st, p);
    return hipGetLastError();
  };
  if constexpr (!Q) {
    if (ring3 && p.b_stream) return go(std::true_type{}, std::true_type{});
    if (ring3) return go(std::true_type{}, std::false_type{});
  }
  return go(std::false_type{}, std::false_type{});
}

// Tile configuration per tile height: (rows, K step, workgroups per CU).
#ifndef MOE_COMBINE_CFG
#define MOE_COMBINE_CFG 128, 32, 2
#endif
// Combine launch below MOE_COMBINE_SMALL_T (MOE_COMBINE_MID_T) tokens: smaller
// token tiles, so that the gather of the o rows runs on more workgroups.  The
// 32-row tiles stop where they no longer fit one round of two workgroups per
// CU at H = 2048 (64 token tiles x 8 column blocks): combine at 2,304 /
// 3,072 / 3,584 tokens 41.0 / 46.0 / 50.0 us with 32-row tiles, 38.0 / 40.4
// / 43.1 us with 64-row tiles.
#ifndef MOE_COMBINE_CFG_SMALL
#define MOE_COMBINE_CFG_SMALL 32, 64, 2
#endif
#ifndef MOE_COMBINE_SMALL_T
#define MOE_COMBINE_SMALL_T 2049
#endif
#ifndef MOE_COMBINE_CFG_MID
#define MOE_COMBINE_CFG_MID 64, 64, 2
#endif
#ifndef MOE_COMBINE_MID_T
#define MOE_COMBINE_MID_T 8192
#endif
#ifndef MOE_GEMM_CFG_128
#define MOE_GEMM_CFG_128 128, 32, 2
#endif
#ifndef MOE_GEMM_CFG_64
#define MOE_GEMM_CFG_64 64, 64, 2
#endif
#ifndef MOE_GEMM_CFG_32
#define MOE_GEMM_CFG_32 32, 64, 2
#endif
// Router launch: (token-tile rows, K step, workgroups per CU).
#ifndef MOE_ROUTER_CFG
#define MOE_ROUTER_CFG 32, 64, 2
#endif
// Down GEMM with 128-row tiles (K = I is short, so its K step may differ).
#ifndef MOE_DOWN_CFG_128
#define MOE_DOWN_CFG_128 MOE_GEMM_CFG_128
#endif

constexpr int router_rows(int bm, int, int) { return bm; }
constexpr int router_bk(int, int bk, int) { return bk; }

template <int MODE, bool Q = false>
hipError_t launch_bm(int BM, const GemmParams& p, int64_t max_items, hipStream_t st, bool ring3 = false) {
  switch (BM) {
    case 32: return launch_mode<MOE_GEMM_CFG_32, MODE, Q>(p, max_items, st);
    case 64: return launch_mode<MOE_GEMM_CFG_64, MODE, Q>(p, max_items, st);
    case 128:
      if constexpr (MODE == DOWN) return launch_mode<MOE_DOWN_CFG_128, MODE, Q>(p, max_items, st);
      return launch_mode<MOE_GEMM_CFG_128, MODE, Q>(p, max_items, st);
    case 256:
      if constexpr (MODE == GATE_UP || MODE == DOWN) return launch_dma<MODE, Q>(p, max_items, st, ring3);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg, int T,
                         int H, int E, int k, float* logits, float* s, int32_t* ids, float* w, hipStream_t st) {
  GemmParams p = {};
  p.a = x;
  p.lda = H;
  p.K = H;
  p.br = w_router;
  p.E = E;
  p.T = T;
  p.k = k;
  p.bias = bias;
  p.logits = logits;
  p.w_sg = w_sg;
  p.gate_s = s;
  p.ids = ids;
  p.wts = w;
  // Small token tiles: one 256-column block per tile, so the tile count is
  // the launch's whole parallelism.
  constexpr int BM = router_rows(MOE_ROUTER_CFG);
  return launch_mode<MOE_ROUTER_CFG, ROUTER>(p, (int64_t)((T + BM - 1) / BM), st);
}

hipError_t launch_gate_up(const uint16_t* x, const void* w_gate, const void* w_up, const int32_t* sorted,
                          const int32_t* tiles, const int32_t* n_tiles, int T, int H, int k, int I, int BM,
                          int64_t max_tiles, uint16_t* h, const void* ws_gate, const void* ws_up, int I_s,
                          uint16_t* h_s, hipStream_t st, const FP8Scales* q, bool ring3, bool stream_w) {
  GemmParams p = {};
  p.b_stream = stream_w ? 1 : 0;
  p.a = x;
  p.lda = H;
  p.K = H;
  p.b0 = static_cast<const uint16_t*>(w_gate);
  p.b1 = static_cast<const uint16_t*>(w_up);
  p.N = I;
  p.sorted = sorted;
  p.tiles = tiles;
  p.n_tiles = n_tiles;
  p.T = T;
  p.k = k;
  p.out = h;
  p.ldo = I;
  if (I_s > 0) {
    p.bs0 = static_cast<const uint16_t*>(ws_gate);
    p.bs1 = static_cast<const uint16_t*>(ws_up);
    p.N_s = I_s;
    p.out_s = h_s;
    p.ldo_s = I_s;
  }
  const int64_t shared_items = I_s > 0 ? (int64_t)((T + BM - 1) / BM) * (I_s / 128) : 0;
  if (q) {
    p.sc0 = q->gate, p.sc1 = q->up, p.ssc0 = q->s_gate, p.ssc1 = q->s_up;
    return launch_bm<GATE_UP, true>(BM, p, max_tiles * (I / 128) + shared_items, st);
  }
  return launch_bm<GATE_UP>(BM, p, max_tiles * (I / 128) + shared_items, st, ring3);
}

hipError_t launch_down(const uint16_t* h, const void* w_down, const int32_t* sorted, const int32_t* tiles,
                       const int32_t* n_tiles, int T, int H, int k, int I, int BM, int64_t max_tiles, uint16_t* o,
                       hipStream_t st, const FP8Scales* q, bool ring3, bool stream_w) {
  GemmParams p = {};
  p.b_stream = stream_w ? 1 : 0;
  p.a = h;
  p.lda = I;
  p.K = I;
  p.b0 = static_cast<const uint16_t*>(w_down);
  p.N = H;
  p.sorted = sorted;
  p.tiles = tiles;
  p.n_tiles = n_tiles;
  p.T = T;
  p.k = k;
  p.out = o;
  p.ldo = H;
  if (q) {
    p.sc0 = q->down;
    return launch_bm<DOWN, true>(BM, p, max_tiles * (H / 256), st);
  }
  return launch_bm<DOWN>(BM, p, max_tiles * (H / 256), st, ring3);
}

hipError_t launch_combine(const uint16_t* o, const float* w, const uint16_t* h_s,
                          const void* ws_down, const float* s, int T, int H, int k, int I_s, uint16_t* y,
                          hipStream_t st, const FP8Scales* q) {
  if (I_s == 0) {
    int64_t n = (int64_t)T * (H / 8);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, o, w, T, H, k, y);
    return hipGetLastError();
  }
  GemmParams p = {};
  p.a = h_s;
  p.lda = I_s;
  p.K = I_s;
  p.bs0 = static_cast<const uint16_t*>(ws_down);
  p.N_s = H;
  p.T = T;
  p.k = k;
  p.out_s = y;
  p.ldo = H;
  p.ldo_s = H;
  p.o = o;
  p.w = w;
  p.s = s;
  if (q) p.ssc0 = q->s_down;
  if (T < MOE_COMBINE_SMALL_T) {
    constexpr int BM = router_rows(MOE_COMBINE_CFG_SMALL);
    const int64_t max_items = (int64_t)((T + BM - 1) / BM) * (H / 256);
    if (q) return launch_mode<MOE_COMBINE_CFG_SMALL, SHARED_COMBINE, true>(p, max_items, st);
    return launch_mode<MOE_COMBINE_CFG_SMALL, SHARED_COMBINE>(p, max_items, st);
  }
  if (T < MOE_COMBINE_MID_T) {
    constexpr int BM = router_rows(MOE_COMBINE_CFG_MID);
    const int64_t max_items = (int64_t)((T + BM - 1) / BM) * (H / 256);
    if (q) return launch_mode<MOE_COMBINE_CFG_MID, SHARED_COMBINE, true>(p, max_items, st);
    return launch_mode<MOE_COMBINE_CFG_MID, SHARED_COMBINE>(p, max_items, st);
  }
  constexpr int BM = router_rows(MOE_COMBINE_CFG);
  const int64_t max_items = (int64_t)((T + BM - 1) / BM) * (H / 256);
  if (q) return launch_mode<MOE_COMBINE_CFG, SHARED_COMBINE, true>(p, max_items, st);
  return launch_mode<MOE_COMBINE_CFG, SHARED_COMBINE>(p, max_items, st);
}

}  // namespace moe
