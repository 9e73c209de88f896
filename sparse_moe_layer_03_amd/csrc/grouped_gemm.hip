// Grouped expert GEMMs of the sparse MoE layer on gfx950 (CDNA4).
//
// Each expert's SwiGLU FFN runs only on the rows routed to it
// (guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B", data path: selected-expert
// MoE; kongchang.com "GFX1151 engine", MoE kernel section: the prefill gain
// came from a rewritten MoE kernel).  After the align stage every expert owns
// a run of padded rows cut into tiles of BM rows; one workgroup computes one
// (tile, column block) item as a dense BF16 GEMM on v_mfma_f32_32x32x16_bf16
// with fp32 accumulation.
//
// One kernel template, three epilogues:
//   GATE_UP         A = gathered token rows of x, B = 128 rows of W_gate and
//                   the matching 128 rows of W_up; epilogue silu(g) * u -> h
//                   (the shared expert is extra tiles over all tokens -> h_s)
//   DOWN            A = h rows, B = 256 rows of W_down -> o (bf16)
//   SHARED_COMBINE  A = h_s rows, B = 256 rows of Ws_down; epilogue is the
//                   deterministic combine y = sum_j w_j o[inv] + s * acc
//
// Data movement: 256 threads (4 wavefronts); per K step of 32 columns the A
// tile (BM x 64 B) and B tile (256 x 64 B) are loaded with 16-byte global
// loads into registers, written to LDS with an XOR swizzle of the 16-byte
// chunk index (conflict-free 16-byte fragment reads), double buffered so
// the next step's global loads are in flight during the MFMAs.  Work items
// are dealt so that each XCD gets one contiguous run (tiles of one expert
// share that XCD's L2).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BNB = 256;     // B rows per tile

enum { GATE_UP = 0, DOWN = 1, SHARED_COMBINE = 2 };

// Wave layout of a BM x 256 tile over 4 wavefronts.
template <int BM>
struct Cfg;
template <>
struct Cfg<256> {
  static constexpr int WAVES_M = 2, WTM = 128, MI = 4, WAVES_N = 2, WTN = 128, NJ = 4;
};
template <>
struct Cfg<128> {
  static constexpr int WAVES_M = 2, WTM = 64, MI = 2, WAVES_N = 2, WTN = 128, NJ = 4;
};
template <>
struct Cfg<64> {
  static constexpr int WAVES_M = 1, WTM = 64, MI = 2, WAVES_N = 4, WTN = 64, NJ = 2;
};
template <>
struct Cfg<32> {
  static constexpr int WAVES_M = 1, WTM = 32, MI = 1, WAVES_N = 4, WTN = 64, NJ = 2;
};

struct GemmParams {
  const uint16_t* a;  // x, h or h_s
  int lda;            // elements per A row
  int K;              // reduction length
  const uint16_t* b0; // routed weights (W_gate or W_down)
  const uint16_t* b1; // W_up
  const uint16_t* bs0;// shared weights (Ws_gate or Ws_down)
  const uint16_t* bs1;// Ws_up
  int N;              // routed output columns per expert
  int N_s;            // shared output columns
  const int32_t* sorted;
  const int32_t* tiles;
  const int32_t* n_tiles;
  int T, k;
  uint16_t* out;      // h, o or y
  uint16_t* out_s;    // h_s
  int ldo, ldo_s;
  const uint16_t* o;  // combine inputs
  const int32_t* inv;
  const float* w;
  const float* s;
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

// ------------------------------------------------------------ shared parts

// One work item: a BM-row tile (routed rows of one expert, or BM tokens of the
// shared expert) times one block of output columns.
struct Item {
  bool shared;
  int expert, row0, nb;
};

// Returns the work item of this workgroup; it.row0 < 0 when there is none.
template <int BM, int MODE>
__device__ __forceinline__ Item decode_item(const GemmParams& p) {
  Item it;
  const int n_routed = (MODE == SHARED_COMBINE) ? 0 : p.n_tiles[0];
  const int n_tok_tiles = (p.T + BM - 1) / BM;
  int n_items, nb_r = 0, nb_s = 0;
  if (MODE == GATE_UP) {
    nb_r = p.N / 128;
    nb_s = p.bs0 ? p.N_s / 128 : 0;
    n_items = n_routed * nb_r + n_tok_tiles * nb_s;
  } else if (MODE == DOWN) {
    nb_r = p.N / 256;
    n_items = n_routed * nb_r;
  } else {
    nb_s = p.N_s / 256;
    n_items = n_tok_tiles * nb_s;
  }
  const int item = xcd_item(blockIdx.x, n_items);
  it.expert = 0;
  it.nb = 0;
  it.shared = false;
  it.row0 = -1;
  if (item < 0) return it;
  if (MODE != SHARED_COMBINE && item < n_routed * nb_r) {
    it.shared = false;
    const int tile = item / nb_r;
    it.nb = item % nb_r;
    it.expert = p.tiles[2 * tile];
    it.row0 = p.tiles[2 * tile + 1];
  } else {
    it.shared = true;
    const int i2 = (MODE == GATE_UP) ? item - n_routed * nb_r : item;
    it.row0 = (i2 / nb_s) * BM;  // first token
    it.nb = i2 % nb_s;
  }
  return it;
}

// Source row of tile row r (r < BM), and whether it carries data.  Rows
// without data (padding, tokens past T) point at row 0 of the source and are
// zeroed when written to LDS, so every load is unconditional.
template <int MODE>
__device__ __forceinline__ const uint16_t* a_row(const GemmParams& p, const Item it, int r, bool& ok) {
  size_t src_row = 0;
  if (it.shared) {
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

// Weight row of tile B-row j (0..255): for GATE_UP rows 0..127 are gate rows
// and 128..255 the up rows of the same 128 intermediate columns.
template <int MODE>
__device__ __forceinline__ const uint16_t* b_row(const GemmParams& p, const Item it, int j) {
  if (MODE == GATE_UP) {
    const size_t col = (size_t)it.nb * 128 + (j & 127);
    const uint16_t* base = (j < 128) ? (it.shared ? p.bs0 : p.b0 + (size_t)it.expert * p.N * p.K)
                                     : (it.shared ? p.bs1 : p.b1 + (size_t)it.expert * p.N * p.K);
    return base + col * p.K;
  }
  const size_t col = (size_t)it.nb * 256 + j;
  return (it.shared ? p.bs0 : p.b0 + (size_t)it.expert * p.N * p.K) + col * p.K;
}

constexpr int EPW = 64;       // epilogue staging: columns per pass
constexpr int ESLD = EPW + 4; // fp32 row stride of the staging tile

// Epilogue: accumulators -> fp32 LDS staging 64 columns at a time -> 16-byte
// stores.  Wave layout: rows wm*WTM + m*32 + (MFMA row), tile columns
// bb[j] + (lane & 31).  GATE_UP pairs column block j (gate) with j + NJ/2 (up).
template <int BM, int MODE, int MI, int NJ, int WTM>
__device__ __forceinline__ void epilogue(const GemmParams& p, const Item it, f32x16 (&acc)[MI][NJ], int wm,
                                         const int (&bb)[NJ], unsigned char* smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  float* sc = reinterpret_cast<float*>(smem);  // [BM][ESLD]
  constexpr int NCOL = (MODE == GATE_UP) ? 128 : 256;
  const int cr = tid >> 3;        // copy-out: row within a 32-row group
  const int cc = (tid & 7) * 8;   // copy-out: first of 8 columns
  for (int pass = 0; pass < NCOL / EPW; ++pass) {
#pragma unroll
    for (int m = 0; m < MI; ++m) {
      constexpr int NOUT = (MODE == GATE_UP) ? NJ / 2 : NJ;
#pragma unroll
      for (int j = 0; j < NOUT; ++j) {
        const int col = bb[j] + (lane & 31) - pass * EPW;
        if (col >= 0 && col < EPW) {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int row = wm * WTM + m * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            sc[row * ESLD + col] = (MODE == GATE_UP) ? silu(acc[m][j][q]) * acc[m][j + NJ / 2][q] : acc[m][j][q];
          }
        }
      }
    }
    __syncthreads();
    for (int r = cr; r < BM; r += 32) {
      const float4 v0 = *reinterpret_cast<const float4*>(sc + r * ESLD + cc);
      const float4 v1 = *reinterpret_cast<const float4*>(sc + r * ESLD + cc + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      const int col = pass * EPW + cc;  // within the item's output columns
      if (MODE == GATE_UP) {
        const u32x4 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7])};
        if (it.shared) {
          const int t = it.row0 + r;
          if (t < p.T) *reinterpret_cast<u32x4*>(p.out_s + (size_t)t * p.ldo_s + it.nb * 128 + col) = pk;
        } else {
          *reinterpret_cast<u32x4*>(p.out + (size_t)(it.row0 + r) * p.ldo + it.nb * 128 + col) = pk;
        }
      } else if (MODE == DOWN) {
        if (p.sorted[it.row0 + r] >= 0) {
          const u32x4 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7])};
          *reinterpret_cast<u32x4*>(p.out + (size_t)(it.row0 + r) * p.ldo + it.nb * 256 + col) = pk;
        }
      } else {
        const int t = it.row0 + r;
        if (t < p.T) {
          const int ocol = it.nb * 256 + col;
          float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          for (int j = 0; j < p.k; ++j) {  // rank order
            const float wj = p.w[(size_t)t * p.k + j];
            const u32x4 ov =
                *reinterpret_cast<const u32x4*>(p.o + (size_t)p.inv[(size_t)t * p.k + j] * p.ldo + ocol);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              y[2 * q] += wj * bf16_to_f32((uint16_t)(ov[q] & 0xffff));
              y[2 * q + 1] += wj * bf16_to_f32((uint16_t)(ov[q] >> 16));
            }
          }
          const float st = p.s[t];
#pragma unroll
          for (int q = 0; q < 8; ++q) y[q] += st * v[q];
          const u32x4 pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                            pack_bf16x2(y[6], y[7])};
          *reinterpret_cast<u32x4*>(p.out_s + (size_t)t * p.ldo_s + ocol) = pk;
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------- kernel 1: B through LDS

template <int BM, int BK>
constexpr size_t lds_bytes_lds() {
  size_t stages = 2 * (size_t)(BM + BNB) * (BK / 8) * 16;
  size_t epi = (size_t)BM * ESLD * 4;
  return stages > epi ? stages : epi;
}

// BM x 256 tile, both operands staged through LDS, K steps of BK columns,
// OCC workgroups per CU (register budget).
template <int BM, int BK, int OCC, int MODE>
__global__ __launch_bounds__(256, OCC) void grouped_gemm_lds_kernel(GemmParams p) {
  using C = Cfg<BM>;
  constexpr int KCH = BK / 8;             // 16-byte chunks per row per K step
  constexpr int RPP = 256 / KCH;          // rows covered by one pass of 256 threads
  constexpr int NA = (BM + RPP - 1) / RPP;// A chunks per thread per K step
  constexpr int NB = BNB / RPP;           // B chunks per thread per K step
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const Item it = decode_item<BM, MODE>(p);
  if (it.row0 < 0) return;

  const int chunk = tid % KCH;
  const int trow = tid / KCH;
  const uint16_t* arow[NA];
  uint32_t amask = 0;  // bit i: chunk i carries data
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = trow + RPP * i;
    bool ok = false;
    arow[i] = (r < BM) ? a_row<MODE>(p, it, r, ok) : p.a;
    amask |= ok ? (1u << i) : 0u;
  }
  const uint16_t* brow[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) brow[i] = b_row<MODE>(p, it, trow + RPP * i);

  u32x4* sA = reinterpret_cast<u32x4*>(smem);            // [2][BM*KCH]
  u32x4* sB = sA + 2 * BM * KCH;                          // [2][BNB*KCH]
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 pa0[NA], pb0[NB], pa1[NA], pb1[NB];
  auto gload = [&](u32x4 (&pa)[NA], u32x4 (&pb)[NB], int kb) {
    const int koff = kb * BK + chunk * 8;
#pragma unroll
    for (int i = 0; i < NA; ++i) pa[i] = *reinterpret_cast<const u32x4*>(arow[i] + koff);
#pragma unroll
    for (int i = 0; i < NB; ++i) pb[i] = *reinterpret_cast<const u32x4*>(brow[i] + koff);
  };
  auto sstore = [&](const u32x4 (&pa)[NA], const u32x4 (&pb)[NB], int st) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int r = trow + RPP * i;
      if (r < BM) sA[st * BM * KCH + r * KCH + swz<KCH>(r, chunk)] = ((amask >> i) & 1u) ? pa[i] : zero;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int r = trow + RPP * i;
      sB[st * BNB * KCH + r * KCH + swz<KCH>(r, chunk)] = pb[i];
    }
  };
  int bb[C::NJ];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    constexpr int half = C::NJ / 2;
    bb[j] = (MODE == GATE_UP) ? (j < half ? wn * half * 32 + j * 32 : 128 + wn * half * 32 + (j - half) * 32)
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
  constexpr int SUB = BK / 16;

  // K loop: two LDS stages, two register sets of prefetched chunks (distance
  // 2), unrolled by two so each buffer has a fixed role; fragments one
  // sub-step ahead of their MFMAs, across the barrier too.  Loads past the end
  // re-read the last K step (unconditional loads keep the waits exact).
  // Order inside a step: the first fragment reads of the step, then the LDS
  // writes of the next step (their buffer was released by the barrier just
  // passed) and the global loads two steps ahead, then the MFMAs.  Writes
  // issued early have completed long before the next barrier, which would
  // otherwise wait for them.
  const int nk = p.K / BK;
  gload(pa0, pb0, 0);
  gload(pa1, pb1, 1);
  sstore(pa0, pb0, 0);
  gload(pa0, pb0, min(2, nk - 1));
  __syncthreads();
  Frag f0, f1;
  bool pending = false;
  auto stage = [&](int st, u32x4 (&pa)[NA], u32x4 (&pb)[NB], int next_kb) {
    read_frags(f0, st, 0);
    __builtin_amdgcn_sched_barrier(0);
    sstore(pa, pb, st ^ 1);
    gload(pa, pb, next_kb);
    __builtin_amdgcn_sched_barrier(0);
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
  };
  for (int kb = 0; kb < nk; kb += 2) {
    stage(0, pa1, pb1, min(kb + 3, nk - 1));  // writes step kb+1 -> LDS[1]
    __syncthreads();
    stage(1, pa0, pb0, min(kb + 4, nk - 1));  // writes step kb+2 -> LDS[0]
    __syncthreads();
  }
  if (pending) mma(f1);
  epilogue<BM, MODE, C::MI, C::NJ, C::WTM>(p, it, acc, wm, bb, smem);
}

// ------------------------------------------- kernel 2: B directly to MFMA

template <int BM, int BK>
constexpr size_t lds_bytes_bd() {
  size_t stages = 2 * (size_t)BM * (BK / 8) * 16;
  size_t epi = (size_t)BM * ESLD * 4;
  return stages > epi ? stages : epi;
}

// BM x 256 tile over 4 wavefronts that split only the columns: wavefront w
// owns 64 weight rows (GATE_UP: 32 gate rows and the 32 matching up rows),
// which no other wavefront needs, so they are loaded from global memory
// straight into MFMA operand registers (lane l: row l % 32, 8 K-values at
// 8 * (l / 32)).  Only the gathered token tile, which all four wavefronts
// share, is staged through LDS.  This halves the LDS traffic per MFMA.
template <int BM, int BK, int OCC, int MODE>
__global__ __launch_bounds__(256, OCC) void grouped_gemm_bd_kernel(GemmParams p) {
  constexpr int MI = BM / 32, NJ = 2;
  constexpr int KCH = BK / 8;
  constexpr int RPP = 256 / KCH;
  constexpr int NA = (BM + RPP - 1) / RPP;
  constexpr int SUB = BK / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wn = tid >> 6;
  const Item it = decode_item<BM, MODE>(p);
  if (it.row0 < 0) return;

  const int chunk = tid % KCH;
  const int trow = tid / KCH;
  const uint16_t* arow[NA];
  uint32_t amask = 0;
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = trow + RPP * i;
    bool ok = false;
    arow[i] = (r < BM) ? a_row<MODE>(p, it, r, ok) : p.a;
    amask |= ok ? (1u << i) : 0u;
  }
  int bb[NJ];
  bb[0] = (MODE == GATE_UP) ? wn * 32 : wn * 64;
  bb[1] = (MODE == GATE_UP) ? 128 + wn * 32 : wn * 64 + 32;
  const uint16_t* bq_row[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) bq_row[j] = b_row<MODE>(p, it, bb[j] + (lane & 31)) + 8 * (lane >> 5);

  u32x4* sA = reinterpret_cast<u32x4*>(smem);  // [2][BM*KCH]
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 pa0[NA], pa1[NA];
  bf16x8 bq0[SUB][NJ], bq1[SUB][NJ];  // B operands of one K step, two steps in flight
  auto gload_a = [&](u32x4 (&pa)[NA], int kb) {
    const int koff = kb * BK + chunk * 8;
#pragma unroll
    for (int i = 0; i < NA; ++i) pa[i] = *reinterpret_cast<const u32x4*>(arow[i] + koff);
  };
  auto gload_b = [&](bf16x8 (&bq)[SUB][NJ], int kb) {
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
      for (int j = 0; j < NJ; ++j) bq[sub][j] = *reinterpret_cast<const bf16x8*>(bq_row[j] + kb * BK + sub * 16);
  };
  auto sstore = [&](const u32x4 (&pa)[NA], int st) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int r = trow + RPP * i;
      if (r < BM) sA[st * BM * KCH + r * KCH + swz<KCH>(r, chunk)] = ((amask >> i) & 1u) ? pa[i] : zero;
    }
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int m = 0; m < MI; ++m)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[m][j][q] = 0.0f;

  auto read_a = [&](bf16x8 (&fa)[MI], int st, int sub) {
    const u32x4* cA = sA + st * BM * KCH;
    const int c = 2 * sub + (lane >> 5);
#pragma unroll
    for (int m = 0; m < MI; ++m) {
      const int r = m * 32 + (lane & 31);
      fa[m] = __builtin_bit_cast(bf16x8, cA[r * KCH + swz<KCH>(r, c)]);
    }
  };
  auto mma = [&](const bf16x8 (&fa)[MI], const bf16x8 (&fb)[NJ]) {
#pragma unroll
    for (int m = 0; m < MI; ++m)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[m], fb[j], acc[m][j], 0, 0, 0);
  };
  // One K step: A fragments from LDS stage st one sub-step ahead of the MFMAs.
  auto stage = [&](int st, const bf16x8 (&bq)[SUB][NJ]) {
    bf16x8 fa0[MI], fa1[MI];
    read_a(fa0, st, 0);
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub) {
      if (sub & 1) {
        if (sub + 1 < SUB) read_a(fa0, st, sub + 1);
        mma(fa1, bq[sub]);
      } else {
        if (sub + 1 < SUB) read_a(fa1, st, sub + 1);
        mma(fa0, bq[sub]);
      }
    }
  };

  // K loop: the token tile through two LDS stages (register prefetch distance
  // 2); the B operands of step kb+2 are loaded once step kb's MFMAs are
  // issued.  Unrolled by two; loads past the end re-read the last K step.
  const int nk = p.K / BK;
  gload_b(bq0, 0);
  gload_a(pa0, 0);
  gload_b(bq1, 1);
  gload_a(pa1, 1);
  sstore(pa0, 0);
  gload_a(pa0, min(2, nk - 1));
  __syncthreads();
  for (int kb = 0; kb < nk; kb += 2) {
    stage(0, bq0);
    gload_b(bq0, min(kb + 2, nk - 1));
    sstore(pa1, 1);
    gload_a(pa1, min(kb + 3, nk - 1));
    __syncthreads();
    stage(1, bq1);
    gload_b(bq1, min(kb + 3, nk - 1));
    sstore(pa0, 0);
    gload_a(pa0, min(kb + 4, nk - 1));
    __syncthreads();
  }
  epilogue<BM, MODE, MI, NJ, BM>(p, it, acc, 0, bb, smem);
}

// Combine without a shared expert: y[t,c] = sum_j w[t,j] o[inv[t*k+j], c].
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int T, int H, int k,
                                                      uint16_t* __restrict__ y) {
  const int per_tok = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)T * per_tok) return;
  const int t = (int)(idx / per_tok);
  const int col = (int)(idx % per_tok) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const u32x4 ov = *reinterpret_cast<const u32x4*>(o + (size_t)inv[(size_t)t * k + j] * H + col);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += wj * bf16_to_f32((uint16_t)(ov[q] & 0xffff));
      acc[2 * q + 1] += wj * bf16_to_f32((uint16_t)(ov[q] >> 16));
    }
  }
  u32x4 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
              pack_bf16x2(acc[6], acc[7])};
  *reinterpret_cast<u32x4*>(y + (size_t)t * H + col) = pk;
}

#ifndef MOE_GEMM_BDIRECT
#define MOE_GEMM_BDIRECT 0
#endif

template <int BM, int BK, int OCC, int MODE>
hipError_t launch_mode(const GemmParams& p, int64_t max_items, hipStream_t st) {
  const int64_t grid = ((max_items + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (grid <= 0) return hipSuccess;
  const void* fn;
  size_t lds;
  if (MOE_GEMM_BDIRECT) {
    fn = (const void*)grouped_gemm_bd_kernel<BM, BK, OCC, MODE>;
    lds = lds_bytes_bd<BM, BK>();
  } else {
    fn = (const void*)grouped_gemm_lds_kernel<BM, BK, OCC, MODE>;
    lds = lds_bytes_lds<BM, BK>();
  }
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (MOE_GEMM_BDIRECT)
    hipLaunchKernelGGL((grouped_gemm_bd_kernel<BM, BK, OCC, MODE>), dim3((unsigned)grid), dim3(256), lds, st, p);
  else
    hipLaunchKernelGGL((grouped_gemm_lds_kernel<BM, BK, OCC, MODE>), dim3((unsigned)grid), dim3(256), lds, st, p);
  return hipGetLastError();
}

// Tile configuration per tile height: (BM, K step, workgroups per CU).
#ifndef MOE_GEMM_CFG_256
#define MOE_GEMM_CFG_256 256, 32, 1
#endif
#ifndef MOE_GEMM_CFG_128
#define MOE_GEMM_CFG_128 128, 32, 2
#endif
#ifndef MOE_GEMM_CFG_64
#define MOE_GEMM_CFG_64 64, 32, 2
#endif
#ifndef MOE_GEMM_CFG_32
#define MOE_GEMM_CFG_32 32, 32, 2
#endif

template <int MODE>
hipError_t launch_bm(int BM, const GemmParams& p, int64_t max_items, hipStream_t st) {
  switch (BM) {
    case 32: return launch_mode<MOE_GEMM_CFG_32, MODE>(p, max_items, st);
    case 64: return launch_mode<MOE_GEMM_CFG_64, MODE>(p, max_items, st);
    case 128: return launch_mode<MOE_GEMM_CFG_128, MODE>(p, max_items, st);
    case 256: return launch_mode<MOE_GEMM_CFG_256, MODE>(p, max_items, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gate_up(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up,
                          const uint16_t* ws_gate, const uint16_t* ws_up, const int32_t* sorted,
                          const int32_t* tiles, const int32_t* n_tiles, int T, int H, int E, int k, int I,
                          int I_s, int BM, int64_t max_tiles, uint16_t* h, uint16_t* h_s, hipStream_t st) {
  (void)E;
  GemmParams p = {};
  p.a = x;
  p.lda = H;
  p.K = H;
  p.b0 = w_gate;
  p.b1 = w_up;
  p.bs0 = I_s > 0 ? ws_gate : nullptr;
  p.bs1 = I_s > 0 ? ws_up : nullptr;
  p.N = I;
  p.N_s = I_s;
  p.sorted = sorted;
  p.tiles = tiles;
  p.n_tiles = n_tiles;
  p.T = T;
  p.k = k;
  p.out = h;
  p.out_s = h_s;
  p.ldo = I;
  p.ldo_s = I_s;
  int64_t n_tok_tiles = (T + BM - 1) / BM;
  int64_t max_items = max_tiles * (I / 128) + (I_s > 0 ? n_tok_tiles * (I_s / 128) : 0);
  return launch_bm<GATE_UP>(BM, p, max_items, st);
}

hipError_t launch_down(const uint16_t* h, const uint16_t* w_down, const int32_t* sorted, const int32_t* tiles,
                       const int32_t* n_tiles, int T, int H, int E, int k, int I, int BM, int64_t max_tiles,
                       uint16_t* o, hipStream_t st) {
  (void)E;
  GemmParams p = {};
  p.a = h;
  p.lda = I;
  p.K = I;
  p.b0 = w_down;
  p.N = H;
  p.sorted = sorted;
  p.tiles = tiles;
  p.n_tiles = n_tiles;
  p.T = T;
  p.k = k;
  p.out = o;
  p.ldo = H;
  return launch_bm<DOWN>(BM, p, max_tiles * (H / 256), st);
}

hipError_t launch_combine(const uint16_t* o, const int32_t* inv, const float* w, const uint16_t* h_s,
                          const uint16_t* ws_down, const float* s, int T, int H, int k, int I_s, uint16_t* y,
                          hipStream_t st) {
  if (I_s == 0) {
    int64_t n = (int64_t)T * (H / 8);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, o, inv, w, T, H, k, y);
    return hipGetLastError();
  }
  constexpr int BM = 128;
  GemmParams p = {};
  p.a = h_s;
  p.lda = I_s;
  p.K = I_s;
  p.bs0 = ws_down;
  p.N_s = H;
  p.T = T;
  p.k = k;
  p.out_s = y;
  p.ldo = H;
  p.ldo_s = H;
  p.o = o;
  p.inv = inv;
  p.w = w;
  p.s = s;
  int64_t max_items = (int64_t)((T + BM - 1) / BM) * (H / 256);
  return launch_mode<MOE_GEMM_CFG_128, SHARED_COMBINE>(p, max_items, st);
}

}  // namespace moe
