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

constexpr int BK = 32;       // K columns per LDS stage
constexpr int KCH = BK / 8;  // 16-byte chunks per row per stage
constexpr int BNB = 256;     // B rows per tile
constexpr int SLD = 132;     // fp32 row stride of the epilogue staging tile

enum { GATE_UP = 0, DOWN = 1, SHARED_COMBINE = 2 };

template <int BM>
struct Cfg;
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

__device__ __forceinline__ int swz4(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }

template <int BM>
constexpr size_t lds_bytes() {
  size_t stages = 2 * (size_t)(BM + BNB) * KCH * 16;
  size_t epi = (size_t)BM * SLD * 4;
  return stages > epi ? stages : epi;
}

template <int BM, int MODE>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(GemmParams p) {
  using C = Cfg<BM>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  // ---------------------------------------------------------------- item
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
  if (item < 0) return;
  bool shared;
  int expert = 0, row0, nb;
  if (MODE == GATE_UP && item < n_routed * nb_r) {
    shared = false;
    int tile = item / nb_r;
    nb = item % nb_r;
    expert = p.tiles[2 * tile];
    row0 = p.tiles[2 * tile + 1];
  } else if (MODE == DOWN) {
    shared = false;
    int tile = item / nb_r;
    nb = item % nb_r;
    expert = p.tiles[2 * tile];
    row0 = p.tiles[2 * tile + 1];
  } else {
    shared = true;
    int it = (MODE == GATE_UP) ? item - n_routed * nb_r : item;
    row0 = (it / nb_s) * BM;  // first token
    nb = it % nb_s;
  }

  // ------------------------------------------------------ row pointers
  constexpr int NA = BM >= 64 ? BM / 64 : 1;  // A chunks per thread per stage
  const uint16_t* arow[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    int r = (tid + 256 * i) >> 2;
    const uint16_t* ptr = nullptr;
    if (r < BM) {
      if (shared) {
        int t = row0 + r;
        if (t < p.T) ptr = p.a + (size_t)t * p.lda;
      } else {
        int a = p.sorted[row0 + r];
        if (a >= 0) {
          size_t src_row = (MODE == GATE_UP) ? (size_t)(a / p.k) : (size_t)(row0 + r);
          ptr = p.a + src_row * p.lda;
        }
      }
    }
    arow[i] = ptr;
  }
  const uint16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int j = (tid >> 2) + 64 * i;  // B row within the tile
    if (MODE == GATE_UP) {
      int col = nb * 128 + (j & 127);
      if (shared)
        brow[i] = (j < 128 ? p.bs0 : p.bs1) + (size_t)col * p.K;
      else
        brow[i] = (j < 128 ? p.b0 : p.b1) + ((size_t)expert * p.N + col) * p.K;
    } else {
      int col = nb * 256 + j;
      if (shared)
        brow[i] = p.bs0 + (size_t)col * p.K;
      else
        brow[i] = p.b0 + ((size_t)expert * p.N + col) * p.K;
    }
  }

  u32x4* sA = reinterpret_cast<u32x4*>(smem);            // [2][BM*KCH]
  u32x4* sB = sA + 2 * BM * KCH;                          // [2][BNB*KCH]
  const int chunk = tid & 3;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 pa[NA], pb[4];

  auto gload = [&](int kb) {
    const int koff = kb * BK + chunk * 8;
#pragma unroll
    for (int i = 0; i < NA; ++i) pa[i] = arow[i] ? *reinterpret_cast<const u32x4*>(arow[i] + koff) : zero;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = *reinterpret_cast<const u32x4*>(brow[i] + koff);
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      int r = (tid + 256 * i) >> 2;
      if (r < BM) sA[st * BM * KCH + r * KCH + swz4(r, chunk)] = pa[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = (tid >> 2) + 64 * i;
      sB[st * BNB * KCH + r * KCH + swz4(r, chunk)] = pb[i];
    }
  };

  // B row (within the tile) of the wave's column block j
  auto bblock = [&](int j) -> int {
    if (MODE == GATE_UP) {
      constexpr int half = C::NJ / 2;
      return j < half ? wn * half * 32 + j * 32 : 128 + wn * half * 32 + (j - half) * 32;
    }
    return wn * C::WTN + j * 32;
  };

  f32x16 acc[C::MI][C::NJ];
#pragma unroll
  for (int m = 0; m < C::MI; ++m)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[m][j][q] = 0.0f;

  const int nk = p.K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < nk) gload(kb + 1);
    const u32x4* cA = sA + st * BM * KCH;
    const u32x4* cB = sB + st * BNB * KCH;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = 2 * s + (lane >> 5);
      bf16x8 af[C::MI], bfr[C::NJ];
#pragma unroll
      for (int m = 0; m < C::MI; ++m) {
        int r = wm * C::WTM + m * 32 + (lane & 31);
        af[m] = __builtin_bit_cast(bf16x8, cA[r * KCH + swz4(r, c)]);
      }
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        int r = bblock(j) + (lane & 31);
        bfr[j] = __builtin_bit_cast(bf16x8, cB[r * KCH + swz4(r, c)]);
      }
#pragma unroll
      for (int m = 0; m < C::MI; ++m)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
          acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr[j], acc[m][j], 0, 0, 0);
    }
    if (kb + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

  // ----------------------------------------------------------- epilogue
  float* sc = reinterpret_cast<float*>(smem);  // [BM][SLD]
  const int npass = (MODE == GATE_UP) ? 1 : 2;
  const int cr = tid >> 4;        // copy-out: row within a 16-row group
  const int cc = (tid & 15) * 8;  // copy-out: first of 8 columns
  for (int pass = 0; pass < npass; ++pass) {
    // accumulators -> staging tile (fp32), 128 columns
#pragma unroll
    for (int m = 0; m < C::MI; ++m) {
      if (MODE == GATE_UP) {
        constexpr int half = C::NJ / 2;
#pragma unroll
        for (int j = 0; j < half; ++j) {
          int col = bblock(j) + (lane & 31);
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            int row = wm * C::WTM + m * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            sc[row * SLD + col] = silu(acc[m][j][q]) * acc[m][j + half][q];
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
          int col = bblock(j) + (lane & 31) - pass * 128;
          if (col >= 0 && col < 128) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              int row = wm * C::WTM + m * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
              sc[row * SLD + col] = acc[m][j][q];
            }
          }
        }
      }
    }
    __syncthreads();
    for (int r = cr; r < BM; r += 16) {
      const float4 v0 = *reinterpret_cast<const float4*>(sc + r * SLD + cc);
      const float4 v1 = *reinterpret_cast<const float4*>(sc + r * SLD + cc + 4);
      float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      if (MODE == GATE_UP) {
        u32x4 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7])};
        if (shared) {
          int t = row0 + r;
          if (t < p.T) *reinterpret_cast<u32x4*>(p.out_s + (size_t)t * p.ldo_s + nb * 128 + cc) = pk;
        } else {
          *reinterpret_cast<u32x4*>(p.out + (size_t)(row0 + r) * p.ldo + nb * 128 + cc) = pk;
        }
      } else if (MODE == DOWN) {
        if (p.sorted[row0 + r] >= 0) {
          u32x4 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7])};
          *reinterpret_cast<u32x4*>(p.out + (size_t)(row0 + r) * p.ldo + nb * 256 + pass * 128 + cc) = pk;
        }
      } else {
        const int t = row0 + r;
        if (t < p.T) {
          const int col = nb * 256 + pass * 128 + cc;
          float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          for (int j = 0; j < p.k; ++j) {
            const float wj = p.w[(size_t)t * p.k + j];
            const u32x4 ov = *reinterpret_cast<const u32x4*>(p.o + (size_t)p.inv[(size_t)t * p.k + j] * p.ldo + col);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              y[2 * q] += wj * bf16_to_f32((uint16_t)(ov[q] & 0xffff));
              y[2 * q + 1] += wj * bf16_to_f32((uint16_t)(ov[q] >> 16));
            }
          }
          const float st = p.s[t];
#pragma unroll
          for (int q = 0; q < 8; ++q) y[q] += st * v[q];
          u32x4 pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                      pack_bf16x2(y[6], y[7])};
          *reinterpret_cast<u32x4*>(p.out_s + (size_t)t * p.ldo_s + col) = pk;
        }
      }
    }
    __syncthreads();
  }
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

template <int BM, int MODE>
hipError_t launch_mode(const GemmParams& p, int64_t max_items, hipStream_t st) {
  constexpr size_t lds = lds_bytes<BM>();
  hipError_t e = hipFuncSetAttribute((const void*)grouped_gemm_kernel<BM, MODE>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int64_t grid = ((max_items + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<BM, MODE>), dim3((unsigned)grid), dim3(256), lds, st, p);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_bm(int BM, const GemmParams& p, int64_t max_items, hipStream_t st) {
  switch (BM) {
    case 32: return launch_mode<32, MODE>(p, max_items, st);
    case 64: return launch_mode<64, MODE>(p, max_items, st);
    case 128: return launch_mode<128, MODE>(p, max_items, st);
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
  return launch_mode<BM, SHARED_COMBINE>(p, max_items, st);
}

}  // namespace moe
