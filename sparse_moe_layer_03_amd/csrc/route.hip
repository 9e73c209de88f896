// Top-k routing on router logits.
//
// The router GEMM (grouped_gemm.hip, ROUTER launch) writes fp32 logits
// (+ bias) and the shared-expert gate, and router_stream_kernel below is the
// router of the tiled forward.  Here one wavefront per token selects
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

// Router GEMM with the selection in its epilogue, for token tiles of 32
// (RS_BM) and one 512-thread workgroup per tile.  The tile's x rows stay in
// LDS (up to RS_KSEG columns at a time, loaded with direct-to-LDS loads);
// W_router is not staged: each wave streams its 32 weight rows straight into
// registers as MFMA operands, RS_D fragments (up to 32 KB per wave) in
// flight, so the load latency is covered by registers rather than by LDS
// stages.  The weights are read from a copy in fragment order
// (router_pack_kernel): one wave's fragment is then 1 KB of consecutive
// bytes, where the [E, H] rows would put its 32 rows in 32 cache lines (the
// load's cost grows with the lines it touches).
//
// Waves: NG = ceil(E / 32) groups of 32 experts; with E <= 128 the groups
// have KS = 2 or 4 waves on consecutive halves / quarters of each K segment,
// whose partial sums are added in LDS in wave order.  The x tile's 16-byte
// units sit in rows of 128 bytes per 64 columns (chunk), swizzled by the row,
// so 16 consecutive rows read at one unit hit 16 distinct bank groups.
constexpr int RS_BM = 32, RS_NT = 512, RS_KSEG = 2048;
constexpr int RS_LD = 256 + 8;  // fp32 row stride of the logits tile

struct RouterStreamArgs {
  const uint16_t* x;
  const uint16_t* wpack;  // W_router in fragment order
  const float* bias;
  const uint16_t* w_sg;
  int T, H, E, k, NG, KS;
  float* logits;
  float* s;
  int32_t* ids;
  float* w;
  int32_t* chunk_hist;  // align's per-chunk expert counts [E][nc] (NULL: not counted), zeroed by the copy launch
  int nc, ch;           // align's chunk count and assignments per chunk (>= 256)
};

__device__ __forceinline__ int rs_swz(int row, int u) { return u ^ (((row >> 1) ^ ((row & 1) << 2)) & 7); }

// 16 bytes per lane from src into LDS at lds + 16 * lane (M0 holds the base);
// waited for with rs_wait_vm0, which the compiler does not do for it
__device__ __forceinline__ void rs_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void rs_wait_vm0() { __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8)); }
// wait until no more than N vector-memory accesses of this wave are outstanding
template <int N>
__device__ __forceinline__ void rs_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// W_router [E, H] -> fragment order [NG][H / 16][64 lanes] of 16 bytes: lane l
// of group g and sub-step n holds row min(32 g + (l & 31), E - 1), columns
// 16 n + 8 (l >> 5) .. + 7 -- its operand of v_mfma_f32_32x32x16_bf16.  The
// same launch zeroes the nzero ints of zero (align's chunk histograms, which
// the router adds its counts to).
__global__ __launch_bounds__(256) void router_pack_kernel(const uint16_t* __restrict__ w, int H, int E, int NG,
                                                          uint16_t* __restrict__ wp, int32_t* __restrict__ zero,
                                                          int64_t nzero) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int NS = H / 16;
  if (u < nzero) zero[u] = 0;
  if (u >= (int64_t)NG * NS * 64) return;
  const int l = (int)(u & 63), n = (int)((u >> 6) % NS), g = (int)((u >> 6) / NS);
  const int e = min(32 * g + (l & 31), E - 1);
  *reinterpret_cast<u32x4*>(wp + u * 8) = *reinterpret_cast<const u32x4*>(w + (size_t)e * H + 16 * n + 8 * (l >> 5));
}

// RS_D: sub-steps (16 columns) per block of the K loop, a divisor of every
// segment's sub-step count nsl (32 for 2048 columns and E > 128).
template <int RS_D>
__global__ __launch_bounds__(RS_NT, 1) void router_stream_kernel(RouterStreamArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = blockIdx.x * RS_BM;
  const int nrow = min(RS_BM, a.T - row0);
  const int NG = a.NG, KS = a.KS;
  const bool active = wave < NG * KS;  // wave-uniform
  const int g = wave % NG, kq = wave / NG;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  const uint32_t lwsg = lds0 + RS_BM * RS_KSEG * 2;  // w_sg segment after the x tile

  // this lane's bias (clamped: columns past E are computed and never selected)
  const float bv = a.bias ? a.bias[min(32 * g + (lane & 31), a.E - 1)] : 0.0f;
  // this wave's weight fragments: 1 KB per sub-step of 16 columns
  const unsigned char* wg = reinterpret_cast<const unsigned char*>(a.wpack) + (size_t)g * (a.H / 16) * 1024;
  // A fragment of sub-step q (16 columns) of a chunk: row lane & 31, unit
  // 2 q + (lane >> 5)
  int aoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) aoff[q] = (lane & 31) * 128 + rs_swz(lane & 31, 2 * q + (lane >> 5)) * 16;
  // direct loads of the x tile: wave w fills row group w & 3 (8 rows) of the
  // chunks c = w / 4 + 2 m; lane l writes row l / 8 of the group at position
  // l & 7, which holds unit rs_swz(row, l & 7)
  const int rg = wave & 3, td = rg * 8 + (lane >> 3);
  const uint16_t* xsrc = a.x + (size_t)min(row0 + td, a.T - 1) * a.H + 8 * rs_swz(td, lane & 7);

  f32x16 acc0, acc1;  // even and odd sub-steps
#pragma unroll
  for (int q = 0; q < 16; ++q) acc0[q] = acc1[q] = 0.0f;
  // shared gate: x . w_sg as an MFMA whose weight operand holds w_sg in
  // column 0 only; wave w takes the sub-steps [w, w + 1) * nsub / 8 of each
  // segment, and the 8 waves' column-0 results are added in wave order
  f32x16 gacc;
#pragma unroll
  for (int q = 0; q < 16; ++q) gacc[q] = 0.0f;

  for (int k0 = 0; k0 < a.H; k0 += RS_KSEG) {
    const int kseg = min(RS_KSEG, a.H - k0), nch = kseg / 64;
    // this wave's sub-steps [n0, n0 + nsl) of 16 columns (nsl % 4 == 0)
    const int nsl = kseg / 16 / KS, n0 = kq * nsl;
    // all 8 waves active (E > 224) and at least 3 blocks of 32 sub-steps:
    // only chunks [0, 16) (the first two blocks) are loaded before the K
    // loop; the rest comes through registers in batches of 8 chunks, each
    // loaded at the start of a block and written to LDS at the start of the
    // next, before its sub-steps (the batches and their barriers are in the
    // active waves' loop, so every wave must be active)
    const bool xstream = RS_D == 32 && KS == 1 && NG == 8 && nsl >= 3 * RS_D;
    const int ndma = xstream ? 2 * RS_D / 4 : nch;
    for (int c = wave >> 2; c < ndma; c += 2) rs_dma16(xsrc + k0 + c * 64, lds0 + c * 4096 + rg * 1024);
    if (a.w_sg) {
      const int nu = kseg / 8;  // 16-byte units; the last instruction's lanes past them repeat the last
      for (int i = wave; i * 64 < nu; i += 8) rs_dma16(a.w_sg + k0 + 8 * min(i * 64 + lane, nu - 1), lwsg + i * 1024);
    }
    const unsigned char* wp = wg + (size_t)(k0 / 16 + n0) * 1024;  // wave-uniform
    const int lo = lane * 16;
    u32x4 wb[RS_D];
    if (active) {
#pragma unroll
      for (int j = 0; j < RS_D; ++j) wb[j] = *reinterpret_cast<const u32x4*>(wp + j * 1024 + lo);
    }
    // the direct loads have completed once no more than the weight loads
    // issued after them are outstanding (accesses complete in issue order)
    if (active)
      rs_wait_vm<RS_D>();
    else
      rs_wait_vm0();
    __syncthreads();
    if (active) {
      const unsigned char* xa = smem + (n0 >> 2) * 4096;
      // sub-step ib + j (ib % 4 == 0, j unrolled)
      auto step = [&](int ib, int j, const u32x4& b, f32x16& acc) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(xa + ((ib >> 2) + (j >> 2)) * 4096 + aoff[j & 3]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
      };
      u32x4 xr[4];
      int pend = -1;  // first chunk of the batch held in xr (-1: none)
      // chunks past the segment are clamped to its last one (loaded and
      // written again, unchanged)
      auto x_issue = [&](int cb) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int c = min(cb + (wave >> 2) + 2 * m, nch - 1);
          xr[m] = *reinterpret_cast<const u32x4*>(xsrc + k0 + c * 64);
        }
        pend = cb;
      };
      auto x_flush = [&]() {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int c = min(pend + (wave >> 2) + 2 * m, nch - 1);
          *reinterpret_cast<u32x4*>(smem + c * 4096 + rg * 1024 + lane * 16) = xr[m];
        }
        pend = -1;
        __syncthreads();
      };
      int i0 = 0;
      // whole blocks of RS_D sub-steps, each refilling its registers with the
      // sub-step RS_D ahead
      for (; i0 + 2 * RS_D <= nsl; i0 += RS_D) {
        if (xstream) {
          if (pend >= 0) x_flush();
          const int cb = 2 * RS_D / 4 + 8 * (i0 / RS_D);  // batch of this block
          if (cb < nch) x_issue(cb);
        }
#pragma unroll
        for (int j = 0; j < RS_D; ++j) {
          step(i0, j, wb[j], (j & 1) ? acc1 : acc0);
          wb[j] = *reinterpret_cast<const u32x4*>(wp + (i0 + RS_D + j) * 1024 + lo);
        }
      }
      if (pend >= 0) x_flush();
      // the last block: its sub-steps are in registers, nothing to load
#pragma unroll
      for (int j = 0; j < RS_D; ++j) step(i0, j, wb[j], (j & 1) ? acc1 : acc0);
    }
    __syncthreads();  // every wave's fragment reads of this x tile are done
    if (a.w_sg) {
      const int nsub = kseg / 16, g0 = wave * nsub / 8, g1 = (wave + 1) * nsub / 8;
      const unsigned char* wsl = smem + RS_BM * RS_KSEG * 2 + 16 * (lane >> 5);
      for (int n = g0; n < g1; ++n) {
        const int t = lane & 31;
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(smem + (n >> 2) * 4096 + t * 128 +
                                                           rs_swz(t, 2 * (n & 3) + (lane >> 5)) * 16);
        u32x4 b = *reinterpret_cast<const u32x4*>(wsl + n * 32);
        if (t != 0) b = u32x4{0u, 0u, 0u, 0u};
        gacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, b), gacc, 0, 0, 0);
      }
      __syncthreads();  // before the next segment's loads (or the logits) overwrite the tile
    }
  }

  // logits tile [32][RS_LD] over the x tile; KS > 1: the partial sums of waves
  // kq > 0 go after it, [kq - 1][g][16][64]
  float* sl = reinterpret_cast<float*>(smem);
  float* part = sl + RS_BM * RS_LD;
  f32x16 accf;
#pragma unroll
  for (int q = 0; q < 16; ++q) accf[q] = acc0[q] + acc1[q];
  if (KS > 1) {
    if (active && kq > 0)
#pragma unroll
      for (int q = 0; q < 16; ++q) part[(((kq - 1) * NG + g) * 16 + q) * 64 + lane] = accf[q];
    __syncthreads();
  }
  if (active && kq == 0) {
    for (int kk = 1; kk < KS; ++kk)
#pragma unroll
      for (int q = 0; q < 16; ++q) accf[q] += part[(((kk - 1) * NG + g) * 16 + q) * 64 + lane];
    const int col = 32 * g + (lane & 31);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      // output block: lane l holds column l & 31, rows 8 (q >> 2) + 4 (l >> 5) + (q & 3)
      const int row = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      float v = accf[q] + bv;
      if (v == 0.0f) v = 0.0f;  // -0 -> +0
      sl[row * RS_LD + col] = v;
    }
  }
  // column 0 of each wave's gate block: lanes 0 and 32
  float* gsum = part + (KS - 1) * NG * 1024;  // [8 waves][32 tokens]
  // the tile's assignments (32 k <= 512) fall in at most three of align's
  // chunks (>= 256 assignments each): their expert counts
  int* thist = reinterpret_cast<int*>(gsum + 8 * RS_BM);  // [3][E]
  if (a.chunk_hist)
    for (int i = tid; i < 3 * a.E; i += RS_NT) thist[i] = 0;
  if (a.w_sg && (lane & 31) == 0)
#pragma unroll
    for (int q = 0; q < 16; ++q) gsum[wave * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)] = gacc[q];
  __syncthreads();
  if (a.w_sg && tid < nrow) {
    float gs = gsum[tid];
#pragma unroll
    for (int w = 1; w < 8; ++w) gs += gsum[w * 32 + tid];
    a.s[row0 + tid] = 1.0f / (1.0f + expf(-gs));
  }
  if (a.logits) {
    float* out = a.logits + (size_t)row0 * a.E;
    for (int i = tid; i < nrow * a.E; i += RS_NT) out[i] = sl[(i / a.E) * RS_LD + i % a.E];
  }
  // selection: 16 lanes per token (row r of wave w: token 4 w + r), sub-lane
  // s holding experts 16 s .. 16 s + 15
  const int sub = lane & 15, tr = 4 * wave + (lane >> 4);
  uint64_t key[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float4 v4 = *reinterpret_cast<const float4*>(sl + tr * RS_LD + 16 * sub + 4 * c);
    const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ex = 16 * sub + 4 * c + q;
      key[4 * c + q] = topk_key64(vv[q], ex, ex < a.E);
    }
  }
  int sel_e;
  float sel_v;
  const float wt = a.k <= 8 ? row16_topk_weights<8>(key, a.k, sub, sel_e, sel_v)
                            : row16_topk_weights<16>(key, a.k, sub, sel_e, sel_v);
  if (tr < nrow && sub < a.k) {
    a.ids[(size_t)(row0 + tr) * a.k + sub] = sel_e;
    a.w[(size_t)(row0 + tr) * a.k + sub] = wt;
  }
  if (a.chunk_hist) {
    // integer counts: the same whatever the order of the additions
    const int c0 = (int)((int64_t)row0 * a.k / a.ch);
    if (tr < nrow && sub < a.k) {
      const int c = (int)(((int64_t)(row0 + tr) * a.k + sub) / a.ch);
      atomicAdd(&thist[(c - c0) * a.E + sel_e], 1);
    }
    __syncthreads();
    for (int i = tid; i < 3 * a.E; i += RS_NT) {
      const int v = thist[i];
      if (v) atomicAdd(&a.chunk_hist[(size_t)(i % a.E) * a.nc + c0 + i / a.E], v);
    }
  }
}

}  // namespace

size_t router_pack_bytes(int H, int E) { return (size_t)((E + 31) / 32) * H * 64; }

hipError_t launch_router_stream(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg,
                                int T, int H, int E, int k, void* wpack, float* logits, float* s, int32_t* ids,
                                float* w, int32_t* chunk_hist, int nc, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  RouterStreamArgs a = {x, static_cast<const uint16_t*>(wpack), bias, w_sg, T, H, E, k, 0, 0, logits, s, ids, w,
                        chunk_hist, nc, align_chunk(T, k)};
  a.NG = (E + 31) / 32;
  a.KS = a.NG >= 5 ? 1 : a.NG >= 3 ? 2 : 4;
  const int64_t units = (int64_t)a.NG * (H / 16) * 64;
  const int64_t nzero = chunk_hist ? (int64_t)nc * E : 0;
  const int64_t nthr = units > nzero ? units : nzero;
  hipLaunchKernelGGL(router_pack_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, st, w_router, H, E,
                     a.NG, static_cast<uint16_t*>(wpack), chunk_hist, nzero);
  const size_t kseg = (size_t)(H < RS_KSEG ? H : RS_KSEG);
  const size_t tile = (size_t)RS_BM * RS_KSEG * 2 + (w_sg ? (kseg * 2 + 1023) / 1024 * 1024 : 0);
  const size_t epi = (size_t)RS_BM * RS_LD * 4 + (size_t)(a.KS - 1) * a.NG * 4096 + 8 * RS_BM * 4 + 3 * E * 4;
  const size_t lds = tile > epi ? tile : epi;
  // sub-steps per block: the largest of 32, 16, 8, 4 that divides the
  // sub-step count of every segment (full segments of RS_KSEG columns, then
  // the rest)
  int D = 32;
  auto fits = [&](int d) {
    for (int k0 = 0; k0 < H; k0 += RS_KSEG) {
      const int ks = H - k0 < RS_KSEG ? H - k0 : RS_KSEG;
      if ((ks / 16 / a.KS) % d) return false;
    }
    return true;
  };
  while (D > 4 && !fits(D)) D /= 2;
  const void* fn = D == 32 ? (const void*)router_stream_kernel<32>
                 : D == 16 ? (const void*)router_stream_kernel<16>
                 : D == 8  ? (const void*)router_stream_kernel<8>
                           : (const void*)router_stream_kernel<4>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((T + RS_BM - 1) / RS_BM));
  switch (D) {
    case 32: hipLaunchKernelGGL(router_stream_kernel<32>, grid, dim3(RS_NT), lds, st, a); break;
    case 16: hipLaunchKernelGGL(router_stream_kernel<16>, grid, dim3(RS_NT), lds, st, a); break;
    case 8: hipLaunchKernelGGL(router_stream_kernel<8>, grid, dim3(RS_NT), lds, st, a); break;
    default: hipLaunchKernelGGL(router_stream_kernel<4>, grid, dim3(RS_NT), lds, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st) {
  dim3 grid((T + 3) / 4);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(256), 0, st, logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
