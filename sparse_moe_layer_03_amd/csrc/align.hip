// Align stage: expert histogram, prefix scan and a stable permutation of the
// token->expert assignments into per-expert row ranges padded to whole tiles.
//
// The layer evaluates each expert's FFN only on the tokens routed to it
// (guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B", data path: selected-expert
// MoE); grouping the assignments by expert turns that into one dense GEMM
// tile sequence per expert (kongchang.com "GFX1151 engine", MoE kernel
// section: sparse routing changes the access pattern, which this grouping
// makes regular again).
//
// Result (bit-exact, independent of scheduling):
//   counts[e]   number of assignments a = t*k + j with ids[a] = e
//   rows of e   floor(counts[e] / BIG) tiles of BIG rows, then the remainder
//               padded to whole tiles of SMALL rows (SMALL divides BIG); with
//               SMALL == BIG, ceil(counts[e] / BIG) tiles, all in the BIG list
//   pad_off[e]  sum of the padded row counts of the experts before e
//   sorted[pad_off[e] + r] = the r-th assignment of expert e in ascending a;
//                            -1 for the padding rows of the expert's last tile
//   inv[a]      the padded row that holds assignment a
//   tiles       (expert, first row) of every BIG tile, experts ascending; the
//               SMALL tiles likewise from entry small_base on
//   n_tiles     {number of BIG tiles, number of SMALL tiles}
//
// Three kernels: per-chunk histograms (LDS integer counters: the counts do
// not depend on the order of the increments), one workgroup that scans the
// chunk histograms and the expert totals, and a scatter in which every chunk
// ranks its assignments in order with wave ballots (no ordering atomics) and
// writes the tile entries and padding rows of a share of the experts.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int CH = 1024;  // assignments per chunk

// chunk_hist[e * nc + c]: assignments of chunk c routed to expert e (expert-major,
// so the scan reads one expert's chunk counts contiguously)
__global__ __launch_bounds__(256) void align_hist_kernel(const int32_t* __restrict__ ids, int n, int E, int nc,
                                                         int32_t* __restrict__ chunk_hist) {
  __shared__ int32_t hist[kMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * CH;
  const int a1 = min(a0 + CH, n);
  for (int a = a0 + tid; a < a1; a += 256) atomicAdd(&hist[ids[a]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 256) chunk_hist[(size_t)e * nc + blockIdx.x] = hist[e];
}

// Exclusive scan of one value per thread over the 256 threads of a block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* sbuf, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sbuf[wave] = incl;
  __syncthreads();
  int wave_off = 0;
  for (int w = 0; w < wave; ++w) wave_off += sbuf[w];
  total = sbuf[0] + sbuf[1] + sbuf[2] + sbuf[3];
  __syncthreads();
  return wave_off + incl - v;
}

__global__ __launch_bounds__(256) void align_scan_kernel(const int32_t* __restrict__ chunk_hist,
                                                         int32_t* __restrict__ chunk_off, int n_chunks, int E,
                                                         int BIG, int SMALL, int32_t* __restrict__ counts, int32_t* __restrict__ pad_off,
                                                         int32_t* __restrict__ tile_off, int32_t* __restrict__ n_tiles) {
  __shared__ int sbuf[4];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    // exclusive offset of every chunk within expert e; the expert's counts are
    // contiguous (nc is a multiple of 4), read 64 at a time with 16-byte loads
    const int4* src = reinterpret_cast<const int4*>(chunk_hist + (size_t)e * n_chunks);
    int4* dst = reinterpret_cast<int4*>(chunk_off + (size_t)e * n_chunks);
    for (int c0 = 0; c0 < n_chunks / 4; c0 += 16) {
      int4 hv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) hv[i] = (c0 + i < n_chunks / 4) ? src[c0 + i] : make_int4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        int4 o;
        o.x = run;
        o.y = o.x + hv[i].x;
        o.z = o.y + hv[i].y;
        o.w = o.z + hv[i].z;
        run = o.w + hv[i].w;
        if (c0 + i < n_chunks / 4) dst[c0 + i] = o;
      }
    }
    counts[e] = run;
  }
  const bool one = SMALL == BIG;
  const int nbig = (e < E) ? (one ? (run + BIG - 1) / BIG : run / BIG) : 0;
  const int rem = (e < E && !one) ? run - nbig * BIG : 0;
  const int nsmall = (rem + SMALL - 1) / SMALL;
  const int padded = nbig * BIG + nsmall * SMALL;
  int total_rows, total_big, total_small;
  const int rows_off = block_exclusive_scan(padded, sbuf, total_rows);
  const int big_off = block_exclusive_scan(nbig, sbuf, total_big);
  const int small_off = block_exclusive_scan(nsmall, sbuf, total_small);
  if (e < E) {
    pad_off[e] = rows_off;
    tile_off[e] = big_off;  // first BIG-list entry of expert e
    tile_off[kMaxE + e] = small_off;
  }
  if (e == 0) {
    pad_off[E] = total_rows;
    n_tiles[0] = total_big;
    n_tiles[1] = total_small;
  }
}

// Also writes, for the experts e = blockIdx.x, blockIdx.x + gridDim.x, ...,
// their tile-table entries and the -1 of their padding rows (all threads of
// the workgroup share each expert's writes).
__global__ __launch_bounds__(256) void align_scatter_kernel(const int32_t* __restrict__ ids, int n, int E, int nc,
                                                            int BIG, int SMALL, int small_base,
                                                            const int32_t* __restrict__ chunk_off,
                                                            const int32_t* __restrict__ pad_off,
                                                            const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ tile_off,
                                                            int32_t* __restrict__ sorted, int32_t* __restrict__ inv,
                                                            int32_t* __restrict__ tiles) {
  __shared__ int32_t base[kMaxE];
  __shared__ int32_t wcnt[4][kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int a0 = blockIdx.x * CH;
  const int a1 = min(a0 + CH, n);
  for (int e = tid; e < E; e += 256) base[e] = pad_off[e] + chunk_off[(size_t)e * nc + blockIdx.x];
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s0 = a0; s0 < a1; s0 += 256) {
    for (int i = tid; i < 4 * kMaxE; i += 256) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const int a = s0 + tid;
    const bool valid = a < a1;
    const int e = valid ? ids[a] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    if (!valid) peers = 0;
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wave][e] = __popcll(peers);  // lowest peer reports the group size
    __syncthreads();
    if (valid) {
      int pos = base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      sorted[pos] = a;
      inv[a] = pos;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += 256) base[ee] += wcnt[0][ee] + wcnt[1][ee] + wcnt[2][ee] + wcnt[3][ee];
    __syncthreads();
  }
  const bool one = SMALL == BIG;
  for (int e = blockIdx.x; e < E; e += gridDim.x) {
    const int run = counts[e];
    const int nbig = one ? (run + BIG - 1) / BIG : run / BIG;
    const int nsmall = one ? 0 : (run - nbig * BIG + SMALL - 1) / SMALL;
    const int padded = nbig * BIG + nsmall * SMALL;
    const int p0 = pad_off[e], b0 = tile_off[e], s0 = small_base + tile_off[kMaxE + e];
    for (int i = tid; i < nbig; i += 256) {
      tiles[2 * (b0 + i)] = e;
      tiles[2 * (b0 + i) + 1] = p0 + i * BIG;
    }
    for (int i = tid; i < nsmall; i += 256) {
      tiles[2 * (s0 + i)] = e;
      tiles[2 * (s0 + i) + 1] = p0 + nbig * BIG + i * SMALL;
    }
    for (int r = run + tid; r < padded; r += 256) sorted[p0 + r] = -1;
  }
}

}  // namespace

// Chunks of CH assignments, rounded up to a multiple of 4 (the scan reads 4
// chunk counts per 16-byte load; chunks past the end are empty).
int align_scratch_ints(int T, int E, int k) { return 2 * align_num_chunks(T, k) * E + 2 * kMaxE; }

int align_num_chunks(int T, int k) { return (int)((((int64_t)T * k + CH - 1) / CH + 3) / 4 * 4); }

hipError_t launch_align(const int32_t* ids, int T, int E, int k, int BIG, int SMALL, int small_base,
                        int32_t* counts, int32_t* pad_off, int32_t* sorted, int32_t* inv, int32_t* tiles,
                        int32_t* n_tiles, int32_t* scratch, hipStream_t st) {
  const int n = T * k;
  const int nc = align_num_chunks(T, k);
  int32_t* chunk_hist = scratch;
  int32_t* chunk_off = scratch + (size_t)nc * E;
  int32_t* tile_off = chunk_off + (size_t)nc * E;  // [2][kMaxE]
  hipLaunchKernelGGL(align_hist_kernel, dim3(nc), dim3(256), 0, st, ids, n, E, nc, chunk_hist);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(256), 0, st, chunk_hist, chunk_off, nc, E, BIG, SMALL, counts,
                     pad_off, tile_off, n_tiles);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(nc), dim3(256), 0, st, ids, n, E, nc, BIG, SMALL, small_base, chunk_off,
                     pad_off, counts, tile_off, sorted, inv, tiles);
  return hipGetLastError();
}

}  // namespace moe
