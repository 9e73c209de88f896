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
// Two kernels: per-chunk histograms (LDS integer counters: the counts do not
// depend on the order of the increments), then one workgroup per chunk that
// reads every chunk's histogram (a few tens of KB from L2), derives the expert
// totals, the padded offsets (block scans over the experts) and its own
// chunk's starting row per expert, ranks its assignments in order with wave
// ballots (no ordering atomics), and writes the tile entries and padding rows
// of a share of the experts.  Every workgroup computes the same totals and
// offsets, so no workgroup waits for another (a single scanning workgroup
// between the two launches cost ~7 us of latency at 65,536 assignments).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int CHMAX = 1024;  // most assignments per chunk (align_chunk)

// chunk_hist[e * nc + c]: assignments of chunk c routed to expert e (expert-major,
// so the scan reads one expert's chunk counts contiguously)
__global__ __launch_bounds__(256) void align_hist_kernel(const int32_t* __restrict__ ids, int n, int E, int nc,
                                                         int ch, int32_t* __restrict__ chunk_hist) {
  __shared__ int32_t hist[kMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * ch;
  const int a1 = min(a0 + ch, n);
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

// One workgroup per chunk c.  Every workgroup derives the totals and padded
// offsets from the chunk histograms (the same integer sums everywhere);
// workgroup 0 stores counts, pad_off and n_tiles.  Then the chunk's
// assignments are ranked in order and scattered, and the tile-table entries
// and padding rows of the experts e = c, c + gridDim.x, ... are written.
__global__ __launch_bounds__(256) void align_scan_scatter_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                 int nc, int ch, int BIG, int SMALL, int small_base,
                                                                 const int32_t* __restrict__ chunk_hist,
                                                                 int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ pad_off,
                                                                 int32_t* __restrict__ n_tiles,
                                                                 int32_t* __restrict__ sorted, int32_t* __restrict__ inv,
                                                                 int32_t* __restrict__ tiles) {
  __shared__ int32_t base[kMaxE];
  __shared__ int32_t wcnt[4][kMaxE];
  __shared__ int32_t s_run[kMaxE], s_poff[kMaxE], s_boff[kMaxE], s_soff[kMaxE];
  __shared__ int sbuf[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  // the chunk's expert ids, loaded before the histograms so that the ranking
  // below waits for no load (clamped, not skipped: a load under a per-lane
  // condition is waited for on its own)
  const int a0 = c * ch;
  const int a1 = min(a0 + ch, n);
  int ea_pre[CHMAX / 256];
#pragma unroll
  for (int it = 0; it < CHMAX / 256; ++it) {
    const int a = a0 + it * 256 + tid;
    const int v = ids[min(a, n - 1)];
    ea_pre[it] = a < a1 ? v : 0;
  }
  // expert e = tid: its total over all chunks and its share in the chunks before c (the chunk
  // counts of one expert are contiguous, nc a multiple of 4, read 64 at a time with 16-byte loads)
  const int e = tid;
  int run = 0, pre = 0;
  if (e < E) {
    const int4* src = reinterpret_cast<const int4*>(chunk_hist + (size_t)e * nc);
    for (int q0 = 0; q0 < nc / 4; q0 += 16) {
      int4 hv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) hv[i] = (q0 + i < nc / 4) ? src[q0 + i] : make_int4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c0 = 4 * (q0 + i);
        run += hv[i].x + hv[i].y + hv[i].z + hv[i].w;
        pre += (c0 < c ? hv[i].x : 0) + (c0 + 1 < c ? hv[i].y : 0) + (c0 + 2 < c ? hv[i].z : 0) +
               (c0 + 3 < c ? hv[i].w : 0);
      }
    }
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
    base[e] = rows_off + pre;
    s_run[e] = run;
    s_poff[e] = rows_off;
    s_boff[e] = big_off;
    s_soff[e] = small_off;
    if (c == 0) {
      counts[e] = run;
      pad_off[e] = rows_off;
    }
  }
  if (c == 0 && e == 0) {
    pad_off[E] = total_rows;
    n_tiles[0] = total_big;
    n_tiles[1] = total_small;
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int it = 0; it < CHMAX / 256; ++it) {
    const int s0 = a0 + it * 256;
    if (s0 >= a1) break;  // uniform (also past a chunk of fewer than CHMAX)
    for (int i = tid; i < 4 * kMaxE; i += 256) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const int a = s0 + tid;
    const bool valid = a < a1;
    const int ea = ea_pre[it];
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (ea >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    if (!valid) peers = 0;
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wave][ea] = __popcll(peers);  // lowest peer reports the group size
    __syncthreads();
    if (valid) {
      int pos = base[ea] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][ea];
      sorted[pos] = a;
      inv[a] = pos;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += 256) base[ee] += wcnt[0][ee] + wcnt[1][ee] + wcnt[2][ee] + wcnt[3][ee];
    __syncthreads();
  }
  for (int e2 = c; e2 < E; e2 += gridDim.x) {
    const int r2 = s_run[e2];
    const int nb2 = one ? (r2 + BIG - 1) / BIG : r2 / BIG;
    const int ns2 = one ? 0 : (r2 - nb2 * BIG + SMALL - 1) / SMALL;
    const int pd2 = nb2 * BIG + ns2 * SMALL;
    const int p0 = s_poff[e2], b0 = s_boff[e2], t0 = small_base + s_soff[e2];
    for (int i = tid; i < nb2; i += 256) {
      tiles[2 * (b0 + i)] = e2;
      tiles[2 * (b0 + i) + 1] = p0 + i * BIG;
    }
    for (int i = tid; i < ns2; i += 256) {
      tiles[2 * (t0 + i)] = e2;
      tiles[2 * (t0 + i) + 1] = p0 + nb2 * BIG + i * SMALL;
    }
    for (int r = r2 + tid; r < pd2; r += 256) sorted[p0 + r] = -1;
  }
}

}  // namespace

// Chunks of align_chunk assignments, rounded up to a multiple of 4 (the scan
// reads 4 chunk counts per 16-byte load; chunks past the end are empty).
int align_scratch_ints(int T, int E, int k) { return align_num_chunks(T, k) * E + 64; }

int align_chunk(int T, int k) {
  const int64_t n = (int64_t)T * k;
  return n >= 65536 ? 1024 : n >= 16384 ? 512 : 256;
}

int align_num_chunks(int T, int k) {
  const int64_t ch = align_chunk(T, k);
  return (int)((((int64_t)T * k + ch - 1) / ch + 3) / 4 * 4);
}

hipError_t launch_align(const int32_t* ids, int T, int E, int k, int BIG, int SMALL, int small_base,
                        int32_t* counts, int32_t* pad_off, int32_t* sorted, int32_t* inv, int32_t* tiles,
                        int32_t* n_tiles, int32_t* scratch, hipStream_t st) {
  const int n = T * k;
  const int nc = align_num_chunks(T, k), ch = align_chunk(T, k);
  int32_t* chunk_hist = scratch;
  hipLaunchKernelGGL(align_hist_kernel, dim3(nc), dim3(256), 0, st, ids, n, E, nc, ch, chunk_hist);
  hipLaunchKernelGGL(align_scan_scatter_kernel, dim3(nc), dim3(256), 0, st, ids, n, E, nc, ch, BIG, SMALL,
                     small_base, chunk_hist, counts, pad_off, n_tiles, sorted, inv, tiles);
  return hipGetLastError();
}

hipError_t launch_align_scan(const int32_t* ids, int T, int E, int k, int BIG, int SMALL, int small_base,
                             int32_t* counts, int32_t* pad_off, int32_t* sorted, int32_t* inv, int32_t* tiles,
                             int32_t* n_tiles, int32_t* scratch, hipStream_t st) {
  const int n = T * k;
  const int nc = align_num_chunks(T, k), ch = align_chunk(T, k);
  hipLaunchKernelGGL(align_scan_scatter_kernel, dim3(nc), dim3(256), 0, st, ids, n, E, nc, ch, BIG, SMALL,
                     small_base, scratch, counts, pad_off, n_tiles, sorted, inv, tiles);
  return hipGetLastError();
}

}  // namespace moe
