// Internal declarations shared by the HIP translation units of libmoe355.
// Nothing here is part of the C ABI (see include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;      // MI355X: 8 accelerator complex dies, workgroups dealt round-robin
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;
constexpr int kSmallMaxT = 32;  // moe_forward takes the small-batch path for 2 <= T <= kSmallMaxT

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Formats of the expert weight matrices.
enum { W_BF16 = 0, W_FP8 = 1, W_Q4 = 2 };

// 8 signed 4-bit weights (weight i in bits 4i..4i+3) and the fp16 bits of
// their group's scale.
struct q4chunk {
  uint32_t w, s;
};

// Eight consecutive weights of one row as one load: 16 bytes of BF16, 8 bytes
// of FP8 E4M3 codes, or 4 bytes of 4-bit weights with their group scale.
template <int F> struct WChunk { typedef u32x4 type; };
template <> struct WChunk<W_FP8> { typedef u32x2 type; };
template <> struct WChunk<W_Q4> { typedef q4chunk type; };
template <int F> using wchunk_t = typename WChunk<F>::type;

// One weight row as the single-token and small-batch kernels read it: chunk
// ch holds weights 8ch .. 8ch+7.
template <int F>
struct WRow {
  const char* p;      // row start
  const uint16_t* s;  // W_Q4: the row's fp16 group scales (one per 32 weights)
  __device__ __forceinline__ wchunk_t<F> operator[](int ch) const {
    if constexpr (F == W_Q4)
      return q4chunk{reinterpret_cast<const uint32_t*>(p)[ch], (uint32_t)s[ch >> 2]};
    else
      return reinterpret_cast<const wchunk_t<F>*>(p)[ch];
  }
};

// Row r (K weights long) of the matrix at m (gs: its group scales for W_Q4).
template <int F>
__device__ __forceinline__ WRow<F> wrow(const void* m, const uint16_t* gs, size_t r, int K) {
  WRow<F> w;
  const size_t bytes = F == W_BF16 ? (size_t)K * 2 : F == W_FP8 ? (size_t)K : (size_t)K / 2;
  w.p = static_cast<const char*>(m) + r * bytes;
  w.s = F == W_Q4 ? gs + r * (size_t)(K / 32) : nullptr;
  return w;
}

__device__ __forceinline__ void chunk_to_f32(const u32x4& w, float* f) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = bf16_to_f32((uint16_t)(w[q] & 0xffff));
    f[2 * q + 1] = bf16_to_f32((uint16_t)(w[q] >> 16));
  }
}

// OCP FP8 E4M3 codes (lowest byte first) to fp32 with the gfx950 conversion
// instruction, two codes per instruction; exact (every E4M3 value is an fp32).
__device__ __forceinline__ void chunk_to_f32(const u32x2& w, float* f) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], true);
    f[4 * q] = lo[0];
    f[4 * q + 1] = lo[1];
    f[4 * q + 2] = hi[0];
    f[4 * q + 3] = hi[1];
  }
}

// 4-bit weights times their group scale (exact in fp32: an 11-bit fp16
// significand times an integer of at most 4 bits).
__device__ __forceinline__ void chunk_to_f32(const q4chunk& c, float* f) {
  const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)c.s);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = sc * (float)((int32_t)(c.w << (28 - 4 * i)) >> 28);
}

// z / (1 + e^-z), with the hardware reciprocal (about 1 ulp) in place of the IEEE division, which
// costs ~10 instructions per element in the epilogues
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Sum over the 64 lanes: inclusive row sums by DPP row_shr 1, 2, 4, 8, then
// row_bcast:15 and row_bcast:31 carry the row totals up; lane 63 holds the
// total, which is returned to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  const int z = 0;
  int b = __float_as_int(v);
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(z, b, 0x111, 0xf, 0xf, false)));
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(z, b, 0x112, 0xf, 0xf, false)));
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(z, b, 0x114, 0xf, 0xf, false)));
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(z, b, 0x118, 0xf, 0xf, false)));
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(z, b, 0x142, 0xa, 0xf, false)));
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(z, b, 0x143, 0xc, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(b, 63));
}

// Map a linear workgroup id to a work item so that each XCD receives one
// contiguous run of items (items sharing an expert's weights stay in one
// XCD's L2).  `n_items` is known only on the device.  Returns -1 when this
// workgroup has no item.
__device__ __forceinline__ int xcd_item(int bid, int n_items) {
  int per = (n_items + kNumXcd - 1) / kNumXcd;
  int xcd = bid % kNumXcd;
  int slot = bid / kNumXcd;
  if (slot >= per) return -1;
  int item = xcd * per + slot;
  return item < n_items ? item : -1;
}

// Expert weights as the single-token and small-batch kernels take them (fmt):
// BF16 matrices; OCP FP8 E4M3 codes with one fp32 scale per output row (sc_*,
// ssc_*); or 4-bit weights, two per byte, with an fp16 scale per group of 32
// weights of a row (gs_*, gss_*).  Routed gate/up [E,I,H], down [E,H,I];
// shared gate/up [I_s,H], down [H,I_s].
struct ExpertWeights {
  const void *gate, *up, *down, *s_gate, *s_up, *s_down;
  const float *sc_gate, *sc_up, *sc_down, *ssc_gate, *ssc_up, *ssc_down;
  const uint16_t *gs_gate, *gs_up, *gs_down, *gss_gate, *gss_up, *gss_down;
  int fmt;
};

// Sections of a workspace: each starts 256-byte aligned and is followed by a
// gap of at least kWsGuard bytes that no kernel touches (moe_workspace_sections
// reports the sections, and a test checks that the gaps keep a fill pattern).
constexpr size_t kWsGuard = 256;
constexpr int kMaxWsSections = 16;
struct WsSections {
  int n = 0;
  size_t off[kMaxWsSections] = {};
  size_t bytes[kMaxWsSections] = {};
  size_t total = 0;
  // appends a section of `b` bytes and returns its offset
  size_t take(size_t b) {
    const size_t at = total;
    if (n < kMaxWsSections) {
      off[n] = at;
      bytes[n] = b;
      ++n;
    }
    total += ((b + 255) & ~(size_t)255) + kWsGuard;
    return at;
  }
};
WsSections decode_sections(int H, int E, int k, int I, int I_s);
WsSections small_batch_sections(int T, int H, int E, int k, int I, int I_s);

// Sets the thread's error message returned by moe_last_error() (cleared for
// MOE_OK) and returns `code`.
int set_error(int code, const char* msg);

// Host-side launch helpers (defined in the .hip files).
// Router GEMM over token tiles: fp32 logits (+ bias, -0 -> +0; stored when
// logits is not NULL), the top-k ids and renormalised weights of every token
// and, when w_sg is given, the shared-expert gate s = sigmoid(x . w_sg) from
// the same x tiles.
hipError_t launch_router(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg, int T,
                         int H, int E, int k, float* logits, float* s, int32_t* ids, float* w, hipStream_t st);
// Router for the tiled forward: 32-token tiles, the tile's x rows resident in
// LDS and W_router streamed into registers from a copy in fragment order
// (written to wpack, router_pack_bytes(H, E) bytes, 16-byte aligned, by a
// first launch), the selection and the shared gate in the same launch; the
// other arguments as launch_router.  chunk_hist (NULL: not counted): align's
// per-chunk expert counts [E][nc] (nc = align_num_chunks(T, k)), zeroed by the
// first launch and counted by the router, for launch_align_scan.
size_t router_pack_bytes(int H, int E);
hipError_t launch_router_stream(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg,
                                int T, int H, int E, int k, void* wpack, float* logits, float* s, int32_t* ids,
                                float* w, int32_t* chunk_hist, int nc, hipStream_t st);
// Top-k ids and renormalised weights from fp32 logits [T, E].
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st);
hipError_t launch_align(const int32_t* ids, int T, int E, int k, int BIG, int SMALL, int small_base,
                        int32_t* counts, int32_t* pad_off, int32_t* sorted, int32_t* inv, int32_t* tiles,
                        int32_t* n_tiles, int32_t* scratch, hipStream_t st);
// Assignments per align chunk (256, 512 or 1024: more and smaller chunks at
// fewer assignments, so that align runs on more workgroups): the histogram and
// scatter unit of align, and of the router's counts.
int align_chunk(int T, int k);
int align_num_chunks(int T, int k);
// The second launch of launch_align alone, on chunk histograms already in
// scratch (counted by launch_router_stream).
hipError_t launch_align_scan(const int32_t* ids, int T, int E, int k, int BIG, int SMALL, int small_base,
                             int32_t* counts, int32_t* pad_off, int32_t* sorted, int32_t* inv, int32_t* tiles,
                             int32_t* n_tiles, int32_t* scratch, hipStream_t st);
int align_scratch_ints(int T, int E, int k);
// Routed gate/up tiles of one tile list; with I_s > 0 the shared expert's
// gate/up over all T tokens (tiles of BM tokens) joins the same launch.
// Row scales of FP8 expert weights for the tiled GEMMs (NULL pointer to the
// struct: BF16 weights).  Routed gate/up [E,I], down [E,H]; shared gate/up
// [I_s], down [H].
struct FP8Scales {
  const float *gate, *up, *down, *s_gate, *s_up, *s_down;
};
// ring3: with 256-row tiles and BF16 weights, the persistent kernel loads the
// weight rows two K steps ahead (three weight stages); see ring3_gate_up.
// stream_w: with 256-row tiles and BF16 weights, the weight rows of an
// expert's only tile are loaded with the non-temporal hint; see stream_weights.
hipError_t launch_gate_up(const uint16_t* x, const void* w_gate, const void* w_up, const int32_t* sorted,
                          const int32_t* tiles, const int32_t* n_tiles, int T, int H, int k, int I, int BM,
                          int64_t max_tiles, uint16_t* h, const void* ws_gate, const void* ws_up, int I_s,
                          uint16_t* h_s, hipStream_t st, const FP8Scales* q = nullptr, bool ring3 = false,
                          bool stream_w = false);
hipError_t launch_down(const uint16_t* h, const void* w_down, const int32_t* sorted, const int32_t* tiles,
                       const int32_t* n_tiles, int T, int H, int k, int I, int BM, int64_t max_tiles, uint16_t* o,
                       hipStream_t st, const FP8Scales* q = nullptr, bool ring3 = true, bool stream_w = false);
// Whether the gate/up launch takes the three-stage weight ring: below a mean
// of 192 rows per expert (tiles partly filled, the launch streams weights).
inline bool ring3_gate_up(int T, int E, int k) { return E > 0 && (int64_t)T * k / E < 192; }
// Whether the persistent routed launches load single-tile experts' weight
// rows with the non-temporal hint: below a mean of 192 rows per expert, where
// the token rows, h and o that later launches read again then stay in the
// Infinity Cache (at larger means o outgrows it and the hint only costs).
inline bool stream_weights(int T, int E, int k) { return E > 0 && (int64_t)T * k / E < 192; }
hipError_t launch_combine(const uint16_t* o, const float* w, const uint16_t* h_s,
                          const void* ws_down, const float* s, int T, int H, int k, int I_s, uint16_t* y,
                          hipStream_t st, const FP8Scales* q = nullptr);
hipError_t launch_decode(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg,
                         const ExpertWeights& W, int H, int E, int k, int I, int I_s, uint16_t* y, void* ws,
                         hipStream_t st);
size_t decode_workspace_size(int H, int E, int k, int I, int I_s);
// Small-batch path (2 <= T <= kSmallMaxT): router, selection and plan, gate/up
// and down over the touched experts' weight rows, combine.
hipError_t launch_small_batch(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg,
                              const ExpertWeights& W, int T, int H, int E, int k, int I, int I_s, uint16_t* y,
                              void* ws, hipStream_t st);
// E4M3 codes to fp32 with the conversion the FP8 kernels use.
hipError_t launch_e4m3_to_f32(const uint8_t* codes, float* out, int64_t n, hipStream_t st);
size_t small_batch_workspace_size(int T, int H, int E, int k, int I, int I_s);
size_t small_batch_ids_offset(int T, int H, int E, int k, int I, int I_s);
size_t decode_ids_offset(int H, int E, int k, int I, int I_s);

}  // namespace moe
