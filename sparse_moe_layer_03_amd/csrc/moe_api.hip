// C ABI of libmoe355: argument validation, workspace carving and the order of
// the stage launches.  Every entry point validates its arguments on the host
// before any HIP call, so argument errors are reported with nothing enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Per-device cache of the architecture check: 0 unknown, 1 gfx950, 2 other.
int g_arch_state[64];

int check_arch() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_ARCH, "no HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_ARCH, "device index %d out of range", dev);
  if (g_arch_state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(MOE_ERR_ARCH, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_arch_state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (g_arch_state[dev] == 2)
      return fail(MOE_ERR_ARCH, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
  }
  if (g_arch_state[dev] != 1) return fail(MOE_ERR_ARCH, "device %d is not gfx950", dev);
  return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Mean rows per expert from which 256-row tiles (the persistent kernel) are
// used.  Measured on the decode-config layer without router bias, forward
// per tile height 64 / 256 rows (BF16 weights): 1,536 tokens (mean 48)
// 406 / 425 us, 2,048 tokens (mean 64) 451 / 438 us, 2,560 tokens 497 /
// 467 us, 4,096 tokens 589 / 521 us, 6,144 tokens 781 / 602 us (128-row
// tiles were between the two from a mean of 64 up).
#ifndef MOE_TILE256_MIN_MEAN
#define MOE_TILE256_MIN_MEAN 64
#endif

int env_rows(const char* name) {
  const char* s = getenv(name);  // tuning only
  const int r = s ? atoi(s) : 0;
  return (r == 32 || r == 64 || r == 128 || r == 256) ? r : 0;
}

int tile_rows_override() {
  static int v = -1;
  if (v < 0) v = env_rows("MOE_TILE_ROWS");
  return v;
}

int small_rows_override() {
  static int v = -1;
  if (v < 0) v = env_rows("MOE_SMALL_ROWS");
  return v;
}

int check_common_shapes(int T, int H, int E, int k) {
  if (T < 0 || T > (1 << 24)) return fail(MOE_ERR_SHAPE, "T=%d outside [0, 2^24]", T);
  if (E < 1 || E > kMaxE) return fail(MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, kMaxE);
  if (k < 1 || k > E || k > kMaxK) return fail(MOE_ERR_SHAPE, "k=%d outside [1, min(E, %d)]", k, kMaxK);
  if (H < 256 || H > 8192 || H % 256 != 0) return fail(MOE_ERR_SHAPE, "H=%d must be a multiple of 256 in [256, 8192]", H);
  return MOE_OK;
}

int check_ffn_shapes(int I, int I_s) {
  if (I < 128 || I % 128 != 0) return fail(MOE_ERR_SHAPE, "I=%d must be a positive multiple of 128", I);
  if (I_s < 0 || I_s % 128 != 0) return fail(MOE_ERR_SHAPE, "I_s=%d must be 0 or a multiple of 128", I_s);
  return MOE_OK;
}

struct Layout {
  int BIG, SMALL;
  bool ring3_gate_up;  // the gate/up launch's persistent kernel with the three-stage weight ring
  bool stream_w;       // the persistent launches load single-tile experts' weight rows non-temporally
  int64_t max_rows, max_big, max_small, max_tiles;
  size_t off_ids, off_w, off_s, off_counts, off_padoff, off_sorted, off_inv, off_tiles, off_ntiles,
      off_scratch, off_h, off_hs, off_o, total;
  WsSections sec;
};

// Tile capacities for tile heights (BIG, SMALL), SMALL <= BIG.
int64_t max_rows_for(int64_t n, int E, int64_t small) {
  const int64_t used = n < E ? n : E;
  return n + used * (small - 1);
}
int64_t max_big_for(int64_t n, int E, int64_t big, int64_t small) {
  const int64_t used = n < E ? n : E;
  if (small == big) return (n + used * (big - 1)) / big;  // sum of ceil(count / BIG)
  return n / big;
}
int64_t max_tiles_for(int64_t n, int E, int64_t big, int64_t small) {
  const int64_t used = n < E ? n : E;
  if (small == big) return max_big_for(n, E, big, small);
  int64_t max_small = used * (big / small);  // at most big/small SMALL tiles per expert
  const int64_t bound = (n + used * (small - 1)) / small;
  if (bound < max_small) max_small = bound;
  return max_big_for(n, E, big, small) + max_small;
}

// Workspace layout of the tiled path (BF16 and FP8 weights alike).
Layout layout(int T, int H, int E, int k, int I, int I_s) {
  Layout L = {};
  L.BIG = moe_align_tile_rows(T, E, k);
  L.SMALL = moe_align_small_tile_rows(T, E, k);
  L.ring3_gate_up = ring3_gate_up(T, E, k);
  L.stream_w = stream_weights(T, E, k);
  const int64_t nA = (int64_t)T * k;
  L.max_rows = max_rows_for(nA, E, L.SMALL);
  L.max_big = max_big_for(nA, E, L.BIG, L.SMALL);
  L.max_tiles = max_tiles_for(nA, E, L.BIG, L.SMALL);
  L.max_small = L.max_tiles - L.max_big;
  const size_t n = (size_t)T * k;
  auto take = [&](size_t bytes) { return L.sec.take(bytes); };
  L.off_ids = take(n * 4);
  L.off_w = take(n * 4);
  L.off_s = take((size_t)T * 4);
  L.off_counts = take((size_t)E * 4);
  L.off_padoff = take((size_t)(E + 1) * 4);
  L.off_sorted = take((size_t)L.max_rows * 4);
  L.off_inv = take(n * 4);
  L.off_tiles = take((size_t)L.max_tiles * 8);
  L.off_ntiles = take(8);
  L.off_scratch = take(moe_align_scratch_size(T, E, k));
  L.off_h = take((size_t)L.max_rows * I * 2);
  L.off_hs = take((size_t)T * (I_s > 0 ? I_s : 0) * 2);
  // o; before the down GEMM writes it, the same bytes hold the router's
  // fragment-order copy of W_router
  const size_t pack = router_pack_bytes(H, E);
  L.off_o = take(n * H * 2 > pack ? n * H * 2 : pack);
  L.total = L.sec.total;
  return L;
}

}  // namespace

int moe::set_error(int code, const char* msg) {
  if (code == MOE_OK) return ok();
  return fail(code, "%s", msg);
}

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_ARCH: return "MOE_ERR_ARCH";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err; }

int moe_align_tile_rows(int T, int E, int k) {
  const int ov = tile_rows_override();
  if (ov) return ov;
  if (E < 1) return 32;
  const int64_t avg = (int64_t)T * k / E;  // mean rows per expert
  if (avg >= MOE_TILE256_MIN_MEAN) return 256;
  // 64 from a mean of 32: with 32-row tiles, experts just above the mean take
  // two tiles and their weights cross HBM twice
  if (avg >= 32) return 64;
  return 32;
}

int moe_align_small_tile_rows(int T, int E, int k) {
  const int big = moe_align_tile_rows(T, E, k);
  const int ov = small_rows_override();
  return (ov && ov <= big) ? ov : big;  // one tile class unless overridden
}

int64_t moe_align_max_rows(int T, int E, int k) {
  return max_rows_for((int64_t)T * k, E, moe_align_small_tile_rows(T, E, k));
}

int64_t moe_align_max_big_tiles(int T, int E, int k) {
  return max_big_for((int64_t)T * k, E, moe_align_tile_rows(T, E, k), moe_align_small_tile_rows(T, E, k));
}

int64_t moe_align_max_tiles(int T, int E, int k) {
  return max_tiles_for((int64_t)T * k, E, moe_align_tile_rows(T, E, k), moe_align_small_tile_rows(T, E, k));
}

size_t moe_align_scratch_size(int T, int E, int k) {
  // per-chunk histograms, per-chunk exclusive offsets, per-expert tile-list offsets
  if (T < 1 || E < 1 || k < 1) return 256;
  return (size_t)align_scratch_ints(T, E, k) * 4;
}

size_t moe_workspace_size(int T, int H, int E, int k, int I, int I_s) {
  if (check_common_shapes(T, H, E, k) != MOE_OK || check_ffn_shapes(I, I_s) != MOE_OK) return 0;
  if (T <= 1) return decode_workspace_size(H, E, k, I, I_s);
  if (T <= kSmallMaxT) return small_batch_workspace_size(T, H, E, k, I, I_s);
  return layout(T, H, E, k, I, I_s).total;
}

size_t moe_forward_ids_offset(int T, int H, int E, int k, int I, int I_s) {
  if (moe_workspace_size(T, H, E, k, I, I_s) == 0) return 0;
  if (T <= 1) return decode_ids_offset(H, E, k, I, I_s);
  if (T <= kSmallMaxT) return small_batch_ids_offset(T, H, E, k, I, I_s);
  return layout(T, H, E, k, I, I_s).off_ids;
}

int moe_workspace_sections(int T, int H, int E, int k, int I, int I_s, size_t* offsets, size_t* bytes, int max) {
  if (moe_workspace_size(T, H, E, k, I, I_s) == 0) return 0;
  const WsSections w = T <= 1 ? decode_sections(H, E, k, I, I_s)
                       : T <= kSmallMaxT ? small_batch_sections(T, H, E, k, I, I_s)
                                         : layout(T, H, E, k, I, I_s).sec;
  for (int i = 0; i < w.n && i < max; ++i) {
    if (offsets) offsets[i] = w.off[i];
    if (bytes) bytes[i] = w.bytes[i];
  }
  return w.n;
}

size_t moe_route_scratch_size(int T, int H, int E) {
  if (check_common_shapes(T, H, E, 1) != MOE_OK) return 0;
  return router_pack_bytes(H, E);
}

int moe_route(const uint16_t* x, const uint16_t* w_router, const float* router_bias, const uint16_t* w_sg, int T,
              int H, int E, int k, int32_t* ids, float* w, float* s, float* logits, void* scratch,
              size_t scratch_bytes, void* stream) {
  int rc = check_common_shapes(T, H, E, k);
  if (rc) return rc;
  if (T == 0) return ok();
  if (!x || !w_router || !ids || !w) return fail(MOE_ERR_NULL, "moe_route: x, w_router, ids and w are required");
  if (w_sg && !s) return fail(MOE_ERR_NULL, "moe_route: s is required when w_sg is given");
  if (!aligned16(x) || !aligned16(w_router) || (w_sg && !aligned16(w_sg)))
    return fail(MOE_ERR_ALIGN, "moe_route: bf16 tensors must be 16-byte aligned");
  if (scratch) {
    const size_t need = router_pack_bytes(H, E);
    if (scratch_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "moe_route: scratch holds %zu bytes, %zu needed", scratch_bytes, need);
    if (!aligned16(scratch)) return fail(MOE_ERR_ALIGN, "moe_route: scratch must be 16-byte aligned");
  }
  if ((rc = check_arch())) return rc;
  const hipStream_t st = (hipStream_t)stream;
  if (scratch)
    return hip_status(launch_router_stream(x, w_router, router_bias, w_sg, T, H, E, k, scratch, logits, s, ids, w,
                                           nullptr, 0, st),
                      "moe_route: streamed router with top-k");
  return hip_status(launch_router(x, w_router, router_bias, w_sg, T, H, E, k, logits, s, ids, w, st),
                    "moe_route: router GEMM with top-k");
}

int moe_route_from_logits(const float* logits, int T, int E, int k, int32_t* ids, float* w, void* stream) {
  if (T < 0 || T > (1 << 24)) return fail(MOE_ERR_SHAPE, "T=%d outside [0, 2^24]", T);
  if (E < 1 || E > kMaxE) return fail(MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, kMaxE);
  if (k < 1 || k > E || k > kMaxK) return fail(MOE_ERR_SHAPE, "k=%d outside [1, min(E, %d)]", k, kMaxK);
  if (T == 0) return ok();
  if (!logits || !ids || !w) return fail(MOE_ERR_NULL, "moe_route_from_logits: logits, ids and w are required");
  int rc = check_arch();
  if (rc) return rc;
  return hip_status(launch_topk(logits, T, E, k, ids, w, (hipStream_t)stream), "moe_route_from_logits");
}

int moe_align(const int32_t* ids, int T, int E, int k, int32_t* counts, int32_t* pad_off, int32_t* sorted,
              int32_t* inv, int32_t* tiles, int32_t* n_tiles, void* scratch, size_t scratch_bytes, void* stream) {
  if (T < 0 || T > (1 << 24)) return fail(MOE_ERR_SHAPE, "T=%d outside [0, 2^24]", T);
  if (E < 1 || E > kMaxE) return fail(MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, kMaxE);
  if (k < 1 || k > E || k > kMaxK) return fail(MOE_ERR_SHAPE, "k=%d outside [1, min(E, %d)]", k, kMaxK);
  if (T == 0) return ok();
  if (!ids || !counts || !pad_off || !sorted || !inv || !tiles || !n_tiles || !scratch)
    return fail(MOE_ERR_NULL, "moe_align: every output and the scratch buffer are required");
  if (!aligned16(scratch)) return fail(MOE_ERR_ALIGN, "moe_align: scratch must be 16-byte aligned");
  if (scratch_bytes < moe_align_scratch_size(T, E, k))
    return fail(MOE_ERR_WORKSPACE, "moe_align: scratch of %zu bytes, %zu needed", scratch_bytes,
                moe_align_scratch_size(T, E, k));
  int rc = check_arch();
  if (rc) return rc;
  return hip_status(launch_align(ids, T, E, k, moe_align_tile_rows(T, E, k), moe_align_small_tile_rows(T, E, k),
                                 (int)moe_align_max_big_tiles(T, E, k), counts, pad_off, sorted, inv, tiles, n_tiles,
                                 static_cast<int32_t*>(scratch), (hipStream_t)stream),
                    "moe_align");
}

namespace {
// The routed GEMMs of both tile classes (tile heights and capacities of L).
hipError_t launch_routed_gate_up(const uint16_t* x, const void* w_gate, const void* w_up, const int32_t* sorted,
                                 const int32_t* tiles, const int32_t* n_tiles, int T, int H, int k, int I,
                                 uint16_t* h, const void* ws_gate, const void* ws_up, int I_s, uint16_t* h_s,
                                 const Layout& L, hipStream_t st, const FP8Scales* q = nullptr) {
  hipError_t e = launch_gate_up(x, w_gate, w_up, sorted, tiles, n_tiles, T, H, k, I, L.BIG, L.max_big, h, ws_gate,
                                ws_up, I_s, h_s, st, q, L.ring3_gate_up, L.stream_w);
  if (e != hipSuccess || L.SMALL == L.BIG) return e;
  return launch_gate_up(x, w_gate, w_up, sorted, tiles + 2 * L.max_big, n_tiles + 1, T, H, k, I, L.SMALL, L.max_small,
                        h, nullptr, nullptr, 0, nullptr, st, q);
}

hipError_t launch_routed_down(const uint16_t* h, const void* w_down, const int32_t* sorted, const int32_t* tiles,
                              const int32_t* n_tiles, int T, int H, int k, int I, uint16_t* o, const Layout& L,
                              hipStream_t st, const FP8Scales* q = nullptr) {
  hipError_t e =
      launch_down(h, w_down, sorted, tiles, n_tiles, T, H, k, I, L.BIG, L.max_big, o, st, q, true, L.stream_w);
  if (e != hipSuccess || L.SMALL == L.BIG) return e;
  return launch_down(h, w_down, sorted, tiles + 2 * L.max_big, n_tiles + 1, T, H, k, I, L.SMALL, L.max_small, o, st,
                     q);
}

// The tiled path of moe_forward / moe_forward_fp8 (T > the small-batch limit)
// on the workspace layout L; q: FP8 row scales (NULL: BF16 weights).
int forward_tiled(const uint16_t* x, const uint16_t* w_router, const float* router_bias, const void* w_gate,
                  const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up, const void* ws_down,
                  const uint16_t* w_sg, int T, int H, int E, int k, int I, int I_s, uint16_t* y, void* workspace,
                  const Layout& L, const FP8Scales* q, hipStream_t st) {
  char* base = static_cast<char*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(base + L.off_ids);
  float* w = reinterpret_cast<float*>(base + L.off_w);
  float* s = reinterpret_cast<float*>(base + L.off_s);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.off_counts);
  int32_t* pad_off = reinterpret_cast<int32_t*>(base + L.off_padoff);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + L.off_sorted);
  int32_t* inv = reinterpret_cast<int32_t*>(base + L.off_inv);
  int32_t* tiles = reinterpret_cast<int32_t*>(base + L.off_tiles);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(base + L.off_ntiles);
  int32_t* scratch = reinterpret_cast<int32_t*>(base + L.off_scratch);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + L.off_h);
  uint16_t* h_s = I_s > 0 ? reinterpret_cast<uint16_t*>(base + L.off_hs) : nullptr;
  uint16_t* o = reinterpret_cast<uint16_t*>(base + L.off_o);

  // router over K slices; the partial logits live in o's bytes until the
  // selection has read them
  // the router also counts align's chunk histograms into the align scratch
  hipError_t e = launch_router_stream(x, w_router, router_bias, I_s > 0 ? w_sg : nullptr, T, H, E, k, o, nullptr,
                                      I_s > 0 ? s : nullptr, ids, w, scratch, align_num_chunks(T, k), st);
  if (e != hipSuccess) return hip_status(e, "moe_forward: router with top-k");
  e = launch_align_scan(ids, T, E, k, L.BIG, L.SMALL, (int)L.max_big, counts, pad_off, sorted, inv, tiles, n_tiles,
                        scratch, st);
  if (e != hipSuccess) return hip_status(e, "moe_forward: align");
  e = launch_routed_gate_up(x, w_gate, w_up, sorted, tiles, n_tiles, T, H, k, I, h, ws_gate, ws_up, I_s, h_s, L, st, q);
  if (e != hipSuccess) return hip_status(e, "moe_forward: gate_up (routed + shared)");
  e = launch_routed_down(h, w_down, sorted, tiles, n_tiles, T, H, k, I, o, L, st, q);
  if (e != hipSuccess) return hip_status(e, "moe_forward: down");
  e = launch_combine(o, w, h_s, ws_down, I_s > 0 ? s : nullptr, T, H, k, I_s, y, st, q);
  return hip_status(e, "moe_forward: combine");
}
}  // namespace

int moe_grouped_gate_up(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* ws_gate,
                        const uint16_t* ws_up, const int32_t* sorted, const int32_t* tiles, const int32_t* n_tiles,
                        int T, int H, int E, int k, int I, int I_s, uint16_t* h, uint16_t* h_s, void* stream) {
  int rc = check_common_shapes(T, H, E, k);
  if (rc || (rc = check_ffn_shapes(I, I_s))) return rc;
  if (T == 0) return ok();
  if (!x || !w_gate || !w_up || !sorted || !tiles || !n_tiles || !h)
    return fail(MOE_ERR_NULL, "moe_grouped_gate_up: missing pointer");
  if (I_s > 0 && (!ws_gate || !ws_up || !h_s)) return fail(MOE_ERR_NULL, "moe_grouped_gate_up: shared tensors");
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(h) ||
      (I_s > 0 && (!aligned16(ws_gate) || !aligned16(ws_up) || !aligned16(h_s))))
    return fail(MOE_ERR_ALIGN, "moe_grouped_gate_up: tensors must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  return hip_status(launch_routed_gate_up(x, w_gate, w_up, sorted, tiles, n_tiles, T, H, k, I, h, ws_gate, ws_up, I_s,
                                          h_s, layout(T, H, E, k, I, I_s), (hipStream_t)stream),
                    "moe_grouped_gate_up");
}

int moe_grouped_down(const uint16_t* h, const uint16_t* w_down, const int32_t* sorted, const int32_t* tiles,
                     const int32_t* n_tiles, int T, int H, int E, int k, int I, uint16_t* o, void* stream) {
  int rc = check_common_shapes(T, H, E, k);
  if (rc || (rc = check_ffn_shapes(I, 0))) return rc;
  if (T == 0) return ok();
  if (!h || !w_down || !sorted || !tiles || !n_tiles || !o) return fail(MOE_ERR_NULL, "moe_grouped_down: missing pointer");
  if (!aligned16(h) || !aligned16(w_down) || !aligned16(o))
    return fail(MOE_ERR_ALIGN, "moe_grouped_down: tensors must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  return hip_status(launch_routed_down(h, w_down, sorted, tiles, n_tiles, T, H, k, I, o, layout(T, H, E, k, I, 0),
                                       (hipStream_t)stream),
                    "moe_grouped_down");
}

int moe_combine(const uint16_t* o, const float* w, const uint16_t* h_s, const uint16_t* ws_down,
                const float* s, int T, int H, int k, int I_s, uint16_t* y, void* stream) {
  if (T < 0 || T > (1 << 24)) return fail(MOE_ERR_SHAPE, "T=%d outside [0, 2^24]", T);
  if (k < 1 || k > kMaxK) return fail(MOE_ERR_SHAPE, "k=%d outside [1, %d]", k, kMaxK);
  if (H < 256 || H > 8192 || H % 256 != 0) return fail(MOE_ERR_SHAPE, "H=%d must be a multiple of 256", H);
  if (I_s < 0 || I_s % 128 != 0) return fail(MOE_ERR_SHAPE, "I_s=%d must be 0 or a multiple of 128", I_s);
  if (T == 0) return ok();
  if (!o || !w || !y) return fail(MOE_ERR_NULL, "moe_combine: missing pointer");
  if (I_s > 0 && (!h_s || !ws_down || !s)) return fail(MOE_ERR_NULL, "moe_combine: shared tensors");
  if (I_s == 0 && (h_s || ws_down || s)) return fail(MOE_ERR_SHAPE, "moe_combine: shared tensors given with I_s = 0");
  if (!aligned16(o) || !aligned16(y) || (I_s > 0 && (!aligned16(h_s) || !aligned16(ws_down))))
    return fail(MOE_ERR_ALIGN, "moe_combine: tensors must be 16-byte aligned");
  int rc = check_arch();
  if (rc) return rc;
  return hip_status(launch_combine(o, w, h_s, ws_down, s, T, H, k, I_s, y, (hipStream_t)stream), "moe_combine");
}

int moe_forward(const uint16_t* x, const uint16_t* w_router, const float* router_bias, const uint16_t* w_gate,
                const uint16_t* w_up, const uint16_t* w_down, const uint16_t* ws_gate, const uint16_t* ws_up,
                const uint16_t* ws_down, const uint16_t* w_sg, int T, int H, int E, int k, int I, int I_s,
                uint16_t* y, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_common_shapes(T, H, E, k);
  if (rc || (rc = check_ffn_shapes(I, I_s))) return rc;
  const int n_shared = (ws_gate != nullptr) + (ws_up != nullptr) + (ws_down != nullptr) + (w_sg != nullptr);
  if (I_s == 0 && n_shared != 0) return fail(MOE_ERR_SHAPE, "shared-expert tensors given with I_s = 0");
  if (I_s > 0 && n_shared != 4) return fail(MOE_ERR_NULL, "I_s > 0 needs ws_gate, ws_up, ws_down and w_sg");
  if (T == 0) return ok();
  if (!x || !w_router || !w_gate || !w_up || !w_down || !y || !workspace)
    return fail(MOE_ERR_NULL, "x, w_router, w_gate, w_up, w_down, y and workspace are required");
  const void* ptrs[] = {x, w_router, w_gate, w_up, w_down, y, ws_gate, ws_up, ws_down, w_sg};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
  const size_t need = moe_workspace_size(T, H, E, k, I, I_s);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  if ((rc = check_arch())) return rc;
  hipStream_t st = (hipStream_t)stream;

  if (T <= kSmallMaxT) {
    ExpertWeights W = {};
    W.gate = w_gate, W.up = w_up, W.down = w_down, W.s_gate = ws_gate, W.s_up = ws_up, W.s_down = ws_down;
    W.fmt = W_BF16;
    if (T == 1)
      return hip_status(launch_decode(x, w_router, router_bias, w_sg, W, H, E, k, I, I_s, y, workspace, st),
                        "moe_forward (decode)");
    return hip_status(launch_small_batch(x, w_router, router_bias, w_sg, W, T, H, E, k, I, I_s, y, workspace, st),
                      "moe_forward (small batch)");
  }

  return forward_tiled(x, w_router, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, w_sg, T, H, E, k, I,
                       I_s, y, workspace, layout(T, H, E, k, I, I_s), nullptr, st);
}

// Workspace of moe_forward_noalloc: one array in every GPU's memory, held until the process ends.
// Host code reaches it only through the per-device address hipGetSymbolAddress returns (the array's
// name is a host-side stand-in there).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_WS_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of `scratch` per device index, set at the first call there

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_ARCH, "no HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_ARCH, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "moe_forward_noalloc: hipGetSymbolAddress of the workspace array: %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

int moe_forward_noalloc(const uint16_t* x, const uint16_t* w_router, const float* router_bias,
                        const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                        const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                        const uint16_t* w_sg, int T, int H, int E, int k, int I, int I_s, uint16_t* y,
                        void* stream) {
  int rc = check_common_shapes(T, H, E, k);
  if (rc || (rc = check_ffn_shapes(I, I_s))) return rc;
  if (T == 0) return ok();
  const size_t need = moe_workspace_size(T, H, E, k, I, I_s);
  if (need > (size_t)MOE_NOALLOC_WS_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_noalloc: these sizes need %zu bytes of workspace, more than its fixed %zu "
                "(use moe_forward with a caller workspace)",
                need, (size_t)MOE_NOALLOC_WS_BYTES);
  if ((rc = check_arch())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return moe_forward(x, w_router, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, w_sg, T, H, E, k, I,
                     I_s, y, ws, (size_t)MOE_NOALLOC_WS_BYTES, stream);
}

int moe_forward_fp8(const uint16_t* x, const uint16_t* w_router, const float* router_bias, const uint8_t* q_gate,
                    const float* sc_gate, const uint8_t* q_up, const float* sc_up, const uint8_t* q_down,
                    const float* sc_down, const uint8_t* qs_gate, const float* ssc_gate, const uint8_t* qs_up,
                    const float* ssc_up, const uint8_t* qs_down, const float* ssc_down, const uint16_t* w_sg, int T,
                    int H, int E, int k, int I, int I_s, uint16_t* y, void* workspace, size_t ws_bytes,
                    void* stream) {
  int rc = check_common_shapes(T, H, E, k);
  if (rc || (rc = check_ffn_shapes(I, I_s))) return rc;
  const int n_shared = (qs_gate != nullptr) + (ssc_gate != nullptr) + (qs_up != nullptr) + (ssc_up != nullptr) +
                       (qs_down != nullptr) + (ssc_down != nullptr) + (w_sg != nullptr);
  if (I_s == 0 && n_shared != 0) return fail(MOE_ERR_SHAPE, "moe_forward_fp8: shared-expert tensors given with I_s = 0");
  if (I_s > 0 && n_shared != 7)
    return fail(MOE_ERR_NULL, "moe_forward_fp8: I_s > 0 needs qs_*, ssc_* (gate, up, down) and w_sg");
  if (T == 0) return ok();
  if (!x || !w_router || !q_gate || !sc_gate || !q_up || !sc_up || !q_down || !sc_down || !y || !workspace)
    return fail(MOE_ERR_NULL, "moe_forward_fp8: x, w_router, q_*/sc_* (gate, up, down), y and workspace are required");
  const void* ptrs[] = {x,       w_router, q_gate, sc_gate, q_up,     sc_up,  q_down,   sc_down, y,
                        qs_gate, ssc_gate, qs_up,  ssc_up,  qs_down, ssc_down, w_sg};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_ALIGN, "moe_forward_fp8: tensor pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MOE_ERR_ALIGN, "moe_forward_fp8: workspace must be 256-byte aligned");
  const size_t need = moe_workspace_size(T, H, E, k, I, I_s);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  if ((rc = check_arch())) return rc;
  hipStream_t st = (hipStream_t)stream;
  ExpertWeights W = {};
  W.gate = q_gate, W.up = q_up, W.down = q_down, W.s_gate = qs_gate, W.s_up = qs_up, W.s_down = qs_down;
  W.sc_gate = sc_gate, W.sc_up = sc_up, W.sc_down = sc_down;
  W.ssc_gate = ssc_gate, W.ssc_up = ssc_up, W.ssc_down = ssc_down;
  W.fmt = W_FP8;
  if (T == 1)
    return hip_status(launch_decode(x, w_router, router_bias, w_sg, W, H, E, k, I, I_s, y, workspace, st),
                      "moe_forward_fp8 (decode)");
  if (T <= kSmallMaxT)
    return hip_status(launch_small_batch(x, w_router, router_bias, w_sg, W, T, H, E, k, I, I_s, y, workspace, st),
                      "moe_forward_fp8 (small batch)");
  const FP8Scales q = {sc_gate, sc_up, sc_down, ssc_gate, ssc_up, ssc_down};
  return forward_tiled(x, w_router, router_bias, q_gate, q_up, q_down, qs_gate, qs_up, qs_down, w_sg, T, H, E, k, I,
                       I_s, y, workspace, layout(T, H, E, k, I, I_s), &q, st);
}

int moe_forward_q4(const uint16_t* x, const uint16_t* w_router, const float* router_bias, const uint8_t* q_gate,
                   const uint16_t* s_gate, const uint8_t* q_up, const uint16_t* s_up, const uint8_t* q_down,
                   const uint16_t* s_down, const uint8_t* qs_gate, const uint16_t* ss_gate, const uint8_t* qs_up,
                   const uint16_t* ss_up, const uint8_t* qs_down, const uint16_t* ss_down, const uint16_t* w_sg, int T,
                   int H, int E, int k, int I, int I_s, uint16_t* y, void* workspace, size_t ws_bytes,
                   void* stream) {
  int rc = check_common_shapes(T, H, E, k);
  if (rc || (rc = check_ffn_shapes(I, I_s))) return rc;
  if (T > MOE_Q4_MAX_T)
    return fail(MOE_ERR_SHAPE, "moe_forward_q4: T=%d; 4-bit expert weights are supported for T <= %d", T, MOE_Q4_MAX_T);
  const int n_shared = (qs_gate != nullptr) + (ss_gate != nullptr) + (qs_up != nullptr) + (ss_up != nullptr) +
                       (qs_down != nullptr) + (ss_down != nullptr) + (w_sg != nullptr);
  if (I_s == 0 && n_shared != 0) return fail(MOE_ERR_SHAPE, "moe_forward_q4: shared-expert tensors given with I_s = 0");
  if (I_s > 0 && n_shared != 7)
    return fail(MOE_ERR_NULL, "moe_forward_q4: I_s > 0 needs qs_*, ss_* (gate, up, down) and w_sg");
  if (T == 0) return ok();
  if (!x || !w_router || !q_gate || !s_gate || !q_up || !s_up || !q_down || !s_down || !y || !workspace)
    return fail(MOE_ERR_NULL, "moe_forward_q4: x, w_router, q_*/s_* (gate, up, down), y and workspace are required");
  const void* ptrs[] = {x,       w_router, q_gate, s_gate, q_up,    s_up,    q_down, s_down, y,
                        qs_gate, ss_gate,  qs_up,  ss_up,  qs_down, ss_down, w_sg};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_ALIGN, "moe_forward_q4: tensor pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MOE_ERR_ALIGN, "moe_forward_q4: workspace must be 256-byte aligned");
  const size_t need = moe_workspace_size(T, H, E, k, I, I_s);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  if ((rc = check_arch())) return rc;
  hipStream_t st = (hipStream_t)stream;
  ExpertWeights W = {};
  W.gate = q_gate, W.up = q_up, W.down = q_down, W.s_gate = qs_gate, W.s_up = qs_up, W.s_down = qs_down;
  W.gs_gate = s_gate, W.gs_up = s_up, W.gs_down = s_down;
  W.gss_gate = ss_gate, W.gss_up = ss_up, W.gss_down = ss_down;
  W.fmt = W_Q4;
  if (T == 1)
    return hip_status(launch_decode(x, w_router, router_bias, w_sg, W, H, E, k, I, I_s, y, workspace, st),
                      "moe_forward_q4 (decode)");
  return hip_status(launch_small_batch(x, w_router, router_bias, w_sg, W, T, H, E, k, I, I_s, y, workspace, st),
                    "moe_forward_q4 (small batch)");
}

int moe_e4m3_to_f32(const uint8_t* codes, float* out, int64_t n, void* stream) {
  if (n < 0) return fail(MOE_ERR_SHAPE, "moe_e4m3_to_f32: n=%lld < 0", (long long)n);
  if (n == 0) return ok();
  if (!codes || !out) return fail(MOE_ERR_NULL, "moe_e4m3_to_f32: codes and out are required");
  if (!aligned16(codes) || !aligned16(out)) return fail(MOE_ERR_ALIGN, "moe_e4m3_to_f32: pointers must be 16-byte aligned");
  int rc = check_arch();
  if (rc) return rc;
  return hip_status(launch_e4m3_to_f32(codes, out, n, (hipStream_t)stream), "moe_e4m3_to_f32");
}

}  // extern "C"
