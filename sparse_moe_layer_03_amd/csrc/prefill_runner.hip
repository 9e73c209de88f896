// Prefill of any token count through fixed-size buckets (native runtime
// around moe_forward).
//
// guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B" (data-path section: any prompt
// is decomposed into optimised q8192 tiles, q1024 and a tail path; runtime
// section: a process keeps q1024/q2048/q4096/q8192 buckets resident, covers
// each prompt with the smallest bucket total and pads only the final
// segment).  Here a bucket is a HIP graph of one moe_forward call over a
// fixed number of tokens, captured once on staging buffers that the runner
// owns.  A prompt of T tokens is covered by the planner's segments (largest
// buckets first, the only partial segment last).  A full segment runs the
// bucket's launches straight on the caller's rows.  For the partial segment
// the runner gathers its rows into the staging input (the padding rows
// repeat the segment's own rows, so the expert loads look like a real
// batch), replays the bucket's graph and copies the real rows out.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <memory>
#include <new>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxBuckets = 16;
constexpr int kMaxBucketTokens = 1 << 16;
constexpr int kMaxPlanUnits = 1 << 20;  // dynamic-programming table bound (entries)

int gcd(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Stage rows: out[r] = x[start + r % len] for r < rows (16-byte chunks).
__global__ __launch_bounds__(256) void gather_pad_kernel(const uint16_t* __restrict__ x, int64_t start, int len,
                                                         int rows, int chunks_per_row, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * chunks_per_row) return;
  const int r = (int)(i / chunks_per_row), c = (int)(i % chunks_per_row);
  const u32x4* src = reinterpret_cast<const u32x4*>(x) + (start + r % len) * chunks_per_row + c;
  reinterpret_cast<u32x4*>(out)[i] = *src;
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace {

int plan_error(int code, const char* msg) { return set_error(code, msg); }

int check_buckets(const int* buckets, int n_buckets, std::vector<int>& sorted_desc, int& g) {
  if (!buckets) return plan_error(MOE_ERR_NULL, "bucket list is NULL");
  if (n_buckets < 1 || n_buckets > kMaxBuckets) return plan_error(MOE_ERR_SHAPE, "1 to 16 buckets");
  sorted_desc.assign(buckets, buckets + n_buckets);
  std::sort(sorted_desc.begin(), sorted_desc.end(), [](int a, int b) { return a > b; });
  for (int i = 0; i < n_buckets; ++i) {
    if (sorted_desc[i] < 1 || sorted_desc[i] > kMaxBucketTokens)
      return plan_error(MOE_ERR_SHAPE, "bucket sizes must lie in [1, 65536]");
    if (i && sorted_desc[i] == sorted_desc[i - 1]) return plan_error(MOE_ERR_SHAPE, "bucket sizes must differ");
  }
  g = 0;
  for (int b : sorted_desc) g = gcd(g, b);
  const int64_t bu = sorted_desc[0] / g;
  if (bu * bu + 2 * bu > kMaxPlanUnits)
    return plan_error(MOE_ERR_SHAPE, "largest bucket / gcd of the buckets must be at most 1022");
  return MOE_OK;
}

// Segments covering T tokens: the smallest total of bucket sizes >= T, with
// the fewest segments among those totals, the lexicographically largest
// sequence in descending order among those; all segments full except the
// last (T - the others' total tokens).
int plan(int T, const std::vector<int>& b_desc, int g, std::vector<int>& seg_bucket, std::vector<int>& seg_len) {
  seg_bucket.clear();
  seg_len.clear();
  if (T == 0) return MOE_OK;
  const int n = (int)b_desc.size();
  std::vector<int> u(n);
  for (int i = 0; i < n; ++i) u[i] = b_desc[i] / g;
  const int64_t Tu = ((int64_t)T + g - 1) / g;  // a total of buckets covers T iff it covers Tu units
  const int64_t bmax = u[0];
  // Every optimal cover uses fewer than bmax buckets other than the largest
  // (a larger set of smaller buckets contains a subset whose sum is a
  // multiple of bmax, replaceable by fewer largest buckets), so at least
  // Tu / bmax - bmax largest buckets: place those first.
  const int64_t q = std::max<int64_t>(0, Tu / bmax - bmax);
  const int64_t R = Tu - q * bmax;
  const int64_t top = R + bmax;  // some total in [R, R + bmax) is reachable (bmax buckets alone)
  const int INF = 1 << 30;
  std::vector<int> cnt((size_t)top + 1, INF);
  cnt[0] = 0;
  for (int64_t t = 1; t <= top; ++t)
    for (int i = 0; i < n; ++i)
      if (u[i] <= t && cnt[t - u[i]] + 1 < cnt[t]) cnt[t] = cnt[t - u[i]] + 1;
  int64_t S = R;
  while (S <= top && cnt[S] == INF) ++S;
  if (S > top) return plan_error(MOE_ERR_SHAPE, "no bucket total covers T");  // not reachable: bmax covers
  for (int64_t j = 0; j < q; ++j) seg_bucket.push_back(b_desc[0]);
  for (int64_t rem = S; rem > 0;) {  // largest bucket that keeps a minimal count
    for (int i = 0; i < n; ++i) {
      if (u[i] <= rem && cnt[rem - u[i]] == cnt[rem] - 1) {
        seg_bucket.push_back(b_desc[i]);
        rem -= u[i];
        break;
      }
    }
  }
  int64_t left = T;
  for (size_t i = 0; i < seg_bucket.size(); ++i) {
    const int len = (int)std::min<int64_t>(left, seg_bucket[i]);
    seg_len.push_back(len);
    left -= len;
  }
  return MOE_OK;
}

}  // namespace

struct moe_prefill_runner {
  int device = -1;
  int H = 0, E = 0, k = 0, I = 0, I_s = 0;
  const uint16_t *w_router = nullptr, *w_sg = nullptr;
  const float* bias = nullptr;
  // BF16 expert weights, or (fp8) E4M3 codes with their row scales
  bool fp8 = false;
  const void *w_gate = nullptr, *w_up = nullptr, *w_down = nullptr;
  const void *ws_gate = nullptr, *ws_up = nullptr, *ws_down = nullptr;
  const float *sc_gate = nullptr, *sc_up = nullptr, *sc_down = nullptr;
  const float *ssc_gate = nullptr, *ssc_up = nullptr, *ssc_down = nullptr;
  std::vector<int> buckets;  // descending
  int g = 1;
  uint16_t* x_stage = nullptr;
  uint16_t* y_stage = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  std::vector<hipGraphExec_t> exec;  // per bucket, same order

  // one layer call over T rows of x / y with the runner's workspace
  int forward(const uint16_t* x, int T, uint16_t* y, hipStream_t st) const {
    if (fp8)
      return moe_forward_fp8(x, w_router, bias, static_cast<const uint8_t*>(w_gate), sc_gate,
                             static_cast<const uint8_t*>(w_up), sc_up, static_cast<const uint8_t*>(w_down), sc_down,
                             static_cast<const uint8_t*>(ws_gate), ssc_gate, static_cast<const uint8_t*>(ws_up),
                             ssc_up, static_cast<const uint8_t*>(ws_down), ssc_down, w_sg, T, H, E, k, I, I_s, y, ws,
                             ws_bytes, st);
    return moe_forward(x, w_router, bias, static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up),
                       static_cast<const uint16_t*>(w_down), static_cast<const uint16_t*>(ws_gate),
                       static_cast<const uint16_t*>(ws_up), static_cast<const uint16_t*>(ws_down), w_sg, T, H, E, k,
                       I, I_s, y, ws, ws_bytes, st);
  }
};

extern "C" {

int moe_bucket_plan(int T, const int* buckets, int n_buckets, int* seg_bucket, int* seg_len, int max_segs,
                    int* n_segs) {
  if (T < 0 || T > (1 << 24)) return plan_error(MOE_ERR_SHAPE, "T outside [0, 2^24]");
  if (!n_segs) return plan_error(MOE_ERR_NULL, "n_segs is required");
  std::vector<int> b;
  int g = 1;
  int rc = check_buckets(buckets, n_buckets, b, g);
  if (rc) return rc;
  std::vector<int> sb, sl;
  if ((rc = plan(T, b, g, sb, sl))) return rc;
  *n_segs = (int)sb.size();
  if ((int)sb.size() > max_segs) return plan_error(MOE_ERR_SHAPE, "more segments than max_segs");
  if (!sb.empty() && (!seg_bucket || !seg_len)) return plan_error(MOE_ERR_NULL, "seg_bucket and seg_len are required");
  for (size_t i = 0; i < sb.size(); ++i) {
    seg_bucket[i] = sb[i];
    seg_len[i] = sl[i];
  }
  return set_error(MOE_OK, "");
}

int moe_prefill_runner_destroy(moe_prefill_runner* r) {
  if (!r) return set_error(MOE_OK, "");
  int prev = -1;
  (void)hipGetDevice(&prev);
  if (r->device >= 0) (void)hipSetDevice(r->device);
  for (hipGraphExec_t e : r->exec)
    if (e) (void)hipGraphExecDestroy(e);
  (void)hipFree(r->x_stage);
  (void)hipFree(r->y_stage);
  (void)hipFree(r->ws);
  if (prev >= 0) (void)hipSetDevice(prev);
  delete r;
  return set_error(MOE_OK, "");
}

}  // extern "C"

namespace {
// Buffers, eager calls and graph capture for a runner whose weights and
// shapes are set in *proto (consumed).
int runner_create(moe_prefill_runner* proto, const int* buckets, int n_buckets, moe_prefill_runner** out) {
  std::unique_ptr<moe_prefill_runner> owned(proto);
  if (!out) return plan_error(MOE_ERR_NULL, "out is required");
  *out = nullptr;
  std::vector<int> b;
  int g = 1;
  int rc = check_buckets(buckets, n_buckets, b, g);
  if (rc) return rc;
  const int H = proto->H, E = proto->E, k = proto->k, I = proto->I, I_s = proto->I_s;
  for (int bt : b)
    if (moe_workspace_size(bt, H, E, k, I, I_s) == 0) return plan_error(MOE_ERR_SHAPE, "unsupported layer shapes");
  if (!proto->w_router || !proto->w_gate || !proto->w_up || !proto->w_down)
    return plan_error(MOE_ERR_NULL, "weights are required");
  moe_prefill_runner* r = owned.release();
  if (hipGetDevice(&r->device) != hipSuccess) {
    delete r;
    return plan_error(MOE_ERR_ARCH, "no HIP device");
  }
  r->buckets = b;
  r->g = g;
  size_t ws_bytes = 0;
  for (int bt : b) ws_bytes = std::max(ws_bytes, moe_workspace_size(bt, H, E, k, I, I_s));
  const size_t io_bytes = (size_t)b[0] * H * 2;
  hipStream_t cap = nullptr;
  hipGraph_t graph = nullptr;
  auto bail = [&](int code, const char* what, hipError_t e) {
    char msg[512];
    if (e != hipSuccess)
      snprintf(msg, sizeof msg, "%s: %s", what, hipGetErrorString(e));
    else
      snprintf(msg, sizeof msg, "moe_prefill_runner_create: %s", moe_last_error());  // set by the failing call
    if (graph) (void)hipGraphDestroy(graph);
    if (cap) (void)hipStreamDestroy(cap);
    moe_prefill_runner_destroy(r);  // clears the message
    return plan_error(code, msg);
  };
  hipError_t e;
  if ((e = hipMalloc(&r->x_stage, io_bytes)) != hipSuccess || (e = hipMalloc(&r->y_stage, io_bytes)) != hipSuccess ||
      (e = hipMalloc(&r->ws, ws_bytes)) != hipSuccess)
    return bail(MOE_ERR_HIP, "moe_prefill_runner_create: device allocation", e);
  r->ws_bytes = ws_bytes;
  if ((e = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking)) != hipSuccess)
    return bail(MOE_ERR_HIP, "moe_prefill_runner_create: stream", e);
  // one eager call per bucket first: validates the arguments and the device
  // outside capture (the staging input is zeroed, so the call is well defined)
  if ((e = hipMemsetAsync(r->x_stage, 0, io_bytes, cap)) != hipSuccess)
    return bail(MOE_ERR_HIP, "moe_prefill_runner_create: clear", e);
  for (int bt : b)
    if ((rc = r->forward(r->x_stage, bt, r->y_stage, cap))) return bail(rc, "", hipSuccess);
  if ((e = hipStreamSynchronize(cap)) != hipSuccess) return bail(MOE_ERR_HIP, "moe_prefill_runner_create: sync", e);
  for (int bt : b) {
    if ((e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal)) != hipSuccess)
      return bail(MOE_ERR_HIP, "moe_prefill_runner_create: begin capture", e);
    rc = r->forward(r->x_stage, bt, r->y_stage, cap);
    e = hipStreamEndCapture(cap, &graph);
    if (rc) return bail(rc, "", hipSuccess);
    if (e != hipSuccess) return bail(MOE_ERR_HIP, "moe_prefill_runner_create: end capture", e);
    hipGraphExec_t ex = nullptr;
    if ((e = hipGraphInstantiate(&ex, graph, nullptr, nullptr, 0)) != hipSuccess)
      return bail(MOE_ERR_HIP, "moe_prefill_runner_create: instantiate", e);
    r->exec.push_back(ex);
    (void)hipGraphDestroy(graph);
    graph = nullptr;
  }
  (void)hipStreamDestroy(cap);
  *out = r;
  return set_error(MOE_OK, "");
}
}  // namespace

extern "C" {

int moe_prefill_runner_create(const uint16_t* w_router, const float* router_bias, const uint16_t* w_gate,
                              const uint16_t* w_up, const uint16_t* w_down, const uint16_t* ws_gate,
                              const uint16_t* ws_up, const uint16_t* ws_down, const uint16_t* w_sg, int H, int E,
                              int k, int I, int I_s, const int* buckets, int n_buckets, moe_prefill_runner** out) {
  if (out) *out = nullptr;
  const int n_shared = (ws_gate != nullptr) + (ws_up != nullptr) + (ws_down != nullptr) + (w_sg != nullptr);
  if ((I_s == 0 && n_shared) || (I_s > 0 && n_shared != 4))
    return plan_error(I_s == 0 ? MOE_ERR_SHAPE : MOE_ERR_NULL, "shared-expert tensors: all four with I_s > 0, none else");
  moe_prefill_runner* r = new (std::nothrow) moe_prefill_runner();
  if (!r) return plan_error(MOE_ERR_HIP, "out of host memory");
  r->H = H, r->E = E, r->k = k, r->I = I, r->I_s = I_s;
  r->w_router = w_router, r->bias = router_bias, r->w_sg = w_sg;
  r->w_gate = w_gate, r->w_up = w_up, r->w_down = w_down, r->ws_gate = ws_gate, r->ws_up = ws_up, r->ws_down = ws_down;
  return runner_create(r, buckets, n_buckets, out);
}

int moe_prefill_runner_create_fp8(const uint16_t* w_router, const float* router_bias, const uint8_t* q_gate,
                                  const float* sc_gate, const uint8_t* q_up, const float* sc_up, const uint8_t* q_down,
                                  const float* sc_down, const uint8_t* qs_gate, const float* ssc_gate,
                                  const uint8_t* qs_up, const float* ssc_up, const uint8_t* qs_down,
                                  const float* ssc_down, const uint16_t* w_sg, int H, int E, int k, int I, int I_s,
                                  const int* buckets, int n_buckets, moe_prefill_runner** out) {
  if (out) *out = nullptr;
  const int n_shared = (qs_gate != nullptr) + (ssc_gate != nullptr) + (qs_up != nullptr) + (ssc_up != nullptr) +
                       (qs_down != nullptr) + (ssc_down != nullptr) + (w_sg != nullptr);
  if ((I_s == 0 && n_shared) || (I_s > 0 && n_shared != 7))
    return plan_error(I_s == 0 ? MOE_ERR_SHAPE : MOE_ERR_NULL, "shared-expert tensors: all seven with I_s > 0, none else");
  if (!sc_gate || !sc_up || !sc_down) return plan_error(MOE_ERR_NULL, "row scales are required");
  moe_prefill_runner* r = new (std::nothrow) moe_prefill_runner();
  if (!r) return plan_error(MOE_ERR_HIP, "out of host memory");
  r->H = H, r->E = E, r->k = k, r->I = I, r->I_s = I_s;
  r->w_router = w_router, r->bias = router_bias, r->w_sg = w_sg;
  r->fp8 = true;
  r->w_gate = q_gate, r->w_up = q_up, r->w_down = q_down, r->ws_gate = qs_gate, r->ws_up = qs_up, r->ws_down = qs_down;
  r->sc_gate = sc_gate, r->sc_up = sc_up, r->sc_down = sc_down;
  r->ssc_gate = ssc_gate, r->ssc_up = ssc_up, r->ssc_down = ssc_down;
  return runner_create(r, buckets, n_buckets, out);
}

int moe_prefill_runner_run(moe_prefill_runner* r, const uint16_t* x, int T, uint16_t* y, void* stream) {
  if (!r) return plan_error(MOE_ERR_NULL, "runner is NULL");
  if (T < 0 || T > (1 << 24)) return plan_error(MOE_ERR_SHAPE, "T outside [0, 2^24]");
  if (T == 0) return set_error(MOE_OK, "");
  if (!x || !y) return plan_error(MOE_ERR_NULL, "x and y are required");
  if (((uintptr_t)x & 15u) || ((uintptr_t)y & 15u)) return plan_error(MOE_ERR_ALIGN, "x and y must be 16-byte aligned");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != r->device)
    return plan_error(MOE_ERR_ARCH, "the current device is not the runner's device");
  std::vector<int> sb, sl;
  int rc = plan(T, r->buckets, r->g, sb, sl);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int cpr = r->H / 8;  // 16-byte chunks per row
  int64_t start = 0;
  for (size_t i = 0; i < sb.size(); ++i) {
    const int bt = sb[i], len = sl[i];
    hipError_t e = hipSuccess;
    if (len == bt) {
      // a full segment: the same launches as the bucket's graph, straight on
      // the caller's rows (no staging copies)
      rc = r->forward(x + start * r->H, bt, y + start * r->H, st);
      if (rc) return rc;
    } else {
      // the padded last segment: staged rows, the bucket's graph, real rows out
      const size_t bi = std::find(r->buckets.begin(), r->buckets.end(), bt) - r->buckets.begin();
      const int64_t n16 = (int64_t)bt * cpr;
      hipLaunchKernelGGL(gather_pad_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st, x, start, len, bt,
                         cpr, r->x_stage);
      e = hipGetLastError();
      if (e == hipSuccess) e = hipGraphLaunch(r->exec[bi], st);
      if (e == hipSuccess)
        e = hipMemcpyAsync(y + start * r->H, r->y_stage, (size_t)len * r->H * 2, hipMemcpyDeviceToDevice, st);
    }
    if (e != hipSuccess) {
      char msg[256];
      snprintf(msg, sizeof msg, "moe_prefill_runner_run: segment %zu: %s", i, hipGetErrorString(e));
      return plan_error(MOE_ERR_HIP, msg);
    }
    start += len;
  }
  return set_error(MOE_OK, "");
}

}  // extern "C"
