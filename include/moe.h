/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts FFN layer.
 *
 * The layer: a router scores every expert for every token, the k best experts
 * are kept, each kept expert's SwiGLU FFN is evaluated on only the tokens
 * routed to it, and the expert outputs are summed with renormalised softmax
 * weights, plus a sigmoid-gated shared expert.  Sources: kongchang.com
 * "GFX1151 engine" (section on the MoE kernel: many expert sub-networks,
 * only a few active per step, sparse routing changes the compute and memory
 * pattern); guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B" (section on the data
 * path: the block runs as a selected-expert MoE, i.e. only chosen experts are
 * computed).  The pages give no formulas; the arithmetic below is the plain
 * reading of a Qwen3-class MoE block.
 *
 * Conventions for every entry point
 *   - Tensors are DEVICE pointers (HIP device memory), row-major, contiguous,
 *     16-byte aligned.  BF16 values are passed as uint16_t bit patterns.
 *   - Weight matrices use the [out, in] convention, so the reduction index is
 *     contiguous: W_router [E,H], W_gate/W_up [E,I,H], W_down [E,H,I],
 *     Ws_gate/Ws_up [I_s,H], Ws_down [H,I_s], w_sg [H].
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work and return; nothing is synchronised and no value is read
 *     back to the host, so a call can be captured in a HIP graph (the prefill
 *     runner's creation and destruction excepted: they allocate, capture and
 *     synchronise).
 *   - Expert weights are BF16 (moe_forward and the stage entry points), OCP
 *     FP8 E4M3 with a row scale (moe_forward_fp8) or signed 4-bit with a
 *     group scale (moe_forward_q4); the router weights are always BF16.
 *   - The caller owns every buffer, including `workspace`.  The library never
 *     allocates or frees device memory and keeps no state between calls
 *     except a per-device cached architecture check -- apart from the
 *     prefill runner (moe_prefill_runner_*), which owns its buffers and
 *     graphs.
 *   - Argument errors are reported before anything is enqueued.  No C++
 *     exception crosses this boundary.  A status other than MOE_OK leaves the
 *     outputs unspecified; moe_last_error() gives a message (thread-local).
 *   - T = 0 is a successful no-op.
 *   - Supported shapes: 1 <= E <= 256, 1 <= k <= min(E, 16), H % 256 == 0,
 *     I % 128 == 0, I_s % 128 == 0 (I_s = 0: no shared expert), T <= 2^24.
 *   - Results are deterministic: identical inputs give bitwise-identical
 *     outputs (no floating-point atomics anywhere).
 */
#ifndef MOE355_MOE_H
#define MOE355_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_NULL (-1)        /* a required pointer is NULL                         */
#define MOE_ERR_SHAPE (-2)       /* unsupported or inconsistent sizes                  */
#define MOE_ERR_ALIGN (-3)       /* a tensor pointer is not 16-byte aligned            */
#define MOE_ERR_WORKSPACE (-4)   /* workspace smaller than moe_workspace_size()        */
#define MOE_ERR_ARCH (-5)        /* the current device is not gfx950 / no device       */
#define MOE_ERR_HIP (-6)         /* a HIP launch failed; see moe_last_error()          */

/* Name of a status code ("MOE_OK", "MOE_ERR_SHAPE", ...). */
const char* moe_status_str(int status);

/* Message describing the last error returned on this host thread ("" if none). */
const char* moe_last_error(void);

/*
 * Tile heights chosen for T tokens.  BIG (moe_align_tile_rows) is 256, 128,
 * 64 or 32 from the mean rows per expert T*k/E (>= 192, >= 128, >= 48, less).
 * SMALL (moe_align_small_tile_rows) equals BIG: every expert's rows are cut
 * into ceil(count / BIG) tiles, the last one padded, and there is one tile
 * list.  The environment variables MOE_TILE_ROWS and MOE_SMALL_ROWS (32, 64,
 * 128 or 256; read once per process; for tuning) override BIG and SMALL.  With SMALL < BIG an expert gets
 * floor(count / BIG) BIG tiles and its remainder is padded to whole SMALL
 * tiles, listed separately.  Depends only on (T, E, k) and those variables;
 * the layer's results do not depend on the tiling.
 */
int moe_align_tile_rows(int T, int E, int k);
int moe_align_small_tile_rows(int T, int E, int k);

/*
 * Upper bound of padded rows: T*k + min(E, T*k) * (SMALL - 1).  Sizes `sorted`
 * in moe_align and the rows of h and o.
 */
int64_t moe_align_max_rows(int T, int E, int k);

/* Capacity of the BIG tile list: (T*k + min(E, T*k) * (BIG - 1)) / BIG with
 * one tile class, floor(T*k / BIG) with two.  The SMALL tiles (if any) start
 * at this entry of the tile table. */
int64_t moe_align_max_big_tiles(int T, int E, int k);

/* Entries of the tile table: BIG capacity + SMALL capacity. */
int64_t moe_align_max_tiles(int T, int E, int k);

/*
 * Bytes of device workspace moe_forward needs for these sizes (worst-case
 * padding included).  Returns 0 for unsupported sizes.
 */
size_t moe_workspace_size(int T, int H, int E, int k, int I, int I_s);

/*
 * Byte offset, within a workspace passed to moe_forward with these shapes, of
 * the expert ids [T,k] int32 (rank order) that the call selected; they stay
 * there until the workspace is reused.  For routing statistics and checks.
 * 0 for unsupported shapes (as moe_workspace_size).
 */
size_t moe_forward_ids_offset(int T, int H, int E, int k, int I, int I_s);

/*
 * Sections of the workspace moe_forward carves for these sizes (the path T
 * selects: single-token, small-batch or tiled), for checking: offsets[i] and
 * bytes[i] (host arrays of `max` entries, either may be NULL) receive the
 * byte offset and the size of section i.  Sections start 256-byte aligned
 * and each is followed by at least 256 bytes that no kernel writes.  Returns
 * the number of sections (entries past `max` are not written), 0 for
 * unsupported sizes.  Host only.
 */
int moe_workspace_sections(int T, int H, int E, int k, int I, int I_s, size_t* offsets, size_t* bytes, int max);

/*
 * The whole layer:  y = sum_{j<k} w[t,j] * FFN_{ids[t,j]}(x_t) + s_t * FFN_s(x_t)
 *
 *   logits[t,e] = sum_h x[t,h] W_router[e,h] (+ router_bias[e]), fp32 accumulation
 *   ids[t,:]    = the k experts with the largest logits, ordered by
 *                 (logit descending, expert index ascending) -- exact ties go
 *                 to the lowest index
 *   w[t,j]      = softmax(logits[t])[ids[t,j]] / sum_j' softmax(logits[t])[ids[t,j']]
 *   FFN_e(x)    = W_down[e] (silu(W_gate[e] x) * (W_up[e] x)),  silu(z) = z/(1+e^-z)
 *   s_t         = sigmoid(x_t . w_sg);  FFN_s uses Ws_gate, Ws_up, Ws_down
 *
 * Inputs:  x [T,H] bf16; W_router [E,H] bf16; router_bias [E] fp32 or NULL;
 *          W_gate, W_up [E,I,H] bf16; W_down [E,H,I] bf16;
 *          Ws_gate, Ws_up [I_s,H], Ws_down [H,I_s], w_sg [H] bf16 -- all four
 *          NULL with I_s = 0, or all four set with I_s > 0.
 * Output:  y [T,H] bf16 (fp32 sum rounded to nearest even).
 * Workspace: at least moe_workspace_size(T,H,E,k,I,I_s) bytes, 256-byte aligned.
 * Internally, for T > MOE_SMALL_BATCH_MAX_T, the call runs the router GEMM
 * with the shared-expert gate and top-k, align, the gate/up GEMM (routed tiles
 * and the shared expert's token tiles in one launch), the routed down GEMM and
 * the combine fused with the shared down projection on `stream`; the
 * arithmetic of every element is the same as that of the stage entry points.
 * With T == 1 it runs the single-token kernels, and with
 * 2 <= T <= MOE_SMALL_BATCH_MAX_T the small-batch kernels (each touched
 * expert's weight rows read once and applied to all of its tokens; h and the
 * expert outputs kept in fp32, the combine in the same rank order).  The
 * selection rule is the same on every path.
 */
#define MOE_SMALL_BATCH_MAX_T 32
int moe_forward(const uint16_t* x, const uint16_t* w_router, const float* router_bias,
                const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                const uint16_t* w_sg, int T, int H, int E, int k, int I, int I_s,
                uint16_t* y, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_forward without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * arithmetic and outputs as moe_forward; the workspace is one array of MOE_NOALLOC_WS_BYTES bytes in
 * each GPU's memory, allocated with the library's code and held until the process ends.  The call
 * allocates and frees nothing.
 *   - Sizes whose moe_workspace_size exceeds MOE_NOALLOC_WS_BYTES give MOE_ERR_WORKSPACE before
 *     anything is enqueued (at hidden 2048, 256 experts, top-8, FFN 512, shared 512: up to 1,198
 *     tokens per call).
 *   - Every call on a GPU uses that GPU's one array and leaves its contents there (no part of it has
 *     to start at zero).  Calls that overlap on one GPU (other streams, other host threads) race:
 *     order them.
 *   - The first call on a device looks up the array's device address (hipGetSymbolAddress).
 */
#define MOE_NOALLOC_WS_BYTES (64u << 20)
int moe_forward_noalloc(const uint16_t* x, const uint16_t* w_router, const float* router_bias,
                        const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                        const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                        const uint16_t* w_sg, int T, int H, int E, int k, int I, int I_s, uint16_t* y,
                        void* stream);

/*
 * The whole layer with FP8 expert weights.  kongchang.com "GFX1151 engine"
 * (section on the two weight formats) describes a HuggingFace-native format
 * whose weights are FP8-quantised, for speed and a smaller memory footprint.
 * Encoding: OCP FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent 0 is subnormal; S.1111.111 is NaN; no infinities; largest
 * magnitude 448), one fp32 scale per output row of every expert matrix:
 *     W[r][c] = scale[r] * e4m3(code[r][c])
 * Same arithmetic and outputs as moe_forward on the dequantised weights (the
 * dot products run over the codes in fp32 and the row scale multiplies each
 * dot product).  The router (W_router, router_bias) and w_sg stay bf16/fp32.
 *
 * Inputs:  q_gate, q_up [E,I,H] and q_down [E,H,I] uint8 codes with scales
 *          sc_gate, sc_up [E,I] and sc_down [E,H] fp32; shared expert
 *          qs_gate, qs_up [I_s,H], qs_down [H,I_s] with ssc_gate, ssc_up
 *          [I_s] and ssc_down [H] -- these six and w_sg all NULL with I_s = 0,
 *          or all set; everything else as in moe_forward.
 * Workspace: moe_workspace_size(T,H,E,k,I,I_s) bytes, 256-byte aligned;
 *          moe_forward_ids_offset() locates the selected ids as for moe_forward.
 * Paths: T == 1 and T <= MOE_SMALL_BATCH_MAX_T run the single-token and
 *          small-batch kernels on the codes (8 bytes per 8 weights); larger
 *          T runs the tiled GEMMs (same tiles as moe_forward) on the codes,
 *          widened exactly to bf16 inside the kernel, with the row scales
 *          applied to the accumulators.  Codes that are NaN give NaN outputs
 *          (not checked).
 */
int moe_forward_fp8(const uint16_t* x, const uint16_t* w_router, const float* router_bias,
                    const uint8_t* q_gate, const float* sc_gate, const uint8_t* q_up, const float* sc_up,
                    const uint8_t* q_down, const float* sc_down,
                    const uint8_t* qs_gate, const float* ssc_gate, const uint8_t* qs_up, const float* ssc_up,
                    const uint8_t* qs_down, const float* ssc_down, const uint16_t* w_sg,
                    int T, int H, int E, int k, int I, int I_s,
                    uint16_t* y, void* workspace, size_t ws_bytes, void* stream);

/*
 * The whole layer with 4-bit expert weights, for 1 <= T <= MOE_Q4_MAX_T
 * (single-token and small-batch steps, where reading the weights bounds the
 * step).  kongchang.com "GFX1151 engine" (section on the two weight formats)
 * names GGUF files with 4-bit integer (Q4) quantisation; the layout here is a
 * plain group-wise one of this library's own (not a GGUF block layout):
 * every output row is cut into groups of 32 consecutive weights along the
 * reduction index, each group has one IEEE fp16 scale, each weight is a
 * signed 4-bit integer q in [-8, 7] (two's complement), two per byte with the
 * even index in the low nibble:  W[r][c] = scale[r][c / 32] * q[r][c].
 * Same arithmetic and outputs as moe_forward on the dequantised weights.
 *
 * Inputs:  q_gate, q_up [E,I,H/2] and q_down [E,H,I/2] uint8 with fp16 scale
 *          bits s_gate, s_up [E,I,H/32] and s_down [E,H,I/32]; shared expert
 *          qs_gate, qs_up [I_s,H/2], qs_down [H,I_s/2] with ss_gate, ss_up
 *          [I_s,H/32], ss_down [H,I_s/32] -- these six and w_sg all NULL with
 *          I_s = 0, or all set; router, bias, w_sg, y and the workspace
 *          (moe_workspace_size) as in moe_forward.
 * T > MOE_Q4_MAX_T gives MOE_ERR_SHAPE.  Non-finite scales give non-finite
 * outputs (not checked).
 */
#define MOE_Q4_MAX_T 32
int moe_forward_q4(const uint16_t* x, const uint16_t* w_router, const float* router_bias,
                   const uint8_t* q_gate, const uint16_t* s_gate, const uint8_t* q_up, const uint16_t* s_up,
                   const uint8_t* q_down, const uint16_t* s_down,
                   const uint8_t* qs_gate, const uint16_t* ss_gate, const uint8_t* qs_up, const uint16_t* ss_up,
                   const uint8_t* qs_down, const uint16_t* ss_down, const uint16_t* w_sg,
                   int T, int H, int E, int k, int I, int I_s,
                   uint16_t* y, void* workspace, size_t ws_bytes, void* stream);

/*
 * out[i] = value of the E4M3 code codes[i] (as defined for moe_forward_fp8),
 * computed with the same device conversion the FP8 kernels use; NaN codes
 * give NaN.  codes [n] uint8 and out [n] fp32, device pointers, 16-byte
 * aligned; n >= 0 (0: no-op).  For checking the conversion.
 */
int moe_e4m3_to_f32(const uint8_t* codes, float* out, int64_t n, void* stream);

/*
 * Prefill of any length through fixed-size buckets.  guanjiawei.ai "AIMA
 * AMD395 Qwen3.6-35B-A3B" (data-path section) decomposes any prompt into
 * optimised 8192- and 1024-token tiles and a tail; its runtime section keeps
 * 1024/2048/4096/8192-token buckets resident, covers each prompt with the
 * smallest bucket total and pads only the final segment.
 *
 * moe_bucket_plan: the segments covering T tokens with the given bucket sizes
 *   (host only, no device call).  Rule: the smallest total of bucket sizes
 *   that is >= T; among covers with that total, the fewest segments; among
 *   those, the lexicographically largest sequence in descending order.  The
 *   segments come in that (descending) order; every segment is full except
 *   the last, which holds T minus the others' tokens (> 0).
 *   buckets [n_buckets] host ints: 1 <= n_buckets <= 16, distinct, each in
 *   [1, 65536], largest / gcd(all) <= 1022.  Outputs (host): *n_segs (set
 *   even when it exceeds max_segs, which is then MOE_ERR_SHAPE),
 *   seg_bucket[i] = bucket size and seg_len[i] = real tokens of segment i.
 *   T = 0 gives no segments.
 */
int moe_bucket_plan(int T, const int* buckets, int n_buckets, int* seg_bucket, int* seg_len, int max_segs,
                    int* n_segs);

/*
 * A prefill runner owns, on the device current at creation: a staging input
 * and output of the largest bucket's size, one workspace and, per bucket, an
 * instantiated HIP graph of one moe_forward call over that many tokens (the
 * weights given here, which must stay valid while the runner lives).
 *   moe_prefill_runner_create: weights and shapes as moe_forward (BF16);
 *     buckets as moe_bucket_plan (each bucket must be a valid moe_forward
 *     size).  Allocates device memory and captures the graphs (the only
 *     entry points that allocate).  *out = NULL on error.
 *   moe_prefill_runner_create_fp8: the same with the expert weights of
 *     moe_forward_fp8 (E4M3 codes and fp32 row scales; the graphs hold
 *     moe_forward_fp8 calls).
 *   moe_prefill_runner_run: y [T,H] = the layer on x [T,H] (device, 16-byte
 *     aligned), enqueued on `stream`, per segment of moe_bucket_plan(T): a
 *     full segment runs the bucket's launches on its rows of x and y
 *     directly; the partial last segment is gathered into the staging input
 *     (its padding rows repeat the segment's own rows), run by the bucket's
 *     graph, and its real rows are copied into y.  The result of every token is that of
 *     moe_forward on the token (tokens do not interact).  Calls on one runner
 *     share its buffers: keep them on one stream (or ordered).  The current
 *     device must be the runner's.
 *   moe_prefill_runner_destroy: frees everything; call it after the last run
 *     has completed.  NULL is a no-op.
 */
typedef struct moe_prefill_runner moe_prefill_runner;
int moe_prefill_runner_create(const uint16_t* w_router, const float* router_bias,
                              const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                              const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                              const uint16_t* w_sg, int H, int E, int k, int I, int I_s,
                              const int* buckets, int n_buckets, moe_prefill_runner** out);
int moe_prefill_runner_create_fp8(const uint16_t* w_router, const float* router_bias,
                                  const uint8_t* q_gate, const float* sc_gate, const uint8_t* q_up,
                                  const float* sc_up, const uint8_t* q_down, const float* sc_down,
                                  const uint8_t* qs_gate, const float* ssc_gate, const uint8_t* qs_up,
                                  const float* ssc_up, const uint8_t* qs_down, const float* ssc_down,
                                  const uint16_t* w_sg, int H, int E, int k, int I, int I_s,
                                  const int* buckets, int n_buckets, moe_prefill_runner** out);
int moe_prefill_runner_run(moe_prefill_runner* runner, const uint16_t* x, int T, uint16_t* y, void* stream);
int moe_prefill_runner_destroy(moe_prefill_runner* runner);

/*
 * Router stage.  kongchang.com "GFX1151 engine" (section on the MoE kernel:
 * of many expert sub-networks only a few are activated for each token) and
 * guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B" (section on the data path: the
 * block runs as a selected-expert MoE) define the selection; the arithmetic
 * is the plain reading of a Qwen3-class router: logits (fp32 accumulation of
 * bf16 products), optional bias, top-k by (logit desc, index asc),
 * renormalised softmax weights, and the shared-expert gate
 * s = sigmoid(x . w_sg).
 *   Outputs: ids [T,k] int32, w [T,k] fp32; logits [T,E] fp32 (includes the
 *   bias; NULL: not stored); s [T] fp32 (required iff w_sg is given, else
 *   ignored).
 *   scratch NULL: one launch, W_router staged through on-chip memory with
 *   the x tiles, the selection reading the logits from on-chip memory.
 *   scratch given (scratch_bytes >= moe_route_scratch_size(T,H,E), which
 *   depends on H and E only; 16-byte aligned, else MOE_ERR_WORKSPACE /
 *   MOE_ERR_ALIGN): the form moe_forward uses for T > 32 -- a first launch
 *   copies W_router into scratch in the order of the matrix-core operands,
 *   then one launch per 32-token tile keeps the tile's x rows on chip,
 *   streams the weights into registers, and selects and computes s in its
 *   epilogue.  Same rule and weights; the two forms' logits differ only by
 *   fp32 summation order.
 */
size_t moe_route_scratch_size(int T, int H, int E);
int moe_route(const uint16_t* x, const uint16_t* w_router, const float* router_bias,
              const uint16_t* w_sg, int T, int H, int E, int k,
              int32_t* ids, float* w, float* s, float* logits,
              void* scratch, size_t scratch_bytes, void* stream);

/*
 * Top-k and weights on caller-supplied fp32 logits [T,E]: the selection of
 * moe_route alone (the same pages and passages: only a few experts per
 * token, chosen by the router).  Same rule and weights as moe_route; -0 and
 * +0 compare equal.  logits [T,E] fp32, ids [T,k] int32, w [T,k] fp32,
 * device pointers; the logits must be finite (NaN is out of contract).
 */
int moe_route_from_logits(const float* logits, int T, int E, int k,
                          int32_t* ids, float* w, void* stream);

/*
 * Expert histogram, prefix scan and stable permutation into padded tiles.
 * kongchang.com "GFX1151 engine" (section on the MoE kernel: sparse routing
 * makes the compute and memory-access pattern unlike a dense layer's) and
 * guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B" (section on the data path: only
 * the selected experts are evaluated): grouping every expert's assignments
 * into contiguous, tile-padded rows turns the selected-expert evaluation into
 * one dense GEMM tile sequence per expert.  Integer work, bit-exact and
 * independent of scheduling (no ordering atomics).
 *   ids [T,k] int32 (values in [0,E)).  BIG, SMALL as moe_align_tile_rows /
 *   moe_align_small_tile_rows.
 *   counts [E]      number of assignments routed to each expert
 *   pad_off [E+1]   first padded row of each expert; pad_off[E] = total rows
 *                   (expert e owns floor(counts[e]/BIG) BIG tiles, then
 *                   ceil((counts[e] mod BIG)/SMALL) SMALL tiles)
 *   sorted [moe_align_max_rows]  assignment a = t*k + j held by each padded row,
 *                   ascending a within an expert; -1 marks a padding row
 *   inv [T*k]       padded row of each assignment
 *   tiles [2*moe_align_max_tiles]  (expert, first row) per tile: the BIG tiles
 *                   in expert order from entry 0, the SMALL tiles in expert
 *                   order from entry moe_align_max_big_tiles
 *   n_tiles [2]     number of BIG tiles, number of SMALL tiles
 *   scratch         at least moe_align_scratch_size(T,E,k) bytes, 16-byte aligned
 */
size_t moe_align_scratch_size(int T, int E, int k);
int moe_align(const int32_t* ids, int T, int E, int k,
              int32_t* counts, int32_t* pad_off, int32_t* sorted, int32_t* inv,
              int32_t* tiles, int32_t* n_tiles, void* scratch, size_t scratch_bytes, void* stream);

/*
 * Grouped gate/up GEMM with fused SwiGLU over the tiles of moe_align:
 *   for a routed padded row p holding assignment a (token t = a / k) of expert e:
 *     h[p,i] = bf16( silu(sum_h x[t,h] W_gate[e,i,h]) * sum_h x[t,h] W_up[e,i,h] )
 *   (padding rows get 0); for every token t when I_s > 0:
 *     h_s[t,i] = bf16( silu(x_t . Ws_gate[i]) * (x_t . Ws_up[i]) )
 *   h [moe_align_max_rows, I] bf16, h_s [T, I_s] bf16 (NULL iff I_s == 0).
 */
int moe_grouped_gate_up(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up,
                        const uint16_t* ws_gate, const uint16_t* ws_up,
                        const int32_t* sorted, const int32_t* tiles, const int32_t* n_tiles,
                        int T, int H, int E, int k, int I, int I_s,
                        uint16_t* h, uint16_t* h_s, void* stream);

/*
 * Grouped down GEMM over the routed tiles:
 *   for every non-padding row p holding assignment a = sorted[p]:
 *     o[a,c] = bf16( sum_i h[p,i] W_down[e,c,i] )
 *   o [T*k, H] bf16, one row per assignment a = t*k + j (token-major), so a
 *   token's k expert outputs are contiguous.
 */
int moe_grouped_down(const uint16_t* h, const uint16_t* w_down,
                     const int32_t* sorted, const int32_t* tiles, const int32_t* n_tiles,
                     int T, int H, int E, int k, int I, uint16_t* o, void* stream);

/*
 * Deterministic, atomic-free combine, fused with the shared expert's down
 * projection when I_s > 0:
 *   y[t,c] = bf16( (((w[t,0] o[t*k] + w[t,1] o[t*k+1]) + ...)
 *                   + w[t,k-1] o[t*k+k-1]) + s[t] (sum_i h_s[t,i] Ws_down[c,i]) )
 *   in fp32, j ascending, then the shared term.  o as moe_grouped_down writes it.
 *   h_s, ws_down and s are NULL iff I_s == 0.
 */
int moe_combine(const uint16_t* o, const float* w,
                const uint16_t* h_s, const uint16_t* ws_down, const float* s,
                int T, int H, int k, int I_s, uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE355_MOE_H */
