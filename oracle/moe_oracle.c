/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU model of the sparse
 * Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP implementation, and the product path
 * never calls it.
 *
 * What the layer is: kongchang.com "GFX1151 engine" (section on the MoE
 * kernel) defines a Mixture of Experts as many expert sub-networks of which
 * only a few are activated for each token, the routing being sparse;
 * guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B" (section on the data path)
 * runs this block as a "selected-expert" MoE, i.e. only the chosen experts
 * are evaluated.  The pages do not spell out the arithmetic; the layer
 * computed here is the plain reading of a Qwen3-class MoE block:
 *
 *   1. router logits  l[t,e] = sum_h x[t,h] * Wr[e,h]   (fp32, ascending h)
 *                      (+ b[e] when a router bias is given), -0 -> +0
 *   2. top-k           experts ordered by (logit desc, index asc), first k
 *   3. weights         p = softmax over all E logits,
 *                      w[t,j] = p[id_j] / sum_j' p[id_j']
 *   4. stable align    assignment a = t*k + j grouped by expert, ascending a
 *   5. expert FFN      h_i = silu(sum_h x*Wg[e,i,h]) * sum_h x*Wu[e,i,h],
 *                      o   = sum_i h_i * Wd[e,:,i],  silu(z) = z/(1+e^-z)
 *   6. shared expert   same SwiGLU with Ws_gate/Ws_up/Ws_down over every
 *                      token, scaled by s[t] = sigmoid(sum_h x*w_sg)
 *   7. combine         y[t] = sum_{j ascending} w[t,j]*o[t*k+j] + s[t]*o_s[t]
 *
 * Precision: the routing decision (step 1-2) is taken on fp32 logits summed
 * sequentially, since the workloads fix router logits as fp32-accumulated and
 * a decision must be taken in one stated precision.  Everything that is not a
 * decision (softmax, renormalisation, gate, FFN, combine) is computed in
 * IEEE double.  BF16 inputs are widened exactly (bits << 16).
 *
 * FP8 expert weights (oracle_forward_fp8): kongchang.com "GFX1151 engine"
 * (section on the two weight formats) says the HuggingFace-native format
 * carries 8-bit floating-point quantised weights and that FP8 loses very
 * little precision; it gives no encoding or scale layout.  Read here as the
 * OCP FP8 E4M3 encoding with one fp32 scale per output row of every expert
 * matrix: W[r][c] = scale[r] * e4m3(code[r][c]).  The router and w_sg stay
 * BF16.  Dequantised weights are exact in double (4 + 24 significant bits),
 * so the layer's arithmetic is otherwise the BF16 one.
 *
 * 4-bit expert weights (oracle_forward_q4): kongchang.com "GFX1151 engine"
 * (section on the two weight formats) names GGUF files with 4-bit integer
 * (Q4) quantisation but gives no block layout.  Read here as a plain
 * group-wise format: every output row is cut into groups of 32 consecutive
 * weights along the reduction index, each group has one IEEE fp16 scale,
 * each weight is a signed 4-bit integer q in [-8, 7] (two's complement),
 * two per byte (even index in the low nibble), and w = scale * q.  The
 * dequantised weights are exact in double.
 *
 * Parallelism: OpenMP over tokens (routing) and over assignments (FFN).
 * Every output element is computed by exactly one thread with a fixed
 * operation order, so results do not depend on the thread count.
 *
 * Built with -ffp-contract=off so that no multiply-add is fused.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_NULL (-1)
#define ORC_ERR_SHAPE (-2)
#define ORC_ERR_NONFINITE (-3)
#define ORC_ERR_NOMEM (-4)

static inline float bf16_to_f32(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static int all_finite_bf16(const uint16_t* p, size_t n) {
    if (!p) return 1;
    for (size_t i = 0; i < n; ++i)
        if ((p[i] & 0x7F80u) == 0x7F80u) return 0;
    return 1;
}

static int all_finite_f32(const float* p, size_t n) {
    if (!p) return 1;
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Dot product of two BF16 rows in fp32, ascending index, accumulator from +0. */
static float dot_bf16_f32(const uint16_t* a, const uint16_t* b, int n) {
    float acc = 0.0f;
    for (int i = 0; i < n; ++i) {
        float p = bf16_to_f32(a[i]) * bf16_to_f32(b[i]);
        acc = acc + p;
    }
    return acc;
}

/* Dot product of two BF16 rows in double, ascending index. */
static double dot_bf16_f64(const uint16_t* a, const uint16_t* b, int n) {
    double acc = 0.0;
    for (int i = 0; i < n; ++i) acc += (double)bf16_to_f32(a[i]) * (double)bf16_to_f32(b[i]);
    return acc;
}

/* OCP FP8 E4M3 ("e4m3fn"): bit 7 sign, bits 6..3 biased exponent (bias 7),
 * bits 2..0 mantissa.  Exponent field 0: subnormal, m/8 * 2^(1-7).
 * Otherwise (1 + m/8) * 2^(e-7).  S.1111.111 is NaN; no infinities, so the
 * largest finite magnitude is 1.75 * 2^8 = 448. */
static double e4m3_value(uint8_t code) {
    int sgn = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = e == 0 ? ldexp((double)m / 8.0, 1 - 7) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sgn ? -mag : mag;
}

/* Decoded values of n codes (NaN for the two NaN codes). */
int oracle_e4m3_decode(const uint8_t* codes, long n, double* out) {
    if (n < 0) return ORC_ERR_SHAPE;
    if (n > 0 && (!codes || !out)) return ORC_ERR_NULL;
    for (long i = 0; i < n; ++i) out[i] = e4m3_value(codes[i]);
    return ORC_OK;
}

static int all_finite_e4m3(const uint8_t* p, size_t n) {
    if (!p) return 1;
    for (size_t i = 0; i < n; ++i)
        if ((p[i] & 0x7Fu) == 0x7Fu) return 0;
    return 1;
}

/* IEEE binary16: bit 15 sign, bits 14..10 biased exponent (bias 15), bits
 * 9..0 mantissa; exponent 0 is subnormal (m/1024 * 2^-14); exponent 31 is
 * infinity (m = 0) or NaN. */
static double f16_value(uint16_t h) {
    int sgn = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double mag;
    if (e == 31) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m / 1024.0, -14);
    else mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return sgn ? -mag : mag;
}

/* Decoded values of n fp16 bit patterns. */
int oracle_f16_decode(const uint16_t* bits, long n, double* out) {
    if (n < 0) return ORC_ERR_SHAPE;
    if (n > 0 && (!bits || !out)) return ORC_ERR_NULL;
    for (long i = 0; i < n; ++i) out[i] = f16_value(bits[i]);
    return ORC_OK;
}

#define Q4_GROUP 32

/* Signed 4-bit weight c of a row of packed nibbles (even c: low nibble). */
static int q4_weight(const uint8_t* row, size_t c) {
    int nib = (c & 1) ? (row[c / 2] >> 4) : (row[c / 2] & 15);
    return nib >= 8 ? nib - 16 : nib;
}

/* Dequantised 4-bit matrix [rows, n] (n a multiple of 32) into out [rows, n]
 * double: out[r][c] = scale[r][c / 32] * q[r][c]. */
int oracle_q4_dequant(const uint8_t* codes, const uint16_t* scales, long rows, int n, double* out) {
    if (rows < 0 || n < Q4_GROUP || n % Q4_GROUP) return ORC_ERR_SHAPE;
    if (rows > 0 && (!codes || !scales || !out)) return ORC_ERR_NULL;
    for (long r = 0; r < rows; ++r)
        for (int c = 0; c < n; ++c)
            out[(size_t)r * n + c] = f16_value(scales[(size_t)r * (n / Q4_GROUP) + c / Q4_GROUP]) *
                                     (double)q4_weight(codes + (size_t)r * (n / 2), (size_t)c);
    return ORC_OK;
}

static int all_finite_f16(const uint16_t* p, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if ((p[i] & 0x7C00u) == 0x7C00u) return 0;
    return 1;
}

/* One expert-weight operand: BF16 bits, E4M3 codes with a scale per row, or
 * 4-bit codes (q4) with an fp16 scale per group of 32.  q_val holds the value
 * of every E4M3 code (e4m3_value of the code, filled once per call), so that
 * the inner loops do not re-derive it per element. */
typedef struct {
    const uint16_t* bf;
    const uint8_t* q;
    const float* scale;
    const uint8_t* q4;
    const uint16_t* s4;
    const double* q_val;
} wmat;

static int wmat_set(wmat m) {
    return m.bf != NULL || (m.q != NULL && m.scale != NULL) || (m.q4 != NULL && m.s4 != NULL);
}

static int wmat_finite(wmat m, size_t rows, size_t cols) {
    if (m.bf) return all_finite_bf16(m.bf, rows * cols);
    if (m.q4) return all_finite_f16(m.s4, rows * (cols / Q4_GROUP));
    return all_finite_e4m3(m.q, rows * cols) && all_finite_f32(m.scale, rows);
}

/* Dot product, in double and ascending index, of a BF16 row x with row r
 * (length n) of an expert operand. */
static double dot_row_f64(const uint16_t* x, wmat m, size_t r, int n) {
    if (m.bf) return dot_bf16_f64(x, m.bf + r * (size_t)n, n);
    double acc = 0.0;
    if (m.q4) {
        const uint8_t* q = m.q4 + r * (size_t)(n / 2);
        const uint16_t* s = m.s4 + r * (size_t)(n / Q4_GROUP);
        for (int i = 0; i < n; ++i)
            acc += (double)bf16_to_f32(x[i]) * (f16_value(s[i / Q4_GROUP]) * (double)q4_weight(q, (size_t)i));
        return acc;
    }
    const uint8_t* q = m.q + r * (size_t)n;
    const double sc = (double)m.scale[r];
    for (int i = 0; i < n; ++i) acc += (double)bf16_to_f32(x[i]) * (sc * m.q_val[q[i]]);
    return acc;
}

/* Element (r, c) of an expert operand with rows of length n, as a double. */
static double wmat_at(wmat m, size_t r, size_t c, int n) {
    if (m.bf) return (double)bf16_to_f32(m.bf[r * (size_t)n + c]);
    if (m.q4)
        return f16_value(m.s4[r * (size_t)(n / Q4_GROUP) + c / Q4_GROUP]) *
               (double)q4_weight(m.q4 + r * (size_t)(n / 2), c);
    return (double)m.scale[r] * m.q_val[m.q[r * (size_t)n + c]];
}

/* Steps 2-3 for one token: select k experts by (logit desc, index asc) and
 * compute their renormalised softmax weights.  Logits are canonical (no -0). */
static void topk_and_weights(const float* l, int E, int k, int32_t* ids, double* w, unsigned char* taken) {
    memset(taken, 0, (size_t)E);
    for (int r = 0; r < k; ++r) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || l[e] > l[best]) best = e; /* strict: lower index keeps ties */
        }
        taken[best] = 1;
        ids[r] = best;
    }
    /* softmax over all E logits, then renormalise over the selected k */
    double m = (double)l[0];
    for (int e = 1; e < E; ++e)
        if ((double)l[e] > m) m = (double)l[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += exp((double)l[e] - m);
    double psum = 0.0;
    for (int r = 0; r < k; ++r) {
        w[r] = exp((double)l[ids[r]] - m) / z;
    }
    for (int r = 0; r < k; ++r) psum += w[r];
    for (int r = 0; r < k; ++r) w[r] = w[r] / psum;
}

/*
 * Router: logits, top-k ids and weights, shared-expert gate.
 *   x[T,H], w_router[E,H], w_sg[H] bf16; bias[E] fp32 or NULL.
 *   logits[T,E] fp32 (out, nullable), ids[T,k] (out), w[T,k] (out),
 *   s[T] (out, nullable; written only when w_sg is given).
 */
int oracle_route(const uint16_t* x, const uint16_t* w_router, const float* bias, const uint16_t* w_sg,
                 int T, int H, int E, int k, float* logits, int32_t* ids, double* w, double* s) {
    if (T < 0 || H < 1 || E < 1 || k < 1 || k > E) return ORC_ERR_SHAPE;
    if (T == 0) return ORC_OK;
    if (!x || !w_router || !ids || !w) return ORC_ERR_NULL;
    if (!all_finite_bf16(x, (size_t)T * H) || !all_finite_bf16(w_router, (size_t)E * H) ||
        !all_finite_f32(bias, bias ? (size_t)E : 0) || !all_finite_bf16(w_sg, w_sg ? (size_t)H : 0))
        return ORC_ERR_NONFINITE;
    int err = ORC_OK;
#pragma omp parallel
    {
        float* l = (float*)malloc(sizeof(float) * (size_t)E);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
        if (!l || !taken) {
#pragma omp atomic write
            err = ORC_ERR_NOMEM;
        } else {
#pragma omp for schedule(static)
            for (int t = 0; t < T; ++t) {
                const uint16_t* xt = x + (size_t)t * H;
                for (int e = 0; e < E; ++e) {
                    float v = dot_bf16_f32(xt, w_router + (size_t)e * H, H);
                    if (bias) v = v + bias[e];
                    if (v == 0.0f) v = 0.0f; /* -0 -> +0 */
                    l[e] = v;
                }
                if (logits) memcpy(logits + (size_t)t * E, l, sizeof(float) * (size_t)E);
                topk_and_weights(l, E, k, ids + (size_t)t * k, w + (size_t)t * k, taken);
                if (s && w_sg) {
                    double c = dot_bf16_f64(xt, w_sg, H);
                    s[t] = 1.0 / (1.0 + exp(-c));
                }
            }
        }
        free(l);
        free(taken);
    }
    return err;
}

/* Top-k and weights on given fp32 logits [T,E] (the same rule as oracle_route). */
int oracle_route_from_logits(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
    if (T < 0 || E < 1 || k < 1 || k > E) return ORC_ERR_SHAPE;
    if (T == 0) return ORC_OK;
    if (!logits || !ids || !w) return ORC_ERR_NULL;
    if (!all_finite_f32(logits, (size_t)T * E)) return ORC_ERR_NONFINITE;
    int err = ORC_OK;
#pragma omp parallel
    {
        float* l = (float*)malloc(sizeof(float) * (size_t)E);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
        if (!l || !taken) {
#pragma omp atomic write
            err = ORC_ERR_NOMEM;
        } else {
#pragma omp for schedule(static)
            for (int t = 0; t < T; ++t) {
                for (int e = 0; e < E; ++e) {
                    float v = logits[(size_t)t * E + e];
                    if (v == 0.0f) v = 0.0f;
                    l[e] = v;
                }
                topk_and_weights(l, E, k, ids + (size_t)t * k, w + (size_t)t * k, taken);
            }
        }
        free(l);
        free(taken);
    }
    return err;
}

/*
 * Stable grouping of assignments by expert (step 4).
 *   ids[T*k] -> counts[E], offsets[E+1] (exclusive prefix of counts),
 *   perm[T*k]: the assignments a = t*k + j with ids[a] = e, ascending a,
 *   concatenated for e = 0 .. E-1 (no padding).
 */
int oracle_align(const int32_t* ids, int T, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm) {
    if (T < 0 || E < 1 || k < 1 || k > E) return ORC_ERR_SHAPE;
    if (!counts || !offsets || (T > 0 && (!ids || !perm))) return ORC_ERR_NULL;
    size_t n = (size_t)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (size_t a = 0; a < n; ++a) {
        if (ids[a] < 0 || ids[a] >= E) return ORC_ERR_SHAPE;
        counts[ids[a]] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (!fill) return ORC_ERR_NOMEM;
    for (size_t a = 0; a < n; ++a) {
        int e = ids[a];
        perm[offsets[e] + fill[e]] = (int32_t)a;
        fill[e] += 1;
    }
    free(fill);
    return ORC_OK;
}

/* SwiGLU hidden of one token under one expert's gate/up matrices [I,H],
 * rows row0 .. row0+I-1 of the operands. */
static void swiglu_hidden(const uint16_t* xt, wmat wg, wmat wu, size_t row0, int H, int I, double* hid) {
    for (int i = 0; i < I; ++i) {
        double g = dot_row_f64(xt, wg, row0 + (size_t)i, H);
        double u = dot_row_f64(xt, wu, row0 + (size_t)i, H);
        hid[i] = silu(g) * u;
    }
}

/* Down projection o[H] = Wd[H,I] . hid[I], rows row0 .. row0+H-1 of wd. */
static void swiglu_down(const double* hid, wmat wd, size_t row0, int H, int I, double* o) {
    for (int c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i) acc += hid[i] * wmat_at(wd, row0 + (size_t)c, (size_t)i, I);
        o[c] = acc;
    }
}

/* The whole layer with expert operands given as BF16 or as FP8 codes with
 * per-row scales; oracle_forward and oracle_forward_fp8 below marshal into it. */
static int forward_impl(const uint16_t* x, const uint16_t* w_router, const float* bias, wmat w_gate, wmat w_up,
                        wmat w_down, wmat ws_gate, wmat ws_up, wmat ws_down, const uint16_t* w_sg, int T, int H,
                        int E, int k, int I, int I_s, const int32_t* ids_in, double* y, int32_t* ids_out,
                        double* w_out, double* s_out, float* logits_out, double* h_out, double* o_out,
                        double* hs_out, double* os_out) {
    if (T < 0 || H < 1 || E < 1 || k < 1 || k > E || I < 1 || I_s < 0) return ORC_ERR_SHAPE;
    int n_shared = wmat_set(ws_gate) + wmat_set(ws_up) + wmat_set(ws_down) + (w_sg != NULL);
    if ((I_s == 0 && n_shared != 0) || (I_s > 0 && n_shared != 4)) return ORC_ERR_SHAPE;
    if (T == 0) return ORC_OK;
    if (!x || !w_router || !wmat_set(w_gate) || !wmat_set(w_up) || !wmat_set(w_down) || !y) return ORC_ERR_NULL;
    if (!wmat_finite(w_gate, (size_t)E * I, (size_t)H) || !wmat_finite(w_up, (size_t)E * I, (size_t)H) ||
        !wmat_finite(w_down, (size_t)E * H, (size_t)I) ||
        (I_s > 0 && (!wmat_finite(ws_gate, (size_t)I_s, (size_t)H) || !wmat_finite(ws_up, (size_t)I_s, (size_t)H) ||
                     !wmat_finite(ws_down, (size_t)H, (size_t)I_s))))
        return ORC_ERR_NONFINITE;

    size_t nA = (size_t)T * k;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * nA);
    double* w = (double*)malloc(sizeof(double) * nA);
    double* s = (double*)calloc((size_t)T, sizeof(double));
    float* lg = (float*)malloc(sizeof(float) * (size_t)T * E);
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * nA);
    double* o = (double*)malloc(sizeof(double) * nA * (size_t)H);
    double* os = I_s > 0 ? (double*)malloc(sizeof(double) * (size_t)T * H) : NULL;
    int err = ORC_OK;
    if (!ids || !w || !s || !lg || !counts || !offsets || !perm || !o || (I_s > 0 && !os)) {
        err = ORC_ERR_NOMEM;
        goto done;
    }

    /* 1-3: route (and, with ids_in, re-weight the given selection) */
    err = oracle_route(x, w_router, bias, w_sg, T, H, E, k, lg, ids, w, s);
    if (err) goto done;
    if (ids_in) {
        /* a selection is k distinct experts of [0, E) */
        for (size_t a = 0; a < nA; ++a) {
            if (ids_in[a] < 0 || ids_in[a] >= E) { err = ORC_ERR_SHAPE; goto done; }
            for (size_t b = a - a % (size_t)k; b < a; ++b)
                if (ids_in[b] == ids_in[a]) { err = ORC_ERR_SHAPE; goto done; }
        }
        for (int t = 0; t < T; ++t) {
            const float* l = lg + (size_t)t * E;
            double m = (double)l[0];
            for (int e = 1; e < E; ++e)
                if ((double)l[e] > m) m = (double)l[e];
            double z = 0.0;
            for (int e = 0; e < E; ++e) z += exp((double)l[e] - m);
            double psum = 0.0;
            for (int j = 0; j < k; ++j) {
                int e = ids_in[(size_t)t * k + j];
                ids[(size_t)t * k + j] = e;
                w[(size_t)t * k + j] = exp((double)l[e] - m) / z;
            }
            for (int j = 0; j < k; ++j) psum += w[(size_t)t * k + j];
            for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = w[(size_t)t * k + j] / psum;
        }
    }

    /* 4: stable align */
    err = oracle_align(ids, T, E, k, counts, offsets, perm);
    if (err) goto done;

    /* 5: every (expert, assignment) pair of the canonical permutation */
#pragma omp parallel
    {
        double* hid = (double*)malloc(sizeof(double) * (size_t)(I > I_s ? I : I_s));
        if (!hid) {
#pragma omp atomic write
            err = ORC_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (long q = 0; q < (long)nA; ++q) {
                int32_t a = perm[q];
                int e = ids[a];
                int t = a / k;
                const uint16_t* xt = x + (size_t)t * H;
                swiglu_hidden(xt, w_gate, w_up, (size_t)e * I, H, I, hid);
                if (h_out) memcpy(h_out + (size_t)a * I, hid, sizeof(double) * (size_t)I);
                swiglu_down(hid, w_down, (size_t)e * H, H, I, o + (size_t)a * H);
            }
            /* 6: shared expert over every token */
            if (I_s > 0) {
#pragma omp for schedule(dynamic, 4)
                for (int t = 0; t < T; ++t) {
                    const uint16_t* xt = x + (size_t)t * H;
                    swiglu_hidden(xt, ws_gate, ws_up, 0, H, I_s, hid);
                    if (hs_out) memcpy(hs_out + (size_t)t * I_s, hid, sizeof(double) * (size_t)I_s);
                    swiglu_down(hid, ws_down, 0, H, I_s, os + (size_t)t * H);
                }
            }
        }
        free(hid);
    }
    if (err) goto done;

    /* 7: combine in rank order, then the gated shared expert */
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double* yt = y + (size_t)t * H;
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) acc = acc + w[(size_t)t * k + j] * o[((size_t)t * k + j) * H + c];
            if (I_s > 0) acc = acc + s[t] * os[(size_t)t * H + c];
            yt[c] = acc;
        }
    }

    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * nA);
    if (w_out) memcpy(w_out, w, sizeof(double) * nA);
    if (s_out) memcpy(s_out, s, sizeof(double) * (size_t)T);
    if (logits_out) memcpy(logits_out, lg, sizeof(float) * (size_t)T * E);
    if (o_out) memcpy(o_out, o, sizeof(double) * nA * (size_t)H);
    if (os_out && I_s > 0) memcpy(os_out, os, sizeof(double) * (size_t)T * H);

done:
    free(ids);
    free(w);
    free(s);
    free(lg);
    free(counts);
    free(offsets);
    free(perm);
    free(o);
    free(os);
    return err;
}

/*
 * The whole layer.
 *   Inputs as in oracle_route plus w_gate/w_up [E,I,H], w_down [E,H,I],
 *   ws_gate/ws_up [I_s,H], ws_down [H,I_s], w_sg [H] (the shared four all
 *   NULL with I_s == 0, or all set).
 *   ids_in [T,k] (nullable): when given, routing selection is replaced by
 *   these ids and the weights are the renormalised softmax probabilities of
 *   these ids (used to evaluate a token under another side's selection).
 *   Each row must hold k distinct experts in [0, E) (else ORC_ERR_SHAPE);
 *   the order of a row is kept (w[t,j] belongs to ids_in[t,j] and the
 *   combine sums in that order).
 *   y [T,H] double (out).
 *   Optional outputs (nullable): ids_out [T,k], w_out [T,k] double,
 *   s_out [T] double, logits_out [T,E] fp32, h_out [T*k, I] double (hidden
 *   of assignment a), o_out [T*k, H] double, hs_out [T, I_s], os_out [T, H].
 */
int oracle_forward(const uint16_t* x, const uint16_t* w_router, const float* bias,
                   const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                   const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down, const uint16_t* w_sg,
                   int T, int H, int E, int k, int I, int I_s,
                   const int32_t* ids_in, double* y,
                   int32_t* ids_out, double* w_out, double* s_out, float* logits_out,
                   double* h_out, double* o_out, double* hs_out, double* os_out) {
    wmat g = {w_gate, NULL, NULL, NULL, NULL, NULL}, u = {w_up, NULL, NULL, NULL, NULL, NULL};
    wmat d = {w_down, NULL, NULL, NULL, NULL, NULL}, sg = {ws_gate, NULL, NULL, NULL, NULL, NULL};
    wmat su = {ws_up, NULL, NULL, NULL, NULL, NULL}, sd = {ws_down, NULL, NULL, NULL, NULL, NULL};
    return forward_impl(x, w_router, bias, g, u, d, sg, su, sd, w_sg, T, H, E, k, I, I_s, ids_in, y, ids_out, w_out,
                        s_out, logits_out, h_out, o_out, hs_out, os_out);
}

/*
 * The whole layer with FP8 expert weights (routed and shared): E4M3 codes
 * q_* in the shapes of the BF16 matrices above, and fp32 scales, one per
 * output row: sc_gate/sc_up [E,I], sc_down [E,H], ssc_gate/ssc_up [I_s],
 * ssc_down [H].  Router, bias, w_sg and every output as in oracle_forward.
 * A NaN code or a non-finite scale gives ORC_ERR_NONFINITE.
 */
int oracle_forward_fp8(const uint16_t* x, const uint16_t* w_router, const float* bias,
                       const uint8_t* q_gate, const float* sc_gate, const uint8_t* q_up, const float* sc_up,
                       const uint8_t* q_down, const float* sc_down,
                       const uint8_t* qs_gate, const float* ssc_gate, const uint8_t* qs_up, const float* ssc_up,
                       const uint8_t* qs_down, const float* ssc_down, const uint16_t* w_sg,
                       int T, int H, int E, int k, int I, int I_s,
                       const int32_t* ids_in, double* y,
                       int32_t* ids_out, double* w_out, double* s_out, float* logits_out,
                       double* h_out, double* o_out, double* hs_out, double* os_out) {
    double val[256];
    for (int c = 0; c < 256; ++c) val[c] = e4m3_value((uint8_t)c);
    wmat g = {NULL, q_gate, sc_gate, NULL, NULL, val}, u = {NULL, q_up, sc_up, NULL, NULL, val};
    wmat d = {NULL, q_down, sc_down, NULL, NULL, val}, sg = {NULL, qs_gate, ssc_gate, NULL, NULL, val};
    wmat su = {NULL, qs_up, ssc_up, NULL, NULL, val}, sd = {NULL, qs_down, ssc_down, NULL, NULL, val};
    return forward_impl(x, w_router, bias, g, u, d, sg, su, sd, w_sg, T, H, E, k, I, I_s, ids_in, y, ids_out, w_out,
                        s_out, logits_out, h_out, o_out, hs_out, os_out);
}

/*
 * The whole layer with 4-bit expert weights (routed and shared): codes
 * q_gate/q_up [E, I, H/2], q_down [E, H, I/2], qs_gate/qs_up [I_s, H/2],
 * qs_down [H, I_s/2] (two weights per byte), and fp16 group scales (bits)
 * s_gate/s_up [E, I, H/32], s_down [E, H, I/32], ss_gate/ss_up [I_s, H/32],
 * ss_down [H, I_s/32].  H, I and I_s must be multiples of 32.  Router, bias,
 * w_sg and every output as in oracle_forward.  A non-finite scale gives
 * ORC_ERR_NONFINITE.
 */
int oracle_forward_q4(const uint16_t* x, const uint16_t* w_router, const float* bias,
                      const uint8_t* q_gate, const uint16_t* s_gate, const uint8_t* q_up, const uint16_t* s_up,
                      const uint8_t* q_down, const uint16_t* s_down,
                      const uint8_t* qs_gate, const uint16_t* ss_gate, const uint8_t* qs_up, const uint16_t* ss_up,
                      const uint8_t* qs_down, const uint16_t* ss_down, const uint16_t* w_sg,
                      int T, int H, int E, int k, int I, int I_s,
                      const int32_t* ids_in, double* y,
                      int32_t* ids_out, double* w_out, double* s_out, float* logits_out,
                      double* h_out, double* o_out, double* hs_out, double* os_out) {
    if (H % Q4_GROUP || I % Q4_GROUP || I_s % Q4_GROUP) return ORC_ERR_SHAPE;
    wmat g = {NULL, NULL, NULL, q_gate, s_gate, NULL}, u = {NULL, NULL, NULL, q_up, s_up, NULL};
    wmat d = {NULL, NULL, NULL, q_down, s_down, NULL}, sg = {NULL, NULL, NULL, qs_gate, ss_gate, NULL};
    wmat su = {NULL, NULL, NULL, qs_up, ss_up, NULL}, sd = {NULL, NULL, NULL, qs_down, ss_down, NULL};
    return forward_impl(x, w_router, bias, g, u, d, sg, su, sd, w_sg, T, H, E, k, I, I_s, ids_in, y, ids_out, w_out,
                        s_out, logits_out, h_out, o_out, hs_out, os_out);
}
