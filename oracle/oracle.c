/*
 * CPU oracle for one batch-1 autoregressive decode step of a Llama-style
 * decoder.  TEST INFRASTRUCTURE ONLY: it is called by the tests, by the smoke
 * check and by the benchmark's CPU-baseline leg, never by the product path.
 * It shares no code, header, table or helper with the GPU library.
 *
 * Plain, slow and deliberately obvious: every value is a float64, every dot
 * product is a single left-to-right sum, nothing is blocked, fused or
 * reordered.  OpenMP only splits independent output rows (and independent
 * attention heads) between threads, so the result does not depend on the
 * thread count.
 *
 * What is computed.  The pages name the operators of a decode step and the
 * order they run in, but write no formulas:
 *   - cloud.baidu.com/article/9434380 ("low-latency single-request LLM
 *     inference: from operator fusion to runtime orchestration"), section 三
 *     (knowledge prerequisites): a forward pass is normalisation, rotary
 *     position encoding, attention, matrix multiply, activation and residual
 *     add; every generated token reads all weights once.
 *   - same page, section 五 step 2: segment A = input norm + Q/K/V linear
 *     maps + rotary encoding; segment B = attention scores + mask + softmax +
 *     attention output projection; segment C = output norm + FFN layer 1 +
 *     activation + FFN layer 2 + residual.
 *   - same page, section 五 step 4: the KV cache is read and written by the
 *     decode step; section 八 Q4: accumulation precision, norm stability and
 *     softmax overflow protection matter for numerical agreement.
 *   - developer.baidu.com/article/detail.html?id=8006242 (MegaKernel 1000 TPS
 *     tutorial), section 3.2: the Llama-3.2-1B single-sequence decode case;
 *     section 4.1.2: the op list is RMSNorm, attention and GEMMs.
 * The formulas below are the plain Llama-family reading of those operators
 * (each function states its reading).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, max_seq;
    double rms_eps, rope_theta;
    int32_t dtype; /* 0: float32 weights and KV cache; 1: bfloat16; 2: weight-only INT8 (the
                      matrices are int8 codes with one float32 scale per output row; the
                      embedding, the norm gains and the KV cache are bfloat16) */
    int32_t tied;  /* 1: the LM head is the token-embedding matrix (dtype 0 and 1 only) */
    /* dtype 2: per-row scales, a table indexed like the weight table below
       (entries of the LM head and the seven layer matrices; others unused) */
    const float *const *scales;
} or_model;

/* Weight pointer table: [0] embed [V][H], [1] final norm gain [H],
   [2] LM head [V][H] (ignored when tied), then per layer l at 3 + 9*l:
   attn_norm [H], wq [nh*d][H], wk [nkv*d][H], wv [nkv*d][H], wo [H][nh*d],
   ffn_norm [H], w_gate [F][H], w_up [F][H], w_down [H][F]; all row-major. */
enum { W_EMBED = 0, W_FINAL_NORM = 1, W_LM_HEAD = 2, W_LAYER0 = 3, W_PER_LAYER = 9 };
enum { L_ATTN_NORM = 0, L_WQ, L_WK, L_WV, L_WO, L_FFN_NORM, L_GATE, L_UP, L_DOWN };

/* ---- storage formats --------------------------------------------------- */

/* bfloat16 -> float64 is exact: the 16 bits are the top half of a binary32. */
double or_f64_from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* float64 -> bfloat16, round to nearest, ties to even, computed directly on
   the float64 value (no intermediate binary32 rounding).  NaN stays NaN,
   overflow goes to infinity, results below the bfloat16 normal range are
   rounded on the subnormal grid. */
uint16_t or_bf16_from_f64(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    /* Spacing of bfloat16 values around a: 2^(e-7) for normal a in
       [2^e, 2^(e+1)); 2^(-133) on the subnormal grid (e < -126). */
    int e;
    frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) -> a in [2^(e-1), 2^e) */
    e -= 1;
    if (e < -126) e = -126;
    double ulp = ldexp(1.0, e - 7);
    double q = a / ulp;          /* exact: division by a power of two */
    double fl = floor(q);
    double r = q - fl;           /* exact */
    double n = fl;
    if (r > 0.5 || (r == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
    double res = n * ulp;        /* exact */
    if (res > 0x1.FEp127) return sign | 0x7F80; /* rounded past the largest finite bfloat16 */
    float f = (float)res;        /* exact: res is a bfloat16 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

static inline double wload(const void *p, int dtype, size_t i) {
    return dtype ? or_f64_from_bf16(((const uint16_t *)p)[i]) : (double)((const float *)p)[i];
}

/* Store a cache entry in the cache's storage type: bfloat16 with RNE, or
   binary32 with the C conversion (IEEE round to nearest even). */
static inline void kvstore(void *p, int dtype, size_t i, double v) {
    if (dtype) ((uint16_t *)p)[i] = or_bf16_from_f64(v);
    else ((float *)p)[i] = (float)v;
}

/* ---- operators --------------------------------------------------------- */

/* RMSNorm: y_i = g_i * x_i / sqrt(mean(x^2) + eps).  eps is added to the
   mean square inside the root.  (Normalisation of segments A and C,
   cloud.baidu.com/article/9434380 §五 step 2; RMSNorm is the op the
   developer.baidu.com MegaKernel tutorial §4.1.2 names.) */
void or_rmsnorm(const double *x, int n, const void *g, int dtype, double eps, double *y) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int i = 0; i < n; ++i) y[i] = wload(g, dtype, (size_t)i) * (x[i] * inv);
}

/* Matrix-vector product y = W h with W row-major [rows][cols] (a Linear
   layer's [out][in] weight); each y_r is one sequential sum over cols. */
void or_gemv(const void *W, int dtype, int rows, int cols, const double *h, double *y) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        double acc = 0.0;
        size_t base = (size_t)r * (size_t)cols;
        for (int c = 0; c < cols; ++c) acc += wload(W, dtype, base + (size_t)c) * h[c];
        y[r] = acc;
    }
}

/* Weight-only INT8 matrix-vector product.  The stored matrix is int8 codes
   q [rows][cols] and one float32 scale per output row, and the weight it
   stands for is W[r][c] = s[r] * q[r][c] (dequantisation; the quantised
   models that www.stapisi.com/news/3904786 section 6.1 names stream these
   codes instead of 16-bit weights).  y = W h, each y_r one sequential sum
   over c of (s_r * q_rc) * h_c in float64. */
void or_gemv_q8(const int8_t *q, const float *s, int rows, int cols, const double *h, double *y) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        double acc = 0.0;
        const double sr = (double)s[r];
        size_t base = (size_t)r * (size_t)cols;
        for (int c = 0; c < cols; ++c) acc += (sr * (double)q[base + (size_t)c]) * h[c];
        y[r] = acc;
    }
}

/* Rotary position encoding, in place, on n_heads vectors of length d laid
   out back to back.  Pairing is "rotate half": element i is paired with
   i + d/2 for i < d/2, and the pair is rotated by the angle
   pos * theta^(-2i/d) (no frequency rescaling).  (Rotary position encoding
   of segment A, cloud.baidu.com/article/9434380 §五 step 2.) */
void or_rope(double *v, int n_heads, int d, int pos, double theta) {
    int half = d / 2;
    for (int h = 0; h < n_heads; ++h) {
        double *x = v + (size_t)h * (size_t)d;
        for (int i = 0; i < half; ++i) {
            double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)d);
            double c = cos(ang), s = sin(ang);
            double a = x[i], b = x[i + half];
            x[i] = a * c - b * s;
            x[i + half] = a * s + b * c;
        }
    }
}

/* Softmax with the maximum subtracted first (overflow protection, page
   cloud.baidu.com/article/9434380 §八 Q4). */
void or_softmax(const double *s, int n, double *p) {
    double m = -INFINITY;
    for (int i = 0; i < n; ++i) if (s[i] > m) m = s[i];
    double sum = 0.0;
    for (int i = 0; i < n; ++i) { p[i] = exp(s[i] - m); sum += p[i]; }
    for (int i = 0; i < n; ++i) p[i] /= sum;
}

/* One query head attending over n_pos cached positions of one KV head:
   K, V are [n_pos][d] in the cache dtype.  Scores q.K_t / sqrt(d), softmax,
   then the probability-weighted sum of V rows.  (Segment B: scores, mask,
   softmax; the causal mask is the choice n_pos = pos + 1.) */
void or_attend(const double *q, const void *K, const void *V, int dtype, int d, int n_pos, double *o) {
    double *s = (double *)malloc(sizeof(double) * (size_t)(n_pos > 0 ? n_pos : 1));
    double *p = (double *)malloc(sizeof(double) * (size_t)(n_pos > 0 ? n_pos : 1));
    double scale = 1.0 / sqrt((double)d);
    for (int t = 0; t < n_pos; ++t) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += q[i] * wload(K, dtype, (size_t)t * d + i);
        s[t] = acc * scale;
    }
    or_softmax(s, n_pos, p);
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    for (int t = 0; t < n_pos; ++t)
        for (int i = 0; i < d; ++i) o[i] += p[t] * wload(V, dtype, (size_t)t * d + i);
    free(s);
    free(p);
}

/* SiLU activation z * sigmoid(z) = z / (1 + e^-z) (the FFN activation of
   segment C, in its SwiGLU form below). */
double or_silu(double z) { return z / (1.0 + exp(-z)); }

/* Index of the largest entry; the lowest index wins ties (greedy decode). */
int or_argmax(const double *v, int n) {
    int best = 0;
    for (int i = 1; i < n; ++i) if (v[i] > v[best]) best = i;
    return best;
}

/* ---- the decode step --------------------------------------------------- */

static size_t kv_off(const or_model *m, int layer, int head, int pos) {
    return (((size_t)layer * m->n_kv_heads + head) * (size_t)m->max_seq + (size_t)pos) * (size_t)m->head_dim;
}

/*
 * One decode step for token `token` at 0-based position `pos`.
 *   x = E[token]
 *   per layer: h = rmsnorm(x, g_attn); q,k,v = Wq h, Wk h, Wv h;
 *              rope(q), rope(k) at pos;
 *              cache[pos] <- k, v (rounded to the cache dtype), then every
 *              query head i attends over cache positions 0..pos of KV head
 *              i / (n_heads / n_kv_heads);
 *              x += Wo o;
 *              h = rmsnorm(x, g_ffn); x += Wd (silu(Wg h) * (Wu h))
 *   logits = W_lm rmsnorm(x, g_final)      (skipped when logits == NULL)
 * Every "W h" is or_gemv, or or_gemv_q8 on the dequantised matrix of a
 * weight-only INT8 model (dtype 2; its LM head is its own int8 matrix).
 * The cache arrays are [n_layers][n_kv_heads][max_seq][head_dim].
 * Returns 0, or a negative code for an out-of-range token/position or an
 * invalid shape.
 */
int or_decode_step(const or_model *m, const void *const *w, void *kc, void *vc, int token, int pos,
                   double *logits) {
    const int H = m->hidden, nh = m->n_heads, nkv = m->n_kv_heads, d = m->head_dim, F = m->ffn;
    const int q8 = m->dtype == 2;
    const int dt = q8 ? 1 : m->dtype; /* storage of the embedding, gains and cache */
    if (token < 0 || token >= m->vocab) return -1;
    if (pos < 0 || pos >= m->max_seq) return -2;
    if (nkv <= 0 || nh % nkv != 0 || d % 2 != 0) return -3;
    if (m->dtype < 0 || m->dtype > 2 || (q8 && (m->tied || !m->scales))) return -3;
    /* matrix i of the weight table times h: plain or dequantised */
#define MAT(i, rows, cols, h, y)                                                              \
    do {                                                                                      \
        if (q8) or_gemv_q8((const int8_t *)w[i], m->scales[i], (rows), (cols), (h), (y));    \
        else or_gemv(w[i], dt, (rows), (cols), (h), (y));                                    \
    } while (0)
    const int group = nh / nkv;

    double *x = (double *)calloc((size_t)H, sizeof(double));
    double *h = (double *)calloc((size_t)H, sizeof(double));
    double *q = (double *)calloc((size_t)nh * d, sizeof(double));
    double *k = (double *)calloc((size_t)nkv * d, sizeof(double));
    double *v = (double *)calloc((size_t)nkv * d, sizeof(double));
    double *o = (double *)calloc((size_t)nh * d, sizeof(double));
    double *t = (double *)calloc((size_t)(H > F ? H : F), sizeof(double));
    double *g = (double *)calloc((size_t)F, sizeof(double));
    double *u = (double *)calloc((size_t)F, sizeof(double));

    for (int i = 0; i < H; ++i) x[i] = wload(w[W_EMBED], dt, (size_t)token * H + i);

    for (int l = 0; l < m->n_layers; ++l) {
        const size_t l0 = W_LAYER0 + (size_t)W_PER_LAYER * l;
        const void *const *lw = w + l0;
        or_rmsnorm(x, H, lw[L_ATTN_NORM], dt, m->rms_eps, h);
        MAT(l0 + L_WQ, nh * d, H, h, q);
        MAT(l0 + L_WK, nkv * d, H, h, k);
        MAT(l0 + L_WV, nkv * d, H, h, v);
        or_rope(q, nh, d, pos, m->rope_theta);
        or_rope(k, nkv, d, pos, m->rope_theta);
        for (int j = 0; j < nkv; ++j)
            for (int i = 0; i < d; ++i) {
                kvstore(kc, dt, kv_off(m, l, j, pos) + i, k[(size_t)j * d + i]);
                kvstore(vc, dt, kv_off(m, l, j, pos) + i, v[(size_t)j * d + i]);
            }
        /* heads are independent: OpenMP splits them between threads, each
           head's sums keep their sequential order */
#pragma omp parallel for schedule(static)
        for (int i = 0; i < nh; ++i) {
            int j = i / group;
            const size_t base = kv_off(m, l, j, 0) * (dt ? 2u : 4u);
            or_attend(q + (size_t)i * d, (const char *)kc + base, (const char *)vc + base, dt, d, pos + 1,
                      o + (size_t)i * d);
        }
        MAT(l0 + L_WO, H, nh * d, o, t);
        for (int i = 0; i < H; ++i) x[i] += t[i];

        or_rmsnorm(x, H, lw[L_FFN_NORM], dt, m->rms_eps, h);
        MAT(l0 + L_GATE, F, H, h, g);
        MAT(l0 + L_UP, F, H, h, u);
        for (int i = 0; i < F; ++i) g[i] = or_silu(g[i]) * u[i];
        MAT(l0 + L_DOWN, H, F, g, t);
        for (int i = 0; i < H; ++i) x[i] += t[i];
    }
    if (logits) {
        or_rmsnorm(x, H, w[W_FINAL_NORM], dt, m->rms_eps, h);
        if (m->tied) or_gemv(w[W_EMBED], dt, m->vocab, H, h, logits);
        else MAT(W_LM_HEAD, m->vocab, H, h, logits);
    }
#undef MAT
    free(x); free(h); free(q); free(k); free(v); free(o); free(t); free(g); free(u);
    return 0;
}

/* Prefill: by definition under causal attention, the cache after a prompt
   is what n successive decode steps at positions start..start+n-1 leave. */
int or_prefill(const or_model *m, const void *const *w, void *kc, void *vc, const int32_t *tokens, int n,
               int start_pos) {
    if (n < 0 || start_pos < 0 || start_pos + n > m->max_seq) return -2;
    for (int i = 0; i < n; ++i) {
        int rc = or_decode_step(m, w, kc, vc, tokens[i], start_pos + i, NULL);
        if (rc) return rc;
    }
    return 0;
}

/* Threads the OpenMP row loops use (reported by the CPU-baseline timing). */
#ifdef _OPENMP
#include <omp.h>
int or_num_threads(void) { return omp_get_max_threads(); }
void or_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int or_num_threads(void) { return 1; }
void or_set_num_threads(int n) { (void)n; }
#endif
