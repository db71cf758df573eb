/*
 * q4moe_oracle.c -- plain, slow CPU oracle of the routed mixture-of-experts
 * FFN layer with group-64 affine 4-bit expert weights.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only code that may load this library.
 * It shares no code, header, table or helper with the HIP path; it includes
 * nothing but the C standard library.
 *
 * Sources.  [Lily-M5] is the page "Perplexity's Lily beats MLX-LM on MacBook
 * M5 because it only runs one model"; sections are named in quotes.
 *   [Lily-M5, "Why Qwen3.6-35B-A3B is a weird workload"]
 *       8 of 256 routed experts per token, plus 1 always-on shared
 *       expert.
 *   [Lily-M5, "Prefill: keep routing on the GPU, dequantize in flight"]
 *       4-bit codes, one bf16 scale and one bf16 bias per group of 64; the
 *       matrix units consume bf16, so each weight is rebuilt as a bf16 value
 *       before it is multiplied; FP32 sums, bf16 results; after each top-k
 *       step the rows are grouped per expert (histogram, prefix scan,
 *       scatter, block map); 32-row tiles.
 *   [Lily-M5, "Decode: minimize bytes per token"]
 *       the gate activation is folded into the input projections, and the
 *       scores and the shared expert into the output projection.
 *
 * Readings where the pages leave a step open (the plainest one the rest of
 * the text supports):
 *   - dequantised weight  w = bf16_round(q * scale + bias), q the 4-bit code
 *     (q*scale+bias is exact in double; it is rounded once, to nearest even);
 *   - code packing: eight codes per 32-bit word along K, lowest nibble first;
 *   - expert:  E(x) = W_down . bf16_round(SiLU(W_gate . x) * (W_up . x)),
 *     SiLU(g) = g / (1 + exp(-g)); h is rounded to bf16 because it is the
 *     next contraction's bf16 operand;
 *   - selection: the k largest fp32 logits, greater first, equal logits
 *     ordered by the lower expert index (softmax is strictly increasing, so
 *     this is top-k of the softmax);
 *   - scores: softmax over all experts, then the selected probabilities are
 *     divided by their sum;
 *   - combine: y_t = sum over slots s = 0..k-1 (in slot order) of
 *     w[t,s] * E_idx[t,s](x_t), then + E_shared(x_t) with weight 1 (the
 *     pages name no gate on the shared expert); y is rounded once to bf16;
 *   - expert-sorted order: assignments a = t*k + s grouped by expert,
 *     ascending a (that is, ascending token) inside an expert;
 *   - block map: for each non-empty expert in ascending order, one entry
 *     (expert, first sorted row) per tile of BM rows.
 *
 * Precision: every dot product accumulates in double, index ascending.  The
 * only roundings are the ones listed above plus the fp32 rounding of the
 * router logits and of the output logits of the token hand-off (both are
 * fp32 logits).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 64

/* ---- bf16 <-> double ---------------------------------------------------- */

static double bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void fail(const char* what) {
    fprintf(stderr, "q4moe oracle: %s\n", what);
    abort();
}

/* Nearest bf16 (8 significant bits, fp32 exponent range) to v, ties to even. */
static uint16_t bf16_round(double v) {
    if (isnan(v) || isinf(v)) fail("non-finite value");
    if (v == 0.0) return signbit(v) ? 0x8000u : 0x0000u;
    int e;
    (void)frexp(fabs(v), &e);              /* |v| in [2^(e-1), 2^e) */
    int qexp = e - 8;                      /* spacing of bf16 numbers in that binade */
    if (qexp < -133) qexp = -133;          /* subnormal bf16 spacing */
    double r = ldexp(rint(ldexp(fabs(v), -qexp)), qexp);  /* rint: ties to even */
    if (r > 3.3895313892515355e38) fail("bf16 overflow");
    float f = (float)r;                    /* exact: at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)((u >> 16) | (v < 0 ? 0x8000u : 0u));
}

/* ---- O1: dequantisation ------------------------------------------------- */

/* code q(n,k) of row n, column k of a [N][K/8]-word matrix */
static unsigned code_at(const uint32_t* q, int64_t K, int64_t n, int64_t k) {
    return (unsigned)((q[n * (K / 8) + k / 8] >> (4 * (k % 8))) & 0xFu);
}

static uint16_t dequant_at(const uint32_t* q, const uint16_t* scale, const uint16_t* bias,
                           int64_t K, int64_t n, int64_t k) {
    int64_t g = n * (K / GROUP) + k / GROUP;
    return bf16_round((double)code_at(q, K, n, k) * bf16_value(scale[g]) + bf16_value(bias[g]));
}

/* w[n*K + k] = bf16_round(q(n,k) * scale(n, k/64) + bias(n, k/64)) */
void oracle_dequant(const uint32_t* q, const uint16_t* scale, const uint16_t* bias,
                    int64_t N, int64_t K, uint16_t* w) {
    if (K % GROUP) fail("K must be a multiple of 64");
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) w[n * K + k] = dequant_at(q, scale, bias, K, n, k);
}

/* ---- the layer ---------------------------------------------------------- */

typedef struct {
    const uint32_t* q;
    const uint16_t* scale;
    const uint16_t* bias;
} oracle_q4;

typedef struct {
    int64_t d, inter, n_experts, top_k;
    const float* w_router;    /* [d][E] */
    const float* router_bias; /* [E] or NULL */
    oracle_q4 gate, up;       /* [E][inter][d/8], [E][inter][d/64] */
    oracle_q4 down;           /* [E][d][inter/8], [E][d][inter/64] */
    oracle_q4 sh_gate, sh_up; /* [inter][d/8] ... */
    oracle_q4 sh_down;        /* [d][inter/8] ... */
} oracle_layer;

/* Matrix `m` of expert e (N rows, K columns) viewed as one [N][K] matrix. */
static oracle_q4 expert_matrix(oracle_q4 m, int64_t e, int64_t N, int64_t K) {
    oracle_q4 r;
    r.q = m.q + e * N * (K / 8);
    r.scale = m.scale + e * N * (K / GROUP);
    r.bias = m.bias + e * N * (K / GROUP);
    return r;
}

/* O2: l[t][e] = fp32( sum_j x[t][j] * W_r[j][e]  (+ b[e]) ) */
void oracle_router_logits(const uint16_t* x, int64_t T, int64_t d, const float* w_router,
                          const float* router_bias, int64_t E, float* logits) {
    double* acc = (double*)malloc(sizeof(double) * (size_t)E);
    for (int64_t t = 0; t < T; ++t) {
        /* every acc[e] still sums its terms j = 0, 1, ..., d-1 in order */
        for (int64_t e = 0; e < E; ++e) acc[e] = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            const double xj = bf16_value(x[t * d + j]);
            for (int64_t e = 0; e < E; ++e) acc[e] += xj * (double)w_router[j * E + e];
        }
        for (int64_t e = 0; e < E; ++e) {
            if (router_bias) acc[e] += (double)router_bias[e];
            logits[t * E + e] = (float)acc[e];
        }
    }
    free(acc);
}

/* O3-O7: selection, scores, histogram, exclusive scan, expert-sorted order. */
void oracle_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* idx, double* w,
                  int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm) {
    if (k < 1 || k > E) fail("need 1 <= k <= E");
    char* taken = (char*)malloc((size_t)E);
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        for (int64_t e = 0; e < E; ++e)
            if (isnan(l[e])) fail("NaN logit");
        /* selection: repeatedly take the largest remaining logit; strict '>'
           while scanning e upward keeps the lower index on equal logits */
        memset(taken, 0, (size_t)E);
        for (int64_t s = 0; s < k; ++s) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            idx[t * k + s] = (int32_t)best;
        }
        /* scores: softmax over all E experts, then renormalise over the selected */
        double m = -INFINITY;
        for (int64_t e = 0; e < E; ++e)
            if ((double)l[e] > m) m = (double)l[e];
        double Z = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - m);
            Z += p[e];
        }
        double S = 0.0;
        for (int64_t s = 0; s < k; ++s) S += p[idx[t * k + s]] / Z;
        for (int64_t s = 0; s < k; ++s) w[t * k + s] = (p[idx[t * k + s]] / Z) / S;
    }
    free(taken);
    free(p);

    const int64_t A = T * k; /* assignments a = t*k + s */
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < A; ++a) counts[idx[a]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t pos = 0;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t a = 0; a < A; ++a)
            if (idx[a] == e) {
                perm[pos] = (int32_t)a;
                inv_perm[a] = (int32_t)pos;
                ++pos;
            }
}

/* O8: block map with tiles of bm rows.  block_map holds (expert, first row)
   pairs; capacity floor(T*k/bm) + E pairs always suffices. */
void oracle_block_map(const int32_t* counts, const int32_t* offsets, int64_t E, int64_t bm,
                      int32_t* block_map, int32_t* n_blocks) {
    int64_t n = 0;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t r = 0; r < counts[e]; r += bm) {
            block_map[2 * n] = (int32_t)e;
            block_map[2 * n + 1] = offsets[e] + (int32_t)r;
            ++n;
        }
    *n_blocks = (int32_t)n;
}

/* One expert applied to one token: h (bf16, optional) and its output P (double).
   gate/up/down are that expert's [N][K] matrices. */
static void expert_apply(oracle_q4 gate, oracle_q4 up, oracle_q4 down, int64_t d, int64_t inter,
                         const uint16_t* x_t, uint16_t* h_out, double* P, uint16_t* hbuf) {
    for (int64_t n = 0; n < inter; ++n) {
        double g = 0.0, u = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            double xj = bf16_value(x_t[j]);
            g += xj * bf16_value(dequant_at(gate.q, gate.scale, gate.bias, d, n, j));
            u += xj * bf16_value(dequant_at(up.q, up.scale, up.bias, d, n, j));
        }
        double silu = g / (1.0 + exp(-g));
        hbuf[n] = bf16_round(silu * u);
        if (h_out) h_out[n] = hbuf[n];
    }
    for (int64_t n2 = 0; n2 < d; ++n2) {
        double acc = 0.0;
        for (int64_t n = 0; n < inter; ++n)
            acc += bf16_value(hbuf[n]) * bf16_value(dequant_at(down.q, down.scale, down.bias,
                                                                inter, n2, n));
        P[n2] = acc;
    }
}

/* Expert e (0..E-1) or the shared expert (e = -1) on one token. */
void oracle_expert(const oracle_layer* L, int64_t e, const uint16_t* x_t, uint16_t* h_out,
                   double* P) {
    const int64_t d = L->d, I = L->inter;
    oracle_q4 g, u, dn;
    if (e < 0) {
        g = L->sh_gate;
        u = L->sh_up;
        dn = L->sh_down;
    } else {
        if (e >= L->n_experts) fail("expert index out of range");
        g = expert_matrix(L->gate, e, I, d);
        u = expert_matrix(L->up, e, I, d);
        dn = expert_matrix(L->down, e, d, I);
    }
    uint16_t* hbuf = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
    expert_apply(g, u, dn, d, I, x_t, h_out, P, hbuf);
    free(hbuf);
}

/* O9-O12 for the listed tokens: y = sum_s w[t,s] E_idx[t,s](x_t) + E_shared(x_t),
   slots in order, then the shared expert.  y_exact is the unrounded sum,
   y the bf16 output. */
void oracle_layer_tokens(const oracle_layer* L, const uint16_t* x, const int32_t* tokens,
                         int64_t n_tokens, const int32_t* idx, const double* w, double* y_exact,
                         uint16_t* y) {
    const int64_t d = L->d, k = L->top_k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_tokens; ++i) {
        const int64_t t = tokens[i];
        const uint16_t* x_t = x + t * d;
        double* P = (double*)malloc(sizeof(double) * (size_t)d);
        double* acc = (double*)calloc((size_t)d, sizeof(double));
        for (int64_t s = 0; s < k; ++s) {
            oracle_expert(L, idx[t * k + s], x_t, NULL, P);
            for (int64_t n = 0; n < d; ++n) acc[n] += w[t * k + s] * P[n];
        }
        oracle_expert(L, -1, x_t, NULL, P);
        for (int64_t n = 0; n < d; ++n) {
            acc[n] += P[n];
            y_exact[i * d + n] = acc[n];
            y[i * d + n] = bf16_round(acc[n]);
        }
        free(P);
        free(acc);
    }
}

/* Threads the OpenMP runtime would use for oracle_layer_tokens (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int oracle_threads(void) { return omp_get_max_threads(); }
#else
int oracle_threads(void) { return 1; }
#endif

/* Test hook: the bf16 rounding used throughout, on an array of doubles. */
void oracle_bf16_round(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(v[i]);
}

/* ---- O13-O15: greedy decoding's token hand-off --------------------------- */
/* [Lily-M5, "Decode: minimize bytes per token"]: the greedy token stays on the
   device between decode steps; the largest output logit selects it and it
   feeds the following step's input directly.
   Readings (the pages give no further detail):
     - the output projection ("LM head") and the input embedding table are V x d
       matrices in the experts' group-64 Q4 format, used as bf16 weights;
     - logit v = fp32( sum_j x[j] * w(v, j) ), summed in double, j ascending;
     - the greedy token is the index of the largest logit, equal logits ordered
       by the lower index, a NaN logit counting as minus infinity (so a vector of
       V NaNs gives token 0);
     - the next step's input is the token's embedding row, i.e. the dequantised
       bf16 row (oracle_dequant of that one row). */

/* O13: logits[v] for v = 0..V-1 of a [V][d] Q4 matrix applied to x (bf16 [d]). */
void oracle_lm_logits(const uint32_t* q, const uint16_t* scale, const uint16_t* bias, int64_t V,
                      int64_t d, const uint16_t* x, float* logits) {
    if (d % GROUP) fail("d must be a multiple of 64");
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t v = 0; v < V; ++v) {
        double acc = 0.0;
        for (int64_t j = 0; j < d; ++j)
            acc += bf16_value(x[j]) * bf16_value(dequant_at(q, scale, bias, d, v, j));
        logits[v] = (float)acc;
    }
}

/* O14: the greedy token. */
int64_t oracle_argmax(const float* logits, int64_t V) {
    int64_t best = 0;
    double best_v = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        const double lv = isnan(logits[v]) ? -INFINITY : (double)logits[v];
        if (v == 0 || lv > best_v) {
            best = v;
            best_v = lv;
        }
    }
    return best;
}
