/*
 * CPU oracle: a plain, slow forward pass of the decode step.  TEST
 * INFRASTRUCTURE ONLY (tests, the smoke check, the benchmark's CPU-baseline leg).
 * It shares no code with the HIP path; see oracle.h for sources and the
 * precision contract.  Threads split output rows (OpenMP); a dot product never
 * spans threads, so results do not depend on the thread count.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

static inline float bf_to_f(uint16_t v) {
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round to nearest even on the 16 dropped bits; NaN stays NaN. */
uint16_t orc_bf16_bits(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

int32_t orc_threads(void) { return (int32_t)omp_get_max_threads(); }

/* dot(w, x) = sum_i w_i x_i (bf16 weights, fp32 activations), accumulated in
 * double in index order (every product is exact in double), rounded once to fp32. */
float orc_dot(const uint16_t* w, const float* x, int32_t n) {
    double s = 0.0;
    for (int32_t i = 0; i < n; ++i) s += (double)bf_to_f(w[i]) * (double)x[i];
    return (float)s;
}

/* RMSNorm: x_i = fp32(h_i * g_i / sqrt(mean(h^2) + eps)), statistics in double. */
void orc_rmsnorm(const float* h, const uint16_t* g, int32_t d, double eps, float* x) {
    double ss = 0.0;
    for (int32_t i = 0; i < d; ++i) ss += (double)h[i] * (double)h[i];
    double r = 1.0 / sqrt(ss / (double)d + eps);
    for (int32_t i = 0; i < d; ++i) x[i] = (float)((double)h[i] * r * (double)bf_to_f(g[i]));
}

/* Rotary embedding, rotate-half pairing: for i < hd/2 the pair (v_i, v_{i+hd/2})
 * turns by the angle pos * theta^(-2i/hd).  Angle, cos and sin in double, cos and
 * sin rounded to fp32, each rotated component rounded once to fp32. */
void orc_rope(float* v, int32_t hd, int32_t pos, double theta) {
    int32_t half = hd / 2;
    for (int32_t i = 0; i < half; ++i) {
        double inv = pow(theta, -2.0 * (double)i / (double)hd);
        double ang = (double)pos * inv;
        float c = (float)cos(ang), s = (float)sin(ang);
        double a = v[i], b = v[i + half];
        v[i] = (float)(a * (double)c - b * (double)s);
        v[i + half] = (float)(a * (double)s + b * (double)c);
    }
}

/* Softmax attention of one query over n cached positions (rows `stride` elements
 * apart): s_j = fp32(q.K_j / sqrt(hd)), p = softmax(s) in double,
 * o = fp32(sum_j p_j V_j) in double. */
void orc_attend(const float* q, const uint16_t* K, const uint16_t* V, int64_t stride, int32_t n, int32_t hd,
                float* o) {
    double* e = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double m = -INFINITY;
    double scale = sqrt((double)hd);
    for (int32_t j = 0; j < n; ++j) {
        double s = 0.0;
        for (int32_t i = 0; i < hd; ++i) s += (double)q[i] * (double)bf_to_f(K[(int64_t)j * stride + i]);
        float sj = (float)(s / scale);
        e[j] = sj;
        if (sj > m) m = sj;
    }
    double z = 0.0;
    for (int32_t j = 0; j < n; ++j) {
        e[j] = exp(e[j] - m);
        z += e[j];
    }
    for (int32_t i = 0; i < hd; ++i) {
        double acc = 0.0;
        for (int32_t j = 0; j < n; ++j) acc += (e[j] / z) * (double)bf_to_f(V[(int64_t)j * stride + i]);
        o[i] = (float)acc;
    }
    free(e);
}

/* SwiGLU product: fp32(silu(z) * u), silu(z) = z / (1 + e^-z) in double. */
float orc_swiglu(float z, float u) {
    double zz = z;
    double silu = zz / (1.0 + exp(-zz));
    return (float)(silu * (double)u);
}

/* Greedy choice: the lowest index attaining the maximum; -1 if any entry is NaN. */
int32_t orc_argmax(const float* v, int32_t n) {
    int32_t best = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (v[i] != v[i]) return -1;
        if (v[i] > v[best]) best = i;
    }
    return n > 0 ? best : -1;
}

/* Router: prob = fp32(softmax(zeta)) in double; sel = the k largest probabilities,
 * ties to the lower expert index, returned in ascending expert order. */
void orc_route(const float* zeta, int32_t E, int32_t k, int32_t* sel, float* prob) {
    if (E <= 0 || k <= 0 || k > E) return;
    double m = -INFINITY, z = 0.0;
    for (int32_t e = 0; e < E; ++e)
        if (zeta[e] > m) m = zeta[e];
    for (int32_t e = 0; e < E; ++e) z += exp((double)zeta[e] - m);
    for (int32_t e = 0; e < E; ++e) prob[e] = (float)(exp((double)zeta[e] - m) / z);
    char* taken = (char*)calloc((size_t)E, 1);
    for (int32_t t = 0; t < k; ++t) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || prob[e] > prob[best])) best = e;
        taken[best] = 1;
    }
    int32_t c = 0;
    for (int32_t e = 0; e < E; ++e)
        if (taken[e]) sel[c++] = e;
    free(taken);
}

/* y[b*ys + r] = dot(W_r, x[b*xs ...]) for rows [0, rows); threads over rows. */
static void gemv(const uint16_t* W, int32_t rows, int32_t cols, const float* x, int32_t xs, int32_t B, float* y,
                 int32_t ys) {
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < rows; ++r)
        for (int32_t b = 0; b < B; ++b) y[(int64_t)b * ys + r] = orc_dot(W + (int64_t)r * cols, x + (int64_t)b * xs, cols);
}

static int32_t* g_moe_sel = 0;
static float* g_moe_prob = 0;
void orc_set_moe_trace(int32_t* sel, float* prob) {
    g_moe_sel = sel;
    g_moe_prob = prob;
}

/* FFN of one layer for B activations; adds the result into h. */
static void ffn_block(const orc_cfg* c, const orc_layer* lw, int32_t layer, int32_t B, float* h) {
    const int32_t d = c->hidden;
    float* x = (float*)malloc(sizeof(float) * (size_t)B * d);
    for (int32_t b = 0; b < B; ++b) orc_rmsnorm(h + (int64_t)b * d, lw->mlp_norm, d, c->rms_eps, x + (int64_t)b * d);
    if (c->n_experts == 0) {
        const int32_t F = c->ffn;
        float* z = (float*)malloc(sizeof(float) * (size_t)B * F);
        float* u = (float*)malloc(sizeof(float) * (size_t)B * F);
        float* dn = (float*)malloc(sizeof(float) * (size_t)B * d);
        gemv(lw->w_gate, F, d, x, d, B, z, F);
        gemv(lw->w_up, F, d, x, d, B, u, F);
        for (int64_t i = 0; i < (int64_t)B * F; ++i) z[i] = orc_swiglu(z[i], u[i]);
        gemv(lw->w_down, d, F, z, F, B, dn, d);
        for (int64_t i = 0; i < (int64_t)B * d; ++i) h[i] = (float)((double)h[i] + (double)dn[i]);
        free(z); free(u); free(dn);
    } else {
        const int32_t E = c->n_experts, K = c->top_k, Fe = c->expert_ffn;
        float* zeta = (float*)malloc(sizeof(float) * (size_t)B * E);
        float* prob = (float*)malloc(sizeof(float) * (size_t)B * E);
        int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * (K > 0 ? K : 1));
        gemv(lw->router, E, d, x, d, B, zeta, E);
        for (int32_t b = 0; b < B; ++b) {
            orc_route(zeta + (int64_t)b * E, E, K, sel + (int64_t)b * K, prob + (int64_t)b * E);
            if (g_moe_sel) memcpy(g_moe_sel + ((int64_t)layer * B + b) * K, sel + (int64_t)b * K, sizeof(int32_t) * K);
            if (g_moe_prob) memcpy(g_moe_prob + ((int64_t)layer * B + b) * E, prob + (int64_t)b * E, sizeof(float) * E);
        }
        float* z = (float*)malloc(sizeof(float) * (size_t)Fe);
        float* u = (float*)malloc(sizeof(float) * (size_t)Fe);
        float* ye = (float*)malloc(sizeof(float) * (size_t)d);
        double* acc = (double*)malloc(sizeof(double) * (size_t)d);
        for (int32_t b = 0; b < B; ++b) {
            const float* xb = x + (int64_t)b * d;
            /* shared expert(s), weight 1 */
            for (int32_t i = 0; i < d; ++i) acc[i] = 0.0;
            for (int32_t s = 0; s < c->n_shared; ++s) {
                gemv(lw->s_gate, Fe, d, xb, d, 1, z, Fe);
                gemv(lw->s_up, Fe, d, xb, d, 1, u, Fe);
                for (int32_t f = 0; f < Fe; ++f) z[f] = orc_swiglu(z[f], u[f]);
                gemv(lw->s_down, d, Fe, z, Fe, 1, ye, d);
                for (int32_t i = 0; i < d; ++i) acc[i] += (double)ye[i];
            }
            /* routed experts in ascending expert order, weighted by their probability */
            for (int32_t t = 0; t < K; ++t) {
                int32_t e = sel[(int64_t)b * K + t];
                double p = prob[(int64_t)b * E + e];
                gemv(lw->e_gate[e], Fe, d, xb, d, 1, z, Fe);
                gemv(lw->e_up[e], Fe, d, xb, d, 1, u, Fe);
                for (int32_t f = 0; f < Fe; ++f) z[f] = orc_swiglu(z[f], u[f]);
                gemv(lw->e_down[e], d, Fe, z, Fe, 1, ye, d);
                for (int32_t i = 0; i < d; ++i) acc[i] += p * (double)ye[i];
            }
            for (int32_t i = 0; i < d; ++i) {
                float y = (float)acc[i];
                h[(int64_t)b * d + i] = (float)((double)h[(int64_t)b * d + i] + (double)y);
            }
        }
        free(z); free(u); free(ye); free(acc); free(zeta); free(prob); free(sel);
    }
    free(x);
}

int orc_ffn(const orc_cfg* c, const orc_layer* lw, int32_t B, float* h) {
    if (B <= 0 || c->hidden <= 0) return ORC_E_ARG;
    ffn_block(c, lw, 0, B, h);
    return ORC_OK;
}

static int valid_cfg(const orc_cfg* c) {
    if (c->n_layers < 0 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
        c->vocab <= 0)
        return 0;
    if (c->n_q_heads % c->n_kv_heads || c->head_dim % 2) return 0;
    if (c->n_experts == 0 && c->ffn <= 0) return 0;
    if (c->n_experts > 0 && (c->top_k <= 0 || c->top_k > c->n_experts || c->expert_ffn <= 0)) return 0;
    return 1;
}

static int head_logits(const orc_cfg* c, const orc_weights* w, int32_t B, const float* h, float* logits,
                       int32_t* next) {
    const int32_t d = c->hidden, V = c->vocab;
    float* x = (float*)malloc(sizeof(float) * (size_t)B * d);
    for (int32_t b = 0; b < B; ++b) orc_rmsnorm(h + (int64_t)b * d, w->final_norm, d, c->rms_eps, x + (int64_t)b * d);
    gemv(w->lm_head, V, d, x, d, B, logits, V);
    free(x);
    int rc = ORC_OK;
    for (int32_t b = 0; b < B; ++b) {
        next[b] = orc_argmax(logits + (int64_t)b * V, V);
        if (next[b] < 0) rc = ORC_E_NAN;
    }
    return rc;
}

int orc_step(const orc_cfg* c, const orc_weights* w, orc_cache* kv, int32_t B, const int32_t* pos,
             const int32_t* tok, float* logits, int32_t* next) {
    if (!valid_cfg(c) || B <= 0 || B > kv->batch) return ORC_E_ARG;
    for (int32_t b = 0; b < B; ++b)
        if (pos[b] < 0 || pos[b] >= kv->max_seq || tok[b] < 0 || tok[b] >= c->vocab) return ORC_E_ARG;
    const int32_t d = c->hidden, Hq = c->n_q_heads, Hkv = c->n_kv_heads, hd = c->head_dim;
    const int32_t group = Hq / Hkv, S = kv->max_seq;
    float* h = (float*)malloc(sizeof(float) * (size_t)B * d);
    float* x = (float*)malloc(sizeof(float) * (size_t)B * d);
    float* q = (float*)malloc(sizeof(float) * (size_t)B * Hq * hd);
    float* k = (float*)malloc(sizeof(float) * (size_t)B * Hkv * hd);
    float* v = (float*)malloc(sizeof(float) * (size_t)B * Hkv * hd);
    float* o = (float*)malloc(sizeof(float) * (size_t)B * Hq * hd);
    float* ao = (float*)malloc(sizeof(float) * (size_t)B * d);
    /* embedding lookup: the residual stream starts as the token's row, widened exactly */
    for (int32_t b = 0; b < B; ++b)
        for (int32_t i = 0; i < d; ++i) h[(int64_t)b * d + i] = bf_to_f(w->embed[(int64_t)tok[b] * d + i]);
    for (int32_t l = 0; l < c->n_layers; ++l) {
        const orc_layer* lw = &w->layers[l];
        for (int32_t b = 0; b < B; ++b) orc_rmsnorm(h + (int64_t)b * d, lw->attn_norm, d, c->rms_eps, x + (int64_t)b * d);
        gemv(lw->wq, Hq * hd, d, x, d, B, q, Hq * hd);
        gemv(lw->wk, Hkv * hd, d, x, d, B, k, Hkv * hd);
        gemv(lw->wv, Hkv * hd, d, x, d, B, v, Hkv * hd);
        for (int32_t b = 0; b < B; ++b) {
            for (int32_t hh = 0; hh < Hq; ++hh) {
                orc_rope(q + ((int64_t)b * Hq + hh) * hd, hd, pos[b], c->rope_theta);
            }
            for (int32_t g = 0; g < Hkv; ++g) {
                float* kg = k + ((int64_t)b * Hkv + g) * hd;
                float* vg = v + ((int64_t)b * Hkv + g) * hd;
                orc_rope(kg, hd, pos[b], c->rope_theta);
                int64_t base = ((((int64_t)l * kv->batch + b) * Hkv + g) * S + pos[b]) * hd;
                for (int32_t i = 0; i < hd; ++i) {
                    kv->k[base + i] = orc_bf16_bits(kg[i]);
                    kv->v[base + i] = orc_bf16_bits(vg[i]);
                }
            }
        }
#pragma omp parallel for schedule(dynamic) collapse(2)
        for (int32_t b = 0; b < B; ++b)
            for (int32_t hh = 0; hh < Hq; ++hh) {
                int32_t g = hh / group;
                int64_t base = (((int64_t)l * kv->batch + b) * Hkv + g) * S * hd;
                orc_attend(q + ((int64_t)b * Hq + hh) * hd, kv->k + base, kv->v + base, hd, pos[b] + 1, hd,
                           o + ((int64_t)b * Hq + hh) * hd);
            }
        gemv(lw->wo, d, Hq * hd, o, Hq * hd, B, ao, d);
        for (int64_t i = 0; i < (int64_t)B * d; ++i) h[i] = (float)((double)h[i] + (double)ao[i]);
        ffn_block(c, lw, l, B, h);
    }
    int rc = head_logits(c, w, B, h, logits, next);
    free(h); free(x); free(q); free(k); free(v); free(o); free(ao);
    return rc;
}

/* P tokens per sequence in one layer-major pass: token t of sequence b sits at
 * position pos[b] + t.  Per layer the K/V of every new position are written into
 * the cache first; the query at position p then attends to cache positions 0..p,
 * so each position sees exactly what P single-position steps would have given it
 * (same primitives, same order inside every dot product).  Writes the logits of
 * each sequence's last position [B][V] and its greedy token next[B]. */
int orc_prefill(const orc_cfg* c, const orc_weights* w, orc_cache* kv, int32_t B, int32_t P, const int32_t* pos,
                const int32_t* tokens, float* logits, int32_t* next) {
    if (!valid_cfg(c) || B <= 0 || B > kv->batch || P <= 0) return ORC_E_ARG;
    for (int32_t b = 0; b < B; ++b) {
        if (pos[b] < 0 || pos[b] + P > kv->max_seq) return ORC_E_ARG;
        for (int32_t t = 0; t < P; ++t)
            if (tokens[(int64_t)b * P + t] < 0 || tokens[(int64_t)b * P + t] >= c->vocab) return ORC_E_ARG;
    }
    const int32_t d = c->hidden, Hq = c->n_q_heads, Hkv = c->n_kv_heads, hd = c->head_dim;
    const int32_t group = Hq / Hkv, S = kv->max_seq, n = B * P;
    int32_t* trace_sel = g_moe_sel; /* the per-step MoE trace is sized for one position per sequence */
    float* trace_prob = g_moe_prob;
    g_moe_sel = 0;
    g_moe_prob = 0;
    float* h = (float*)malloc(sizeof(float) * (size_t)n * d);
    float* x = (float*)malloc(sizeof(float) * (size_t)n * d);
    float* q = (float*)malloc(sizeof(float) * (size_t)n * Hq * hd);
    float* k = (float*)malloc(sizeof(float) * (size_t)n * Hkv * hd);
    float* v = (float*)malloc(sizeof(float) * (size_t)n * Hkv * hd);
    float* o = (float*)malloc(sizeof(float) * (size_t)n * Hq * hd);
    float* ao = (float*)malloc(sizeof(float) * (size_t)n * d);
    float* hl = (float*)malloc(sizeof(float) * (size_t)B * d);
    for (int32_t r = 0; r < n; ++r)
        for (int32_t i = 0; i < d; ++i) h[(int64_t)r * d + i] = bf_to_f(w->embed[(int64_t)tokens[r] * d + i]);
    for (int32_t l = 0; l < c->n_layers; ++l) {
        const orc_layer* lw = &w->layers[l];
        for (int32_t r = 0; r < n; ++r) orc_rmsnorm(h + (int64_t)r * d, lw->attn_norm, d, c->rms_eps, x + (int64_t)r * d);
        gemv(lw->wq, Hq * hd, d, x, d, n, q, Hq * hd);
        gemv(lw->wk, Hkv * hd, d, x, d, n, k, Hkv * hd);
        gemv(lw->wv, Hkv * hd, d, x, d, n, v, Hkv * hd);
        for (int32_t r = 0; r < n; ++r) {
            const int32_t b = r / P, p = pos[b] + r % P;
            for (int32_t hh = 0; hh < Hq; ++hh) orc_rope(q + ((int64_t)r * Hq + hh) * hd, hd, p, c->rope_theta);
            for (int32_t g = 0; g < Hkv; ++g) {
                float* kg = k + ((int64_t)r * Hkv + g) * hd;
                float* vg = v + ((int64_t)r * Hkv + g) * hd;
                orc_rope(kg, hd, p, c->rope_theta);
                int64_t base = ((((int64_t)l * kv->batch + b) * Hkv + g) * S + p) * hd;
                for (int32_t i = 0; i < hd; ++i) {
                    kv->k[base + i] = orc_bf16_bits(kg[i]);
                    kv->v[base + i] = orc_bf16_bits(vg[i]);
                }
            }
        }
#pragma omp parallel for schedule(dynamic) collapse(2)
        for (int32_t r = 0; r < n; ++r)
            for (int32_t hh = 0; hh < Hq; ++hh) {
                const int32_t b = r / P, p = pos[b] + r % P, g = hh / group;
                int64_t base = (((int64_t)l * kv->batch + b) * Hkv + g) * S * hd;
                orc_attend(q + ((int64_t)r * Hq + hh) * hd, kv->k + base, kv->v + base, hd, p + 1, hd,
                           o + ((int64_t)r * Hq + hh) * hd);
            }
        gemv(lw->wo, d, Hq * hd, o, Hq * hd, n, ao, d);
        for (int64_t i = 0; i < (int64_t)n * d; ++i) h[i] = (float)((double)h[i] + (double)ao[i]);
        ffn_block(c, lw, l, n, h);
    }
    for (int32_t b = 0; b < B; ++b) memcpy(hl + (int64_t)b * d, h + ((int64_t)b * P + P - 1) * d, sizeof(float) * d);
    int rc = head_logits(c, w, B, hl, logits, next);
    free(h); free(x); free(q); free(k); free(v); free(o); free(ao); free(hl);
    g_moe_sel = trace_sel;
    g_moe_prob = trace_prob;
    return rc;
}

int orc_sequence(const orc_cfg* c, const orc_weights* w, const int32_t* tokens, int32_t n, float* logits) {
    if (!valid_cfg(c) || n <= 0) return ORC_E_ARG;
    for (int32_t t = 0; t < n; ++t)
        if (tokens[t] < 0 || tokens[t] >= c->vocab) return ORC_E_ARG;
    const int32_t d = c->hidden, Hq = c->n_q_heads, Hkv = c->n_kv_heads, hd = c->head_dim;
    const int32_t group = Hq / Hkv, kvw = Hkv * hd;
    float* h = (float*)malloc(sizeof(float) * (size_t)n * d);
    float* x = (float*)malloc(sizeof(float) * (size_t)n * d);
    float* q = (float*)malloc(sizeof(float) * (size_t)n * Hq * hd);
    float* k = (float*)malloc(sizeof(float) * (size_t)n * kvw);
    float* v = (float*)malloc(sizeof(float) * (size_t)n * kvw);
    uint16_t* Kl = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n * kvw); /* [t][Hkv][hd] */
    uint16_t* Vl = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n * kvw);
    float* o = (float*)malloc(sizeof(float) * (size_t)n * Hq * hd);
    float* ao = (float*)malloc(sizeof(float) * (size_t)n * d);
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    for (int32_t t = 0; t < n; ++t)
        for (int32_t i = 0; i < d; ++i) h[(int64_t)t * d + i] = bf_to_f(w->embed[(int64_t)tokens[t] * d + i]);
    for (int32_t l = 0; l < c->n_layers; ++l) {
        const orc_layer* lw = &w->layers[l];
        for (int32_t t = 0; t < n; ++t) orc_rmsnorm(h + (int64_t)t * d, lw->attn_norm, d, c->rms_eps, x + (int64_t)t * d);
        gemv(lw->wq, Hq * hd, d, x, d, n, q, Hq * hd);
        gemv(lw->wk, kvw, d, x, d, n, k, kvw);
        gemv(lw->wv, kvw, d, x, d, n, v, kvw);
        for (int32_t t = 0; t < n; ++t) {
            for (int32_t hh = 0; hh < Hq; ++hh) {
                orc_rope(q + ((int64_t)t * Hq + hh) * hd, hd, t, c->rope_theta);
            }
            for (int32_t g = 0; g < Hkv; ++g) orc_rope(k + (int64_t)t * kvw + (int64_t)g * hd, hd, t, c->rope_theta);
            for (int32_t i = 0; i < kvw; ++i) {
                Kl[(int64_t)t * kvw + i] = orc_bf16_bits(k[(int64_t)t * kvw + i]);
                Vl[(int64_t)t * kvw + i] = orc_bf16_bits(v[(int64_t)t * kvw + i]);
            }
        }
        /* causal: position t attends to positions 0..t */
#pragma omp parallel for schedule(dynamic) collapse(2)
        for (int32_t t = 0; t < n; ++t)
            for (int32_t hh = 0; hh < Hq; ++hh) {
                int32_t g = hh / group;
                orc_attend(q + ((int64_t)t * Hq + hh) * hd, Kl + (int64_t)g * hd, Vl + (int64_t)g * hd, kvw, t + 1, hd,
                           o + ((int64_t)t * Hq + hh) * hd);
            }
        gemv(lw->wo, d, Hq * hd, o, Hq * hd, n, ao, d);
        for (int64_t i = 0; i < (int64_t)n * d; ++i) h[i] = (float)((double)h[i] + (double)ao[i]);
        ffn_block(c, lw, l, n, h);
    }
    int rc = head_logits(c, w, n, h, logits, next);
    free(h); free(x); free(q); free(k); free(v); free(Kl); free(Vl); free(o); free(ao); free(next);
    return rc;
}
