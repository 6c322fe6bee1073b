/*
 * Plain CPU oracle of one batch-1 greedy decode step of a Llama-family transformer.
 *
 * TEST INFRASTRUCTURE ONLY. This file defines the correct result that the GPU path is
 * checked against. It shares no code with the GPU path. The tests, the smoke check and the
 * cpu_baseline leg of the bench may use it; the product path never does.
 *
 * What is computed follows the AutoMegaKernel pages: the method is a faster schedule of the
 * standard Llama decode step, and its correctness criterion is logit equivalence plus
 * greedy-token agreement with eager execution (page 1, "What's built" and "Honesty rules";
 * page 3, "How it works"). The ops listed there are RMSNorm, the QKV/O/gate/up/down GEMVs,
 * RoPE, attention over a persistent KV cache, SwiGLU and weight dequantisation (page 3,
 * "Layer 1, instructions"); the int8/int4 weight-only formats are the pages' quantised
 * kernels (page 2, "Quantisation support and performance").
 *
 * Arithmetic: every sum, product and transcendental is evaluated in IEEE double. Values are
 * rounded only where the method stores them in a narrower format: the activations and the
 * KV cache (fp32 or bf16), the int8/int4 codes and their fp16 scales. The pages do not fix
 * rounding points; the readings taken here (one rounding per op output, residual in the
 * activation format, logits not rounded, argmax decided on fp32 logits, lowest index wins)
 * are listed with the other readings in the design notes.
 *
 * No fast-math, no BLAS, no intrinsics. Built with -O2 -fopenmp -ffp-contract=off; OpenMP
 * only splits independent output rows and attention heads over threads (each row's sum is
 * evaluated in the same order regardless of the thread count).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_INT8 2
#define ORC_INT4 3

#define ORC_FMT_F32 0
#define ORC_FMT_BF16 1
#define ORC_FMT_F16 2

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENAN 2

/* ------------------------------------------------------------------ rounding */

/* Round a double to a binary floating-point format with `mant` significant bits, smallest
 * exponent of a normal number `emin` and largest finite value `maxv`, round-to-nearest-even.
 * Subnormals keep the fixed spacing 2^(emin - mant + 1). Overflow gives +-inf. */
static double round_fmt(double x, int mant, int emin, double maxv) {
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    frexp(x, &e);                 /* x = f * 2^e, 0.5 <= |f| < 1, so the leading bit is 2^(e-1) */
    int ulp_e = (e - 1) - (mant - 1);
    int min_ulp_e = emin - (mant - 1);
    if (ulp_e < min_ulp_e) ulp_e = min_ulp_e;
    double scaled = ldexp(x, -ulp_e);            /* exact: only the exponent changes */
    double r = nearbyint(scaled);                /* current rounding mode: to nearest, ties even */
    double y = ldexp(r, ulp_e);
    if (fabs(y) > maxv) return x > 0 ? INFINITY : -INFINITY;
    return y;
}

double orc_round(double x, int fmt) {
    switch (fmt) {
    case ORC_FMT_F32: return round_fmt(x, 24, -126, 3.4028234663852886e38);
    case ORC_FMT_BF16: return round_fmt(x, 8, -126, 3.3895313892515355e38);
    case ORC_FMT_F16: return round_fmt(x, 11, -14, 65504.0);
    default: return NAN;
    }
}

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------ quantisation */

/* Symmetric absmax quantisation of a bf16 master matrix [rows, cols] (row-major).
 * group == 0: one scale per output row; else one scale per (row, group of `group` columns).
 * qmax = 127 (int8) or 7 (int4). Scale s = fp16(fp32(A / qmax)) with A the group's absmax;
 * code q = clamp(round_half_even(fp32(w) / fp32(s)), -qmax, qmax); s == 0 gives q = 0.
 * The divisions are evaluated in fp32 because they decide integer codes, and the GPU path
 * takes the same decision in fp32. */
int orc_quantize(const uint16_t* w, int64_t rows, int64_t cols, int group, int qmax, int8_t* q, float* s) {
    if (!w || !q || !s || rows < 0 || cols <= 0 || qmax <= 0) return ORC_EINVAL;
    int64_t g = group > 0 ? group : cols;
    if (cols % g) return ORC_EINVAL;
    int64_t ng = cols / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < ng; ++b) {
            const uint16_t* wr = w + r * cols + b * g;
            double a = 0.0;
            for (int64_t k = 0; k < g; ++k) {
                double v = fabs(bf16_to_double(wr[k]));
                if (v > a) a = v;
            }
            float a32 = (float)a;                       /* exact: a is a bf16 value */
            float ratio = a32 / (float)qmax;            /* fp32 division */
            float sc = (float)orc_round((double)ratio, ORC_FMT_F16);
            s[r * ng + b] = sc;
            int8_t* qr = q + r * cols + b * g;
            for (int64_t k = 0; k < g; ++k) {
                if (sc == 0.0f) { qr[k] = 0; continue; }
                float t = (float)bf16_to_double(wr[k]) / sc;   /* fp32 division */
                float n = nearbyintf(t);
                if (n > (float)qmax) n = (float)qmax;
                if (n < -(float)qmax) n = -(float)qmax;
                qr[k] = (int8_t)n;
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ the ops */

/* RMSNorm: h_i = round_act(x_i * r * g_i), r = 1 / sqrt(mean(x^2) + eps). */
void orc_rmsnorm(const double* x, const double* g, int n, double eps, int act_fmt, double* h) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int i = 0; i < n; ++i) h[i] = orc_round(x[i] * r * g[i], act_fmt);
}

/* Rotary embedding of one head (half-split pairs (i, i + hd/2)), in place, not rounded.
 * Pair i is rotated by the angle pos * theta^(-2i/hd). */
void orc_rope(double* u, int hd, int pos, double theta) {
    int half = hd / 2;
    for (int i = 0; i < half; ++i) {
        double inv_freq = pow(theta, -2.0 * (double)i / (double)hd);
        double ang = (double)pos * inv_freq;
        double c = cos(ang), s = sin(ang);
        double a = u[i], b = u[i + half];
        u[i] = a * c - b * s;
        u[i + half] = b * c + a * s;
    }
}

/* Decode attention of one query head over cache rows [0, n): K, V are [n][hd] (fp32 storage
 * of act-format values). o_d = round_act(sum_s p_s V_sd), p = softmax(q.K^T / sqrt(hd)). */
void orc_attention(const double* q, const float* K, const float* V, int n, int hd, int act_fmt, double* o,
                   double* scratch /* [n] */) {
    double scale = 1.0 / sqrt((double)hd);
    double m = -INFINITY;
    for (int s = 0; s < n; ++s) {
        double d = 0.0;
        for (int k = 0; k < hd; ++k) d += q[k] * (double)K[(int64_t)s * hd + k];
        scratch[s] = d * scale;
        if (scratch[s] > m) m = scratch[s];
    }
    double z = 0.0;
    for (int s = 0; s < n; ++s) {
        scratch[s] = exp(scratch[s] - m);
        z += scratch[s];
    }
    for (int k = 0; k < hd; ++k) {
        double acc = 0.0;
        for (int s = 0; s < n; ++s) acc += scratch[s] * (double)V[(int64_t)s * hd + k];
        o[k] = orc_round(acc / z, act_fmt);
    }
}

/* SwiGLU: round_act(silu(g) * u), silu(g) = g / (1 + exp(-g)). */
double orc_swiglu(double g, double u, int act_fmt) {
    return orc_round(g / (1.0 + exp(-g)) * u, act_fmt);
}

/* Greedy choice: the lowest index among the maxima; -1 if any value is NaN. */
int orc_argmax_f32(const float* v, int64_t n) {
    int best = -1;
    float bv = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (isnan(v[i])) return -1;
        if (best < 0 || v[i] > bv) { best = (int)i; bv = v[i]; }
    }
    return best;
}

/* ------------------------------------------------------------------ model */

typedef struct {
    int hidden, n_layers, n_heads, n_kv_heads, head_dim, intermediate, vocab, max_ctx;
    int tied;      /* LM head is the embedding matrix */
    int wfmt;      /* ORC_F32 / ORC_BF16 / ORC_INT8 / ORC_INT4: format of the projection weights */
    int act_f32;   /* 1: activations and KV cache in fp32; 0: bf16 */
    double rope_theta, rms_eps;
} orc_desc;

/* One projection matrix [rows, cols] as the oracle holds it. */
typedef struct {
    int64_t rows, cols;
    const float* f32;        /* ORC_F32 master (borrowed) */
    const uint16_t* bf16;    /* ORC_BF16 master (borrowed) */
    int8_t* q;               /* ORC_INT8 / ORC_INT4 codes (owned) */
    float* s;                /* scales: [rows] (int8) or [rows][cols/128] (int4) (owned) */
    int group;
} orc_mat;

enum { W_EMBED = 0, W_FINAL_NORM = 1, W_LM_HEAD = 2, W_ATTN_NORM = 10, W_WQ, W_WK, W_WV, W_WO, W_MLP_NORM, W_WG, W_WU, W_WD };

typedef struct {
    orc_desc d;
    int act_fmt;
    /* embedding rows and norm gains stay in their master format (fp32 or bf16) */
    const void* embed;
    const void* final_norm;
    const void** attn_norm;
    const void** mlp_norm;
    orc_mat lm;
    orc_mat* wq; orc_mat* wk; orc_mat* wv; orc_mat* wo; orc_mat* wg; orc_mat* wu; orc_mat* wd;
    float* kv;               /* [L][2][nKV][max_ctx][hd], act-format values stored in fp32 */
    /* scratch */
    double *x, *h, *q, *k, *v, *o, *g, *u, *a, *acc, *att_scratch;
    float* logits32;
} orc_ctx;

static int64_t kv_index(const orc_ctx* c, int layer, int kv, int grp, int pos) {
    const orc_desc* d = &c->d;
    return ((((int64_t)layer * 2 + kv) * d->n_kv_heads + grp) * d->max_ctx + pos) * d->head_dim;
}

static double master_at(const orc_ctx* c, const void* p, int64_t i) {
    if (c->d.wfmt == ORC_F32) return (double)((const float*)p)[i];
    return bf16_to_double(((const uint16_t*)p)[i]);
}

static void mat_free(orc_mat* m) {
    free(m->q);
    free(m->s);
    memset(m, 0, sizeof(*m));
}

orc_ctx* orc_create(const orc_desc* d) {
    if (!d || d->hidden <= 0 || d->n_layers < 0 || d->n_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 ||
        (d->head_dim & 1) || d->intermediate <= 0 || d->vocab <= 0 || d->max_ctx <= 0 ||
        d->n_heads % d->n_kv_heads || d->wfmt < 0 || d->wfmt > 3)
        return NULL;
    orc_ctx* c = (orc_ctx*)calloc(1, sizeof(orc_ctx));
    if (!c) return NULL;
    c->d = *d;
    c->act_fmt = d->act_f32 ? ORC_FMT_F32 : ORC_FMT_BF16;
    int L = d->n_layers;
    c->attn_norm = (const void**)calloc(L + 1, sizeof(void*));
    c->mlp_norm = (const void**)calloc(L + 1, sizeof(void*));
    c->wq = (orc_mat*)calloc(L + 1, sizeof(orc_mat));
    c->wk = (orc_mat*)calloc(L + 1, sizeof(orc_mat));
    c->wv = (orc_mat*)calloc(L + 1, sizeof(orc_mat));
    c->wo = (orc_mat*)calloc(L + 1, sizeof(orc_mat));
    c->wg = (orc_mat*)calloc(L + 1, sizeof(orc_mat));
    c->wu = (orc_mat*)calloc(L + 1, sizeof(orc_mat));
    c->wd = (orc_mat*)calloc(L + 1, sizeof(orc_mat));
    int64_t kvn = (int64_t)L * 2 * d->n_kv_heads * d->max_ctx * d->head_dim;
    c->kv = (float*)calloc(kvn > 0 ? kvn : 1, sizeof(float));
    int qd = d->n_heads * d->head_dim, kd = d->n_kv_heads * d->head_dim;
    int big = d->hidden;
    if (qd > big) big = qd;
    if (d->intermediate > big) big = d->intermediate;
    if (d->vocab > big) big = d->vocab;
    c->x = (double*)calloc(d->hidden, sizeof(double));
    c->h = (double*)calloc(d->hidden, sizeof(double));
    c->q = (double*)calloc(qd, sizeof(double));
    c->k = (double*)calloc(kd, sizeof(double));
    c->v = (double*)calloc(kd, sizeof(double));
    c->o = (double*)calloc(qd, sizeof(double));
    c->g = (double*)calloc(d->intermediate, sizeof(double));
    c->u = (double*)calloc(d->intermediate, sizeof(double));
    c->a = (double*)calloc(d->intermediate, sizeof(double));
    c->acc = (double*)calloc(big, sizeof(double));
    c->att_scratch = (double*)calloc((int64_t)d->n_heads * d->max_ctx, sizeof(double));
    c->logits32 = (float*)calloc(d->vocab, sizeof(float));
    if (!c->kv || !c->x || !c->h || !c->q || !c->k || !c->v || !c->o || !c->g || !c->u || !c->a || !c->acc ||
        !c->att_scratch || !c->logits32 || !c->wq || !c->wk || !c->wv || !c->wo || !c->wg || !c->wu || !c->wd ||
        !c->attn_norm || !c->mlp_norm) {
        /* leak-free enough for an allocation failure in a test tool */
        return NULL;
    }
    return c;
}

void orc_destroy(orc_ctx* c) {
    if (!c) return;
    for (int l = 0; l <= c->d.n_layers; ++l) {
        mat_free(&c->wq[l]); mat_free(&c->wk[l]); mat_free(&c->wv[l]); mat_free(&c->wo[l]);
        mat_free(&c->wg[l]); mat_free(&c->wu[l]); mat_free(&c->wd[l]);
    }
    mat_free(&c->lm);
    free(c->wq); free(c->wk); free(c->wv); free(c->wo); free(c->wg); free(c->wu); free(c->wd);
    free(c->attn_norm); free(c->mlp_norm);
    free(c->kv); free(c->x); free(c->h); free(c->q); free(c->k); free(c->v); free(c->o);
    free(c->g); free(c->u); free(c->a); free(c->acc); free(c->att_scratch); free(c->logits32);
    free(c);
}

static int mat_set(orc_ctx* c, orc_mat* m, const void* master, int64_t rows, int64_t cols) {
    mat_free(m);
    m->rows = rows;
    m->cols = cols;
    switch (c->d.wfmt) {
    case ORC_F32: m->f32 = (const float*)master; return ORC_OK;
    case ORC_BF16: m->bf16 = (const uint16_t*)master; return ORC_OK;
    default: {
        int group = c->d.wfmt == ORC_INT4 ? 128 : 0;
        int qmax = c->d.wfmt == ORC_INT4 ? 7 : 127;
        if (group && cols % group) return ORC_EINVAL;
        int64_t ns = group ? rows * (cols / group) : rows;
        m->q = (int8_t*)malloc((size_t)(rows * cols));
        m->s = (float*)malloc((size_t)ns * sizeof(float));
        if (!m->q || !m->s) return ORC_EINVAL;
        m->group = group;
        return orc_quantize((const uint16_t*)master, rows, cols, group, qmax, m->q, m->s);
    }
    }
}

/* Register a master tensor (borrowed for the context's lifetime when fp32/bf16; quantised
 * into owned codes for int8/int4). Layout row-major [out, in]. */
int orc_set_weight(orc_ctx* c, int kind, int layer, const void* master) {
    if (!c || !master) return ORC_EINVAL;
    const orc_desc* d = &c->d;
    int H = d->hidden, qd = d->n_heads * d->head_dim, kd = d->n_kv_heads * d->head_dim, I = d->intermediate;
    if (kind >= W_ATTN_NORM && (layer < 0 || layer >= d->n_layers)) return ORC_EINVAL;
    switch (kind) {
    case W_EMBED: c->embed = master; if (d->tied) return mat_set(c, &c->lm, master, d->vocab, H); return ORC_OK;
    case W_FINAL_NORM: c->final_norm = master; return ORC_OK;
    case W_LM_HEAD: if (d->tied) return ORC_EINVAL; return mat_set(c, &c->lm, master, d->vocab, H);
    case W_ATTN_NORM: c->attn_norm[layer] = master; return ORC_OK;
    case W_MLP_NORM: c->mlp_norm[layer] = master; return ORC_OK;
    case W_WQ: return mat_set(c, &c->wq[layer], master, qd, H);
    case W_WK: return mat_set(c, &c->wk[layer], master, kd, H);
    case W_WV: return mat_set(c, &c->wv[layer], master, kd, H);
    case W_WO: return mat_set(c, &c->wo[layer], master, H, qd);
    case W_WG: return mat_set(c, &c->wg[layer], master, I, H);
    case W_WU: return mat_set(c, &c->wu[layer], master, I, H);
    case W_WD: return mat_set(c, &c->wd[layer], master, H, I);
    default: return ORC_EINVAL;
    }
}

/* y = W h in double. int8: y_j = s_j * sum_k q_jk h_k. int4: y_j = sum_b s_jb * sum_{k in b} q_jk h_k. */
static void gemv(const orc_ctx* c, const orc_mat* m, const double* h, double* y) {
    const int64_t R = m->rows, K = m->cols;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < R; ++j) {
        double acc = 0.0;
        if (m->f32) {
            const float* w = m->f32 + j * K;
            for (int64_t k = 0; k < K; ++k) acc += (double)w[k] * h[k];
        } else if (m->bf16) {
            const uint16_t* w = m->bf16 + j * K;
            for (int64_t k = 0; k < K; ++k) acc += bf16_to_double(w[k]) * h[k];
        } else if (m->group == 0) {
            const int8_t* w = m->q + j * K;
            for (int64_t k = 0; k < K; ++k) acc += (double)w[k] * h[k];
            acc *= (double)m->s[j];
        } else {
            const int8_t* w = m->q + j * K;
            const int64_t ng = K / m->group;
            for (int64_t b = 0; b < ng; ++b) {
                double part = 0.0;
                for (int64_t k = b * m->group; k < (b + 1) * m->group; ++k) part += (double)w[k] * h[k];
                acc += (double)m->s[j * ng + b] * part;
            }
        }
        y[j] = acc;
    }
    (void)c;
}

static void load_gains(const orc_ctx* c, const void* p, int n, double* out) {
    for (int i = 0; i < n; ++i) out[i] = master_at(c, p, i);
}

/* Write `n` cache rows [pos0, pos0+n) of (layer, K or V, kv group) from fp32 values (which
 * must already be act-format values). */
int orc_set_kv(orc_ctx* c, int layer, int kv, int grp, int pos0, int n, const float* vals) {
    if (!c || !vals || layer < 0 || layer >= c->d.n_layers || kv < 0 || kv > 1 || grp < 0 ||
        grp >= c->d.n_kv_heads || pos0 < 0 || n < 0 || pos0 + n > c->d.max_ctx)
        return ORC_EINVAL;
    memcpy(c->kv + kv_index(c, layer, kv, grp, pos0), vals, (size_t)n * c->d.head_dim * sizeof(float));
    return ORC_OK;
}

int orc_get_kv(const orc_ctx* c, int layer, int kv, int grp, int pos0, int n, float* out) {
    if (!c || !out || layer < 0 || layer >= c->d.n_layers || kv < 0 || kv > 1 || grp < 0 ||
        grp >= c->d.n_kv_heads || pos0 < 0 || n < 0 || pos0 + n > c->d.max_ctx)
        return ORC_EINVAL;
    memcpy(out, c->kv + kv_index(c, layer, kv, grp, pos0), (size_t)n * c->d.head_dim * sizeof(float));
    return ORC_OK;
}

/* One decode step: token at position pos. Reads cache rows [0, pos), writes row pos.
 * logits (double, [vocab]) and logits32 ([vocab], the fp32 rounding the greedy choice is
 * made on) are optional outputs; *token_out gets the greedy token (-1 on NaN). */
int orc_step(orc_ctx* c, int token, int pos, double* logits, float* logits32, int* token_out) {
    if (!c) return ORC_EINVAL;
    const orc_desc* d = &c->d;
    if (token < 0 || token >= d->vocab || pos < 0 || pos >= d->max_ctx || !c->embed || !c->final_norm)
        return ORC_EINVAL;
    const int H = d->hidden, hd = d->head_dim, nH = d->n_heads, nKV = d->n_kv_heads, I = d->intermediate;
    const int act = c->act_fmt;
    double* gain = (double*)malloc(sizeof(double) * (size_t)H);
    if (!gain) return ORC_EINVAL;
    /* embedding: the master row is already an act-format value */
    for (int i = 0; i < H; ++i) c->x[i] = master_at(c, c->embed, (int64_t)token * H + i);
    for (int l = 0; l < d->n_layers; ++l) {
        if (!c->attn_norm[l] || !c->mlp_norm[l]) { free(gain); return ORC_EINVAL; }
        /* attention block */
        load_gains(c, c->attn_norm[l], H, gain);
        orc_rmsnorm(c->x, gain, H, d->rms_eps, act, c->h);
        gemv(c, &c->wq[l], c->h, c->q);
        gemv(c, &c->wk[l], c->h, c->k);
        gemv(c, &c->wv[l], c->h, c->v);
        for (int hh = 0; hh < nH; ++hh) orc_rope(c->q + hh * hd, hd, pos, d->rope_theta);
        for (int g = 0; g < nKV; ++g) orc_rope(c->k + g * hd, hd, pos, d->rope_theta);
        for (int i = 0; i < nH * hd; ++i) c->q[i] = orc_round(c->q[i], act);
        for (int i = 0; i < nKV * hd; ++i) {
            c->k[i] = orc_round(c->k[i], act);
            c->v[i] = orc_round(c->v[i], act);
        }
        for (int g = 0; g < nKV; ++g) {
            float* kr = c->kv + kv_index(c, l, 0, g, pos);
            float* vr = c->kv + kv_index(c, l, 1, g, pos);
            for (int i = 0; i < hd; ++i) {
                kr[i] = (float)c->k[g * hd + i];
                vr[i] = (float)c->v[g * hd + i];
            }
        }
#pragma omp parallel for schedule(static)
        for (int hh = 0; hh < nH; ++hh) {
            int g = (int)(((int64_t)hh * nKV) / nH);
            orc_attention(c->q + hh * hd, c->kv + kv_index(c, l, 0, g, 0), c->kv + kv_index(c, l, 1, g, 0), pos + 1, hd,
                          act, c->o + hh * hd, c->att_scratch + (int64_t)hh * d->max_ctx);
        }
        gemv(c, &c->wo[l], c->o, c->acc);
        for (int i = 0; i < H; ++i) c->x[i] = orc_round(c->x[i] + c->acc[i], act);
        /* MLP block */
        load_gains(c, c->mlp_norm[l], H, gain);
        orc_rmsnorm(c->x, gain, H, d->rms_eps, act, c->h);
        gemv(c, &c->wg[l], c->h, c->g);
        gemv(c, &c->wu[l], c->h, c->u);
        for (int j = 0; j < I; ++j) c->a[j] = orc_swiglu(c->g[j], c->u[j], act);
        gemv(c, &c->wd[l], c->a, c->acc);
        for (int i = 0; i < H; ++i) c->x[i] = orc_round(c->x[i] + c->acc[i], act);
    }
    load_gains(c, c->final_norm, H, gain);
    orc_rmsnorm(c->x, gain, H, d->rms_eps, act, c->h);
    free(gain);
    if (!c->lm.rows) return ORC_EINVAL;
    gemv(c, &c->lm, c->h, c->acc);
    for (int j = 0; j < d->vocab; ++j) {
        c->logits32[j] = (float)c->acc[j];       /* round to nearest fp32 */
        if (logits) logits[j] = c->acc[j];
        if (logits32) logits32[j] = c->logits32[j];
    }
    int t = orc_argmax_f32(c->logits32, d->vocab);
    if (token_out) *token_out = t;
    return t < 0 ? ORC_ENAN : ORC_OK;
}

/* Dequantised view of a registered projection (for tests): out[r][k] = s * q (double). */
int orc_get_codes(const orc_ctx* c, int kind, int layer, int8_t* q, float* s) {
    if (!c) return ORC_EINVAL;
    const orc_mat* m = NULL;
    switch (kind) {
    case W_LM_HEAD: m = &c->lm; break;
    case W_WQ: m = &c->wq[layer]; break;
    case W_WK: m = &c->wk[layer]; break;
    case W_WV: m = &c->wv[layer]; break;
    case W_WO: m = &c->wo[layer]; break;
    case W_WG: m = &c->wg[layer]; break;
    case W_WU: m = &c->wu[layer]; break;
    case W_WD: m = &c->wd[layer]; break;
    default: return ORC_EINVAL;
    }
    if (!m->q) return ORC_EINVAL;
    int64_t ns = m->group ? m->rows * (m->cols / m->group) : m->rows;
    if (q) memcpy(q, m->q, (size_t)(m->rows * m->cols));
    if (s) memcpy(s, m->s, (size_t)ns * sizeof(float));
    return ORC_OK;
}

int orc_rounding_mode_is_nearest(void) { return fegetround() == FE_TONEAREST; }

/* Threads of the OpenMP loops from now on (the CPU baseline's one-thread figure); returns the
   count in effect. Results do not depend on it: every parallel loop writes disjoint outputs and
   each output's sum runs in one thread in a fixed order. */
int orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
