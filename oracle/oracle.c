/*
 * oracle.c — plain CPU reference of the decoder forward pass.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): loaded by the tests, the smoke
 * check and the benchmark's CPU-baseline leg, never by the GPU library.
 *
 * Written for a reader checking it against the pages by eye: one function
 * per op of the step list, no blocking, no fusion, no reordering. OpenMP
 * only splits independent output rows (matvec) and heads (attention) across
 * threads; each output is computed by one thread in index order, so results
 * do not depend on the thread count.
 */
#include "oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int32_t g_mutation = ORC_MUT_NONE;
static int32_t g_f32_acc = 0;

void orc_set_mutation(int32_t code) { g_mutation = code; }
void orc_set_f32_accumulate(int32_t on) { g_f32_acc = on; }

void orc_set_threads(int32_t n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int32_t orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * IEEE-754 binary16 -> binary32. binary16: 1 sign bit, 5 exponent bits (bias
 * 15), 10 fraction bits. Exponent 0 encodes zero and subnormals
 * (fraction * 2^-24); exponent 31 encodes inf / NaN; otherwise the value is
 * (1024 + fraction) * 2^(exponent - 25). Every binary16 value is exactly
 * representable in binary32, so the conversion is exact. The table holds all
 * 65536 results, computed once from this definition.
 * ------------------------------------------------------------------------- */
static float g_f16_table[65536];
static int g_f16_ready = 0;

static float f16_by_definition(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exponent = (h >> 10) & 0x1f;
    int fraction = h & 0x3ff;
    float v;
    if (exponent == 0)
        v = ldexpf((float)fraction, -24);
    else if (exponent == 31)
        v = fraction ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + fraction), exponent - 25);
    return sign ? -v : v;
}

static void f16_table_init(void)
{
    if (g_f16_ready) return;
    for (int i = 0; i < 65536; ++i) g_f16_table[i] = f16_by_definition((uint16_t)i);
    g_f16_ready = 1;
}

static inline float f16(uint16_t h) { return g_f16_table[h]; }

void orc_f16_to_f32(const uint16_t* in, float* out, int64_t n)
{
    f16_table_init();
    for (int64_t i = 0; i < n; ++i) out[i] = f16(in[i]);
}

/* Element i of a vector-shaped weight (norm weights, embedding rows). */
static float weight_elem(const orc_tensor* w, int64_t i)
{
    if (w->dtype == ORC_F32) return ((const float*)w->data)[i];
    return f16(((const uint16_t*)w->data)[i]);
}

/* ---------------------------------------------------------------------------
 * embed: x = f32(E[row]) (section "The format": prologue).
 * ------------------------------------------------------------------------- */
void orc_embed(const orc_tensor* E, int64_t row, int64_t d, float* x)
{
    f16_table_init();
    for (int64_t i = 0; i < d; ++i) x[i] = weight_elem(E, row * d + i);
}

/* ---------------------------------------------------------------------------
 * rms_norm (section "The format": block and epilogue):
 *   r = 1 / sqrt(sum_i x_i^2 / n + eps),  out_i = w_i * (x_i * r).
 * The sum of squares is accumulated in f64; r is rounded to f32 and the two
 * multiplications are f32 multiplications, each rounded once.
 * ------------------------------------------------------------------------- */
void orc_rmsnorm(const float* x, const orc_tensor* w, int32_t n, double eps,
                 float* out)
{
    f16_table_init();
    double ss = 0.0;
    for (int32_t i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    double mean = ss / (double)n;
    float r;
    if (g_mutation == ORC_MUT_EPS_OUTSIDE)
        r = (float)(1.0 / (sqrt(mean) + eps));
    else
        r = (float)(1.0 / sqrt(mean + eps));
    for (int32_t i = 0; i < n; ++i) {
        float xr = x[i] * r;
        out[i] = weight_elem(w, i) * xr;
    }
}

/* ---------------------------------------------------------------------------
 * matmul (section "The format"): y = W h, W stored [N][K] row-major.
 * y_n = f32( sum_k W[n][k] * h[k] ), products exact in f64 (24 + 24 bit
 * mantissas fit in 53), summed in f64 in index order, rounded once.
 * An 8-bit block contributes scale * q_j for its 32 values; f32(scale) *
 * f32(q) is exact in f32 (11-bit mantissa times an 8-bit integer).
 * ------------------------------------------------------------------------- */
static double dot_row(const orc_tensor* W, int64_t n, int64_t K, const float* h)
{
    double acc = 0.0;
    float accf = 0.0f;
    if (W->dtype == ORC_F32) {
        const float* row = (const float*)W->data + n * K;
        for (int64_t k = 0; k < K; ++k) {
            if (g_f32_acc) accf += row[k] * h[k];
            else acc += (double)row[k] * (double)h[k];
        }
    } else if (W->dtype == ORC_F16) {
        const uint16_t* row = (const uint16_t*)W->data + n * K;
        for (int64_t k = 0; k < K; ++k) {
            if (g_f32_acc) accf += f16(row[k]) * h[k];
            else acc += (double)f16(row[k]) * (double)h[k];
        }
    } else {
        const int64_t nblk = K / 32;
        const uint8_t* row = (const uint8_t*)W->data + n * nblk * 34;
        for (int64_t b = 0; b < nblk; ++b) {
            const uint8_t* blk = row + b * 34;
            uint16_t sbits = (uint16_t)(blk[0] | (blk[1] << 8));
            float scale = f16(sbits);
            for (int j = 0; j < 32; ++j) {
                float w = scale * (float)(int8_t)blk[2 + j];
                if (g_f32_acc) accf += w * h[b * 32 + j];
                else acc += (double)w * (double)h[b * 32 + j];
            }
        }
    }
    return g_f32_acc ? (double)accf : acc;
}

/* Element (n, k) of an f32 / f16 matrix, for the transposed planted mistake. */
static float matrix_elem(const orc_tensor* W, int64_t n, int64_t k, int64_t K)
{
    if (W->dtype == ORC_F32) return ((const float*)W->data)[n * K + k];
    return f16(((const uint16_t*)W->data)[n * K + k]);
}

void orc_matvec(const orc_tensor* W, int64_t N, int64_t K, const float* h,
                float* y)
{
    f16_table_init();
    if (g_mutation == ORC_MUT_MATVEC_TRANSPOSE && N == K && W->dtype != ORC_Q8) {
        #pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)matrix_elem(W, k, n, K) * (double)h[k];
            y[n] = (float)acc;
        }
        return;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) y[n] = (float)dot_row(W, n, K, h);
}

/* ---------------------------------------------------------------------------
 * RoPE position cache (page "Execution contract", "Memory lifecycle",
 * "Position caches": cos/sin, positions x half head_dim, built at load).
 * Angle for position p and pair i: p * theta^(-2i/hd), in f64, rounded.
 * ------------------------------------------------------------------------- */
void orc_rope_table(int32_t n_pos, int32_t hd, double theta, float* cos_out,
                    float* sin_out)
{
    const int32_t half = hd / 2;
    for (int32_t p = 0; p < n_pos; ++p) {
        for (int32_t i = 0; i < half; ++i) {
            double inv_freq = pow(theta, -2.0 * (double)i / (double)hd);
            double angle = (double)p * inv_freq;
            cos_out[(int64_t)p * half + i] = (float)cos(angle);
            sin_out[(int64_t)p * half + i] = (float)sin(angle);
        }
    }
}

/* rope (section "The format"): each head's pair i, (a, b) = (t[i],
 * t[i+hd/2]) with rotate-half pairing or (t[2i], t[2i+1]) with adjacent
 * pairing, becomes (a c - b s, a s + b c) with the angle of pair i; computed
 * in f64 and rounded once. */
void orc_rope_pairs(float* t, int32_t n_heads, int32_t hd, const float* cos_row,
                    const float* sin_row, int32_t pairing)
{
    const int32_t half = hd / 2;
    int32_t adjacent = pairing == ORC_ROPE_ADJACENT;
    if (g_mutation == ORC_MUT_ROPE_INTERLEAVED) adjacent = !adjacent;
    for (int32_t j = 0; j < n_heads; ++j) {
        float* v = t + (int64_t)j * hd;
        for (int32_t i = 0; i < half; ++i) {
            const int32_t ia = adjacent ? 2 * i : i;
            const int32_t ib = adjacent ? 2 * i + 1 : i + half;
            double a = v[ia], b = v[ib];
            double c = cos_row[i], s = sin_row[i];
            v[ia] = (float)(a * c - b * s);
            v[ib] = (float)(a * s + b * c);
        }
    }
}

void orc_rope(float* t, int32_t n_heads, int32_t hd, const float* cos_row,
              const float* sin_row)
{
    orc_rope_pairs(t, n_heads, hd, cos_row, sin_row, ORC_ROPE_HALVES);
}

/* add_bias (section "The operations"): the bias vector added to the matmul
 * output just computed; one f32 rounding of the exact sum. */
void orc_add_bias(float* y, const orc_tensor* b, int64_t n)
{
    f16_table_init();
    for (int64_t i = 0; i < n; ++i) y[i] = (float)((double)y[i] + (double)weight_elem(b, i));
}

/* ---------------------------------------------------------------------------
 * attention (section "The format"): for query head j, KV head
 * g = j / (n_heads / n_kv_heads); scores z_t = (q_j . K_t) / sqrt(hd) for
 * t = 0 .. n_pos-1; softmax with the maximum subtracted; a_j = sum_t
 * softmax_t V_t. All in f64, rounded to f32 at the end.
 * ------------------------------------------------------------------------- */
void orc_attention(const float* q, int32_t n_heads, int32_t n_kv, int32_t hd,
                   const float* K, const float* V, int64_t head_stride,
                   int32_t n_pos, float* out)
{
    const int32_t group = n_heads / n_kv;
    const double scale = (g_mutation == ORC_MUT_SCALE_1_OVER_HD)
                             ? 1.0 / (double)hd : 1.0 / sqrt((double)hd);
    #pragma omp parallel for schedule(static)
    for (int32_t j = 0; j < n_heads; ++j) {
        int32_t g = (g_mutation == ORC_MUT_GQA_MODULO) ? j % n_kv : j / group;
        const float* qj = q + (int64_t)j * hd;
        const float* Kg = K + (int64_t)g * head_stride;
        const float* Vg = V + (int64_t)g * head_stride;
        double* z = (double*)malloc(sizeof(double) * (size_t)(n_pos > 0 ? n_pos : 1));
        double* acc = (double*)calloc((size_t)hd, sizeof(double));
        double zmax = -INFINITY;
        for (int32_t t = 0; t < n_pos; ++t) {
            double s = 0.0;
            for (int32_t e = 0; e < hd; ++e)
                s += (double)qj[e] * (double)Kg[(int64_t)t * hd + e];
            z[t] = s * scale;
            if (z[t] > zmax) zmax = z[t];
        }
        double den = 0.0;
        for (int32_t t = 0; t < n_pos; ++t) {
            double e = exp(z[t] - zmax);
            den += e;
            for (int32_t c = 0; c < hd; ++c)
                acc[c] += e * (double)Vg[(int64_t)t * hd + c];
        }
        for (int32_t c = 0; c < hd; ++c)
            out[(int64_t)j * hd + c] = (float)(acc[c] / den);
        free(z);
        free(acc);
    }
}

/* silu (section "The operations"), in place: g = g / (1 + exp(-g)). */
void orc_silu(float* g, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        double z = g[i];
        g[i] = (float)(z / (1.0 + exp(-z)));
    }
}

/* gelu_tanh (section "The operations": the tanh approximation, not the erf
 * form), in place: g = g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3))). */
void orc_gelu_tanh(float* g, int64_t n)
{
    const double c = sqrt(2.0 / acos(-1.0));
    for (int64_t i = 0; i < n; ++i) {
        double z = g[i];
        if (g_mutation == ORC_MUT_GELU_ERF)
            g[i] = (float)(0.5 * z * (1.0 + erf(z / sqrt(2.0))));
        else
            g[i] = (float)(0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z))));
    }
}

/* scale (section "The operations"), in place: x = x * s, one f32 rounding
 * of the exact product. */
void orc_scale(float* x, int64_t n, float s)
{
    for (int64_t i = 0; i < n; ++i) x[i] = (float)((double)x[i] * (double)s);
}

/* mul, in place: g = g * u (one f32 rounding). */
void orc_mul(float* g, const float* u, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) g[i] = g[i] * u[i];
}

/* add, in place: x = x + o (one f32 rounding). */
static void add_inplace(float* x, const float* o, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) x[i] = x[i] + o[i];
}

/* ---------------------------------------------------------------------------
 * The model.
 * ------------------------------------------------------------------------- */
#define TRACE_CAP 4096

struct orc_model {
    orc_config cfg;
    orc_tensor token_embd, output_norm, output;
    orc_tensor* layers;
    float* kc;    /* [L][n_kv][max_ctx][hd] */
    float* vc;
    float* cos_t; /* [max_ctx][hd/2] */
    float* sin_t;
    float* cos_l; /* local layers' table (rope_theta_local) */
    float* sin_l;
    int32_t n_past;
    float *x, *h, *q, *k, *v, *a, *o, *g, *u, *dn, *y;
    char trace[TRACE_CAP];
    size_t trace_len;
};

static void trace_reset(orc_model* m) { m->trace_len = 0; m->trace[0] = 0; }

static void trace_op(orc_model* m, const char* op, char sep)
{
    size_t n = strlen(op);
    if (m->trace_len + n + 2 >= TRACE_CAP) return;
    if (m->trace_len > 0) m->trace[m->trace_len++] = sep;
    memcpy(m->trace + m->trace_len, op, n);
    m->trace_len += n;
    m->trace[m->trace_len] = 0;
}

orc_model* orc_create(const orc_config* cfg, const orc_tensor* token_embd,
                      const orc_tensor* output_norm, const orc_tensor* output,
                      const orc_tensor* layers)
{
    f16_table_init();
    if (!cfg || cfg->n_layers < 0 || cfg->d_model <= 0 || cfg->n_heads <= 0 ||
        cfg->n_kv_heads <= 0 || cfg->n_heads % cfg->n_kv_heads ||
        cfg->head_dim <= 0 || cfg->head_dim % 2 || cfg->ffn_dim <= 0 ||
        cfg->vocab <= 0 || cfg->max_ctx <= 0 ||
        (cfg->arch != ORC_LLAMA && cfg->arch != ORC_QWEN3 && cfg->arch != ORC_QWEN2 &&
         cfg->arch != ORC_GEMMA3) ||
        (cfg->rope_pairing != ORC_ROPE_HALVES && cfg->rope_pairing != ORC_ROPE_ADJACENT) ||
        cfg->sliding_window < 0 || (cfg->sliding_window > 0 && cfg->window_pattern < 1) ||
        cfg->rope_theta_local < 0)
        return NULL;
    orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
    if (!m) return NULL;
    m->cfg = *cfg;
    m->token_embd = *token_embd;
    m->output_norm = *output_norm;
    m->output = (output && output->data) ? *output : *token_embd;
    size_t nl = (size_t)cfg->n_layers * ORC_NSLOT;
    m->layers = (orc_tensor*)calloc(nl ? nl : 1, sizeof(orc_tensor));
    if (nl) memcpy(m->layers, layers, nl * sizeof(orc_tensor));
    const int64_t hd = cfg->head_dim, d = cfg->d_model;
    const int64_t kv_elems = (int64_t)cfg->n_layers * cfg->n_kv_heads *
                             (int64_t)cfg->max_ctx * hd;
    m->kc = (float*)calloc((size_t)(kv_elems ? kv_elems : 1), sizeof(float));
    m->vc = (float*)calloc((size_t)(kv_elems ? kv_elems : 1), sizeof(float));
    m->cos_t = (float*)malloc(sizeof(float) * (size_t)cfg->max_ctx * (size_t)(hd / 2));
    m->sin_t = (float*)malloc(sizeof(float) * (size_t)cfg->max_ctx * (size_t)(hd / 2));
    m->cos_l = (float*)malloc(sizeof(float) * (size_t)cfg->max_ctx * (size_t)(hd / 2));
    m->sin_l = (float*)malloc(sizeof(float) * (size_t)cfg->max_ctx * (size_t)(hd / 2));
    const int64_t qd = (int64_t)cfg->n_heads * hd, kvd = (int64_t)cfg->n_kv_heads * hd;
    m->x = (float*)malloc(sizeof(float) * (size_t)d);
    m->h = (float*)malloc(sizeof(float) * (size_t)d);
    m->y = (float*)malloc(sizeof(float) * (size_t)d);
    m->q = (float*)malloc(sizeof(float) * (size_t)qd);
    m->a = (float*)malloc(sizeof(float) * (size_t)qd);
    m->k = (float*)malloc(sizeof(float) * (size_t)kvd);
    m->v = (float*)malloc(sizeof(float) * (size_t)kvd);
    m->o = (float*)malloc(sizeof(float) * (size_t)d);
    m->dn = (float*)malloc(sizeof(float) * (size_t)d);
    m->g = (float*)malloc(sizeof(float) * (size_t)cfg->ffn_dim);
    m->u = (float*)malloc(sizeof(float) * (size_t)cfg->ffn_dim);
    if (!m->layers || !m->kc || !m->vc || !m->cos_t || !m->sin_t || !m->cos_l ||
        !m->sin_l || !m->x ||
        !m->h || !m->y || !m->q || !m->a || !m->k || !m->v || !m->o ||
        !m->dn || !m->g || !m->u) {
        orc_destroy(m);
        return NULL;
    }
    orc_rope_table(cfg->max_ctx, cfg->head_dim, cfg->rope_theta, m->cos_t, m->sin_t);
    orc_rope_table(cfg->max_ctx, cfg->head_dim,
                   cfg->rope_theta_local > 0 ? cfg->rope_theta_local : cfg->rope_theta,
                   m->cos_l, m->sin_l);
    return m;
}

void orc_destroy(orc_model* m)
{
    if (!m) return;
    free(m->layers); free(m->kc); free(m->vc); free(m->cos_t); free(m->sin_t);
    free(m->cos_l); free(m->sin_l);
    free(m->x); free(m->h); free(m->y); free(m->q); free(m->a); free(m->k);
    free(m->v); free(m->o); free(m->dn); free(m->g); free(m->u);
    free(m);
}

static float* kv_row(const orc_model* m, float* base, int32_t layer, int32_t g,
                     int32_t pos)
{
    const orc_config* c = &m->cfg;
    int64_t off = (((int64_t)layer * c->n_kv_heads + g) * c->max_ctx + pos) *
                  (int64_t)c->head_dim;
    return base + off;
}

/* norm_heads (section "The format", qwen3 only): RMSNorm of every head_dim
 * slice with one shared weight. */
static void norm_heads(float* t, int32_t n_heads, int32_t hd,
                       const orc_tensor* w, double eps, float* tmp)
{
    for (int32_t j = 0; j < n_heads; ++j) {
        orc_rmsnorm(t + (int64_t)j * hd, w, hd, eps, tmp);
        memcpy(t + (int64_t)j * hd, tmp, sizeof(float) * (size_t)hd);
    }
}

/* One token through the step list at position p = n_past. */
static void forward_one(orc_model* m, int32_t tok, float* logits)
{
    const orc_config* c = &m->cfg;
    const int32_t d = c->d_model, hd = c->head_dim, F = c->ffn_dim;
    const int32_t nh = c->n_heads, nkv = c->n_kv_heads;
    const int32_t qd = nh * hd, kvd = nkv * hd;
    const double eps = c->rms_eps;
    const int32_t p = m->n_past;
    const int32_t half = hd / 2;
    int32_t rp = (g_mutation == ORC_MUT_ROPE_POS_PLUS1) ? p + 1 : p;
    if (rp >= c->max_ctx) rp = c->max_ctx - 1;
    const int gemma = (c->arch == ORC_GEMMA3);
    float tmp[4096];
    float* hbuf = hd <= 4096 ? tmp : NULL;
    char sec = '|';

    trace_reset(m);
    trace_op(m, "embed", sec);
    orc_embed(&m->token_embd, tok, d, m->x);
    if (gemma) {
        trace_op(m, "scale", ',');
        orc_scale(m->x, d, (float)sqrt((double)d));
    }

    for (int32_t l = 0; l < c->n_layers; ++l) {
        const orc_tensor* w = m->layers + (int64_t)l * ORC_NSLOT;
        /* local layer: attends through the window, rotates with the local
         * theta; the pattern's every P-th layer is global. */
        const int local = c->sliding_window > 0 && (l + 1) % c->window_pattern != 0;
        const int local_theta = local && g_mutation != ORC_MUT_GLOBAL_THETA;
        const float* cos_row = (local_theta ? m->cos_l : m->cos_t) + (int64_t)rp * half;
        const float* sin_row = (local_theta ? m->sin_l : m->sin_t) + (int64_t)rp * half;
        sec = '|';
        trace_op(m, "rms_norm", sec); sec = ',';
        orc_rmsnorm(m->x, &w[ORC_ATTN_NORM], d, eps, m->h);
        const int bias = (c->arch == ORC_QWEN2);
        trace_op(m, "matmul", sec);
        orc_matvec(&w[ORC_ATTN_Q], qd, d, m->h, m->q);
        if (bias) { trace_op(m, "add_bias", sec); orc_add_bias(m->q, &w[ORC_ATTN_Q_BIAS], qd); }
        trace_op(m, "matmul", sec);
        orc_matvec(&w[ORC_ATTN_K], kvd, d, m->h, m->k);
        const int k_bias_late = (g_mutation == ORC_MUT_K_BIAS_AFTER_ROPE);
        if (bias && !k_bias_late) { trace_op(m, "add_bias", sec); orc_add_bias(m->k, &w[ORC_ATTN_K_BIAS], kvd); }
        trace_op(m, "matmul", sec);
        orc_matvec(&w[ORC_ATTN_V], kvd, d, m->h, m->v);
        if (bias) { trace_op(m, "add_bias", sec); orc_add_bias(m->v, &w[ORC_ATTN_V_BIAS], kvd); }
        const int qk_norm = (c->arch == ORC_QWEN3 || gemma);
        const int norm_first = (g_mutation != ORC_MUT_NORM_AFTER_ROPE);
        if (qk_norm && norm_first) {
            trace_op(m, "norm_heads", sec);
            norm_heads(m->q, nh, hd, &w[ORC_ATTN_Q_NORM], eps, hbuf);
            trace_op(m, "norm_heads", sec);
            norm_heads(m->k, nkv, hd, &w[ORC_ATTN_K_NORM], eps, hbuf);
        }
        trace_op(m, "rope", sec);
        orc_rope_pairs(m->q, nh, hd, cos_row, sin_row, c->rope_pairing);
        trace_op(m, "rope", sec);
        orc_rope_pairs(m->k, nkv, hd, cos_row, sin_row, c->rope_pairing);
        if (bias && k_bias_late) orc_add_bias(m->k, &w[ORC_ATTN_K_BIAS], kvd);
        if (qk_norm && !norm_first) {
            trace_op(m, "norm_heads", sec);
            norm_heads(m->q, nh, hd, &w[ORC_ATTN_Q_NORM], eps, hbuf);
            trace_op(m, "norm_heads", sec);
            norm_heads(m->k, nkv, hd, &w[ORC_ATTN_K_NORM], eps, hbuf);
        }
        /* attention appends this position's k (after rope) and v to the
         * cache, then attends over positions 0..p. */
        for (int32_t g = 0; g < nkv; ++g) {
            memcpy(kv_row(m, m->kc, l, g, p), m->k + (int64_t)g * hd, sizeof(float) * (size_t)hd);
            memcpy(kv_row(m, m->vc, l, g, p), m->v + (int64_t)g * hd, sizeof(float) * (size_t)hd);
        }
        trace_op(m, "attention", sec);
        int32_t n_pos = (g_mutation == ORC_MUT_EXCLUDE_SELF) ? p : p + 1;
        int32_t lo = 0;  /* first position inside the window */
        if (local) {
            const int32_t W = c->sliding_window + (g_mutation == ORC_MUT_WINDOW_PLUS1 ? 1 : 0);
            lo = p - W + 1 > 0 ? p - W + 1 : 0;
        }
        orc_attention(m->q, nh, nkv, hd, kv_row(m, m->kc, l, 0, lo),
                      kv_row(m, m->vc, l, 0, lo), (int64_t)c->max_ctx * hd,
                      n_pos - lo, m->a);
        trace_op(m, "matmul", sec);
        orc_matvec(&w[ORC_ATTN_OUTPUT], d, qd, m->a, m->o);
        if (gemma) {
            trace_op(m, "rms_norm", sec);
            if (g_mutation != ORC_MUT_NO_POST_ATTN_NORM) {
                orc_rmsnorm(m->o, &w[ORC_POST_ATTN_NORM], d, eps, m->y);
                memcpy(m->o, m->y, sizeof(float) * (size_t)d);
            }
        }
        trace_op(m, "add", sec);
        if (g_mutation == ORC_MUT_NO_ATTN_RESIDUAL)
            memcpy(m->x, m->o, sizeof(float) * (size_t)d);
        else
            add_inplace(m->x, m->o, d);

        trace_op(m, "rms_norm", sec);
        orc_rmsnorm(m->x, &w[ORC_FFN_NORM], d, eps, m->h);
        trace_op(m, "matmul", sec);
        orc_matvec(&w[ORC_FFN_GATE], F, d, m->h, m->g);
        if (gemma) {
            trace_op(m, "gelu_tanh", sec);
            orc_gelu_tanh(m->g, F);
        } else if (g_mutation != ORC_MUT_SILU_ON_UP) {
            trace_op(m, "silu", sec);
            orc_silu(m->g, F);
        }
        trace_op(m, "matmul", sec);
        orc_matvec(&w[ORC_FFN_UP], F, d, m->h, m->u);
        if (!gemma && g_mutation == ORC_MUT_SILU_ON_UP) {
            trace_op(m, "silu", sec);
            orc_silu(m->u, F);
        }
        trace_op(m, "mul", sec);
        orc_mul(m->g, m->u, F);
        trace_op(m, "matmul", sec);
        orc_matvec(&w[ORC_FFN_DOWN], d, F, m->g, m->dn);
        if (gemma) {
            trace_op(m, "rms_norm", sec);
            orc_rmsnorm(m->dn, &w[ORC_POST_FFN_NORM], d, eps, m->y);
            memcpy(m->dn, m->y, sizeof(float) * (size_t)d);
        }
        trace_op(m, "add", sec);
        add_inplace(m->x, m->dn, d);
    }

    m->n_past = p + 1;
    if (!logits) return;
    sec = '|';
    trace_op(m, "rms_norm", sec); sec = ',';
    orc_rmsnorm(m->x, &m->output_norm, d, eps, m->y);
    trace_op(m, "last", sec);  /* one row per call: the last row is the row */
    trace_op(m, "matmul", sec);
    orc_matvec(&m->output, c->vocab, d, m->y, logits);
}

int orc_forward(orc_model* m, const int32_t* tokens, int32_t n, float* logits)
{
    if (!m || !tokens || n <= 0) return ORC_ERR_BAD_ARGUMENT;
    if ((int64_t)m->n_past + n > m->cfg.max_ctx) return ORC_ERR_CONTEXT_FULL;
    if (m->cfg.head_dim > 4096) return ORC_ERR_BAD_ARGUMENT;
    for (int32_t s = 0; s < n; ++s)
        if (tokens[s] < 0 || tokens[s] >= m->cfg.vocab) return ORC_ERR_BAD_TOKEN;
    for (int32_t s = 0; s < n; ++s)
        forward_one(m, tokens[s], s == n - 1 ? logits : NULL);
    return ORC_OK;
}

void orc_reset(orc_model* m)
{
    if (m) m->n_past = 0;
}

int32_t orc_kv_len(const orc_model* m) { return m ? m->n_past : -1; }

int orc_set_kv_len(orc_model* m, int32_t n)
{
    if (!m || n < 0 || n > m->cfg.max_ctx) return ORC_ERR_BAD_ARGUMENT;
    m->n_past = n;
    return ORC_OK;
}

static int kv_copy(const orc_model* m, int32_t layer, int32_t which, int32_t pos0,
                   int32_t n, float* host, int to_host)
{
    const orc_config* c = &m->cfg;
    if (layer < 0 || layer >= c->n_layers || (which != 0 && which != 1) ||
        pos0 < 0 || n < 0 || (int64_t)pos0 + n > c->max_ctx)
        return ORC_ERR_BAD_ARGUMENT;
    float* base = which ? m->vc : m->kc;
    const size_t row = sizeof(float) * (size_t)c->head_dim;
    for (int32_t g = 0; g < c->n_kv_heads; ++g)
        for (int32_t t = 0; t < n; ++t) {
            float* dev = kv_row(m, base, layer, g, pos0 + t);
            float* h = host + ((int64_t)g * n + t) * c->head_dim;
            if (to_host) memcpy(h, dev, row);
            else memcpy(dev, h, row);
        }
    return ORC_OK;
}

int orc_kv_read(const orc_model* m, int32_t layer, int32_t which, int32_t pos0,
                int32_t n, float* out)
{
    if (!m || !out) return ORC_ERR_BAD_ARGUMENT;
    return kv_copy(m, layer, which, pos0, n, out, 1);
}

int orc_kv_write(orc_model* m, int32_t layer, int32_t which, int32_t pos0,
                 int32_t n, const float* in)
{
    if (!m || !in) return ORC_ERR_BAD_ARGUMENT;
    return kv_copy(m, layer, which, pos0, n, (float*)in, 0);
}

const char* orc_trace(const orc_model* m) { return m ? m->trace : ""; }
