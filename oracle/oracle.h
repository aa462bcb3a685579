/*
 * oracle.h — plain CPU reference of the decoder forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the GPU library includes, links or
 * calls this code; only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg load it. It shares no code with the GPU path.
 *
 * What it computes: the per-layer step list of a llama / qwen3 / qwen2 /
 * gemma3-style decoder as the architecture-definition file lays it out
 * (page "Local inference and architectures", section "The format": prologue
 * embed; block
 * rms_norm, q/k/v matmul (each followed by add_bias in qwen2, whose
 * definition differs from llama's by those three lines, section "Adding an
 * architecture"), norm_heads q/k (qwen3 only), rope q/k, attention, o matmul,
 * add, rms_norm, gate matmul, silu, up matmul, mul, down matmul, add;
 * epilogue rms_norm, last, logits matmul with the output weight or, if that
 * is absent, the token embedding). gemma3 (20 steps per layer, section
 * "What is in effect right now"; gelu_tanh, section "The operations"; a
 * window pattern, section "Rules") is read as: prologue embed, scale by
 * sqrt(d_model); block rms_norm, q/k/v matmul, norm_heads q/k, rope q/k,
 * attention (through a sliding window on the pattern's local layers), o
 * matmul, rms_norm of o, add, rms_norm, gate matmul, gelu_tanh, up matmul,
 * mul, down matmul, rms_norm of down, add. Multiplication is in f32 on f32 values
 * (same page, section "Choosing the engine": the engine multiplies in f32
 * rather than quantising activations). Every dot product is formed from
 * exact f32×f32 products accumulated in f64 and rounded once to f32, so the
 * oracle's own error is far below the tolerances it is used to check.
 *
 * Runtime contract followed (page "Execution contract"): tokens go through
 * one at a time (section "Forward phase", "Text generation"); a bulk call
 * with n > 1 tokens produces the same result as n single calls; the KV cache
 * is sized to max context at creation, appended on every token and cleared by
 * reset (section "Memory lifecycle", "KV cache"); cos/sin position caches
 * are precomputed at creation (same section, "Position caches").
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - RMSNorm: y_i = w_i * (x_i / sqrt(mean(x^2) + eps)), weight multiplies.
 *  - norm_heads: the same RMSNorm over each head_dim slice, one shared weight.
 *  - RoPE: rotate-half pairs (i, i + hd/2) by default, or adjacent pairs
 *    (2i, 2i+1) when the config asks for them; pair i turns by the angle
 *    p * theta^(-2i/hd) either way.
 *  - add_bias: y_i = y_i + b_i in f32, right after the matmul it follows.
 *  - attention: causal over positions 0..p including p, scale 1/sqrt(hd),
 *    grouped-query head j reads KV head j / (n_heads / n_kv_heads).
 *  - K is cached after RoPE, V as computed.
 *  - sliding window W (gemma3's local layers): position p attends to the
 *    positions t with p - W < t <= p; with window_pattern P, layer l is
 *    global when (l + 1) % P == 0 and local otherwise; local layers rotate
 *    with rope_theta_local, global ones with rope_theta.
 *  - gelu_tanh(x) = x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))).
 *  - scale: x_i = x_i * s with s = f32(sqrt(d_model)), one rounding.
 *  - 8-bit blocks: 32 int8 along K with one f16 scale, w = scale * q.
 */
#ifndef DECFWD_ORACLE_H
#define DECFWD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_Q8 = 2 };
enum { ORC_LLAMA = 0, ORC_QWEN3 = 1, ORC_QWEN2 = 2, ORC_GEMMA3 = 3 };
enum { ORC_ROPE_HALVES = 0, ORC_ROPE_ADJACENT = 1 };

enum {
    ORC_OK = 0,
    ORC_ERR_CONTEXT_FULL = 1,
    ORC_ERR_BAD_TOKEN = 2,
    ORC_ERR_BAD_ARGUMENT = 3,
    ORC_ERR_NO_MEMORY = 4
};

/* Per-layer weight slots, in the order the block uses them. */
enum {
    ORC_ATTN_NORM = 0, ORC_ATTN_Q, ORC_ATTN_K, ORC_ATTN_V, ORC_ATTN_Q_NORM,
    ORC_ATTN_K_NORM, ORC_ATTN_OUTPUT, ORC_FFN_NORM, ORC_FFN_GATE,
    ORC_FFN_UP, ORC_FFN_DOWN, ORC_ATTN_Q_BIAS, ORC_ATTN_K_BIAS,
    ORC_ATTN_V_BIAS, ORC_POST_ATTN_NORM, ORC_POST_FFN_NORM, ORC_NSLOT
};

/* Planted mistakes, used only by tests that prove the pins catch them. */
enum {
    ORC_MUT_NONE = 0,
    ORC_MUT_NORM_AFTER_ROPE = 1,  /* norm_heads after rope instead of before */
    ORC_MUT_ROPE_INTERLEAVED = 2, /* the other rope pairing than configured */
    ORC_MUT_NO_ATTN_RESIDUAL = 3, /* x = o instead of x += o */
    ORC_MUT_SCALE_1_OVER_HD = 4,  /* scores / hd instead of / sqrt(hd) */
    ORC_MUT_GQA_MODULO = 5,       /* kv head j % n_kv instead of j / group */
    ORC_MUT_EPS_OUTSIDE = 6,      /* 1/(sqrt(mean)+eps) */
    ORC_MUT_EXCLUDE_SELF = 7,     /* attend to 0..p-1 only */
    ORC_MUT_SILU_ON_UP = 8,       /* silu(up) * gate */
    ORC_MUT_ROPE_POS_PLUS1 = 9,   /* rotate by p+1 */
    ORC_MUT_MATVEC_TRANSPOSE = 10, /* y = W^T h on square weights */
    ORC_MUT_K_BIAS_AFTER_ROPE = 11, /* qwen2's k bias added after rope */
    ORC_MUT_GELU_ERF = 12,         /* erf gelu where gelu_tanh is asked for */
    ORC_MUT_WINDOW_PLUS1 = 13,     /* the window one position wider */
    ORC_MUT_NO_POST_ATTN_NORM = 14, /* o added without its rms_norm */
    ORC_MUT_GLOBAL_THETA = 15      /* local layers rotate with rope_theta */
};

typedef struct {
    int32_t arch;
    int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab;
    int32_t max_ctx;
    int32_t rope_pairing;  /* ORC_ROPE_HALVES or ORC_ROPE_ADJACENT */
    double rope_theta, rms_eps;
    int32_t sliding_window; /* 0: every layer attends to all positions */
    int32_t window_pattern; /* >= 1 when sliding_window > 0 */
    double rope_theta_local; /* theta of the local layers; 0: rope_theta */
} orc_config;

/* A weight as the caller holds it. f32 / f16: [rows][cols] row-major.
 * Q8: rows * cols/32 blocks of 34 bytes (f16 scale little-endian, then 32
 * int8). The oracle borrows `data`; the caller keeps it alive. */
typedef struct {
    int32_t dtype;
    int32_t pad_;
    const void* data;
} orc_tensor;

typedef struct orc_model orc_model;

/* Single steps, exposed so that each can be pinned on its own. */
void orc_f16_to_f32(const uint16_t* in, float* out, int64_t n);
void orc_rmsnorm(const float* x, const orc_tensor* w, int32_t n, double eps,
                 float* out);
void orc_matvec(const orc_tensor* W, int64_t N, int64_t K, const float* h,
                float* y);
void orc_embed(const orc_tensor* E, int64_t row, int64_t d, float* x);
void orc_rope_table(int32_t n_pos, int32_t hd, double theta, float* cos_out,
                    float* sin_out);
void orc_rope(float* t, int32_t n_heads, int32_t hd, const float* cos_row,
              const float* sin_row);
/* orc_rope with the pairing given (ORC_ROPE_HALVES or ORC_ROPE_ADJACENT). */
void orc_rope_pairs(float* t, int32_t n_heads, int32_t hd, const float* cos_row,
                    const float* sin_row, int32_t pairing);
/* y[i] = f32(y[i] + b[i]) for i < n; b is f32 or f16. */
void orc_add_bias(float* y, const orc_tensor* b, int64_t n);
/* q [n_heads][hd]; K, V: [n_kv][head_stride floats], row t of kv head g at
 * K + g*head_stride + t*hd; n_pos positions; out [n_heads][hd]. */
void orc_attention(const float* q, int32_t n_heads, int32_t n_kv, int32_t hd,
                   const float* K, const float* V, int64_t head_stride,
                   int32_t n_pos, float* out);
void orc_silu(float* g, int64_t n);
/* gelu_tanh in place (f64 inside, one rounding). */
void orc_gelu_tanh(float* g, int64_t n);
/* x_i = f32(x_i * s) for i < n. */
void orc_scale(float* x, int64_t n, float s);
void orc_mul(float* g, const float* u, int64_t n);

/* The model. `layers` holds n_layers * ORC_NSLOT tensors; slots an
 * architecture does not use (q/k norm outside qwen3 and gemma3, biases
 * outside qwen2, post norms outside gemma3) are ignored. `output` with data == NULL means tied weights. */
orc_model* orc_create(const orc_config* cfg, const orc_tensor* token_embd,
                      const orc_tensor* output_norm, const orc_tensor* output,
                      const orc_tensor* layers);
/* Appends n tokens; writes the last position's logits [vocab] unless
 * logits == NULL. Returns ORC_OK or an error; on error nothing changes. */
int orc_forward(orc_model* m, const int32_t* tokens, int32_t n, float* logits);
void orc_reset(orc_model* m);
int32_t orc_kv_len(const orc_model* m);
/* which: 0 = K, 1 = V. out / in: [n_kv][n][hd]. */
int orc_kv_read(const orc_model* m, int32_t layer, int32_t which,
                int32_t pos0, int32_t n, float* out);
int orc_kv_write(orc_model* m, int32_t layer, int32_t which, int32_t pos0,
                 int32_t n, const float* in);
int orc_set_kv_len(orc_model* m, int32_t n);
/* Op names of the last token, "|"-separated per section. */
const char* orc_trace(const orc_model* m);
void orc_destroy(orc_model* m);

void orc_set_mutation(int32_t code);
void orc_set_f32_accumulate(int32_t on);
void orc_set_threads(int32_t n);
int32_t orc_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
