/*
 * decfwd.h — C ABI of the MI355X decoder forward pass (gfx950, HIP).
 *
 * One loaded decoder (llama, qwen3, qwen2 or gemma3 step list) on one GPU: load(config,
 * weights) -> model; forward(model, tokens) -> logits of the last position;
 * reset_kv_cache; free. Plain pointers and sizes only; no C++ or PyTorch
 * types cross this boundary, and no call aborts, exits or throws.
 *
 * Sources (all passages cited by page title and section):
 *  - the step list: page "Local inference and architectures", section "The
 *    format" (prologue embed; per layer rms_norm, q/k/v matmul, norm_heads
 *    q and k for qwen3, rope q and k, attention, o matmul, add, rms_norm,
 *    gate matmul, silu, up matmul, mul, down matmul, add; epilogue rms_norm,
 *    last, logits matmul with the output weight or the token embedding);
 *  - tensor names are the GGUF names (same page, "The format"), and "a | b"
 *    tensor fallback gives tied embeddings (same page, "Rules");
 *  - f32 multiplication of f32 activations (same page, "Choosing the
 *    engine"); 8-bit weights are dequantised, activations never are;
 *  - load steps, idempotent load, one forward for prefill and decode, bulk
 *    prefill equal to token-by-token within epsilon: page "Execution
 *    contract", sections "Load phase" and "Forward phase";
 *  - weights, KV cache sized to max context, frame allocator bucketed by
 *    exact size, cos/sin position cache: same page, "Memory lifecycle";
 *  - structured, actionable errors: same page, "Error semantics";
 *  - one forward at a time per KV cache: same page, "Concurrency";
 *  - timing breakdown: same page, "Observability";
 *  - idempotent release of all device memory: same page, "Shutdown".
 *
 * Threading: calls on one model are serialised by the caller; a second
 * concurrent df_forward / df_generate on the same model returns DF_ERR_BUSY.
 * Different models may be used from different threads.
 *
 * Streams: all device work of a model is ordered on one HIP stream (given
 * at load, or created by the library). Device outputs are valid once that
 * stream has been synchronised.
 */
#ifndef DECFWD_H
#define DECFWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. The first seven mirror the runtime's structured error kinds
 * (page "Execution contract", "Error semantics"). */
typedef int32_t df_status;
#define DF_OK 0
#define DF_ERR_UNSUPPORTED_OP 1          /* no kernel for this dtype / shape */
#define DF_ERR_SHAPE_MISMATCH 2          /* a tensor's rows / cols are wrong */
#define DF_ERR_MISSING_TENSOR 3          /* a required tensor is absent */
#define DF_ERR_WEIGHT_FORMAT_MISMATCH 4  /* dtype and byte count disagree */
#define DF_ERR_OUT_OF_MEMORY 5           /* a device allocation failed */
#define DF_ERR_BACKEND_INIT 6            /* no usable gfx950 device / HIP error at load */
#define DF_ERR_INVALID_CONFIG 7          /* a config field is out of range */
#define DF_ERR_CONTEXT_FULL 8            /* kv_len + n would pass max_ctx */
#define DF_ERR_BUSY 9                    /* another forward is running on this model */
#define DF_ERR_INVALID_ARGUMENT 10       /* NULL / out-of-range argument, bad token id */
#define DF_ERR_DEVICE 11                 /* a HIP call failed after load */

/* Architectures: the step lists of page "Local inference and
 * architectures" ("What is in effect right now": llama 16 steps per layer,
 * qwen3 18, qwen2 19). qwen3 adds norm_heads on q and k before rope (section
 * "The format"); qwen2 adds a bias to each of the q, k and v matmul outputs
 * (the three bias lines of the same section), tensors
 * "blk.<i>.attn_{q,k,v}.bias", f32 or f16 vectors of n_heads*head_dim and
 * n_kv_heads*head_dim values. */
#define DF_ARCH_LLAMA 0
#define DF_ARCH_QWEN3 1
#define DF_ARCH_QWEN2 2
/* gemma3 (20 steps per layer, page "Local inference and architectures",
 * "What is in effect right now"; gelu_tanh, "The operations"; a window
 * pattern, "Rules"). Read as: the embedding scaled by f32(sqrt(d_model));
 * per layer rms_norm, q/k/v matmul, norm_heads q and k, rope, attention
 * (through the sliding window on the pattern's local layers), o matmul,
 * rms_norm of o ("blk.<i>.post_attention_norm.weight"), add, rms_norm, gate
 * matmul, gelu_tanh, up matmul, mul, down matmul, rms_norm of down
 * ("blk.<i>.post_ffw_norm.weight"), add. */
#define DF_ARCH_GEMMA3 3

/* RoPE pairing within a head (the pages name rope without fixing the
 * pairing): DF_ROPE_HALVES rotates (t[i], t[i + head_dim/2]),
 * DF_ROPE_ADJACENT rotates (t[2i], t[2i+1]); pair i turns by
 * p * theta^(-2i/head_dim) either way. */
#define DF_ROPE_HALVES 0
#define DF_ROPE_ADJACENT 1

/* Widest matmul input: a decode matvec keeps its whole f32 input vector in
 * LDS (128 KiB at this width, of the 160 KiB a gfx950 work-group may use). */
#define DF_MAX_WIDTH 32768

/* Weight dtypes. DF_Q8_32: blocks of 32 consecutive int8 values along a row
 * with one f16 scale each; the host layout of one block is the scale
 * (little-endian f16) followed by the 32 values, 34 bytes; value = scale * q.
 * Embeddings and norm weights are DF_F32 or DF_F16. */
#define DF_F32 0
#define DF_F16 1
#define DF_Q8_32 2

typedef struct df_config {
    int32_t arch;        /* DF_ARCH_LLAMA, DF_ARCH_QWEN3, DF_ARCH_QWEN2 or DF_ARCH_GEMMA3 */
    int32_t n_layers;    /* >= 0 */
    int32_t d_model;     /* multiple of 32, <= DF_MAX_WIDTH */
    int32_t n_heads;     /* query heads */
    int32_t n_kv_heads;  /* divides n_heads; n_heads / n_kv_heads <= 8 */
    int32_t head_dim;    /* 16, 32, 64, 128 or 256; n_heads * head_dim <= DF_MAX_WIDTH */
    int32_t ffn_dim;     /* multiple of 32, <= DF_MAX_WIDTH */
    int32_t vocab;       /* >= 1 */
    int32_t max_ctx;     /* KV capacity in positions, 1 .. 1048576 */
    int32_t rope_pairing; /* DF_ROPE_HALVES (0) or DF_ROPE_ADJACENT */
    double rope_theta;   /* > 0; angle p * theta^(-2i/head_dim) */
    double rms_eps;      /* >= 0; inside the square root */
    /* Sliding-window attention (any arch): with sliding_window W > 0, layer
     * i is local when (i + 1) % window_pattern != 0 and its position p then
     * attends to the positions p - W < t <= p only, rotating with
     * rope_theta_local (0: rope_theta); the other layers are global. W = 0:
     * every layer global. */
    int32_t sliding_window;  /* >= 0 */
    int32_t window_pattern;  /* >= 1 when sliding_window > 0 */
    double rope_theta_local; /* >= 0 */
} df_config;

/* One weight. name is the GGUF name ("token_embd.weight",
 * "blk.<i>.attn_q.weight", ..., "output_norm.weight", optional
 * "output.weight"). Matrices are [rows = outputs][cols = inputs] row-major
 * (y = W h); vectors (norm weights) have rows == 1. data points to host
 * memory (on_device == 0) or device memory of the model's GPU
 * (on_device == 1); nbytes must equal the size the dtype implies. The
 * library copies the data during df_load; the caller keeps ownership and may
 * free it when df_load returns. */
typedef struct df_tensor {
    const char* name;
    int32_t dtype;
    int32_t on_device;
    int64_t rows;
    int64_t cols;
    const void* data;
    uint64_t nbytes;
} df_tensor;

typedef struct df_options {
    void* stream;        /* hipStream_t to order all work on; NULL: the library makes one */
    int32_t device;      /* HIP device ordinal; used when stream is NULL */
    int32_t flags;       /* reserved: must be 0 (no flags are defined) */
} df_options;

typedef struct df_timings {
    double load_ms;          /* wall time of df_load, upload included */
    double last_prefill_ms;  /* device time of the last df_forward with n > 1 */
    double last_step_ms;     /* device time of the last df_forward with n == 1 */
    int64_t n_forward;       /* df_forward calls that succeeded */
    int64_t weight_bytes;    /* device bytes held for weights */
    int64_t kv_bytes;        /* device bytes held for the KV cache */
    int64_t pool_bytes;      /* device bytes held by the activation frame pool */
} df_timings;

typedef struct df_model df_model;

/* Validate config and tensor table, allocate device weights (repacking
 * 8-bit blocks into separate value and scale planes), the KV cache for
 * max_ctx positions and the cos/sin table, and upload. Validation happens
 * before any device call. On error *out = NULL, nothing is leaked and
 * df_last_error(NULL) names the tensor / field / bytes involved. opt may be
 * NULL (device 0, own stream). */
df_status df_load(const df_config* cfg, const df_tensor* tensors,
                  size_t n_tensors, const df_options* opt, df_model** out);

/* Open another conversation on a loaded model (page "Execution contract",
 * "Concurrency": each conversation has its own KV cache, and several share
 * one loaded model). The session shares the model's device weights and
 * cos/sin table and gets its own KV cache of max_ctx positions (1 .. the
 * model's max_ctx), decode state, activation pool and stream (opt->stream,
 * or one the library makes; opt->device is ignored: the model's device is
 * used; opt->flags must be 0). *out is a df_model handle on which every
 * other call works as on a loaded model; it starts empty (kv_len 0). Forwards
 * on different handles of one model may run concurrently from different
 * threads; one handle still takes one forward at a time (DF_ERR_BUSY). The
 * weights stay allocated until the model and all its sessions are freed,
 * in any order, each with df_free. On error *out = NULL and
 * df_last_error(NULL) says why. */
df_status df_session(const df_model* model, int32_t max_ctx, const df_options* opt,
                     df_model** out);

/* Append n tokens (host array of ids in [0, vocab)) at positions kv_len ..
 * kv_len+n-1 and write the logits of the last position, vocab f32 values,
 * to logits_dev (device memory, caller-owned; NULL skips the logits).
 * n == 1 runs the decode path; n > 1 runs bulk prefill on matrix cores
 * (f16 or 8-bit block weights; 8-bit blocks are dequantised to f16 on the
 * way into the GEMM; f32 weights run the decode path n times), which matches
 * n single calls within the prefill tolerance. Arguments are checked
 * before any launch (n < 1 or a NULL `tokens` is DF_ERR_INVALID_ARGUMENT,
 * kv_len + n > max_ctx DF_ERR_CONTEXT_FULL, an id outside [0, vocab)
 * DF_ERR_INVALID_ARGUMENT); on error kv_len is unchanged. Stream-ordered:
 * the host may reuse `tokens` on return. */
df_status df_forward(df_model* m, const int32_t* tokens, int32_t n,
                     float* logits_dev);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * result as n df_forward calls of one token each, with no allocation in the
 * call. The n tokens run through the decode kernels one position at a time
 * (never the bulk matrix-core path, whose buffers grow with n). The
 * activations that pass between the step's kernels live in one fixed device
 * array of DF_NOALLOC_SCRATCH_BYTES bytes per GPU,
 * held by the library until the process ends and shared by every call on
 * that GPU: calls that overlap on one GPU (two models, or two sessions, on
 * different streams) race on it and must be ordered by the caller. Nothing
 * in the array needs clearing between calls: every value is written before
 * it is read. A model whose step activations (d_model + q|k|v + n_heads *
 * head_dim + ffn_dim floats, plus d_model + 1 for gemma3, each rounded up to
 * 256 bytes) exceed the array is refused with DF_ERR_UNSUPPORTED_OP; the
 * llama-8B shape takes 112 KiB. Also refused while df_profile is on. Other
 * arguments and errors as df_forward: an argument error leaves kv_len
 * unchanged; a failed launch (DF_ERR_DEVICE) leaves it at the positions
 * completed before it. */
#define DF_NOALLOC_SCRATCH_BYTES (256 * 1024)
df_status df_forward_noalloc(df_model* m, const int32_t* tokens, int32_t n,
                             float* logits_dev);

/* Greedy decode on the device: step i feeds token t_i (t_0 = first_token),
 * computes the logits, takes t_{i+1} = argmax (lowest index on ties) and
 * writes it to tokens_dev[i], for i < n_steps, with no host round trip.
 * The last step's logits go to logits_dev unless it is NULL. Equivalent to
 * n_steps df_forward(n = 1) + df_argmax calls. */
df_status df_generate(df_model* m, int32_t first_token, int32_t n_steps,
                      int32_t* tokens_dev, float* logits_dev);

/* kv_len = 0. The cache memory is kept; nothing reads past kv_len. */
df_status df_reset_kv_cache(df_model* m);

/* Release every device allocation and set *m = NULL. NULL or an already
 * released handle is a no-op. */
void df_free(df_model** m);

/* Text of the last error on this model, or, for m == NULL, the last df_load
 * failure on the calling thread. Valid until the next call on the model. */
const char* df_last_error(const df_model* m);

/* Timing breakdown and memory footprint. Synchronises the model's stream. */
df_status df_get_timings(df_model* m, df_timings* out);

/* Number of positions in the KV cache. */
df_status df_kv_length(const df_model* m, int32_t* out);

/* argmax of vocab f32 values in device memory; lowest index on ties, NaN
 * never wins. Synchronises the stream and writes the id to *token_host. */
df_status df_argmax(df_model* m, const float* logits_dev, int32_t* token_host);

/* Copy KV rows [pos0, pos0+n) of one layer (which: 0 = K after RoPE, 1 = V)
 * to host memory laid out [n_kv_heads][n][head_dim] f32. Synchronises. */
df_status df_read_kv(df_model* m, int32_t layer, int32_t which, int32_t pos0,
                     int32_t n, float* host);

/* Overwrite KV rows [pos0, pos0+n) of one layer from host memory laid out
 * as df_read_kv's, and set kv_len to kv_len_after (<= max_ctx). Restores a
 * saved context without recomputing it. Synchronises. */
df_status df_write_kv(df_model* m, int32_t layer, int32_t which, int32_t pos0,
                      int32_t n, const float* host, int32_t kv_len_after);

/* The HIP stream the model orders its work on (a hipStream_t). */
void* df_stream(const df_model* m);

/* Kernel classes for df_profile (observability, page "Execution contract",
 * "Observability": a timing breakdown of every forward). */
#define DF_K_EMBED 0        /* token row gather */
#define DF_K_QKV 1          /* rms_norm + q/k/v matvec */
#define DF_K_ATTN 2         /* norm_heads + rope + KV append + split attention */
#define DF_K_O 3            /* o matvec + residual add */
#define DF_K_GATE_UP 4      /* rms_norm + gate/up matvec + silu * up */
#define DF_K_DOWN 5         /* down matvec + residual add */
#define DF_K_LOGITS 6       /* final rms_norm + logits matvec */
#define DF_K_ARGMAX 7       /* greedy token */
#define DF_K_ATTN_MERGE 8   /* merge of the attention splits */
#define DF_K_COUNT 9
/* Bulk-prefill launch classes, for df_time_prefill. */
#define DF_K_PF_QKV 10      /* rms_norm rows + q/k/v GEMM */
#define DF_K_PF_ATTN 11     /* causal attention */
#define DF_K_PF_O 12        /* o GEMM + residual add */
#define DF_K_PF_GATE_UP 13  /* rms_norm rows + gate/up GEMM + gate activation * up */
#define DF_K_PF_DOWN 14     /* down GEMM + residual add */
#define DF_K_PF_ROWS 15     /* row pass before the attention: bias / norm_heads / rope of q and k,
                               KV append, and the cache's f16 copies of the new rows */

/* Time every launch of one kernel class (enable = 1) with start / end
 * stamps taken by the kernel dispatch itself, or stop (enable = 0). The
 * device-resident step graph is not used while a class is profiled. */
df_status df_profile(df_model* m, int32_t kernel, int32_t enable);

/* Synchronise, then report the launches timed since the last read and their
 * summed device time in milliseconds; clears the record. */
df_status df_profile_read(df_model* m, int32_t kernel, int64_t* launches,
                          double* total_ms);

/* Mean device time of one launch of a kernel class in the decode step's
 * launch configuration: the class's launches of one step (one per layer, or
 * one for embed / logits / argmax) are replayed `reps` times back to back on
 * the model's stream between one pair of HIP events, with no other work in
 * between. Activation buffers and the cache row at kv_len are overwritten
 * (the next df_forward / df_generate starts from its own inputs as always).
 * The row at kv_len is free, so the cached context stays intact; on a full
 * cache (kv_len == max_ctx) DF_K_ATTN returns DF_ERR_CONTEXT_FULL.
 * Synchronises. */
df_status df_time_kernel(df_model* m, int32_t kernel, int32_t reps,
                         double* mean_us);

/* Mean device time of one layer's launches of a bulk-prefill class
 * (DF_K_PF_QKV .. DF_K_PF_ROWS) for `rows` rows (1 .. max_ctx - kv_len) at
 * positions kv_len .. kv_len+rows-1: each layer's launches in turn, `reps`
 * times, back to back between one pair of HIP events, on activation buffers
 * filled with pseudo-random values in [-1, 1) (the clocks depend on the
 * operands). DF_K_PF_ROWS writes the cache rows kv_len .. kv_len+rows-1,
 * which no later call reads before overwriting them, and kv_len is left as
 * it was, so the cached context stays intact; DF_K_PF_ATTN first runs the
 * row pass once per layer, untimed, so that it attends over those rows. Needs f16 or 8-bit block
 * weights (else DF_ERR_UNSUPPORTED_OP). Synchronises. */
df_status df_time_prefill(df_model* m, int32_t kernel, int32_t rows, int32_t reps,
                          double* mean_us);

/* Debug query: the matrix-core kernels a bulk prefill of `rows` rows runs
 * for the q/k/v, o, gate/up and down GEMMs (plan[0..3]), each a tile code
 * DF_GEMM_* with the DF_GEMM_Q8_* flags or'ed in, and in bits 8..11
 * (DF_GEMM_SPLIT_MASK) the number of work-groups each tile's K loop is split
 * over (1: none); all 0 when the model has no layers or no bulk path (f32
 * weights). The same host function picks the kernel at launch, so tests can
 * check which kernels a run exercises. */
#define DF_GEMM_T128x128 1        /* 4 waves, operands staged through registers */
#define DF_GEMM_T128x256 2        /* 8 waves, staged through registers */
#define DF_GEMM_T256x256 3        /* 8 waves, staged through registers */
#define DF_GEMM_T256x256_LDS 4    /* 8 waves, operand tiles loaded straight into LDS */
#define DF_GEMM_T256x192_LDS 5    /* 8 waves of 64 x 96, loaded straight into LDS */
#define DF_GEMM_TILE_MASK 15
#define DF_GEMM_Q8_IN_GEMM 16     /* 8-bit weight tiles dequantised on their way into LDS */
#define DF_GEMM_Q8_DEQUANT_FIRST 32 /* 8-bit matrices converted to f16 before the GEMM */
#define DF_GEMM_SPLIT_SHIFT 8
#define DF_GEMM_SPLIT_MASK 0xF00
df_status df_prefill_plan(const df_model* m, int32_t rows, int32_t* plan);

#ifdef __cplusplus
}
#endif
#endif
