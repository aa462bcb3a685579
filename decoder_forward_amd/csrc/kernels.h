// kernels.h — launchers of the gfx950 kernels, used by the runtime (host
// C++). Internal to the library; the public surface is include/decfwd.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace dfk {

// Events that the next launch stamps with its own start and end (set by the
// runtime around a profiled launch; both null otherwise). The stamps come
// from the dispatch itself, so they measure the kernel without the cost of
// separate event records.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchTiming& launch_timing();

#define DFK_LAUNCH(kernel, grid, block, lds, stream, ...)                                      \
    do {                                                                                      \
        ::dfk::LaunchTiming& lt_ = ::dfk::launch_timing();                                    \
        if (lt_.start || lt_.stop)                                                            \
            hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, lt_.start, lt_.stop, 0u,  \
                                  __VA_ARGS__);                                               \
        else                                                                                  \
            hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                \
    } while (0)

enum WType { W_F32 = 0, W_F16 = 1, W_Q8 = 2 };

// Widest activation row a kernel handles (d_model, ffn_dim, n_heads*hd).
constexpr int MAX_WIDTH = 32768;

// A device matrix [rows][cols] (y = W h). f32 / f16: `data` holds the
// values row-major. Q8: `data` holds the int8 values row-major and `scales`
// the f16 scale of every 32-value block, [rows][cols / 32].
struct Weight {
    int dtype = W_F16;
    const void* data = nullptr;
    const uint16_t* scales = nullptr;
    int64_t rows = 0, cols = 0;
};

// Epilogues of the decode matvec.
//   MV_STORE : out[n]  = r * (W (x . w))[n]
//   MV_RESID : out[n] += r * (W (x . w))[n]            (residual add)
//   MV_SWIGLU: out[f]  = act(r (W (x . w))[f]) * r (W (x . w))[f + up_rows]
// where (x . w) is x times the norm weight and r = 1/sqrt(mean(x^2) + eps)
// when a norm weight is given, else x and r = 1; act is silu or gelu_tanh.
// MV_STORE2 / MV_RESID2 are MV_STORE / MV_RESID with two rows per unit, n
// and n + up_rows (= half the rows), so that each activation value a lane
// reads from LDS serves two weights of the same column, as in MV_SWIGLU;
// launch_matvec picks them for an even number of rows (MV_RESID always runs
// as MV_RESID2: its outputs, d_model rows, are a multiple of 32).
enum MatvecMode { MV_STORE = 0, MV_RESID = 1, MV_SWIGLU = 2, MV_STORE2 = 3, MV_RESID2 = 4 };
// Gate activation of the gated FFN.
enum GateAct { ACT_SILU = 0, ACT_GELU_TANH = 1 };
// Gate activation of the gated FFN (GateAct): silu(g) = g / (1 + e^-g), or
// gelu_tanh(g) = g/2 (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))), the tanh
// form of gelu (page "Local inference and architectures", "The operations").
__device__ inline float gate_act(float g, int act)
{
    if (act == ACT_GELU_TANH) {
        constexpr float k = 0.7978845608028654f;  // sqrt(2/pi)
        return 0.5f * g * (1.0f + tanhf(k * fmaf(0.044715f * g, g * g, g)));
    }
    return g / (1.0f + expf(-g));
}

// Work layout of a decode matvec over a grid of blocks of waves (see
// device_common.h): units per block, K slices per unit, chunks per slice,
// items per wave.
struct MvLayout {
    int64_t K, n_out, up_rows;
    int upb;
    int log_s;
    int cps;
    int ipw;
    int act = ACT_SILU;  // MV_SWIGLU's gate activation
    int wdtype = W_F16;  // weight dtype the layout was made for (chunk width)
};
// Layout for at most max_blocks blocks of nwaves waves; *blocks gets the
// blocks it uses.
MvLayout make_mv_layout(int wdtype, int64_t K, int64_t n_out, int64_t up_rows, int max_blocks,
                        int nwaves, int64_t* blocks);
// LDS bytes a block needs: the staged activation and the (unit, slice) sums.
size_t mv_lds_bytes(const MvLayout& L, int mode);

// Device-side decode state: the position and the token of the step being
// computed, so that a captured step needs no per-step arguments.
struct DevState {
    int pos;        // position of the token being decoded
    int tok;        // its id
    int step;       // index of the next generated token
    int argmax_count;
    float part_val[256];
    int part_idx[256];
};

// Decode attention: rows per tile, most work-groups per KV head (the
// partition of tiles over work-groups depends only on the position), and
// query heads per KV head (1, 2, 4 or 8).
constexpr int ATTN_T = 64;
constexpr int ATTN_MAX_SPLIT = 128;
// Floats of one attention partial (one item of G query heads): the
// accumulators [G][hd], then the G running maxima, the G sums, padded to a
// multiple of 4 floats so that every item starts 16-byte aligned.
inline constexpr int attn_part_stride(int G, int hd) { return G * hd + ((2 * G + 3) & ~3); }
constexpr int ATTN_MAX_GROUP = 8;

// First position decode attention reads at position p: 0, or inside a
// sliding window of `window` positions, p - window + 1.
__host__ __device__ inline int attn_first_pos(int p, int window)
{
    return window > 0 && p - window + 1 > 0 ? p - window + 1 : 0;
}
// Work-groups per KV head that decode attention uses at position p.
inline int attn_splits(int p, int window = 0)
{
    const int tiles = (p + 1 - attn_first_pos(p, window) + ATTN_T - 1) / ATTN_T;
    const int tpw = (tiles + ATTN_MAX_SPLIT - 1) / ATTN_MAX_SPLIT;
    return (tiles + tpw - 1) / tpw;
}

hipError_t launch_matvec(const Weight& W, int mode, const float* x,
                         const float* norm_w, float eps, int64_t n_out,
                         int64_t up_rows, float* out, hipStream_t s,
                         int act = ACT_SILU);

// x[row] = f32(E[token]) * scale.
hipError_t launch_embed(const Weight& E, const int* tokens_dev,
                        const int* state_tok, int n_rows, float* x,
                        hipStream_t s, float scale = 1.0f);

// x[row] += w . t[row] / sqrt(mean(t[row]^2) + eps) for `rows` rows of d
// floats: an rms_norm of a matmul output added to the residual stream.
hipError_t launch_norm_add_rows(float* x, const float* t, const float* w, int rows, int d,
                                float eps, hipStream_t s);

struct AttnDecodeArgs {
    const float* qkv;          // [n_heads*hd | n_kv*hd | n_kv*hd]
    const float* q_norm;       // [hd] or null (llama)
    const float* k_norm;
    const float* bias;         // [qd + 2 kvd] q|k|v bias (qwen2) or null
    float eps;
    int adjacent;              // rope pairing: (2i, 2i+1) if set, else (i, i + hd/2)
    int window;                // > 0: attend to positions p - window < t <= p only
    const float* cos_t;        // [max_ctx][hd/2]
    const float* sin_t;
    float* kc;                 // this layer's K cache [n_kv][max_ctx][hd]
    float* vc;
    uint16_t* k16;             // f16 copies for bulk prefill, or null: K [n_kv][max_ctx][hd],
    uint16_t* vt16;            // V transposed [n_kv][hd][max_ctx]; the step's row p goes to both
    int max_ctx, n_heads, n_kv, head_dim;
    const int* state_pos;      // device int: position p
    float* part;               // [n_kv][ATTN_MAX_SPLIT] items of attn_part_stride floats
    float* out;                // [n_heads][hd]
    int grid_splits;           // work-groups launched per KV head (>= in use)
};
hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t s);
// Merge of the split partials into `out` (no-op when one split covers p).
hipError_t launch_attn_combine(const AttnDecodeArgs& a, hipStream_t s);

// argmax over n values, lowest index on ties, NaN never wins. Writes the id
// to *out_dev. When `advance` is set it also stores the id as the next token
// of the state, appends it to gen_out[state->step] and advances pos / step.
hipError_t launch_argmax(const float* v, int n, DevState* st, int* out_dev,
                         int advance, int* gen_out, hipStream_t s);

hipError_t launch_set_state(DevState* st, int pos, int tok, int step,
                            hipStream_t s);

// ---- bulk prefill ----------------------------------------------------------

// out[s] = f16(w . x[s] / rms(x[s])) for `rows` rows of d floats.
hipError_t launch_rmsnorm_rows(const float* x, const float* w, int rows, int d, float eps,
                               uint16_t* out, hipStream_t s);

// C[M][N] = A[M][K] B[N][K]^T on matrix cores, f16 operands, f32 accumulation.
enum GemmMode {
    GEMM_STORE_F32 = 0,   // C f32  = A B^T
    GEMM_ADD_F32 = 1,     // C f32 += A B^T (residual)
    GEMM_STORE_F16 = 2,   // C f16  = A B^T
    GEMM_SWIGLU_F16 = 3,  // C f16 [M][N] = act(A Bg^T) * (A Bu^T); Bu = B + up_rows rows
};
struct GemmArgs {
    const uint16_t* A;
    int64_t lda;
    const uint16_t* B;
    int64_t ldb;
    void* C;
    int64_t ldc;
    int M, N, K;
    int64_t up_rows;
    const uint16_t* zeros;     // >= 16 zero bytes (device): source of out-of-range chunks
    // 8-bit block weights: B holds int8 values [N][ldb] (bytes) and Bsc the
    // f16 scale of every 32 values [N][ldb / 32]; B rows are dequantised to
    // f16 (scale * q) on their way into LDS. Null for f16 weights.
    const uint16_t* Bsc;
    int act;                   // GEMM_SWIGLU_F16's gate activation (GateAct)
    // K split of small grids (register-staged tiles; launch_gemm fills split
    // from gemm_plan when ws and tickets are given): `split` work-groups per
    // tile, each on a contiguous range of K stages, store their partial sums
    // in ws; the last of a tile's work-groups to finish adds them in split
    // order and runs the epilogue.
    float* ws;                 // gemm_split_ws_bytes(...) bytes (device)
    int* tickets;              // >= GEMM_SPLIT_TICKETS ints, zero (device); left zero
    int split;
};
hipError_t launch_gemm(const GemmArgs& g, int mode, hipStream_t s);
// The GEMM kernel launch_gemm runs for an M x N problem in `mode` (q8:
// 8-bit block weights dequantised inside the GEMM): a GEMM_PLAN_* tile
// code, plus GEMM_PLAN_Q8_IN_GEMM for q8. Host only.
enum GemmPlan {
    GEMM_PLAN_128x128 = 1,      // 4 waves, register-staged operand loads
    GEMM_PLAN_128x256 = 2,      // 8 waves, register-staged
    GEMM_PLAN_256x256 = 3,      // 8 waves, register-staged (8-bit weights)
    GEMM_PLAN_256x256_LDS = 4,  // 8 waves, operand tiles loaded straight into LDS
    GEMM_PLAN_256x192_LDS = 5,  // 8 waves (64 x 96 each), loaded straight into LDS
    GEMM_PLAN_TILE_MASK = 15,
    GEMM_PLAN_Q8_IN_GEMM = 16,  // weight tiles dequantised on their way into LDS
    GEMM_PLAN_DEQUANT_FIRST = 32,  // 8-bit weights converted to f16 before the GEMM (runtime)
    GEMM_PLAN_SPLIT_SHIFT = 8,  // bits 8..11: work-groups per tile along K (1: no split)
    GEMM_PLAN_SPLIT_MASK = 0xF00,
};
int gemm_plan(int64_t M, int64_t N, int64_t K, int64_t up_rows, int mode, bool q8);
constexpr int GEMM_SPLIT_TICKETS = 1024;
// Bytes of partial sums the plan's split needs (0 without a split).
size_t gemm_split_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t up_rows, int mode, bool q8);

// 8-bit block rows to f16 rows: out[r][k] = f16(scale[r][k / 32] * q[r][k]),
// the values the 8-bit GEMM stores in LDS; cols a multiple of 32.
hipError_t launch_dequant_q8(const void* values, const uint16_t* scales, int64_t rows, int64_t cols,
                             uint16_t* out, hipStream_t s);
// Bulk prefill of at least this many rows dequantises each layer's 8-bit
// matrices to f16 first and runs the f16 GEMMs: the conversion costs less
// than the 8-bit GEMM's slower register-staged loads from about here on
// (measured faster at 1024 rows, slower at 512).
constexpr int PF_DEQUANT_MIN_ROWS = 1024;

struct QkPostArgs {
    const float* qkv;     // [S][qd | kvd | kvd] f32
    const float* q_norm;  // [hd] or null
    const float* k_norm;
    const float* bias;    // [qd | kvd | kvd] bias (qwen2) or null
    float eps;
    int adjacent;         // rope pairing, as in AttnDecodeArgs
    const float* cos_t;
    const float* sin_t;
    float* kc;            // layer K cache [n_kv][max_ctx][hd]
    float* vc;
    uint16_t* q16;        // [S][n_heads][hd] f16
    int S, p0, n_heads, n_kv, head_dim, max_ctx;
};
hipError_t launch_qk_post_rows(const QkPostArgs& a, hipStream_t s);

struct AttnPrefillArgs {
    const uint16_t* q16;  // [S][n_heads][hd] f16 (after RoPE)
    const float* kc;      // layer K cache [n_kv][max_ctx][hd]
    const float* vc;
    const uint16_t* k16;  // the layer's f16 copies (KvShadowArgs), or null: then K and V are
    const uint16_t* vt16; // read from kc / vc and rounded to f16 in the kernel
    uint16_t* out16;      // [S][n_heads * hd] f16
    int S, p0, n_heads, n_kv, head_dim, max_ctx;
    int window;           // > 0: each query sees the keys p - window < t <= p only
};
hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s);

// f16 copies of cache rows [pos0, pos0 + n) of one layer for the bulk-prefill
// attention: k16[g][t][d] = f16(kc[g][t][d]) and vt16[g][d][t] =
// f16(vc[g][t][d]) (V transposed, so that a tile of keys is contiguous per
// dim); do_k / do_v select the halves. The same rounding as the conversion
// the attention would otherwise do in LDS.
struct KvShadowArgs {
    const float* kc;
    const float* vc;
    uint16_t* k16;
    uint16_t* vt16;
    int pos0, n, n_kv, head_dim, max_ctx;
    int do_k, do_v;
};
hipError_t launch_kv_shadow(const KvShadowArgs& a, hipStream_t s);
// True when the bulk-prefill attention reads the f16 copies for this head
// dim (the copies are then kept for every layer).
inline bool kv_shadow_head_dim(int hd) { return hd == 64 || hd == 128; }

// Deterministic pseudo-random values in [-1, 1) (f32, or f16 when f16 is
// set): inputs for timing replays, whose power draw, and so clocks, depend
// on the data.
hipError_t launch_fill_random(void* dst, int64_t n, int f16, uint32_t seed, hipStream_t s);

// Upload helpers.
hipError_t launch_to_f32(const void* src, int src_dtype, int64_t n, float* dst,
                         hipStream_t s);
// Split host-format 8-bit blocks (34 bytes: f16 scale, 32 int8) of a
// [rows][cols] matrix into a value plane and a scale plane.
hipError_t launch_q8_split(const uint8_t* blocks, int64_t rows, int64_t cols,
                           int8_t* values, uint16_t* scales, hipStream_t s);

}  // namespace dfk
