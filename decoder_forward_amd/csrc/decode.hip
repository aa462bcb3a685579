// decode.hip — bs=1 decode kernels for gfx950 (CDNA4, wave64).
//
// One token per step (page "Execution contract", "Forward phase": prefill
// and decode both run forward on one token). At one token every matmul is a
// matrix-vector product that reads each weight once: the step is bound by
// HBM bandwidth, not by arithmetic. The kernels therefore stream weights with
// 16-byte coalesced loads, keep the activation vector in LDS, multiply in
// f32 (page "Local inference and architectures", "Choosing the engine") and
// reduce across the 64 lanes of a wave with shuffles. RMSNorm is folded into
// the matvec that consumes it: y = r * W (x . w) with r = 1/sqrt(mean x^2 +
// eps), so the norm needs no pass of its own. norm_heads, RoPE and the KV
// append are folded into the attention kernel's prologue.
#include "attn_core.h"

#include <hip/hip_fp16.h>

namespace dfk {
namespace {

using namespace dev;

// Decode matvec as its own launch (see mv_begin / mv_finish).
template <int WT, int MODE, bool NORM>
__global__ void __launch_bounds__(512)
matvec_kernel(const void* __restrict__ W, const uint16_t* __restrict__ scales, MvLayout L,
              const float* __restrict__ x, const float* __restrict__ norm_w, float eps,
              float* __restrict__ out)
{
    extern __shared__ float hs[];
    __shared__ float red[16];
    MvState<WT, MODE> st;
    mv_begin<WT, MODE>(W, scales, L, blockIdx.x, st, threadIdx.x);
    mv_finish<WT, MODE, NORM>(scales, W, L, st, x, norm_w, eps, out, hs, red, threadIdx.x);
}

template <int WT, int MODE, bool NORM>
hipError_t launch_mv_t(const Weight& W, const float* x, const float* nw,
                       float eps, int64_t n_out, int64_t up_rows, float* out,
                       hipStream_t s, int act)
{
    int64_t blocks = 0;
    MvLayout L = make_mv_layout(WT, W.cols, n_out, up_rows, 512, 8, &blocks);
    L.act = act;
    const size_t lds = mv_lds_bytes(L, MODE);
    if (lds > 65536) {  // x of more than 16384 values: opt in to the larger LDS
        const hipError_t r = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&matvec_kernel<WT, MODE, NORM>),
            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (r != hipSuccess) return r;
    }
    DFK_LAUNCH((matvec_kernel<WT, MODE, NORM>), dim3(unsigned(blocks)),
                       dim3(512), lds, s, W.data, W.scales, L, x, nw, eps, out);
    return hipGetLastError();
}

template <int WT>
hipError_t launch_mv_w(const Weight& W, int mode, const float* x,
                       const float* nw, float eps, int64_t n_out,
                       int64_t up_rows, float* out, hipStream_t s, int act)
{
    const bool norm = nw != nullptr;
    switch (mode) {
    case MV_STORE:
        return norm ? launch_mv_t<WT, MV_STORE, true>(W, x, nw, eps, n_out, up_rows, out, s, act)
                    : launch_mv_t<WT, MV_STORE, false>(W, x, nw, eps, n_out, up_rows, out, s, act);
    case MV_SWIGLU:
        return norm ? launch_mv_t<WT, MV_SWIGLU, true>(W, x, nw, eps, n_out, up_rows, out, s, act)
                    : launch_mv_t<WT, MV_SWIGLU, false>(W, x, nw, eps, n_out, up_rows, out, s, act);
    case MV_STORE2:
        return norm ? launch_mv_t<WT, MV_STORE2, true>(W, x, nw, eps, n_out, up_rows, out, s, act)
                    : launch_mv_t<WT, MV_STORE2, false>(W, x, nw, eps, n_out, up_rows, out, s, act);
    case MV_RESID2:
        return norm ? launch_mv_t<WT, MV_RESID2, true>(W, x, nw, eps, n_out, up_rows, out, s, act)
                    : launch_mv_t<WT, MV_RESID2, false>(W, x, nw, eps, n_out, up_rows, out, s, act);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// embed: x[row] = f32(E[token]) (prologue of the step list).
// ---------------------------------------------------------------------------
template <int WT>
__global__ void embed_kernel(const void* __restrict__ E, int64_t d,
                             const int* __restrict__ tokens,
                             const int* __restrict__ state_tok,
                             float* __restrict__ x, float scale)
{
    const int row = blockIdx.x;
    const int t = tokens ? tokens[row] : *state_tok;
    for (int64_t i = threadIdx.x; i < d; i += blockDim.x) {
        float v;
        if constexpr (WT == W_F32) v = static_cast<const float*>(E)[int64_t(t) * d + i];
        else v = f16_bits_to_f32(static_cast<const uint16_t*>(E)[int64_t(t) * d + i]);
        x[int64_t(row) * d + i] = v * scale;
    }
}

// ---------------------------------------------------------------------------
// rms_norm of a matmul output added to the residual stream (gemma3's norms
// after o and after down): x[row] += w . t[row] / sqrt(mean(t[row]^2) + eps).
// One block per row; the row is held in registers between the two passes.
// ---------------------------------------------------------------------------
constexpr int NA_THREADS = 1024;
constexpr int NA_PER_THREAD = (MAX_WIDTH + NA_THREADS - 1) / NA_THREADS;

__global__ void __launch_bounds__(NA_THREADS)
norm_add_rows_kernel(float* __restrict__ x, const float* __restrict__ t,
                     const float* __restrict__ w, int d, float eps)
{
    __shared__ float red[NA_THREADS / WAVE];
    const int64_t row = blockIdx.x;
    const float* tr = t + row * d;
    float* xr = x + row * d;
    float v[NA_PER_THREAD];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NA_PER_THREAD; ++i) {
        const int k = threadIdx.x + i * NA_THREADS;
        v[i] = k < d ? tr[k] : 0.f;
        ss = fmaf(v[i], v[i], ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < NA_THREADS / WAVE; ++i) tot += red[i];
    const float r = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
#pragma unroll
    for (int i = 0; i < NA_PER_THREAD; ++i) {
        const int k = threadIdx.x + i * NA_THREADS;
        if (k < d) xr[k] += w[k] * (v[i] * r);
    }
}

// ---------------------------------------------------------------------------
// Decode attention (split-K "flash decoding") for one KV head g: grid
// (splits, n_kv), 4 waves per work-group.
//
// The positions 0..p are cut into tiles of ATTN_T rows; work-group `split`
// takes a contiguous run of tiles (the same partition for every launch shape,
// so results are bitwise reproducible) and runs attn_core on it: norm_heads
// and rope of the query heads (and of the new key in the work-group that owns
// position p, which also appends k and v at slot p), then per-wave online
// softmax over its rows. One work-group per head writes the output itself;
// otherwise each writes its (acc, max, sum) partial for the merge kernel.
// ---------------------------------------------------------------------------
template <int HD>
constexpr int attn_waves() { return HD >= 256 ? 8 : 4; }

template <int HD, int G>
__global__ void __launch_bounds__(64 * attn_waves<HD>())
attn_decode_kernel(AttnDecodeArgs a)
{
    constexpr int NW = attn_waves<HD>();
    __shared__ float lds[attn_core_lds_floats<HD, G, NW>()];
    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int p = *gmem(a.state_pos);
    const int lo = attn_first_pos(p, a.window);
    const int tiles = (p + 1 - lo + ATTN_T - 1) / ATTN_T;
    const int tpw = (tiles + ATTN_MAX_SPLIT - 1) / ATTN_MAX_SPLIT;  // tiles per work-group
    const int n_active = (tiles + tpw - 1) / tpw;
    if (split >= n_active) return;
    AttnItem it;
    it.qkv = a.qkv;
    it.q_norm = a.q_norm;
    it.k_norm = a.k_norm;
    it.bias = a.bias;
    it.eps = a.eps;
    it.adjacent = a.adjacent;
    it.cos_row = a.cos_t + int64_t(p) * (HD / 2);
    it.sin_row = a.sin_t + int64_t(p) * (HD / 2);
    it.kc = a.kc + int64_t(g) * a.max_ctx * HD;
    it.vc = a.vc + int64_t(g) * a.max_ctx * HD;
    it.k16 = a.k16 ? a.k16 + int64_t(g) * a.max_ctx * HD : nullptr;
    it.vt16 = a.vt16 ? a.vt16 + int64_t(g) * HD * a.max_ctx : nullptr;
    it.ctx = a.max_ctx;
    it.qd = a.n_heads * HD;
    it.kvd = a.n_kv * HD;
    it.g = g;
    it.p = p;
    it.pos0 = lo + split * tpw * ATTN_T;
    it.pos1 = min(p + 1, lo + (split + 1) * tpw * ATTN_T);
    it.out = n_active == 1 ? a.out : nullptr;
    it.part = a.part + (int64_t(g) * ATTN_MAX_SPLIT + split) * attn_part_stride(G, HD);
    attn_core<HD, G, NW, ATTN_T / (NW * 4), false>(it, lds, threadIdx.x);
}

// Merge of the split partials of one query head (launched after the split
// kernel, so its stores are visible): weights 2^(m_c - M) (base-2 maxima), total sum, and
// the weighted sum of the accumulators in split order. Four groups of HD
// threads take every fourth split; their sums meet in LDS in fixed order.
template <int HD>
__global__ void __launch_bounds__(4 * HD)
attn_combine_kernel(AttnDecodeArgs a)
{
    constexpr int T = ATTN_T;
    constexpr int CB = 8;
    __shared__ float w[ATTN_MAX_SPLIT];
    __shared__ float lsum[ATTN_MAX_SPLIT];
    __shared__ float ps[4][HD];
    __shared__ float s_L;
    const int hq = blockIdx.x;
    const int G = a.n_heads / a.n_kv;
    const int g = hq / G, j = hq % G;
    const int tid = threadIdx.x;
    const int p = *a.state_pos;
    const int tiles = (p + 1 - attn_first_pos(p, a.window) + T - 1) / T;
    const int tpw = (tiles + ATTN_MAX_SPLIT - 1) / ATTN_MAX_SPLIT;
    const int n_active = (tiles + tpw - 1) / tpw;
    if (n_active == 1) return;  // the split kernel wrote the output itself
    const int64_t cs = attn_part_stride(G, HD);
    const float* pg = a.part + int64_t(g) * ATTN_MAX_SPLIT * cs;
    for (int c = tid; c < n_active; c += blockDim.x) {
        w[c] = pg[c * cs + G * HD + j];
        lsum[c] = pg[c * cs + G * HD + G + j];
    }
    __syncthreads();
    if (tid < WAVE) {
        float M = -INFINITY;
        for (int c = tid; c < n_active; c += WAVE) M = fmaxf(M, w[c]);
        M = wave_max(M);
        float L = 0.f;
        for (int c = tid; c < n_active; c += WAVE) {
            const float e = exp2_fast(w[c] - M);  // maxima in base-2 units
            w[c] = e;
            L = fmaf(lsum[c], e, L);
        }
        L = wave_sum(L);
        if (tid == 0) s_L = L;
    }
    __syncthreads();
    const int grp = tid / HD;
    const int d = tid % HD;
    float acc = 0.f;
    for (int c0 = grp; c0 < n_active; c0 += 4 * CB) {
        float x[CB];
#pragma unroll
        for (int b2 = 0; b2 < CB; ++b2) {
            const int c = c0 + 4 * b2;
            x[b2] = c < n_active ? pg[c * cs + j * HD + d] : 0.f;
        }
#pragma unroll
        for (int b2 = 0; b2 < CB; ++b2) {
            const int c = c0 + 4 * b2;
            if (c < n_active) acc = fmaf(w[c], x[b2], acc);
        }
    }
    ps[grp][d] = acc;
    __syncthreads();
    if (grp == 0)
        a.out[int64_t(hq) * HD + d] = (ps[0][d] + ps[1][d] + ps[2][d] + ps[3][d]) / s_L;
}

// ---------------------------------------------------------------------------
// argmax, two stages: per-block (max, lowest index), then the last block to
// finish (atomic ticket) merges the block results in block order.
// ---------------------------------------------------------------------------
__device__ inline bool better(float v, int i, float bv, int bi)
{
    return v > bv || (v == bv && i < bi);
}

__device__ inline void argmax_wave(float& bv, int& bi)
{
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, WAVE);
        const int oi = __shfl_xor(bi, o, WAVE);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
}

// Block-wide (max, lowest index) of the per-thread candidates.
__device__ inline void argmax_block(float& bv, int& bi, float* sv, int* si)
{
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x >> 6;
    argmax_wave(bv, bi);
    if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
    __syncthreads();
    bv = -INFINITY;
    bi = 0x7fffffff;
    for (int w = 0; w < int(blockDim.x >> 6); ++w)
        if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
}

__global__ void __launch_bounds__(256)
argmax_kernel(const float* __restrict__ v, int n, DevState* st, int* out_dev,
              int advance, int* gen_out)
{
    __shared__ float sv[4];
    __shared__ int si[4];
    __shared__ int is_last;
    const int tid = threadIdx.x;
    const int per = (n + gridDim.x - 1) / gridDim.x;
    const int lo = blockIdx.x * per;
    const int hi = min(n, lo + per);
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    // Up to 8 loads in flight per thread.
    for (int base = lo; base < hi; base += 256 * 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = base + u * 256 + tid;
            x[u] = i < hi ? v[i] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = base + u * 256 + tid;
            if (i < hi && better(x[u], i, bv, bi)) { bv = x[u]; bi = i; }
        }
    }
    argmax_block(bv, bi, sv, si);
    if (tid == 0) {
        st_shared_f(&st->part_val[blockIdx.x], bv);
        st_shared_i(&st->part_idx[blockIdx.x], bi);
    }
    if (!last_to_arrive(&st->argmax_count, int(gridDim.x), &is_last)) return;
    bv = -INFINITY;
    bi = 0x7fffffff;
    if (tid < int(gridDim.x)) {
        bv = ld_shared_f(&st->part_val[tid]);
        bi = ld_shared_i(&st->part_idx[tid]);
    }
    __syncthreads();
    argmax_block(bv, bi, sv, si);
    if (tid != 0) return;
    if (bi == 0x7fffffff) bi = 0;  // all NaN
    if (out_dev) *out_dev = bi;
    if (advance) {
        gen_out[st->step] = bi;
        st->tok = bi;
        st->pos += 1;
        st->step += 1;
    }
}

__global__ void set_state_kernel(DevState* st, int pos, int tok, int step)
{
    if (threadIdx.x == 0) {
        st->pos = pos;
        st->tok = tok;
        st->step = step;
    }
}

__global__ void to_f32_kernel(const void* __restrict__ src, int src_dtype,
                              int64_t n, float* __restrict__ dst)
{
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        dst[i] = src_dtype == W_F32 ? static_cast<const float*>(src)[i]
                                    : f16_bits_to_f32(static_cast<const uint16_t*>(src)[i]);
    }
}

// Deterministic pseudo-random values, uniform in [-1, 1), for timing
// replays: element i gets a 32-bit integer hash of (i, seed) (the
// multiply-xorshift finaliser of MurmurHash3) scaled to [-1, 1).
__global__ void fill_random_kernel(void* __restrict__ dst, int64_t n, int f16, uint32_t seed)
{
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        uint32_t h = uint32_t(i) ^ (uint32_t(i >> 32) * 0x9e3779b9u) ^ seed;
        h ^= h >> 16;
        h *= 0x85ebca6bu;
        h ^= h >> 13;
        h *= 0xc2b2ae35u;
        h ^= h >> 16;
        const float v = float(int32_t(h)) * (1.0f / 2147483648.0f);
        if (f16) static_cast<_Float16*>(dst)[i] = static_cast<_Float16>(v);
        else static_cast<float*>(dst)[i] = v;
    }
}

__global__ void q8_split_kernel(const uint8_t* __restrict__ blocks,
                                int64_t n_blocks, int8_t* __restrict__ values,
                                uint16_t* __restrict__ scales)
{
    for (int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; b < n_blocks;
         b += int64_t(gridDim.x) * blockDim.x) {
        const uint8_t* src = blocks + b * 34;
        scales[b] = uint16_t(src[0]) | uint16_t(uint16_t(src[1]) << 8);
        uint32_t* dst = reinterpret_cast<uint32_t*>(values + b * 32);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint8_t* q = src + 2 + 4 * j;
            dst[j] = uint32_t(q[0]) | (uint32_t(q[1]) << 8) | (uint32_t(q[2]) << 16) |
                     (uint32_t(q[3]) << 24);
        }
    }
}

}  // namespace

MvLayout make_mv_layout(int wdtype, int64_t K, int64_t n_out, int64_t up_rows, int max_blocks,
                        int nwaves, int64_t* blocks)
{
    const int E = wdtype == W_F32 ? 4 : wdtype == W_F16 ? 8 : 16;
    MvLayout L;
    L.K = K;
    L.n_out = n_out;
    L.up_rows = up_rows;
    L.wdtype = wdtype;
    const int64_t CH = int64_t(64) * E;
    const int64_t nchunks = (K + CH - 1) / CH;
    const int64_t upb = n_out > 0 ? (n_out + max_blocks - 1) / max_blocks : 1;
    L.upb = int(upb);
    *blocks = n_out > 0 ? (n_out + upb - 1) / upb : 0;
    L.log_s = 0;
    if (upb % nwaves != 0 && upb < 64) {
        for (int ls = 1; ls <= 3; ++ls) {
            const int S = 1 << ls;
            if (nchunks % S == 0 && (upb * S) % nwaves == 0) { L.log_s = ls; break; }
        }
    }
    const int S = 1 << L.log_s;
    L.cps = int(nchunks / S);
    L.ipw = int((upb * S + nwaves - 1) / nwaves);
    return L;
}

size_t mv_lds_bytes(const MvLayout& L, int mode)
{
    const int NR = (mode == MV_SWIGLU || mode == MV_STORE2 || mode == MV_RESID2) ? 2 : 1;
    const int S = 1 << L.log_s;
    return size_t(dev::mv_staged_floats(L.wdtype, L.K)) * sizeof(float) +
           size_t(L.upb) * S * NR * sizeof(float);
}

hipError_t launch_matvec(const Weight& W, int mode, const float* x,
                         const float* norm_w, float eps, int64_t n_out,
                         int64_t up_rows, float* out, hipStream_t s, int act)
{
    if (n_out <= 0) return hipSuccess;
    // An even number of rows runs as pairs (n, n + n_out / 2): one LDS read
    // of the activation per two weights. Residual outputs (d_model rows, a
    // multiple of 32) are always even; an odd MV_STORE (a vocabulary) runs
    // one row per unit.
    if (mode == MV_RESID && n_out % 2 != 0) return hipErrorInvalidValue;
    if ((mode == MV_STORE || mode == MV_RESID) && n_out % 2 == 0) {
        mode = mode == MV_STORE ? MV_STORE2 : MV_RESID2;
        up_rows = n_out / 2;
        n_out /= 2;
    }
    switch (W.dtype) {
    case W_F32: return launch_mv_w<W_F32>(W, mode, x, norm_w, eps, n_out, up_rows, out, s, act);
    case W_F16: return launch_mv_w<W_F16>(W, mode, x, norm_w, eps, n_out, up_rows, out, s, act);
    case W_Q8: return launch_mv_w<W_Q8>(W, mode, x, norm_w, eps, n_out, up_rows, out, s, act);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_embed(const Weight& E, const int* tokens_dev,
                        const int* state_tok, int n_rows, float* x,
                        hipStream_t s, float scale)
{
    if (E.dtype == W_F32)
        DFK_LAUNCH(embed_kernel<W_F32>, dim3(n_rows), dim3(256), 0, s,
                           E.data, E.cols, tokens_dev, state_tok, x, scale);
    else
        DFK_LAUNCH(embed_kernel<W_F16>, dim3(n_rows), dim3(256), 0, s,
                           E.data, E.cols, tokens_dev, state_tok, x, scale);
    return hipGetLastError();
}

template <int HD>
hipError_t launch_attn_hd(const AttnDecodeArgs& a, dim3 grid, hipStream_t s)
{
    switch (a.n_heads / a.n_kv) {
    case 1: DFK_LAUNCH((attn_decode_kernel<HD, 1>), grid, dim3(64 * attn_waves<HD>()), 0, s, a); break;
    case 2: DFK_LAUNCH((attn_decode_kernel<HD, 2>), grid, dim3(64 * attn_waves<HD>()), 0, s, a); break;
    case 3: DFK_LAUNCH((attn_decode_kernel<HD, 3>), grid, dim3(64 * attn_waves<HD>()), 0, s, a); break;
    case 4: DFK_LAUNCH((attn_decode_kernel<HD, 4>), grid, dim3(64 * attn_waves<HD>()), 0, s, a); break;
    case 5: DFK_LAUNCH((attn_decode_kernel<HD, 5>), grid, dim3(64 * attn_waves<HD>()), 0, s, a); break;
    case 6: DFK_LAUNCH((attn_decode_kernel<HD, 6>), grid, dim3(64 * attn_waves<HD>()), 0, s, a); break;
    case 7: DFK_LAUNCH((attn_decode_kernel<HD, 7>), grid, dim3(64 * attn_waves<HD>()), 0, s, a); break;
    case 8: DFK_LAUNCH((attn_decode_kernel<HD, 8>), grid, dim3(64 * attn_waves<HD>()), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t s)
{
    const dim3 grid(a.grid_splits, a.n_kv);
    switch (a.head_dim) {
    case 16: return launch_attn_hd<16>(a, grid, s);
    case 32: return launch_attn_hd<32>(a, grid, s);
    case 64: return launch_attn_hd<64>(a, grid, s);
    case 128: return launch_attn_hd<128>(a, grid, s);
    case 256: return launch_attn_hd<256>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(const AttnDecodeArgs& a, hipStream_t s)
{
    const dim3 grid(a.n_heads);
    switch (a.head_dim) {
    case 16: DFK_LAUNCH(attn_combine_kernel<16>, grid, dim3(64), 0, s, a); break;
    case 32: DFK_LAUNCH(attn_combine_kernel<32>, grid, dim3(128), 0, s, a); break;
    case 64: DFK_LAUNCH(attn_combine_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: DFK_LAUNCH(attn_combine_kernel<128>, grid, dim3(512), 0, s, a); break;
    case 256: DFK_LAUNCH(attn_combine_kernel<256>, grid, dim3(1024), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_norm_add_rows(float* x, const float* t, const float* w, int rows, int d,
                                float eps, hipStream_t s)
{
    if (rows <= 0) return hipSuccess;
    if (d > MAX_WIDTH) return hipErrorInvalidValue;
    DFK_LAUNCH(norm_add_rows_kernel, dim3(rows), dim3(NA_THREADS), 0, s, x, t, w, d, eps);
    return hipGetLastError();
}

hipError_t launch_argmax(const float* v, int n, DevState* st, int* out_dev,
                         int advance, int* gen_out, hipStream_t s)
{
    int blocks = (n + 1023) / 1024;
    if (blocks > 256) blocks = 256;
    if (blocks < 1) blocks = 1;
    DFK_LAUNCH(argmax_kernel, dim3(blocks), dim3(256), 0, s, v, n, st,
                       out_dev, advance, gen_out);
    return hipGetLastError();
}

hipError_t launch_set_state(DevState* st, int pos, int tok, int step,
                            hipStream_t s)
{
    DFK_LAUNCH(set_state_kernel, dim3(1), dim3(64), 0, s, st, pos, tok, step);
    return hipGetLastError();
}

hipError_t launch_fill_random(void* dst, int64_t n, int f16, uint32_t seed, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    DFK_LAUNCH(fill_random_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, dst, n, f16, seed);
    return hipGetLastError();
}

hipError_t launch_to_f32(const void* src, int src_dtype, int64_t n, float* dst,
                         hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    DFK_LAUNCH(to_f32_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                       src, src_dtype, n, dst);
    return hipGetLastError();
}

hipError_t launch_q8_split(const uint8_t* blocks, int64_t rows, int64_t cols,
                           int8_t* values, uint16_t* scales, hipStream_t s)
{
    const int64_t nb = rows * (cols / 32);
    if (nb <= 0) return hipSuccess;
    int64_t g = (nb + 255) / 256;
    if (g > 8192) g = 8192;
    DFK_LAUNCH(q8_split_kernel, dim3(unsigned(g)), dim3(256), 0, s,
                       blocks, nb, values, scales);
    return hipGetLastError();
}

}  // namespace dfk
