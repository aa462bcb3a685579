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
#include "kernels.h"

#include <hip/hip_fp16.h>

namespace dfk {
namespace {

constexpr int WAVE = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads marked non-temporal: streamed data is read once.
__device__ inline uint4 load16_nt(const void* p)
{
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline float4 load16f_nt(const float* p)
{
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ inline float f16_bits_to_f32(uint16_t b)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// Cross-work-group hand-off without cache-wide fences. Values another
// work-group will read are stored with relaxed agent-scope atomics (written
// through to the coherence point, bypassing the per-XCD L2), every wave waits
// for its stores to be acknowledged before the block takes its ticket, and
// the reader loads with relaxed agent-scope atomics (bypassing stale L2
// lines). A device-scope fence would instead write back and invalidate the
// whole L2 of the XCD once per work-group.
__device__ inline void st_shared_f(float* p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_shared_i(int* p, int v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_shared_f(const float* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int ld_shared_i(const int* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's memory operations are complete.
__device__ inline void drain_memory() { __builtin_amdgcn_s_waitcnt(0); }
// Ticket: returns true in the last of `n` work-groups to arrive (all
// threads). Call after every thread has issued its hand-off stores.
__device__ inline bool last_to_arrive(int* counter, int n, int* flag_lds)
{
    drain_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == n - 1;
        if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag_lds = last;
    }
    __syncthreads();
    return *flag_lds != 0;
}

// Cross-lane reductions with DPP row operations (no LDS traffic):
// quad_perm [1,0,3,2] and [2,3,0,1] combine lanes within quads, row half
// mirror and row mirror combine quads within a 16-lane row. After
// row16_sum every lane of a row holds the row's sum; the four rows of a
// wave are then combined with readlane into a wave-uniform value.
template <int CTRL>
__device__ inline float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

constexpr int DPP_QUAD_XOR1 = 0xB1;
constexpr int DPP_QUAD_XOR2 = 0x4E;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

__device__ inline float row16_sum(float v)
{
    v += dpp_f<DPP_QUAD_XOR1>(v);
    v += dpp_f<DPP_QUAD_XOR2>(v);
    v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
    v += dpp_f<DPP_ROW_MIRROR>(v);
    return v;
}

__device__ inline float row16_max(float v)
{
    v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
    v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
    v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
    return v;
}

__device__ inline float lane_value(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the 64 lanes, the same value in every lane.
__device__ inline float wave_sum(float v)
{
    v = row16_sum(v);
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

__device__ inline float wave_max(float v)
{
    v = row16_max(v);
    return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
                 fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// Elements of a weight row covered by one lane's 16-byte load.
template <int WT> struct Epl;
template <> struct Epl<W_F32> { static constexpr int v = 4; };
template <> struct Epl<W_F16> { static constexpr int v = 8; };
template <> struct Epl<W_Q8> { static constexpr int v = 16; };

template <int WT>
__device__ inline uint4 load_w(const void* base, int64_t elem)
{
    const char* p = static_cast<const char*>(base) +
                    elem * (WT == W_F32 ? 4 : WT == W_F16 ? 2 : 1);
    return load16_nt(p);
}

// dot of a lane's 16-byte weight vector with hs[k .. k + Epl).
template <int WT>
__device__ inline float lane_dot(uint4 w, const float* hs, int64_t k,
                                 const uint16_t* srow)
{
    if constexpr (WT == W_F32) {
        const float4 h = *reinterpret_cast<const float4*>(hs + k);
        float a = __uint_as_float(w.x) * h.x;
        a = fmaf(__uint_as_float(w.y), h.y, a);
        a = fmaf(__uint_as_float(w.z), h.z, a);
        return fmaf(__uint_as_float(w.w), h.w, a);
    } else if constexpr (WT == W_F16) {
        const half8 hw = __builtin_bit_cast(half8, w);
        const float4 h0 = *reinterpret_cast<const float4*>(hs + k);
        const float4 h1 = *reinterpret_cast<const float4*>(hs + k + 4);
        float a = static_cast<float>(hw[0]) * h0.x;
        float b = static_cast<float>(hw[1]) * h0.y;
        a = fmaf(static_cast<float>(hw[2]), h0.z, a);
        b = fmaf(static_cast<float>(hw[3]), h0.w, b);
        a = fmaf(static_cast<float>(hw[4]), h1.x, a);
        b = fmaf(static_cast<float>(hw[5]), h1.y, b);
        a = fmaf(static_cast<float>(hw[6]), h1.z, a);
        b = fmaf(static_cast<float>(hw[7]), h1.w, b);
        return a + b;
    } else {
        // 16 int8 of one 32-value block: scale * sum(q * h)
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 h = *reinterpret_cast<const float4*>(hs + k + 4 * j);
            const uint32_t v = ww[j];
            a = fmaf(static_cast<float>(static_cast<int8_t>(v & 0xff)), h.x, a);
            b = fmaf(static_cast<float>(static_cast<int8_t>((v >> 8) & 0xff)), h.y, b);
            a = fmaf(static_cast<float>(static_cast<int8_t>((v >> 16) & 0xff)), h.z, a);
            b = fmaf(static_cast<float>(static_cast<int8_t>(v >> 24)), h.w, b);
        }
        return f16_bits_to_f32(srow[k >> 5]) * (a + b);
    }
}

// Decode matvec: out = epilogue(r * W (x . w)).
//
// Work layout. A block owns `upb` consecutive output units (a row, or a
// gate row with its up row) and splits each unit's K range into S equal
// slices of whole 64-lane chunks, so that its 8 waves get equal numbers of
// (unit, slice) items: the kernel has no straggler waves. Each wave walks its
// items as one stream of chunks, U chunks per batch, and issues the loads of
// batch i+1 before it consumes batch i; the very first batch is issued before
// the activation is staged in LDS. With S > 1, slice sums meet in LDS and are
// added in slice order, so results do not depend on timing.
template <int WT, int NR, int U>
struct ChunkBatch {
    uint4 w[U][NR];
};

struct MvLayout {
    int64_t K, n_out, up_rows;
    int upb;         // units per block
    int log_s;       // K slices per unit = 1 << log_s
    int cps;         // chunks per slice
    int ipw;         // items per wave
};

// Position in a block's stream of (unit, slice) items, chunk by chunk.
// Advanced incrementally: no division on the hot path. Wave-uniform.
struct Cursor {
    int item;
    int within;
};

__device__ inline void advance(Cursor& c, int cps)
{
    if (++c.within == cps) {
        c.within = 0;
        ++c.item;
    }
}

template <int WT, int NR, int U>
__device__ inline void fetch(const void* W, const MvLayout& L, int64_t unit0, Cursor& c,
                             int item_end, int lane, ChunkBatch<WT, NR, U>& b)
{
    constexpr int E = Epl<WT>::v;
    constexpr int64_t CH = int64_t(WAVE) * E;
    const int smask = (1 << L.log_s) - 1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t unit = unit0 + (c.item >> L.log_s);
        const int64_t k = (int64_t((c.item & smask) * L.cps + c.within)) * CH + int64_t(lane) * E;
        const bool ok = c.item < item_end && unit < L.n_out && k < L.K;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int64_t row = unit + (r == 1 ? L.up_rows : 0);
            b.w[u][r] = ok ? load_w<WT>(W, row * L.K + k) : make_uint4(0u, 0u, 0u, 0u);
        }
        advance(c, L.cps);
    }
}

template <int WT, int MODE, bool NORM>
__global__ void __launch_bounds__(512)
matvec_kernel(const void* __restrict__ W, const uint16_t* __restrict__ scales, MvLayout L,
              const float* __restrict__ x, const float* __restrict__ norm_w, float eps,
              float* __restrict__ out)
{
    constexpr int NR = (MODE == MV_SWIGLU) ? 2 : 1;
    constexpr int U = (WT == W_F32) ? 8 : (NR == 1 ? 8 : 4);
    extern __shared__ float hs[];  // K floats, then NR * upb * S slice sums
    __shared__ float red[16];
    constexpr int E = Epl<WT>::v;
    constexpr int64_t CH = int64_t(WAVE) * E;
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nwaves = blockDim.x >> 6;
    const int64_t unit0 = int64_t(blockIdx.x) * L.upb;
    const int S = 1 << L.log_s;
    const int item_begin = wave * L.ipw;
    const int item_end = min(item_begin + L.ipw, L.upb * S);
    const int n_chunks = (item_end > item_begin ? item_end - item_begin : 0) * L.cps;
    float* part = hs + L.K;

    Cursor fc{item_begin, 0};  // next chunk to fetch
    Cursor uc{item_begin, 0};  // next chunk to use
    ChunkBatch<WT, NR, U> cur;
    if (n_chunks > 0) fetch<WT, NR, U>(W, L, unit0, fc, item_end, lane, cur);

    // Stage the activation (times the norm weight) in LDS; K % 4 == 0.
    float ss = 0.f;
    for (int64_t k = int64_t(tid) * 4; k < L.K; k += int64_t(blockDim.x) * 4) {
        float4 v = *reinterpret_cast<const float4*>(x + k);
        if constexpr (NORM) {
            ss = fmaf(v.x, v.x, ss);
            ss = fmaf(v.y, v.y, ss);
            ss = fmaf(v.z, v.z, ss);
            ss = fmaf(v.w, v.w, ss);
            const float4 w = *reinterpret_cast<const float4*>(norm_w + k);
            v.x *= w.x; v.y *= w.y; v.z *= w.z; v.w *= w.w;
        }
        *reinterpret_cast<float4*>(hs + k) = v;
    }
    float r = 1.f;
    if constexpr (NORM) {
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        float tot = 0.f;
        for (int i = 0; i < nwaves; ++i) tot += red[i];
        r = 1.0f / sqrtf(tot / static_cast<float>(L.K) + eps);
    } else {
        __syncthreads();
    }

    auto finish = [&](int64_t unit, float (&acc)[NR]) {
        if constexpr (MODE == MV_SWIGLU) {
            const float g = acc[0] * r;
            const float u = acc[1] * r;
            out[unit] = (g / (1.0f + expf(-g))) * u;
        } else if constexpr (MODE == MV_RESID) {
            out[unit] += acc[0] * r;
        } else {
            out[unit] = acc[0] * r;
        }
    };

    float acc[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) acc[i] = 0.f;
    const int smask = S - 1;
    for (int q = 0; q < n_chunks; q += U) {
        ChunkBatch<WT, NR, U> nxt;
        const bool more = q + U < n_chunks;
        if (more) fetch<WT, NR, U>(W, L, unit0, fc, item_end, lane, nxt);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (uc.item >= item_end) break;
            const int64_t unit = unit0 + (uc.item >> L.log_s);
            if (unit >= L.n_out) break;
            const int64_t k = (int64_t((uc.item & smask) * L.cps + uc.within)) * CH +
                              int64_t(lane) * E;
            if (k < L.K) {
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    const uint16_t* srow = nullptr;
                    if constexpr (WT == W_Q8)
                        srow = scales + (unit + (i == 1 ? L.up_rows : 0)) * (L.K >> 5);
                    acc[i] += lane_dot<WT>(cur.w[u][i], hs, k, srow);
                }
            }
            if (uc.within == L.cps - 1) {
#pragma unroll
                for (int i = 0; i < NR; ++i) acc[i] = wave_sum(acc[i]);
                if (lane == 0) {
                    if (S == 1) {
                        finish(unit, acc);
                    } else {
#pragma unroll
                        for (int i = 0; i < NR; ++i) part[uc.item * NR + i] = acc[i];
                    }
                }
#pragma unroll
                for (int i = 0; i < NR; ++i) acc[i] = 0.f;
            }
            advance(uc, L.cps);
        }
        if (more) cur = nxt;
    }
    if (S > 1) {
        __syncthreads();
        for (int j = tid; j < L.upb; j += blockDim.x) {
            const int64_t unit = unit0 + j;
            if (unit >= L.n_out) break;
            float sum[NR];
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                sum[i] = 0.f;
                for (int s2 = 0; s2 < S; ++s2) sum[i] += part[(j * S + s2) * NR + i];
            }
            finish(unit, sum);
        }
    }
}

template <int WT, int MODE, bool NORM>
hipError_t launch_mv_t(const Weight& W, const float* x, const float* nw,
                       float eps, int64_t n_out, int64_t up_rows, float* out,
                       hipStream_t s)
{
    constexpr int E = Epl<WT>::v;
    const int threads = 512;
    const int nwaves = threads / WAVE;
    MvLayout L;
    L.K = W.cols;
    L.n_out = n_out;
    L.up_rows = up_rows;
    const int64_t CH = int64_t(WAVE) * E;
    const int64_t nchunks = (L.K + CH - 1) / CH;
    const int64_t max_blocks = 512;  // two 8-wave blocks per CU, all resident
    const int64_t upb = (n_out + max_blocks - 1) / max_blocks;
    L.upb = int(upb);
    const int64_t blocks = (n_out + upb - 1) / upb;
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
    const int NR = MODE == MV_SWIGLU ? 2 : 1;
    const size_t lds = size_t(L.K) * sizeof(float) +
                       (S > 1 ? size_t(upb * S * NR) * sizeof(float) : 0);
    DFK_LAUNCH((matvec_kernel<WT, MODE, NORM>), dim3(unsigned(blocks)),
                       dim3(threads), lds, s, W.data, W.scales, L, x, nw, eps, out);
    return hipGetLastError();
}

template <int WT>
hipError_t launch_mv_w(const Weight& W, int mode, const float* x,
                       const float* nw, float eps, int64_t n_out,
                       int64_t up_rows, float* out, hipStream_t s)
{
    const bool norm = nw != nullptr;
    switch (mode) {
    case MV_STORE:
        return norm ? launch_mv_t<WT, MV_STORE, true>(W, x, nw, eps, n_out, up_rows, out, s)
                    : launch_mv_t<WT, MV_STORE, false>(W, x, nw, eps, n_out, up_rows, out, s);
    case MV_RESID:
        return norm ? launch_mv_t<WT, MV_RESID, true>(W, x, nw, eps, n_out, up_rows, out, s)
                    : launch_mv_t<WT, MV_RESID, false>(W, x, nw, eps, n_out, up_rows, out, s);
    case MV_SWIGLU:
        return norm ? launch_mv_t<WT, MV_SWIGLU, true>(W, x, nw, eps, n_out, up_rows, out, s)
                    : launch_mv_t<WT, MV_SWIGLU, false>(W, x, nw, eps, n_out, up_rows, out, s);
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
                             float* __restrict__ x)
{
    const int row = blockIdx.x;
    const int t = tokens ? tokens[row] : *state_tok;
    for (int64_t i = threadIdx.x; i < d; i += blockDim.x) {
        float v;
        if constexpr (WT == W_F32) v = static_cast<const float*>(E)[int64_t(t) * d + i];
        else v = f16_bits_to_f32(static_cast<const uint16_t*>(E)[int64_t(t) * d + i]);
        x[int64_t(row) * d + i] = v;
    }
}

// ---------------------------------------------------------------------------
// Decode attention (split-K "flash decoding") for one KV head g.
//
// The positions 0..p are cut into tiles of ATTN_T rows; work-group `split`
// takes a contiguous run of tiles (the same partition for every launch shape,
// so results are bitwise reproducible). Prologue: the group's query heads
// (and, in the work-group that owns position p, this head's new key) get
// norm_heads (qwen3) and RoPE at p from the cos/sin table; the owner appends
// k and v at slot p. Each row of K / V is read by 16 lanes (a 512-byte
// coalesced row for head_dim 128) straight into registers; the 16 lanes
// reduce a row's dot products with four shuffles. Softmax runs online across
// tiles in f32. Work-groups write (max, sum, acc) partials; the last one of a
// head to finish (atomic ticket) merges them in split order.
// ---------------------------------------------------------------------------
template <int N>
__device__ inline void load_slice(const float* p, float (&v)[N])
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 x = load16f_nt(p + i);
            v[i] = x.x; v[i + 1] = x.y; v[i + 2] = x.z; v[i + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = p[i];
    }
}

template <int HD, int G>
__global__ void __launch_bounds__(256)
attn_decode_kernel(AttnDecodeArgs a)
{
    constexpr int T = ATTN_T;          // rows per tile
    constexpr int LPR = 16;            // lanes per row
    constexpr int DPL = HD / LPR;      // dims per lane
    constexpr int RPI = WAVE / LPR;    // rows per wave per iteration
    constexpr int ITER = T / (4 * RPI);
    constexpr int HALF = HD / 2;
    __shared__ float qs[G][HD];
    __shared__ float knew[HD];
    __shared__ float vnew[HD];
    __shared__ float sc[G][T];
    __shared__ float s_m[G], s_l[G], s_resc[G];
    __shared__ float red[4 * (WAVE / 16)][G][HD];

    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wave = tid >> 6;
    const int p = *a.state_pos;
    const int n_pos = p + 1;
    const int tiles = (n_pos + T - 1) / T;
    const int tpw = (tiles + ATTN_MAX_SPLIT - 1) / ATTN_MAX_SPLIT;  // tiles per work-group
    const int n_active = (tiles + tpw - 1) / tpw;
    if (split >= n_active) return;
    const int tile0 = split * tpw;
    const int tile1 = min(tiles, tile0 + tpw);
    const bool owner = (split == n_active - 1);
    const int qd = a.n_heads * HD;
    const int kvd = a.n_kv * HD;
    const int64_t head_base = int64_t(g) * a.max_ctx * HD;
    const float* kbase = a.kc + head_base;
    const float* vbase = a.vc + head_base;
    const int rg = lane / LPR;          // row within the wave's group of RPI rows
    const int ds = (lane % LPR) * DPL;  // first dim of this lane's slice

    // K and V rows of the first tile: issued before anything else so that
    // their latency covers the q prologue. Row p (the new one) is filled in
    // from LDS once the owner has computed it.
    float kr[ITER][DPL], vr[ITER][DPL];
    auto load_tile = [&](int tile) {
        const int t0 = tile * T;
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int t = t0 + wave * (T / 4) + it * RPI + rg;
            if (t < p) {
                load_slice<DPL>(kbase + int64_t(t) * HD + ds, kr[it]);
                load_slice<DPL>(vbase + int64_t(t) * HD + ds, vr[it]);
            } else {
#pragma unroll
                for (int d = 0; d < DPL; ++d) { kr[it][d] = 0.f; vr[it][d] = 0.f; }
            }
        }
    };
    load_tile(tile0);

    // Raw q of the group's heads (and the new k, v for the owner) into LDS.
    for (int i = tid; i < G * HD; i += 256)
        qs[i / HD][i % HD] = a.qkv[int64_t(g) * G * HD + i];
    if (owner) {
        for (int i = tid; i < HD; i += 256) {
            knew[i] = a.qkv[qd + g * HD + i];
            vnew[i] = a.qkv[qd + kvd + g * HD + i];
        }
    }
    if (tid < G) { s_m[tid] = -INFINITY; s_l[tid] = 0.f; }
    __syncthreads();

    // norm_heads (qwen3): RMSNorm of each head with the shared weight.
    if (a.q_norm) {
        const int nvec = G + (owner ? 1 : 0);
        for (int j = wave; j < nvec; j += 4) {
            float* v = (j < G) ? qs[j] : knew;
            const float* w = (j < G) ? a.q_norm : a.k_norm;
            float ss = 0.f;
            for (int i = lane; i < HD; i += WAVE) ss = fmaf(v[i], v[i], ss);
            ss = wave_sum(ss);
            const float r = 1.0f / sqrtf(ss / static_cast<float>(HD) + a.eps);
            for (int i = lane; i < HD; i += WAVE) v[i] = w[i] * (v[i] * r);
        }
        __syncthreads();
    }

    // RoPE at position p: pair (i, i + HD/2) -> (a c - b s, a s + b c).
    {
        const float* cosr = a.cos_t + int64_t(p) * HALF;
        const float* sinr = a.sin_t + int64_t(p) * HALF;
        const int nvec = G + (owner ? 1 : 0);
        for (int i = tid; i < nvec * HALF; i += 256) {
            const int j = i / HALF;
            const int k = i % HALF;
            float* v = (j < G) ? qs[j] : knew;
            const float x0 = v[k], x1 = v[k + HALF];
            const float cs = cosr[k], sn = sinr[k];
            v[k] = fmaf(x0, cs, -x1 * sn);
            v[k + HALF] = fmaf(x0, sn, x1 * cs);
        }
        __syncthreads();
    }

    // Append k (after RoPE) and v at slot p.
    if (owner) {
        for (int i = tid; i < HD; i += 256) {
            a.kc[head_base + int64_t(p) * HD + i] = knew[i];
            a.vc[head_base + int64_t(p) * HD + i] = vnew[i];
        }
    }

    float q[G][DPL];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int d = 0; d < DPL; ++d) q[j][d] = qs[j][ds + d];
    float acc[G][DPL];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[j][d] = 0.f;
    const float scale = 1.0f / sqrtf(static_cast<float>(HD));

    for (int tile = tile0; tile < tile1; ++tile) {
        const int t0 = tile * T;
        if (tile != tile0) load_tile(tile);
        // The new row p, if it falls in this tile, comes from LDS.
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int t = t0 + wave * (T / 4) + it * RPI + rg;
            if (t == p) {
#pragma unroll
                for (int d = 0; d < DPL; ++d) { kr[it][d] = knew[ds + d]; vr[it][d] = vnew[ds + d]; }
            }
        }
        // Scores of this wave's rows, reduced over the 16 lanes of a row.
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int row = wave * (T / 4) + it * RPI + rg;
            const bool valid = t0 + row < n_pos;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float s = 0.f;
#pragma unroll
                for (int d = 0; d < DPL; ++d) s = fmaf(q[j][d], kr[it][d], s);
                s = row16_sum(s);
                if ((lane % LPR) == 0) sc[j][row] = valid ? s * scale : -INFINITY;
            }
        }
        __syncthreads();
        // Online softmax: tile maximum, probabilities, rescale of the past.
        for (int j = wave; j < G; j += 4) {
            const float s = sc[j][lane];
            const float mt = wave_max(s);
            const float mo = s_m[j];
            const float mn = fmaxf(mo, mt);
            const float pr = (s == -INFINITY) ? 0.f : expf(s - mn);
            const float lt = wave_sum(pr);
            sc[j][lane] = pr;
            if (lane == 0) {
                const float resc = (mo == -INFINITY) ? 0.f : expf(mo - mn);
                s_resc[j] = resc;
                s_l[j] = s_l[j] * resc + lt;
                s_m[j] = mn;
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float resc = s_resc[j];
#pragma unroll
            for (int d = 0; d < DPL; ++d) acc[j][d] *= resc;
        }
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int row = wave * (T / 4) + it * RPI + rg;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float pr = sc[j][row];
#pragma unroll
                for (int d = 0; d < DPL; ++d) acc[j][d] = fmaf(pr, vr[it][d], acc[j][d]);
            }
        }
        __syncthreads();
    }

    // Sum the 16 row groups (4 per wave, 4 waves) through LDS, fixed order.
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int d = 0; d < DPL; ++d) red[wave * RPI + rg][j][ds + d] = acc[j][d];
    __syncthreads();
    auto red_sum = [&](int j, int d) {
        float v = 0.f;
#pragma unroll
        for (int r2 = 0; r2 < 4 * RPI; ++r2) v += red[r2][j][d];
        return v;
    };

    const int hq0 = g * G;
    if (n_active == 1) {
        for (int i = tid; i < G * HD; i += 256) {
            const int j = i / HD, d = i % HD;
            a.out[int64_t(hq0 + j) * HD + d] = red_sum(j, d) / s_l[j];
        }
        return;
    }
    float* part = a.part + (int64_t(g) * ATTN_MAX_SPLIT + split) * G * (HD + 2);
    for (int i = tid; i < G * HD; i += 256) {
        const int j = i / HD, d = i % HD;
        part[j * (HD + 2) + d] = red_sum(j, d);
    }
    if (tid < G) {
        part[tid * (HD + 2) + HD] = s_m[tid];
        part[tid * (HD + 2) + HD + 1] = s_l[tid];
    }
}

// Merge of the split partials of one query head (launched after the split
// kernel, so its stores are visible): weights exp(m_c - M), total sum, and
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
    const int tiles = (p + 1 + T - 1) / T;
    const int tpw = (tiles + ATTN_MAX_SPLIT - 1) / ATTN_MAX_SPLIT;
    const int n_active = (tiles + tpw - 1) / tpw;
    if (n_active == 1) return;  // the split kernel wrote the output itself
    const int64_t cs = int64_t(G) * (HD + 2);
    const float* pg = a.part + int64_t(g) * ATTN_MAX_SPLIT * cs + int64_t(j) * (HD + 2);
    for (int c = tid; c < n_active; c += blockDim.x) {
        w[c] = pg[c * cs + HD];
        lsum[c] = pg[c * cs + HD + 1];
    }
    __syncthreads();
    if (tid < WAVE) {
        float M = -INFINITY;
        for (int c = tid; c < n_active; c += WAVE) M = fmaxf(M, w[c]);
        M = wave_max(M);
        float L = 0.f;
        for (int c = tid; c < n_active; c += WAVE) {
            const float e = expf(w[c] - M);
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
            x[b2] = c < n_active ? pg[c * cs + d] : 0.f;
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

hipError_t launch_matvec(const Weight& W, int mode, const float* x,
                         const float* norm_w, float eps, int64_t n_out,
                         int64_t up_rows, float* out, hipStream_t s)
{
    if (n_out <= 0) return hipSuccess;
    switch (W.dtype) {
    case W_F32: return launch_mv_w<W_F32>(W, mode, x, norm_w, eps, n_out, up_rows, out, s);
    case W_F16: return launch_mv_w<W_F16>(W, mode, x, norm_w, eps, n_out, up_rows, out, s);
    case W_Q8: return launch_mv_w<W_Q8>(W, mode, x, norm_w, eps, n_out, up_rows, out, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_embed(const Weight& E, const int* tokens_dev,
                        const int* state_tok, int n_rows, float* x,
                        hipStream_t s)
{
    if (E.dtype == W_F32)
        DFK_LAUNCH(embed_kernel<W_F32>, dim3(n_rows), dim3(256), 0, s,
                           E.data, E.cols, tokens_dev, state_tok, x);
    else
        DFK_LAUNCH(embed_kernel<W_F16>, dim3(n_rows), dim3(256), 0, s,
                           E.data, E.cols, tokens_dev, state_tok, x);
    return hipGetLastError();
}

template <int HD>
hipError_t launch_attn_hd(const AttnDecodeArgs& a, dim3 grid, hipStream_t s)
{
    switch (a.n_heads / a.n_kv) {
    case 1: DFK_LAUNCH((attn_decode_kernel<HD, 1>), grid, dim3(256), 0, s, a); break;
    case 2: DFK_LAUNCH((attn_decode_kernel<HD, 2>), grid, dim3(256), 0, s, a); break;
    case 4: DFK_LAUNCH((attn_decode_kernel<HD, 4>), grid, dim3(256), 0, s, a); break;
    case 8: DFK_LAUNCH((attn_decode_kernel<HD, 8>), grid, dim3(256), 0, s, a); break;
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
    default: return hipErrorInvalidValue;
    }
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
