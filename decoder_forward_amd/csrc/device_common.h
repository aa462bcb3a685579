// device_common.h — device-side building blocks of the decode kernels: 16-byte
// streaming loads, hand-off between work-groups of one kernel, DPP
// reductions, and the per-lane dot product of a weight vector.
#pragma once

#include "kernels.h"

namespace dfk {
namespace dev {

constexpr int WAVE = 64;

// Global address space. Pointers the compiler cannot place are generic:
// accesses through them become flat instructions, which also count against
// the LDS wait counter, so every LDS access would wait for all loads in
// flight. Casting to the global address space gives global instructions.
#define DFK_GLOBAL __attribute__((address_space(1)))

template <class T>
__device__ inline DFK_GLOBAL T* gmem(T* p)
{
    return (DFK_GLOBAL T*)(p);
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads marked non-temporal: streamed data is read once.
__device__ inline uint4 load16_nt(const void* p)
{
    const u32x4 v = __builtin_nontemporal_load(gmem(static_cast<const u32x4*>(p)));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline float4 load16f_nt(const float* p)
{
    const f32x4 v = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4*>(p)));
    return make_float4(v.x, v.y, v.z, v.w);
}

// Plain 16-byte load of 4 floats from global memory.
__device__ inline float4 load4f(const float* p)
{
    const f32x4 v = *gmem(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ inline float f16_bits_to_f32(uint16_t b)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// f16 bits of v, rounded to nearest even.
__device__ inline uint16_t f32_to_f16_bits(float v) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v)); }

// 2^x on the hardware exponential (v_exp_f32); softmax weights only, where
// results below the normal range may flush to zero.
__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }


// Cross-work-group hand-off without cache-wide fences. Values another
// work-group will read are stored with relaxed agent-scope atomics (written
// through to the coherence point, bypassing the per-XCD L2), every wave waits
// for its stores to be acknowledged before the block takes its ticket, and
// the reader loads with relaxed agent-scope atomics (bypassing stale L2
// lines). A device-scope fence would instead write back and invalidate the
// whole L2 of the XCD once per work-group.
__device__ inline void st_shared_f(float* p, float v)
{
    __hip_atomic_store(gmem(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_shared_i(int* p, int v)
{
    __hip_atomic_store(gmem(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_shared_f(const float* p)
{
    return __hip_atomic_load(gmem(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int ld_shared_i(const int* p)
{
    return __hip_atomic_load(gmem(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        const int prev = __hip_atomic_fetch_add(gmem(counter), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == n - 1;
        if (last) __hip_atomic_store(gmem(counter), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// The activation a matvec stages in LDS is stored lane-permuted: within
// each chunk of 64 * E values (E = Epl, one 16-byte weight load per lane),
// value j of lane l's E sits at (j / 4) * 256 + 4 l + j % 4. A lane then
// reads its E activations as E / 4 float4 at a 16-byte stride across the
// wave: every LDS read instruction is free of bank conflicts (consecutive
// 32-byte slices per lane would put four lanes of each 16 on the same
// banks). The staged region is padded to whole chunks.
template <int WT>
__device__ inline int64_t lds_pos(int64_t k)
{
    constexpr int E = Epl<WT>::v;
    constexpr int64_t CH = int64_t(WAVE) * E;
    const int64_t c = k / CH, w = k - c * CH;
    const int64_t l = w / E, j = w - l * E;
    return c * CH + (j >> 2) * 256 + l * 4 + (j & 3);
}

// Floats of LDS the staged activation of width K takes (whole chunks).
__host__ __device__ inline int64_t mv_staged_floats(int wdtype, int64_t K)
{
    const int64_t CH = int64_t(64) * (wdtype == W_F32 ? 4 : wdtype == W_F16 ? 8 : 16);
    return (K + CH - 1) / CH * CH;
}

// dot of a lane's 16-byte weight vector with its activations: hl points at
// the lane's first float4 in the permuted layout (chunk start + 4 lane); the
// others follow 256 floats apart.
template <int WT>
__device__ inline float lane_dot(uint4 w, const float* hl, uint16_t scale_bits)
{
    if constexpr (WT == W_F32) {
        const float4 h = *reinterpret_cast<const float4*>(hl);
        float a = __uint_as_float(w.x) * h.x;
        a = fmaf(__uint_as_float(w.y), h.y, a);
        a = fmaf(__uint_as_float(w.z), h.z, a);
        return fmaf(__uint_as_float(w.w), h.w, a);
    } else if constexpr (WT == W_F16) {
        const half8 hw = __builtin_bit_cast(half8, w);
        const float4 h0 = *reinterpret_cast<const float4*>(hl);
        const float4 h1 = *reinterpret_cast<const float4*>(hl + 256);
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
            const float4 h = *reinterpret_cast<const float4*>(hl + 256 * j);
            const uint32_t v = ww[j];
            a = fmaf(static_cast<float>(static_cast<int8_t>(v & 0xff)), h.x, a);
            b = fmaf(static_cast<float>(static_cast<int8_t>((v >> 8) & 0xff)), h.y, b);
            a = fmaf(static_cast<float>(static_cast<int8_t>((v >> 16) & 0xff)), h.z, a);
            b = fmaf(static_cast<float>(static_cast<int8_t>(v >> 24)), h.w, b);
        }
        return f16_bits_to_f32(scale_bits) * (a + b);
    }
}


// ---------------------------------------------------------------------------
// Decode matvec: out = epilogue(r * W (x . w)).
//
// Work layout (MvLayout, computed on the host by make_mv_layout). A block
// owns `upb` consecutive output units (a row; a gate row with its up row; or
// rows n and n + up_rows of an even row count, whose weights of one column
// share the lane's activation value) and splits each unit's K range into S equal slices of whole 64-lane chunks
// so that its 8 waves get equal numbers of (unit, slice) items: no straggler
// waves. Each wave walks its items as one stream of chunks, U chunks per
// batch, and issues the loads of batch i+1 before it consumes batch i. The
// first batch is issued by mv_begin, before the activation is staged. The
// (unit, slice) sums meet in LDS and are added in slice order after the
// streaming loop, so results do not depend on timing.
// ---------------------------------------------------------------------------
template <int WT, int NR, int U>
struct ChunkBatch {
    uint4 w[U][NR];
    uint16_t s[WT == W_Q8 ? U : 1][NR];  // 8-bit blocks: the chunk's block scale (f16 bits)
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
__device__ inline void fetch(const void* W, const uint16_t* scales, const MvLayout L, int64_t unit0,
                             Cursor& c, int item_end, int lane, ChunkBatch<WT, NR, U>& b)
{
    constexpr int E = Epl<WT>::v;
    constexpr int64_t CH = int64_t(WAVE) * E;
    const int smask = (1 << L.log_s) - 1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // the chunk's unit and row offsets are wave-uniform (scalar); only
        // the lane's K offset (32-bit: K < 2^31) is per lane
        const int k = ((c.item & smask) * L.cps + c.within) * int(CH) + lane * E;
        const int64_t unit = unit0 + (c.item >> L.log_s);
        // Chunks past the end are loaded from the start of W (a valid
        // address) and never consumed; lanes past K load from their row's
        // start. The loads stay unconditional, so the wait before consuming
        // a batch can leave the next batch in flight (a branch around each
        // load makes the compiler wait for all).
        const bool ok = c.item < item_end && unit < L.n_out;  // uniform
        const int kl = (ok && k < int(L.K)) ? k : 0;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int64_t row = unit + (r == 1 ? L.up_rows : 0);
            b.w[u][r] = load_w<WT>(W, (ok ? row * L.K : 0) + kl);
            // the scale travels with its weights, so that no dependent load
            // is left for the consuming step
            if constexpr (WT == W_Q8) b.s[u][r] = *gmem(scales + (ok ? row * (L.K >> 5) : 0) + (kl >> 5));
        }
        advance(c, L.cps);
    }
}

template <int WT, int MODE>
struct MvState {
    static constexpr int NR = (MODE == MV_SWIGLU || MODE == MV_STORE2 || MODE == MV_RESID2) ? 2 : 1;
    static constexpr int U = (WT == W_F32) ? 8 : (NR == 1 ? 8 : 4);
    ChunkBatch<WT, NR, U> cur;
    Cursor fc, uc;
    int item_end;
    int n_chunks;
    int64_t unit0;
};

// Part 1: the block's item range and its first batch of weight loads.
template <int WT, int MODE>
__device__ inline void mv_begin(const void* W, const uint16_t* scales, const MvLayout L, int block,
                                MvState<WT, MODE>& st, int tid)
{
    const int lane = tid & (WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = 1 << L.log_s;
    const int item_begin = wave * L.ipw;
    st.unit0 = int64_t(block) * L.upb;
    st.item_end = min(item_begin + L.ipw, L.upb * S);
    st.n_chunks = (st.item_end > item_begin ? st.item_end - item_begin : 0) * L.cps;
    if (st.unit0 >= L.n_out) st.n_chunks = 0;
    st.fc = Cursor{item_begin, 0};
    st.uc = Cursor{item_begin, 0};
    if (st.n_chunks > 0) {
        fetch<WT, MvState<WT, MODE>::NR, MvState<WT, MODE>::U>(W, scales, L, st.unit0, st.fc, st.item_end,
                                                               lane, st.cur);
    } else {
        // Defined contents: an undefined batch lets the register allocator
        // merge it with other live ranges.
#pragma unroll
        for (int u = 0; u < MvState<WT, MODE>::U; ++u)
#pragma unroll
            for (int r = 0; r < MvState<WT, MODE>::NR; ++r) {
                st.cur.w[u][r] = make_uint4(0u, 0u, 0u, 0u);
                if constexpr (WT == W_Q8) st.cur.s[u][r] = 0;
            }
    }
}

// Part 2: stage x (times the norm weight, if NORM) in LDS (hs: the staged
// activation, then the slice sums), then consume the batches and write the
// epilogue selected by MODE (MV_SWIGLU: gate and up rows together;
// MV_STORE2 / MV_RESID2: rows n and n + up_rows together; the others one
// row).
template <int WT, int MODE, bool NORM>
__device__ inline void mv_finish(const uint16_t* scales, const void* W, const MvLayout L,
                                 MvState<WT, MODE>& st, const float* __restrict__ x,
                                 const float* __restrict__ norm_w, float eps,
                                 float* __restrict__ out, float* hs, float* red, int tid)
{
    constexpr int NR = MvState<WT, MODE>::NR;
    constexpr int U = MvState<WT, MODE>::U;
    constexpr int E = Epl<WT>::v;
    constexpr int64_t CH = int64_t(WAVE) * E;
    const int lane = tid & (WAVE - 1);
    const int wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int S = 1 << L.log_s;
    float* part = hs + mv_staged_floats(WT, L.K);

    // The residual value of this thread's first output unit, loaded now so
    // that its latency passes while the activation is staged and the weights
    // stream.
    float resid0 = 0.f, resid1 = 0.f;
    if constexpr (MODE == MV_RESID2) {
        if (tid < L.upb && st.unit0 + tid < L.n_out) {
            resid0 = *gmem(out + st.unit0 + tid);
            resid1 = *gmem(out + st.unit0 + tid + L.up_rows);
        }
    }

    float ss = 0.f;
    for (int k = tid * 4; k < L.K; k += blockDim.x * 4) {
        float4 v = load4f(x + k);
        if constexpr (NORM) {
            ss = fmaf(v.x, v.x, ss);
            ss = fmaf(v.y, v.y, ss);
            ss = fmaf(v.z, v.z, ss);
            ss = fmaf(v.w, v.w, ss);
            const float4 w = load4f(norm_w + k);
            v.x *= w.x; v.y *= w.y; v.z *= w.z; v.w *= w.w;
        }
        *reinterpret_cast<float4*>(hs + lds_pos<WT>(k)) = v;
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
            *gmem(out + unit) = gate_act(g, L.act) * u;
        } else if constexpr (MODE == MV_RESID2) {
            const bool own = unit == st.unit0 + tid;
            const float old0 = own ? resid0 : *gmem(out + unit);
            const float old1 = own ? resid1 : *gmem(out + unit + L.up_rows);
            *gmem(out + unit) = old0 + acc[0] * r;
            *gmem(out + unit + L.up_rows) = old1 + acc[1] * r;
        } else if constexpr (MODE == MV_STORE2) {
            *gmem(out + unit) = acc[0] * r;
            *gmem(out + unit + L.up_rows) = acc[1] * r;
        } else {
            *gmem(out + unit) = acc[0] * r;
        }
    };

    // Each (unit, slice) sum goes to LDS; the epilogues (global loads and
    // stores) run after the streaming loop, so that no wait inside the loop
    // covers anything but the batch being consumed.
    float acc[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) acc[i] = 0.f;
    const int smask = S - 1;
    auto consume = [&](const ChunkBatch<WT, NR, U>& cb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (st.uc.item >= st.item_end) break;
            const int64_t unit = st.unit0 + (st.uc.item >> L.log_s);
            if (unit >= L.n_out) break;
            // 32-bit: K < 2^31. A lane past K (only in a row's last chunk)
            // reads the staged region's padding (whole chunks are
            // allocated), and its product is dropped by a select rather than
            // a branch around the dot.
            const int k = ((st.uc.item & smask) * L.cps + st.uc.within) * int(CH) + lane * E;
            const bool kin = k < int(L.K);
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const float dv = lane_dot<WT>(cb.w[u][i], hs + (k - lane * (E - 4)), cb.s[WT == W_Q8 ? u : 0][i]);
                acc[i] += kin ? dv : 0.f;
            }
            if (st.uc.within == L.cps - 1) {
#pragma unroll
                for (int i = 0; i < NR; ++i) acc[i] = wave_sum(acc[i]);
                if (lane == 0) {
#pragma unroll
                    for (int i = 0; i < NR; ++i) part[st.uc.item * NR + i] = acc[i];
                }
#pragma unroll
                for (int i = 0; i < NR; ++i) acc[i] = 0.f;
            }
            advance(st.uc, L.cps);
        }
    };
    // Batch i+1 is in flight while batch i is consumed; the last batch is
    // consumed on its own (no fetch past the end). Two named buffers
    // alternate: copying one batch into the other would wait for its loads.
    ChunkBatch<WT, NR, U> nb;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r2 = 0; r2 < NR; ++r2) {  // defined (see mv_begin)
            nb.w[u][r2] = make_uint4(0u, 0u, 0u, 0u);
            if constexpr (WT == W_Q8) nb.s[u][r2] = 0;
        }
    for (int q = 0; q < st.n_chunks;) {
        if (q + U >= st.n_chunks) { consume(st.cur); break; }
        fetch<WT, NR, U>(W, scales, L, st.unit0, st.fc, st.item_end, lane, nb);
        consume(st.cur);
        q += U;
        if (q + U >= st.n_chunks) { consume(nb); break; }
        fetch<WT, NR, U>(W, scales, L, st.unit0, st.fc, st.item_end, lane, st.cur);
        consume(nb);
        q += U;
    }
    __syncthreads();
    for (int j = tid; j < L.upb; j += blockDim.x) {
        const int64_t unit = st.unit0 + j;
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

}  // namespace dev
}  // namespace dfk
