// decode_persistent.hip — one decode step as one cooperative launch.
//
// The step list (page "Local inference and architectures", "The format")
// runs as a sequence of phases over a grid of one block per compute unit,
// all resident at once: embed; per layer [rms_norm + q/k/v matvec]
// [norm_heads + rope + KV append + split attention, the last split of a KV
// head to finish merging the head's splits] [o matvec + add] [rms_norm +
// gate/up matvec + silu * up] [down matvec + add]; then [rms_norm + logits
// matvec] [argmax]. Phases are separated by a grid barrier. Before a block
// waits at a barrier it issues the first weight loads of its next phase
// (weights do not depend on the barrier), so HBM keeps streaming while the
// grid synchronises, and the ramp of every separate launch disappears.
//
// Activations that one block writes and another reads within the launch go
// through write-through stores and loads that bypass the per-XCD L2
// (relaxed agent-scope atomics, 16-byte coherent buffer loads); weights and
// the KV cache rows of earlier positions use ordinary streaming loads.
//
// Every wait is bounded: a barrier that does not complete within its spin
// limit sets an error word, after which every block stops waiting and the
// launch ends; the host reports the error.
#include "attn_core.h"

#include <algorithm>

namespace dfk {
namespace {

using namespace dev;

constexpr int NT = STEP_THREADS;  // threads per block
constexpr int NWV = NT / 64;  // waves per block
constexpr unsigned SPIN_LIMIT = 1u << 22;
constexpr int MV_DEPTH = 1;         // matvec batch depth
constexpr unsigned ERR_POLL = 256;  // spins between reads of the error word

// ---------------------------------------------------------------------------
// Grid barrier on per-block flags. Barrier k of a launch publishes the value
// (epoch << 10) + k, where epoch = words[3] counts the launches so far: the
// block's thread 0 stores it in its own flag word (a write-through store,
// no read-modify-write on a shared address), and wave 0 then polls all nb
// flags, four per lane with one 16-byte L2-bypassing load, until every one
// has reached the value (signed difference, so a faster block already at
// barrier k + 1 counts). Values of earlier launches are smaller, so the
// flags need no reset. Callers make their stores complete (drain_memory in
// every thread) before the barrier; loads issued after the drain (the next
// phase's weights) stay in flight across it. words[2] is the error flag:
// a wait that runs out of spins sets it and every later wait gives up.
// ---------------------------------------------------------------------------
constexpr int MAX_BARRIERS = 1 << 10;  // per launch

__device__ inline void grid_sync(int* words, int* flags, int value)
{
    __syncthreads();
    if (threadIdx.x < WAVE) {
        const int lane = threadIdx.x;
        if (lane == 0) st_shared_i(flags + blockIdx.x, value);
        const int nb = gridDim.x;
        unsigned spins = 0;
        for (;;) {
            bool done = true;
            for (int i0 = 0; i0 < nb; i0 += 4 * WAVE) {
                const int i = i0 + 4 * lane;
                if (i < nb) {
                    const float4 f4 = coh_load4(reinterpret_cast<const float*>(flags), i);
                    const int f[4] = {__float_as_int(f4.x), __float_as_int(f4.y), __float_as_int(f4.z),
                                      __float_as_int(f4.w)};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (i + j < nb && int(unsigned(f[j]) - unsigned(value)) < 0) done = false;
                }
            }
            if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
            __builtin_amdgcn_s_sleep(1);
            if (++spins % ERR_POLL == 0 && (spins >= SPIN_LIMIT || ld_shared_i(words + 2) != 0)) {
                if (lane == 0) st_shared_i(words + 2, 1);
                break;
            }
        }
    }
    __syncthreads();
}

// Block 0 counts the launch once every block has passed a barrier (so has
// read the epoch at its start).
__device__ inline void grid_exit(int* words, int epoch)
{
    drain_memory();
    if (blockIdx.x == 0 && threadIdx.x == 0) st_shared_i(words + 3, int(unsigned(epoch) + 1u));
}

// The value of x, hidden from the optimiser: per-lane values a phase derives
// from it cannot be hoisted out of the layer loop and kept live across the
// other phases.
__device__ inline int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

__device__ inline bool am_better(float v, int i, float bv, int bi)
{
    return v > bv || (v == bv && i < bi);
}

// Block-wide argmax of per-thread candidates (lowest index on ties).
__device__ inline void am_block(float& bv, int& bi, float* sv, int* si)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (am_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) { sv[wv] = bv; si[wv] = bi; }
    __syncthreads();
    bv = -INFINITY;
    bi = 0x7fffffff;
    for (int k = 0; k < NWV; ++k)
        if (am_better(sv[k], si[k], bv, bi)) { bv = sv[k]; bi = si[k]; }
    __syncthreads();
}

// The step description lives in device memory and is read through a
// constant-space pointer (scalar loads). Each phase re-reads the fields it
// needs through a pointer the optimiser cannot see through, so that the
// uniform values of all phases are not loaded at entry and kept live.
__device__ inline const DFK_CONST StepArgs* fresh(const StepArgs* p)
{
    const DFK_CONST StepArgs* q = (const DFK_CONST StepArgs*)(p);
    asm volatile("" : "+s"(q));
    return q;
}

__device__ inline MvLayout mv_layout(const DFK_CONST MvLayout& m)
{
    MvLayout L;
    L.K = m.K;
    L.n_out = m.n_out;
    L.up_rows = m.up_rows;
    L.upb = m.upb;
    L.log_s = m.log_s;
    L.cps = m.cps;
    L.ipw = m.ipw;
    return L;
}

__device__ inline const DFK_CONST StepLayer& layer_of(const DFK_CONST StepArgs& A, int l)
{
    return ((const DFK_CONST StepLayer*)(A.layers))[l];
}

template <int WT, int WO, int HD, int G>
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(4)))
decode_step_kernel(const StepArgs* __restrict__ Ap, float* logits_out, int advance)
{
    extern __shared__ float lds[];
    __shared__ float red[16];
    __shared__ float sv[NWV];
    __shared__ int si[NWV];
    __shared__ int flag;
    const int b = blockIdx.x;
    const int nb = gridDim.x;
    const int tid = threadIdx.x;
    const int epoch = ld_shared_i(fresh(Ap)->bar + 3);
    int n_bar = 0;
    auto sync = [&]() {
        grid_sync(fresh(Ap)->bar, fresh(Ap)->bar_flags, int(unsigned(epoch) * MAX_BARRIERS + unsigned(++n_bar)));
    };
    const int p = gmem(fresh(Ap)->st)->pos;
    const int tok = gmem(fresh(Ap)->st)->tok;

    // embed: x = E[tok], a slice per block.
    {
        const DFK_CONST StepArgs& A = *fresh(Ap);
        const int per = (A.d + nb - 1) / nb;
        for (int i = b * per + tid; i < min(A.d, (b + 1) * per); i += NT) {
            const float v = A.embd_dtype == W_F32
                                ? *gmem(static_cast<const float*>(A.embd) + int64_t(tok) * A.d + i)
                                : f16_bits_to_f32(*gmem(static_cast<const uint16_t*>(A.embd) + int64_t(tok) * A.d + i));
            st_shared_f(A.x + i, v);
        }
        drain_memory();
    }
    // attention partition over (KV head, split) items: at most one per block
    const int n_kv = Ap->n_kv;
    const int n_layers = Ap->n_layers;
    const int n_pos = p + 1;
    const int tiles = (n_pos + ATTN_T - 1) / ATTN_T;
    const int want = max(1, nb / n_kv);
    const int n_splits_max = min(tiles, min(want, Ap->max_splits));
    const int tpw = (tiles + n_splits_max - 1) / n_splits_max;
    const int n_splits = (tiles + tpw - 1) / tpw;
    const int n_items = n_kv * n_splits;

    // Every phase drains its stores, issues its successor's first weight
    // loads, then waits at the barrier that publishes its output.
    for (int l = 0; l < n_layers; ++l) {
        {
            const DFK_CONST StepArgs& A = *fresh(Ap);
            const DFK_CONST StepLayer& Ly = layer_of(A, l);
            const int t = opaque(tid);
            MvState<WT, MV_STORE, MV_DEPTH> st;
            mv_begin<WT, MV_STORE>(Ly.wqkv, Ly.sqkv, mv_layout(A.mv_qkv), b, st, t);
            sync();
            mv_finish<WT, MV_STORE, true, true, MV_DEPTH, false>(Ly.sqkv, Ly.wqkv, mv_layout(A.mv_qkv), st, A.x,
                                                Ly.attn_norm, A.eps, A.qkv, lds, red, t);
            drain_memory();
        }
        sync();
        if (b < n_items) {
            const DFK_CONST StepArgs& A = *fresh(Ap);
            const DFK_CONST StepLayer& Ly = layer_of(A, l);
            const int t = opaque(tid);
            const int g = b / n_splits, split = b % n_splits;
            AttnItem it;
            it.qkv = A.qkv;
            it.q_norm = Ly.q_norm;
            it.k_norm = Ly.k_norm;
            it.bias = Ly.bias;
            it.eps = A.eps;
            it.adjacent = A.adjacent;
            it.cos_row = A.cos_t + int64_t(p) * (HD / 2);
            it.sin_row = A.sin_t + int64_t(p) * (HD / 2);
            it.kc = Ly.kc + int64_t(g) * A.max_ctx * HD;
            it.vc = Ly.vc + int64_t(g) * A.max_ctx * HD;
            it.qd = A.qd;
            it.kvd = A.kvd;
            it.g = g;
            it.p = p;
            it.pos0 = split * tpw * ATTN_T;
            it.pos1 = min(n_pos, (split + 1) * tpw * ATTN_T);
            it.out = n_splits == 1 ? A.att : nullptr;
            float* part_g = A.part + int64_t(g) * A.max_splits * attn_part_stride(G, HD);
            it.part = part_g + int64_t(split) * attn_part_stride(G, HD);
            attn_core<HD, G, NWV, 2, false, true>(it, lds, t);
            if (n_splits > 1 && last_to_arrive(A.attn_cnt + g, n_splits, &flag))
                attn_merge_group<HD, G, true>(part_g, n_splits, A.att + int64_t(g) * G * HD, lds, t, NT);
            drain_memory();
        }
        {
            const DFK_CONST StepArgs& A = *fresh(Ap);
            const DFK_CONST StepLayer& Ly = layer_of(A, l);
            const int t = opaque(tid);
            MvState<WT, MV_RESID, MV_DEPTH> st;
            mv_begin<WT, MV_RESID>(Ly.wo, Ly.so, mv_layout(A.mv_o), b, st, t);
            sync();
            mv_finish<WT, MV_RESID, false, true, MV_DEPTH, false>(Ly.so, Ly.wo, mv_layout(A.mv_o), st, A.att, nullptr,
                                                 A.eps, A.x, lds, red, t);
            drain_memory();
        }
        {
            const DFK_CONST StepArgs& A = *fresh(Ap);
            const DFK_CONST StepLayer& Ly = layer_of(A, l);
            const int t = opaque(tid);
            MvState<WT, MV_SWIGLU, MV_DEPTH> st;
            mv_begin<WT, MV_SWIGLU>(Ly.wgu, Ly.sgu, mv_layout(A.mv_gu), b, st, t);
            sync();
            mv_finish<WT, MV_SWIGLU, true, true, MV_DEPTH, false>(Ly.sgu, Ly.wgu, mv_layout(A.mv_gu), st, A.x,
                                                 Ly.ffn_norm, A.eps, A.mid, lds, red, t);
            drain_memory();
        }
        {
            const DFK_CONST StepArgs& A = *fresh(Ap);
            const DFK_CONST StepLayer& Ly = layer_of(A, l);
            const int t = opaque(tid);
            MvState<WT, MV_RESID, MV_DEPTH> st;
            mv_begin<WT, MV_RESID>(Ly.wd, Ly.sd, mv_layout(A.mv_down), b, st, t);
            sync();
            mv_finish<WT, MV_RESID, false, true, MV_DEPTH, false>(Ly.sd, Ly.wd, mv_layout(A.mv_down), st, A.mid,
                                                 nullptr, A.eps, A.x, lds, red, t);
            drain_memory();
        }
    }

    if (logits_out) {
        // logits = W_out rms_norm(x)
        {
            const DFK_CONST StepArgs& A = *fresh(Ap);
            const int t = opaque(tid);
            MvState<WO, MV_STORE, MV_DEPTH> st;
            mv_begin<WO, MV_STORE>(A.wout, A.sout, mv_layout(A.mv_logits), b, st, t);
            sync();
            mv_finish<WO, MV_STORE, true, true, MV_DEPTH, false>(A.sout, A.wout, mv_layout(A.mv_logits), st, A.x,
                                                A.out_norm, A.eps, logits_out, lds, red, t);
            drain_memory();
        }
        if (advance) {
            sync();
            // greedy token: per-block (max, lowest index), then block 0 merges.
            {
                const DFK_CONST StepArgs& A = *fresh(Ap);
                const int per = (A.V + nb - 1) / nb;
                const int lo = b * per, hi = min(A.V, lo + per);
                float bv = -INFINITY;
                int bi = 0x7fffffff;
                for (int i = lo + tid; i < hi; i += NT) {
                    const float v = ld_shared_f(logits_out + i);
                    if (am_better(v, i, bv, bi)) { bv = v; bi = i; }
                }
                am_block(bv, bi, sv, si);
                if (tid == 0) {
                    st_shared_f(A.amax_val + b, bv);
                    st_shared_i(A.amax_idx + b, bi);
                }
                drain_memory();
            }
            sync();
            if (b == 0) {
                const DFK_CONST StepArgs& A = *fresh(Ap);
                float bv = -INFINITY;
                int bi = 0x7fffffff;
                for (int k = tid; k < nb; k += NT) {
                    const float v = ld_shared_f(A.amax_val + k);
                    const int i = ld_shared_i(A.amax_idx + k);
                    if (am_better(v, i, bv, bi)) { bv = v; bi = i; }
                }
                am_block(bv, bi, sv, si);
                if (tid == 0) {
                    if (bi == 0x7fffffff) bi = 0;
                    DFK_GLOBAL DevState* st = gmem(A.st);
                    const int step = st->step;
                    *gmem(A.gen_out + step) = bi;
                    st->tok = bi;
                    st->pos = p + 1;
                    st->step = step + 1;
                }
            }
        }
    }
    grid_exit(fresh(Ap)->bar, epoch);
}

template <int WT, int WO, int HD, int G>
const void* step_kernel_ptr()
{
    return reinterpret_cast<const void*>(&decode_step_kernel<WT, WO, HD, G>);
}

const void* pick(int wdtype, int odtype, int hd, int G)
{
#define DF_PICK_G(WT, WO, HD)                                             \
    switch (G) {                                                          \
    case 1: return step_kernel_ptr<WT, WO, HD, 1>();                      \
    case 2: return step_kernel_ptr<WT, WO, HD, 2>();                      \
    case 3: return step_kernel_ptr<WT, WO, HD, 3>();                      \
    case 4: return step_kernel_ptr<WT, WO, HD, 4>();                      \
    case 5: return step_kernel_ptr<WT, WO, HD, 5>();                      \
    case 6: return step_kernel_ptr<WT, WO, HD, 6>();                      \
    case 7: return step_kernel_ptr<WT, WO, HD, 7>();                      \
    case 8: return step_kernel_ptr<WT, WO, HD, 8>();                      \
    }                                                                     \
    return nullptr;
#define DF_PICK_HD(WT, WO)                                                \
    if (hd == 64) { DF_PICK_G(WT, WO, 64) }                               \
    if (hd == 128) { DF_PICK_G(WT, WO, 128) }                             \
    return nullptr;
    if (wdtype == W_F16 && odtype == W_F16) { DF_PICK_HD(W_F16, W_F16) }
    if (wdtype == W_Q8 && odtype == W_Q8) { DF_PICK_HD(W_Q8, W_Q8) }
    if (wdtype == W_Q8 && odtype == W_F16) { DF_PICK_HD(W_Q8, W_F16) }
    return nullptr;
#undef DF_PICK_HD
#undef DF_PICK_G
}

}  // namespace

bool step_fits(const StepArgs& a, int wdtype, int odtype, size_t* lds)
{
    const int G = a.n_heads / a.n_kv;
    const void* k = pick(wdtype, odtype, a.hd, G);
    if (!k) return false;
    if (6 * a.n_layers + 4 >= MAX_BARRIERS) return false;  // barrier values of one launch
    size_t need = 0;
    need = std::max(need, mv_lds_bytes(a.mv_qkv, MV_STORE));
    need = std::max(need, mv_lds_bytes(a.mv_o, MV_RESID));
    need = std::max(need, mv_lds_bytes(a.mv_gu, MV_SWIGLU));
    need = std::max(need, mv_lds_bytes(a.mv_down, MV_RESID));
    need = std::max(need, mv_lds_bytes(a.mv_logits, MV_STORE));
    const size_t hd = size_t(a.hd);
    need = std::max(need, (G * hd + 2 * hd + NWV * G * hd + 2 * NWV * G) * sizeof(float));  // attn_core
    const size_t cols = size_t(G) * hd / 4, P = NT / cols;
    need = std::max(need, (size_t(2) * a.max_splits * G + 4 + P * cols * 4 + P * G) * sizeof(float));  // merge
    *lds = need;
    if (need > 65536 &&
        hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, int(need)) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, NT, need) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return per_cu >= 1;
}

hipError_t launch_decode_step(const StepArgs& a, const StepArgs* a_dev, float* logits, int advance,
                              int wdtype, int odtype, int blocks, size_t lds, hipStream_t s)
{
    const int G = a.n_heads / a.n_kv;
    const void* k = pick(wdtype, odtype, a.hd, G);
    if (!k) return hipErrorInvalidValue;
    void* args[] = {&a_dev, &logits, &advance};
    const LaunchTiming& t = launch_timing();
    if (t.start) {
        const hipError_t r = hipEventRecord(t.start, s);
        if (r != hipSuccess) return r;
    }
    const hipError_t r = hipLaunchCooperativeKernel(k, dim3(blocks), dim3(NT), args, unsigned(lds), s);
    if (r == hipSuccess && t.stop) return hipEventRecord(t.stop, s);
    return r;
}

}  // namespace dfk
