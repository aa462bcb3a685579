// attn_core.h — decode attention for one (KV head, row range) item, and the
// merge of the partial results of one KV head's items.
//
// Page "Local inference and architectures", "The format" (the attention
// step of the step list): for each query head j of KV head g,
//   s_t = q_j . k_t / sqrt(hd),  out_j = sum_t softmax(s)_t v_t
// over the cache rows t = 0 .. p, where row p is this step's k (after
// norm_heads and rope) and v, appended to the cache by the item that covers
// it. q and k get norm_heads (qwen3) and rope at position p first.
//
// Work layout. A block of NW waves walks its rows in sweeps of NW*4*ITER
// rows: wave w takes rows w*4*ITER .. w*4*ITER + 4*ITER - 1 of a sweep, 16
// lanes per row (4 rows per wave instruction, hd/16 dims per lane). For
// hd >= 64 a lane's dims are float4 groups 64 floats apart (lane l of the
// row holds dims 64c + 4l .. 64c + 4l + 3 for c = 0 .. hd/64 - 1), so each
// 16-byte load instruction covers whole contiguous 256-byte runs of a row:
// no cache line is requested by two instructions. Each wave keeps its own online
// softmax (running max m, running sum l, accumulator) across sweeps: no
// block-wide synchronisation inside the row loop. With DBUF the next sweep's
// rows are loaded while the current one is consumed (twice the registers).
// At the end the waves' states meet in LDS and are merged with weights
// exp(m_w - M) in wave order.
//
// The softmax runs in base 2: q is multiplied once by log2(e)/sqrt(hd), so
// a dot product is s_t * log2(e) and e^{s_t - M} = 2^{s'_t - M'} (one
// v_exp_f32 per weight); maxima M are kept in these base-2 units.
//
// Result: with `out` set (the item covers every row) the normalised output
// of the G heads; otherwise the partial (sum_t e^{s_t - M} v_t, M, sum_t
// e^{s_t - M}) per head, merged across items by the combine kernel.
#pragma once

#include "device_common.h"

namespace dfk {
namespace dev {

struct AttnItem {
    const float* qkv;      // this step's q (all heads) | k | v
    const float* q_norm;   // norm_heads weights (qwen3), null for llama
    const float* k_norm;
    const float* bias;     // qwen2's q | k | v bias, laid out as qkv; else null
    float eps;
    int adjacent;          // rope pairs (2i, 2i+1) if set, else (i, i + hd/2)
    const float* cos_row;  // rope cos / sin at position p, hd/2 each
    const float* sin_row;
    float* kc;             // this KV head's cache rows [max_ctx][hd]
    float* vc;
    uint16_t* k16;         // this KV head's f16 copies (or null): rows [max_ctx][hd] and
    uint16_t* vt16;        // V transposed [hd][max_ctx]
    int ctx;               // max_ctx: the row stride of vt16
    int qd, kvd;           // widths of q and of k (= v) inside qkv
    int g;                 // KV head
    int p;                 // position of this step's row
    int pos0, pos1;        // rows [pos0, pos1) of the item; pos1 <= p + 1
    float* out;            // [n_heads][hd], or null: write `part`
    float* part;           // attn_part_stride floats: acc [G][hd], max [G], sum [G]
};

template <int HD, int G, int NW>
constexpr int attn_core_lds_floats()
{
    return G * HD + 2 * HD + NW * G * HD + 2 * NW * G;
}

// Offset within a row of a lane's d-th dim; l16 is the lane's index within
// its 16-lane row group (see the work layout above).
template <int DPL>
__device__ inline int attn_dim(int l16, int d)
{
    if constexpr (DPL % 4 == 0) return (d >> 2) * 64 + l16 * 4 + (d & 3);
    else return l16 * DPL + d;
}

// The lane's DPL dims of the row at p (in attn_dim order).
template <int N>
__device__ inline void load_row_slice(const float* p, int l16, float (&v)[N])
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 x = load16f_nt(p + attn_dim<N>(l16, i));
            v[i] = x.x; v[i + 1] = x.y; v[i + 2] = x.z; v[i + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = *gmem(p + attn_dim<N>(l16, i));
    }
}

// The lane's K / V registers for one sweep of ITER row groups.
template <int HD, int ITER>
struct AttnRows {
    float k[ITER][HD / 16];
    float v[ITER][HD / 16];
};

// Row t of sweep s for lane group rg of wave w (see the work layout above).
template <int NW, int ITER>
__device__ inline int attn_row(const AttnItem& a, int s, int w, int it, int rg)
{
    return a.pos0 + s * (NW * 4 * ITER) + w * (4 * ITER) + it * 4 + rg;
}

// Loads of sweep s into r: the cache rows below min(pos1, p) it covers.
// Every load is issued: a row past that bound reads the bound's last row (or
// row 0), a valid address, and is replaced when consumed (row p by this
// step's k and v, rows past it by zeros), so that no wait on these loads is
// needed before the rows are consumed (a branch or a select on the loaded
// values here would make the compiler wait for them at once). Needs only the
// item's rows and cache pointers, so a caller may issue the first sweep
// before the q / k / v of this step exist.
template <int HD, int NW, int ITER>
__device__ inline void attn_load(const AttnItem& a, int s, int tid, AttnRows<HD, ITER>& r)
{
    constexpr int DPL = HD / 16;
    const int lane = tid & (WAVE - 1);
    const int w = tid >> 6;
    const int rg = lane >> 4;
    const int l16 = lane & 15;
    const int last = max(min(a.pos1, a.p) - 1, 0);
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int t = min(attn_row<NW, ITER>(a, s, w, it, rg), last);
        load_row_slice<DPL>(a.kc + int64_t(t) * HD, l16, r.k[it]);
        load_row_slice<DPL>(a.vc + int64_t(t) * HD, l16, r.v[it]);
    }
}

template <int HD, int G, int NW, int ITER, bool DBUF>
__device__ void attn_run(const AttnItem& a, float* lds, int tid, AttnRows<HD, ITER>& first);

// The whole item: first sweep's loads, then attn_run.
template <int HD, int G, int NW, int ITER, bool DBUF>
__device__ void attn_core(const AttnItem& a, float* lds, int tid)
{
    AttnRows<HD, ITER> first;
    attn_load<HD, NW, ITER>(a, 0, tid, first);
    attn_run<HD, G, NW, ITER, DBUF>(a, lds, tid, first);
}

// The item after its first sweep's loads were issued into `first`.
template <int HD, int G, int NW, int ITER, bool DBUF>
__device__ void attn_run(const AttnItem& a, float* lds, int tid, AttnRows<HD, ITER>& first)
{
    constexpr int LPR = 16;
    constexpr int RG = WAVE / LPR;               // rows per wave instruction
    constexpr int DPL = HD / LPR;                // dims per lane
    constexpr int SW = NW * RG * ITER;           // rows per sweep
    constexpr int HALF = HD / 2;
    float* qs = lds;                  // [G][HD]
    float* knew = qs + G * HD;        // [HD]
    float* vnew = knew + HD;          // [HD]
    float* red = vnew + HD;           // [NW][G][HD]
    float* sm = red + NW * G * HD;    // [NW][G]
    float* sl = sm + NW * G;          // [NW][G]
    const int lane = tid & (WAVE - 1);
    const int w = tid >> 6;
    const int rg = lane >> 4;
    const int l16 = lane & (LPR - 1);
    const int p = a.p;
    const bool owner = a.pos1 == p + 1;
    const int n_sweeps = (a.pos1 - a.pos0 + SW - 1) / SW;

    auto row_of = [&](int s, int it) { return attn_row<NW, ITER>(a, s, w, it, rg); };
    AttnRows<HD, ITER> second;  // the next sweep's rows (DBUF only)

    // q of the group's heads (and, for the owner, this step's k): one wave
    // per vector, lane l holding rope pairs l, l + 64, ... (< hd/2), pair i
    // being elements (i0, i1); bias (qwen2), norm_heads, then rope, then
    // into LDS.
    constexpr int PPL = (HALF + WAVE - 1) / WAVE;  // rope pairs per lane
    const int nv = G + (owner ? 1 : 0);
    for (int j = w; j < nv; j += NW) {
        const int off = j < G ? (a.g * G + j) * HD : a.qd + a.g * HD;
        const float* src = a.qkv + off;
        float x0[PPL], x1[PPL];
        int i0[PPL], i1[PPL];
#pragma unroll
        for (int r = 0; r < PPL; ++r) {
            const int i = lane + r * WAVE;
            i0[r] = a.adjacent ? 2 * i : i;
            i1[r] = a.adjacent ? 2 * i + 1 : i + HALF;
            x0[r] = 0.f;
            x1[r] = 0.f;
            if (i < HALF) {
                x0[r] = *gmem(src + i0[r]);
                x1[r] = *gmem(src + i1[r]);
                if (a.bias) {
                    x0[r] += *gmem(a.bias + off + i0[r]);
                    x1[r] += *gmem(a.bias + off + i1[r]);
                }
            }
        }
        if (a.q_norm) {
            float ss = 0.f;
#pragma unroll
            for (int r = 0; r < PPL; ++r) ss += fmaf(x0[r], x0[r], x1[r] * x1[r]);
            ss = wave_sum(ss);
            const float rs = 1.0f / sqrtf(ss / static_cast<float>(HD) + a.eps);
            const float* nw = j < G ? a.q_norm : a.k_norm;
#pragma unroll
            for (int r = 0; r < PPL; ++r) {
                if (lane + r * WAVE < HALF) {
                    x0[r] = *gmem(nw + i0[r]) * (x0[r] * rs);
                    x1[r] = *gmem(nw + i1[r]) * (x1[r] * rs);
                }
            }
        }
        float* dst = j < G ? qs + j * HD : knew;
#pragma unroll
        for (int r = 0; r < PPL; ++r) {
            const int i = lane + r * WAVE;
            if (i < HALF) {
                const float c = *gmem(a.cos_row + i), s = *gmem(a.sin_row + i);
                const float y0 = fmaf(x0[r], c, -x1[r] * s);
                const float y1 = fmaf(x0[r], s, x1[r] * c);
                dst[i0[r]] = y0;
                dst[i1[r]] = y1;
                if (j == G) {  // append k at slot p
                    *gmem(a.kc + int64_t(p) * HD + i0[r]) = y0;
                    *gmem(a.kc + int64_t(p) * HD + i1[r]) = y1;
                    if (a.k16) {
                        *gmem(a.k16 + int64_t(p) * HD + i0[r]) = f32_to_f16_bits(y0);
                        *gmem(a.k16 + int64_t(p) * HD + i1[r]) = f32_to_f16_bits(y1);
                    }
                }
            }
        }
    }
    if (owner) {
        const int voff = a.qd + a.kvd + a.g * HD;
        for (int i = tid; i < HD; i += NW * WAVE) {
            float v = *gmem(a.qkv + voff + i);
            if (a.bias) v += *gmem(a.bias + voff + i);
            vnew[i] = v;
            *gmem(a.vc + int64_t(p) * HD + i) = v;  // append v at slot p
            if (a.vt16) *gmem(a.vt16 + int64_t(i) * a.ctx + p) = f32_to_f16_bits(v);
        }
    }
    __syncthreads();

    // log2(e) / sqrt(hd): scores in base-2 units
    const float qscale = 1.4426950408889634f / sqrtf(static_cast<float>(HD));
    float q[G][DPL], acc[G][DPL], m[G], l[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) {
            q[j][d] = qs[j * HD + attn_dim<DPL>(l16, d)] * qscale;
            acc[j][d] = 0.f;
        }
        m[j] = -INFINITY;
        l[j] = 0.f;
    }

    const int lim = min(a.pos1, p);  // rows below come from the cache
    auto consume = [&](int s, float (&kk)[ITER][DPL], float (&vv)[ITER][DPL]) {
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int t = row_of(s, it);
            if (t == p) {
#pragma unroll
                for (int d = 0; d < DPL; ++d) {
                    kk[it][d] = knew[attn_dim<DPL>(l16, d)];
                    vv[it][d] = vnew[attn_dim<DPL>(l16, d)];
                }
            } else if (t >= lim) {
                // past the item: its score is masked; zero values so that
                // the rows it was loaded from cannot reach the output
#pragma unroll
                for (int d = 0; d < DPL; ++d) {
                    kk[it][d] = 0.f;
                    vv[it][d] = 0.f;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float sc[ITER];
            float mt = -INFINITY;
#pragma unroll
            for (int it = 0; it < ITER; ++it) {
                float x = 0.f;
#pragma unroll
                for (int d = 0; d < DPL; ++d) x = fmaf(q[j][d], kk[it][d], x);
                x = row16_sum(x);
                sc[it] = row_of(s, it) < a.pos1 ? x : -INFINITY;
                mt = fmaxf(mt, sc[it]);
            }
            mt = fmaxf(fmaxf(lane_value(mt, 0), lane_value(mt, 16)),
                       fmaxf(lane_value(mt, 32), lane_value(mt, 48)));
            const float mn = fmaxf(m[j], mt);
            const float resc = m[j] == -INFINITY ? 0.f : exp2_fast(m[j] - mn);
            float ps = 0.f;
#pragma unroll
            for (int d = 0; d < DPL; ++d) acc[j][d] *= resc;
#pragma unroll
            for (int it = 0; it < ITER; ++it) {
                const float pr = sc[it] == -INFINITY ? 0.f : exp2_fast(sc[it] - mn);
                ps += pr;
#pragma unroll
                for (int d = 0; d < DPL; ++d) acc[j][d] = fmaf(pr, vv[it][d], acc[j][d]);
            }
            l[j] = fmaf(l[j], resc, ps);
            m[j] = mn;
        }
    };
    if constexpr (DBUF) {
        for (int s = 0; s < n_sweeps; s += 2) {
            if (s + 1 < n_sweeps) attn_load<HD, NW, ITER>(a, s + 1, tid, second);
            consume(s, first.k, first.v);
            if (s + 1 < n_sweeps) {
                if (s + 2 < n_sweeps) attn_load<HD, NW, ITER>(a, s + 2, tid, first);
                consume(s + 1, second.k, second.v);
            }
        }
    } else {
        for (int s = 0; s < n_sweeps; ++s) {
            if (s > 0) attn_load<HD, NW, ITER>(a, s, tid, first);
            consume(s, first.k, first.v);
        }
    }

    // The wave's four row groups, then the waves, in fixed order.
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) {
            acc[j][d] += __shfl_xor(acc[j][d], 16, WAVE);
            acc[j][d] += __shfl_xor(acc[j][d], 32, WAVE);
        }
        const float lw = (lane_value(l[j], 0) + lane_value(l[j], 16)) +
                         (lane_value(l[j], 32) + lane_value(l[j], 48));
        if (lane < LPR) {
#pragma unroll
            for (int d = 0; d < DPL; ++d) red[(w * G + j) * HD + attn_dim<DPL>(l16, d)] = acc[j][d];
        }
        if (lane == 0) {
            sm[w * G + j] = m[j];
            sl[w * G + j] = lw;
        }
    }
    __syncthreads();
    for (int i = tid; i < G * HD; i += NW * WAVE) {
        const int j = i / HD, d = i % HD;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm[ww * G + j]);
        float v = 0.f, L = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = sm[ww * G + j];
            const float f = mw == -INFINITY ? 0.f : exp2_fast(mw - M);
            v = fmaf(f, red[(ww * G + j) * HD + d], v);
            L = fmaf(f, sl[ww * G + j], L);
        }
        if (a.out) {
            *gmem(a.out + (a.g * G + j) * HD + d) = v / L;
        } else {
            *gmem(a.part + j * HD + d) = v;
            if (d == 0) {
                *gmem(a.part + G * HD + j) = M;
                *gmem(a.part + G * HD + G + j) = L;
            }
        }
    }
    __syncthreads();
}

}  // namespace dev
}  // namespace dfk
