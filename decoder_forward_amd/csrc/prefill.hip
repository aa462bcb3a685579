// prefill.hip — bulk prefill kernels for gfx950: S tokens in one forward.
//
// Bulk prefill runs the same step list over S rows at positions p0..p0+S-1
// and has to agree with S single-token forwards within epsilon (page
// "Execution contract", "Forward phase"). With S rows the four weight
// matmuls are dense contractions, so they run on the CDNA4 matrix cores
// (v_mfma_f32_32x32x16_f16: f16 operands, f32 accumulation); the activation
// operands are rounded to f16 once, by the kernel that produces them.
// Attention is a causal flash attention on v_mfma_f32_16x16x32_f16 that
// reads the f32 KV cache and rounds K and V to f16 in LDS.
#include "kernels.h"

namespace dfk {
namespace {

constexpr int WAVE = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline float h2f(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }
__device__ inline uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }

template <int CTRL>
__device__ inline float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum / max over the 16 lanes of a DPP row (quad xor 1, quad xor 2, half
// mirror, mirror); every lane of the row gets the result.
__device__ inline float row16_sum(float v)
{
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return v;
}
__device__ inline float row16_max(float v)
{
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return v;
}
__device__ inline float wave_sum(float v)
{
    v = row16_sum(v);
    auto rl = [](float x, int l) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
    };
    return (rl(v, 0) + rl(v, 16)) + (rl(v, 32) + rl(v, 48));
}

// ---------------------------------------------------------------------------
// rms_norm of S rows, rounded to f16 as the next GEMM's A operand:
// out[s][k] = f16(w[k] * (x[s][k] * r_s)), r_s = 1/sqrt(mean(x_s^2) + eps).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
rmsnorm_rows_kernel(const float* __restrict__ x, const float* __restrict__ w,
                    int d, float eps, uint16_t* __restrict__ out)
{
    __shared__ float red[4];
    const int s = blockIdx.x;
    const float* xr = x + int64_t(s) * d;
    float ss = 0.f;
    for (int k = threadIdx.x * 4; k < d; k += 1024) {
        const float4 v = *reinterpret_cast<const float4*>(xr + k);
        ss = fmaf(v.x, v.x, ss); ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss); ss = fmaf(v.w, v.w, ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / static_cast<float>(d) + eps);
    uint16_t* o = out + int64_t(s) * d;
    for (int k = threadIdx.x * 4; k < d; k += 1024) {
        const float4 v = *reinterpret_cast<const float4*>(xr + k);
        const float4 g = *reinterpret_cast<const float4*>(w + k);
        ushort4 h;
        h.x = f2h(g.x * (v.x * r)); h.y = f2h(g.y * (v.y * r));
        h.z = f2h(g.z * (v.z * r)); h.w = f2h(g.w * (v.w * r));
        *reinterpret_cast<ushort4*>(o + k) = h;
    }
}

// ---------------------------------------------------------------------------
// GEMM C[M][N] = A[M][K] B[N][K]^T, f16 operands (both K-contiguous), f32
// accumulation on v_mfma_f32_32x32x16_f16. 128x128 work-group tile, 64-deep
// K stages double-buffered in LDS (rows padded by 16 bytes), four waves in a
// 2x2 arrangement of 64x64 wave tiles (2x2 MFMA blocks each).
//
// Lane layout of v_mfma_f32_32x32x16_f16 (checked on the device): lane l
// supplies A[l%32][(l/32)*8 + i] and B[(l/32)*8 + i][l%32] for i < 8 and
// receives C[(i/4)*8 + (l/32)*4 + i%4][l%32] for i < 16.
//
// Epilogues: store f32; add into f32 (residual); store f16; SwiGLU — the
// tile's 128 B rows are gate rows f0..f0+63 and up rows f0..f0+63 in blocks
// of 32 (gate, up, gate, up) so that each lane holds matching gate and up
// sums, and writes f16(silu(g) * u).
// ---------------------------------------------------------------------------
constexpr int GBM = 128, GBN = 128, GBK = 64, GPAD = GBK + 8;

template <int MODE>
__global__ void __launch_bounds__(256)
gemm_kernel(GemmArgs g)
{
    __shared__ _Float16 As[2][GBM][GPAD];
    __shared__ _Float16 Bs[2][GBN][GPAD];
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int ncols = (MODE == GEMM_SWIGLU_F16) ? GBN / 2 : GBN;  // outputs per tile
    const int ntn = (g.N + ncols - 1) / ncols;
    const int ntm = (g.M + GBM - 1) / GBM;
    // XCD-aware order: blocks b, b+8, b+16, ... run on one XCD; give them the
    // same n tile (weights) so its rows are reused from that XCD's L2.
    const int b = blockIdx.x;
    int tn, tm;
    if (ntn % 8 == 0) {
        const int x = b & 7, y = b >> 3;
        tn = (y / ntm) * 8 + x;
        tm = y % ntm;
    } else {
        tn = b / ntm;
        tm = b % ntm;
    }
    const int m0 = tm * GBM;
    const int n0 = tn * ncols;

    // Global rows this thread copies: 4 chunks of 16 bytes for A and for B.
    const uint16_t* aptr[4];
    const uint16_t* bptr[4];
    int srow[4], scol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + i * 256;
        const int row = c >> 3;
        const int kc = (c & 7) * 8;
        srow[i] = row;
        scol[i] = kc;
        const int am = m0 + row;
        aptr[i] = am < g.M ? g.A + int64_t(am) * g.lda + kc : nullptr;
        int bn;
        bool ok;
        if constexpr (MODE == GEMM_SWIGLU_F16) {
            const int cb = row >> 5, within = row & 31;
            const int f = n0 + (cb >> 1) * 32 + within;
            ok = f < g.N;
            bn = f + ((cb & 1) ? int(g.up_rows) : 0);
        } else {
            bn = n0 + row;
            ok = bn < g.N;
        }
        bptr[i] = ok ? g.B + int64_t(bn) * g.ldb + kc : nullptr;
    }
    uint4 ra[4], rb[4];
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool kin = k0 + scol[i] < g.K;
            ra[i] = (aptr[i] && kin) ? *reinterpret_cast<const uint4*>(aptr[i] + k0) : make_uint4(0, 0, 0, 0);
            rb[i] = (bptr[i] && kin) ? *reinterpret_cast<const uint4*>(bptr[i] + k0) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint4*>(&As[buf][srow[i]][scol[i]]) = ra[i];
            *reinterpret_cast<uint4*>(&Bs[buf][srow[i]][scol[i]]) = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;

    const int nst = (g.K + GBK - 1) / GBK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) load_stage((st + 1) * GBK);
#pragma unroll
        for (int kk = 0; kk < GBK / 16; ++kk) {
            half8 af[2], bf[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                af[mi] = *reinterpret_cast<const half8*>(&As[buf][wm * 64 + mi * 32 + (l & 31)][kk * 16 + (l >> 5) * 8]);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                bf[ni] = *reinterpret_cast<const half8*>(&Bs[buf][wn * 64 + ni * 32 + (l & 31)][kk * 16 + (l >> 5) * 8]);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
        }
        if (st + 1 < nst) store_stage(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = m0 + wm * 64 + mi * 32 + (i >> 2) * 8 + (l >> 5) * 4 + (i & 3);
            if (r >= g.M) continue;
            if constexpr (MODE == GEMM_SWIGLU_F16) {
                const int f = n0 + wn * 32 + (l & 31);
                if (f < g.N) {
                    const float gt = acc[mi][0][i];
                    const float up = acc[mi][1][i];
                    static_cast<uint16_t*>(g.C)[int64_t(r) * g.ldc + f] = f2h((gt / (1.0f + expf(-gt))) * up);
                }
            } else {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int c = n0 + wn * 64 + ni * 32 + (l & 31);
                    if (c >= g.N) continue;
                    const int64_t o = int64_t(r) * g.ldc + c;
                    if constexpr (MODE == GEMM_STORE_F32) static_cast<float*>(g.C)[o] = acc[mi][ni][i];
                    else if constexpr (MODE == GEMM_ADD_F32) static_cast<float*>(g.C)[o] += acc[mi][ni][i];
                    else static_cast<uint16_t*>(g.C)[o] = f2h(acc[mi][ni][i]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Per row s (position p0 + s) and head: norm_heads (qwen3), RoPE at the
// position, then q -> Q16[s][head][d] (f16, the attention's A operand) and
// k (after RoPE), v -> the f32 KV cache at slot p0 + s.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64)
qk_post_rows_kernel(QkPostArgs a)
{
    extern __shared__ float v[];  // head_dim floats
    const int s = blockIdx.x;
    const int h = blockIdx.y;     // < n_heads: query head; else KV head h - n_heads
    const int lane = threadIdx.x;
    const int HD = a.head_dim, half = HD / 2;
    const int qd = a.n_heads * HD, kvd = a.n_kv * HD;
    const int pos = a.p0 + s;
    const bool is_q = h < a.n_heads;
    const int g = h - a.n_heads;
    const float* src = a.qkv + int64_t(s) * (qd + 2 * kvd) + (is_q ? h * HD : qd + g * HD);
    for (int i = lane; i < HD; i += WAVE) v[i] = src[i];
    __syncthreads();
    const float* nw = is_q ? a.q_norm : a.k_norm;
    if (nw) {
        float ss = 0.f;
        for (int i = lane; i < HD; i += WAVE) ss = fmaf(v[i], v[i], ss);
        ss = wave_sum(ss);
        const float r = 1.0f / sqrtf(ss / static_cast<float>(HD) + a.eps);
        for (int i = lane; i < HD; i += WAVE) v[i] = nw[i] * (v[i] * r);
        __syncthreads();
    }
    const float* cs = a.cos_t + int64_t(pos) * half;
    const float* sn = a.sin_t + int64_t(pos) * half;
    for (int i = lane; i < half; i += WAVE) {
        const float x0 = v[i], x1 = v[i + half];
        v[i] = fmaf(x0, cs[i], -x1 * sn[i]);
        v[i + half] = fmaf(x0, sn[i], x1 * cs[i]);
    }
    __syncthreads();
    if (is_q) {
        uint16_t* q = a.q16 + (int64_t(s) * a.n_heads + h) * HD;
        for (int i = lane; i < HD; i += WAVE) q[i] = f2h(v[i]);
    } else {
        const int64_t slot = (int64_t(g) * a.max_ctx + pos) * HD;
        const float* vs = a.qkv + int64_t(s) * (qd + 2 * kvd) + qd + kvd + g * HD;
        for (int i = lane; i < HD; i += WAVE) {
            a.kc[slot + i] = v[i];
            a.vc[slot + i] = vs[i];
        }
    }
}

// ---------------------------------------------------------------------------
// Causal flash attention over the cache for 16 query rows and one KV head;
// wave w handles query head g*G + w of the group, so each K/V tile is staged
// once for G heads. Per tile of 32 keys: S = Q K^T (16x32) on
// v_mfma_f32_16x16x32_f16, mask keys past each row's position, online
// softmax in f32 (row statistics reduced over the 16 lanes of a DPP row),
// P rounded to f16 through LDS, O += P V on the same instruction.
//
// Lane layout of v_mfma_f32_16x16x32_f16 (checked on the device): lane l
// supplies A[l%16][(l/16)*8 + i] and B[(l/16)*8 + i][l%16] for i < 8 and
// receives C[(l/16)*4 + i][l%16] for i < 4.
// ---------------------------------------------------------------------------
template <int HD, int G>
__global__ void __launch_bounds__(64 * G)
attn_prefill_kernel(AttnPrefillArgs a)
{
    constexpr int KQ = HD < 32 ? 32 : HD;  // QK depth, zero padded to 32
    constexpr int TK = 32;                  // keys per tile
    constexpr int DB = HD / 16;             // 16-wide output blocks
    __shared__ _Float16 Ks[TK][KQ + 8];
    __shared__ _Float16 Vt[HD][TK + 8];
    __shared__ _Float16 Ps[G][16][TK + 8];
    const int qb = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = tid >> 6;
    const int j = g * G + w;  // query head
    const int s0 = qb * 16;
    const float scale = 1.0f / sqrtf(static_cast<float>(HD));
    const int64_t head_base = int64_t(g) * a.max_ctx * HD;

    // Q fragments: A[q = l%16][d = kq*32 + (l/16)*8 + i].
    half8 qa[KQ / 32];
    {
        const int s = s0 + (l & 15);
#pragma unroll
        for (int kq = 0; kq < KQ / 32; ++kq) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int d = kq * 32 + (l >> 4) * 8 + i;
                qa[kq][i] = (s < a.S && d < HD)
                                ? __builtin_bit_cast(_Float16, a.q16[(int64_t(s) * a.n_heads + j) * HD + d])
                                : _Float16(0);
            }
        }
    }
    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m[4], lsum[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { m[i] = -INFINITY; lsum[i] = 0.f; }

    const int s_last = min(a.S, s0 + 16) - 1;
    const int n_keys = a.p0 + s_last + 1;
    const int tiles = (n_keys + TK - 1) / TK;
    for (int kt = 0; kt < tiles; ++kt) {
        const int t0 = kt * TK;
        // K tile (row-major, zero-padded depth) and V tile (transposed).
        for (int e = tid; e < TK * (KQ / 4); e += 64 * G) {
            const int r = e / (KQ / 4);
            const int c = (e % (KQ / 4)) * 4;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
            float4 vv = kv;
            if (t0 + r < n_keys && c < HD) {
                kv = *reinterpret_cast<const float4*>(a.kc + head_base + int64_t(t0 + r) * HD + c);
                vv = *reinterpret_cast<const float4*>(a.vc + head_base + int64_t(t0 + r) * HD + c);
            }
            Ks[r][c] = _Float16(kv.x); Ks[r][c + 1] = _Float16(kv.y);
            Ks[r][c + 2] = _Float16(kv.z); Ks[r][c + 3] = _Float16(kv.w);
            if (c < HD) {
                Vt[c][r] = _Float16(vv.x); Vt[c + 1][r] = _Float16(vv.y);
                Vt[c + 2][r] = _Float16(vv.z); Vt[c + 3][r] = _Float16(vv.w);
            }
        }
        __syncthreads();
        // Scores for keys kb*16 + l%16, rows (l/16)*4 + i.
        f32x4 sc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kq = 0; kq < KQ / 32; ++kq) {
                const half8 kf = *reinterpret_cast<const half8*>(&Ks[kb * 16 + (l & 15)][kq * 32 + (l >> 4) * 8]);
                sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kq], kf, sc[kb], 0, 0, 0);
            }
        }
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qpos = a.p0 + s0 + (l >> 4) * 4 + i;
            float x0 = sc[0][i] * scale, x1 = sc[1][i] * scale;
            if (t0 + (l & 15) > qpos) x0 = -INFINITY;
            if (t0 + 16 + (l & 15) > qpos) x1 = -INFINITY;
            const float mt = row16_max(fmaxf(x0, x1));
            const float mn = fmaxf(m[i], mt);
            const float p0v = (x0 == -INFINITY) ? 0.f : expf(x0 - mn);
            const float p1v = (x1 == -INFINITY) ? 0.f : expf(x1 - mn);
            const float rs = row16_sum(p0v + p1v);
            alpha[i] = (m[i] == -INFINITY) ? 0.f : expf(m[i] - mn);
            lsum[i] = lsum[i] * alpha[i] + rs;
            m[i] = mn;
            Ps[w][(l >> 4) * 4 + i][l & 15] = _Float16(p0v);
            Ps[w][(l >> 4) * 4 + i][16 + (l & 15)] = _Float16(p1v);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[db][i] *= alpha[i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // P as the A operand: A[q = l%16][key = (l/16)*8 + i].
        const half8 pa = *reinterpret_cast<const half8*>(&Ps[w][l & 15][(l >> 4) * 8]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const half8 vb = *reinterpret_cast<const half8*>(&Vt[db * 16 + (l & 15)][(l >> 4) * 8]);
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, o[db], 0, 0, 0);
        }
        __syncthreads();
    }
    // O / l -> out[s][j*HD + d] in f16 (the o matmul's A operand).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s = s0 + (l >> 4) * 4 + i;
        if (s >= a.S) continue;
        const float inv = 1.0f / lsum[i];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d = db * 16 + (l & 15);
            a.out16[int64_t(s) * a.n_heads * HD + j * HD + d] = f2h(o[db][i] * inv);
        }
    }
}

template <int HD>
hipError_t launch_attn_prefill_hd(const AttnPrefillArgs& a, hipStream_t s)
{
    const dim3 grid((a.S + 15) / 16, a.n_kv);
    switch (a.n_heads / a.n_kv) {
    case 1: DFK_LAUNCH((attn_prefill_kernel<HD, 1>), grid, dim3(64), 0, s, a); break;
    case 2: DFK_LAUNCH((attn_prefill_kernel<HD, 2>), grid, dim3(128), 0, s, a); break;
    case 4: DFK_LAUNCH((attn_prefill_kernel<HD, 4>), grid, dim3(256), 0, s, a); break;
    case 8: DFK_LAUNCH((attn_prefill_kernel<HD, 8>), grid, dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_rows(const float* x, const float* w, int rows, int d, float eps,
                               uint16_t* out, hipStream_t s)
{
    if (rows <= 0) return hipSuccess;
    DFK_LAUNCH(rmsnorm_rows_kernel, dim3(rows), dim3(256), 0, s, x, w, d, eps, out);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, int mode, hipStream_t s)
{
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    const int ncols = mode == GEMM_SWIGLU_F16 ? GBN / 2 : GBN;
    const int blocks = ((g.N + ncols - 1) / ncols) * ((g.M + GBM - 1) / GBM);
    switch (mode) {
    case GEMM_STORE_F32: DFK_LAUNCH(gemm_kernel<GEMM_STORE_F32>, dim3(blocks), dim3(256), 0, s, g); break;
    case GEMM_ADD_F32: DFK_LAUNCH(gemm_kernel<GEMM_ADD_F32>, dim3(blocks), dim3(256), 0, s, g); break;
    case GEMM_STORE_F16: DFK_LAUNCH(gemm_kernel<GEMM_STORE_F16>, dim3(blocks), dim3(256), 0, s, g); break;
    case GEMM_SWIGLU_F16: DFK_LAUNCH(gemm_kernel<GEMM_SWIGLU_F16>, dim3(blocks), dim3(256), 0, s, g); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_qk_post_rows(const QkPostArgs& a, hipStream_t s)
{
    if (a.S <= 0) return hipSuccess;
    DFK_LAUNCH(qk_post_rows_kernel, dim3(a.S, a.n_heads + a.n_kv), dim3(64),
                       size_t(a.head_dim) * sizeof(float), s, a);
    return hipGetLastError();
}

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s)
{
    if (a.S <= 0) return hipSuccess;
    switch (a.head_dim) {
    case 16: return launch_attn_prefill_hd<16>(a, s);
    case 32: return launch_attn_prefill_hd<32>(a, s);
    case 64: return launch_attn_prefill_hd<64>(a, s);
    case 128: return launch_attn_prefill_hd<128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dfk
