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

#include <atomic>
#include <type_traits>

namespace dfk {
namespace {

constexpr int WAVE = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float h2f(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }
__device__ inline uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }
// Two floats rounded to f16, a in the low half.
__device__ inline uint32_t pack_h2(float a, float b) { return uint32_t(f2h(a)) | (uint32_t(f2h(b)) << 16); }

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
// accumulation on v_mfma_f32_32x32x16_f16. BM x BN work-group tile, 64-deep
// K stages double-buffered in LDS (rows padded by 16 bytes), four waves in a
// 2x2 arrangement of (BM/2) x (BN/2) wave tiles. A wave reads BM/64 A and
// BN/64 B fragments from LDS per 16-deep step and issues (BM/64)(BN/64)
// MFMAs, so larger tiles need less LDS bandwidth per flop.
//
// Lane layout of v_mfma_f32_32x32x16_f16 (checked on the device): lane l
// supplies A[l%32][(l/32)*8 + i] and B[(l/32)*8 + i][l%32] for i < 8 and
// receives C[(i/4)*8 + (l/32)*4 + i%4][l%32] for i < 16.
//
// Epilogues: store f32; add into f32 (residual); store f16; SwiGLU — the
// tile's B rows are gate and up rows in alternating blocks of 32 (gate
// f..f+31, up f..f+31, ...) so that each lane holds matching gate and up
// sums, and writes f16(silu(g) * u).
// ---------------------------------------------------------------------------
constexpr int GBK = 64, GPAD = GBK + 8;
// Work-group tile of the prefill GEMMs. The gate/up GEMM (twice the columns)
// takes 256 x 256: half the LDS traffic per flop, and still enough tiles to
// fill the device at prefill sizes; the others keep 128 x 128 for tile count.
constexpr int GBM_ = 128, GBN_ = 128;

template <int BM, int BN>
constexpr size_t gemm_lds_bytes() { return size_t(2) * (BM + BN) * GPAD * sizeof(_Float16); }

template <int BM, int BN, int MODE, bool WQ8>
__global__ void __launch_bounds__(256)
gemm_kernel(GemmArgs g)
{
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int MI = WTM / 32, NI = WTN / 32;
    constexpr int CA = BM / 32, CB = BN / 32;  // 16-byte chunks per thread per stage
    extern __shared__ _Float16 gsm[];
    _Float16 (*As)[BM][GPAD] = reinterpret_cast<_Float16 (*)[BM][GPAD]>(gsm);
    _Float16 (*Bs)[BN][GPAD] = reinterpret_cast<_Float16 (*)[BN][GPAD]>(gsm + 2 * BM * GPAD);
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    constexpr int ncols = (MODE == GEMM_SWIGLU_F16) ? BN / 2 : BN;  // outputs per tile
    const int ntn = (g.N + ncols - 1) / ncols;
    const int ntm = (g.M + BM - 1) / BM;
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
    const int m0 = tm * BM;
    const int n0 = tn * ncols;

    // Global rows this thread copies: chunk c of a stage is row c / 8, K
    // offset (c % 8) * 8.
    const uint16_t* aptr[CA];
    const uint16_t* bptr[CB];
    const uint16_t* sptr[WQ8 ? CB : 1];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int c = tid + i * 256;
        const int am = m0 + (c >> 3);
        aptr[i] = am < g.M ? g.A + int64_t(am) * g.lda + (c & 7) * 8 : nullptr;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
        const int c = tid + i * 256;
        const int row = c >> 3;
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
        if constexpr (WQ8) {
            // values: 1 byte per weight (8 per chunk); scales: one f16 per 32
            bptr[i] = ok ? reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(g.B) +
                                                            int64_t(bn) * g.ldb + (c & 7) * 8)
                         : nullptr;
            sptr[i] = ok ? g.Bsc + int64_t(bn) * (g.ldb >> 5) : nullptr;
        } else {
            bptr[i] = ok ? g.B + int64_t(bn) * g.ldb + (c & 7) * 8 : nullptr;
        }
    }
    // Two register sets: the loads of stage s+2 are issued while stage s is
    // computed, so each load has two stages of MFMA work to arrive. Loads
    // are unconditional: rows or K chunks past the end read 16 zero bytes
    // (g.zeros), so nothing is masked after the load and the waits count
    // exactly.
    // B registers: 16 bytes of f16, or for 8-bit blocks 8 value bytes (in
    // .x, .y) and the block's f16 scale (in .z).
    u32x4 ra0[CA], rb0[CB], ra1[CA], rb1[CB];
    auto load_stage = [&](auto set_c, int k0) {
        constexpr int set = decltype(set_c)::value;
        u32x4* ra = set == 0 ? ra0 : ra1;
        u32x4* rb = set == 0 ? rb0 : rb1;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const bool ok = aptr[i] && k0 + ((tid + i * 256) & 7) * 8 < g.K;
            ra[i] = *reinterpret_cast<const u32x4*>(ok ? aptr[i] + k0 : g.zeros);
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int kc = k0 + ((tid + i * 256) & 7) * 8;
            const bool ok = bptr[i] && kc < g.K;
            if constexpr (WQ8) {
                const uint2 q = *reinterpret_cast<const uint2*>(
                    ok ? reinterpret_cast<const uint8_t*>(bptr[i]) + k0 : reinterpret_cast<const uint8_t*>(g.zeros));
                const uint16_t sc = *(ok ? sptr[i] + (kc >> 5) : g.zeros);
                rb[i] = u32x4{q.x, q.y, uint32_t(sc), 0u};
            } else {
                rb[i] = *reinterpret_cast<const u32x4*>(ok ? bptr[i] + k0 : g.zeros);
            }
        }
    };
    // 8 int8 values times the f16 scale, rounded to f16 (RNE).
    auto dequant = [](u32x4 r) {
        const float sc = h2f(uint16_t(r.z));
        u32x4 o;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t v = h == 0 ? r.x : r.y;
            const float f0 = static_cast<float>(static_cast<int8_t>(v & 0xff)) * sc;
            const float f1 = static_cast<float>(static_cast<int8_t>((v >> 8) & 0xff)) * sc;
            const float f2 = static_cast<float>(static_cast<int8_t>((v >> 16) & 0xff)) * sc;
            const float f3 = static_cast<float>(static_cast<int8_t>(v >> 24)) * sc;
            o[2 * h] = pack_h2(f0, f1);
            o[2 * h + 1] = pack_h2(f2, f3);
        }
        return o;
    };
    auto store_stage = [&](auto set_c) {
        constexpr int set = decltype(set_c)::value, buf = set;
        const u32x4* ra = set == 0 ? ra0 : ra1;
        const u32x4* rb = set == 0 ? rb0 : rb1;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = tid + i * 256;
            *reinterpret_cast<u32x4*>(&As[buf][c >> 3][(c & 7) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = tid + i * 256;
            if constexpr (WQ8) *reinterpret_cast<u32x4*>(&Bs[buf][c >> 3][(c & 7) * 8]) = dequant(rb[i]);
            else *reinterpret_cast<u32x4*>(&Bs[buf][c >> 3][(c & 7) * 8]) = rb[i];
        }
    };

    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;

    auto compute = [&](auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
#pragma unroll
        for (int kk = 0; kk < GBK / 16; ++kk) {
            half8 af[MI], bf[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                af[mi] = *reinterpret_cast<const half8*>(&As[buf][wm * WTM + mi * 32 + (l & 31)][kk * 16 + (l >> 5) * 8]);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                bf[ni] = *reinterpret_cast<const half8*>(&Bs[buf][wn * WTN + ni * 32 + (l & 31)][kk * 16 + (l >> 5) * 8]);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
        }
    };

    // Stage s lives in LDS buffer s & 1. A register set is stored to LDS two
    // stages of compute after its loads were issued: while stage s is
    // computed, the set holding stage s+1 is stored and reloaded with stage
    // s+3, and the other set holds stage s+2 in flight.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    const int nst = (g.K + GBK - 1) / GBK;
    // Loads and stores run unconditionally (past the last stage they repeat
    // the last stage into a buffer nobody reads again), so every path keeps
    // the same loads in flight and the waits stay exact.
    auto kof = [&](int stage) { return min(stage, nst - 1) * GBK; };
    load_stage(S0{}, 0);
    load_stage(S1{}, kof(1));
    store_stage(S0{});
    load_stage(S0{}, kof(2));
    __syncthreads();
    int st = 0;
    for (; st + 1 < nst; st += 2) {
        // even stage st (LDS 0); set 1 holds stage st+1, set 0 stage st+2
        store_stage(S1{});
        load_stage(S1{}, kof(st + 3));
        compute(S0{});
        __syncthreads();
        // odd stage st+1 (LDS 1); set 0 holds stage st+2, set 1 stage st+3
        store_stage(S0{});
        load_stage(S0{}, kof(st + 4));
        compute(S1{});
        __syncthreads();
    }
    if (st < nst) compute(S0{});  // odd number of stages: the last one

    // Epilogue.
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = m0 + wm * WTM + mi * 32 + (i >> 2) * 8 + (l >> 5) * 4 + (i & 3);
            if (r >= g.M) continue;
            if constexpr (MODE == GEMM_SWIGLU_F16) {
#pragma unroll
                for (int ni = 0; ni < NI; ni += 2) {
                    const int f = n0 + ((wn * WTN) / 64 + ni / 2) * 32 + (l & 31);
                    if (f < g.N) {
                        const float gt = acc[mi][ni][i];
                        const float up = acc[mi][ni + 1][i];
                        static_cast<uint16_t*>(g.C)[int64_t(r) * g.ldc + f] = f2h(gate_act(gt, g.act) * up);
                    }
                }
            } else {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    const int c = n0 + wn * WTN + ni * 32 + (l & 31);
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

template <int BM, int BN, int MODE, bool WQ8>
hipError_t launch_gemm_q(const GemmArgs& g, hipStream_t s)
{
    constexpr size_t lds = gemm_lds_bytes<BM, BN>();
    static std::atomic<bool> attr_set{false};  // sessions may launch from several threads
    if (!attr_set.load(std::memory_order_acquire)) {
        const hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<BM, BN, MODE, WQ8>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (r != hipSuccess) return r;
        attr_set.store(true, std::memory_order_release);
    }
    constexpr int ncols = (MODE == GEMM_SWIGLU_F16) ? BN / 2 : BN;
    const int blocks = ((g.N + ncols - 1) / ncols) * ((g.M + BM - 1) / BM);
    DFK_LAUNCH((gemm_kernel<BM, BN, MODE, WQ8>), dim3(blocks), dim3(256), lds, s, g);
    return hipGetLastError();
}

template <int BM, int BN, int MODE>
hipError_t launch_gemm_t(const GemmArgs& g, hipStream_t s)
{
    return g.Bsc ? launch_gemm_q<BM, BN, MODE, true>(g, s) : launch_gemm_q<BM, BN, MODE, false>(g, s);
}

// ---------------------------------------------------------------------------
// Per row s (position p0 + s) and head: bias (qwen2), norm_heads (qwen3),
// RoPE at the position, then q -> Q16[s][head][d] (f16, the attention's A
// operand) and k (after RoPE), v (+ bias) -> the f32 KV cache at slot p0 + s.
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
    const int off = is_q ? h * HD : qd + g * HD;
    const float* src = a.qkv + int64_t(s) * (qd + 2 * kvd) + off;
    for (int i = lane; i < HD; i += WAVE) v[i] = a.bias ? src[i] + a.bias[off + i] : src[i];
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
        const int i0 = a.adjacent ? 2 * i : i, i1 = a.adjacent ? 2 * i + 1 : i + half;
        const float x0 = v[i0], x1 = v[i1];
        v[i0] = fmaf(x0, cs[i], -x1 * sn[i]);
        v[i1] = fmaf(x0, sn[i], x1 * cs[i]);
    }
    __syncthreads();
    if (is_q) {
        uint16_t* q = a.q16 + (int64_t(s) * a.n_heads + h) * HD;
        for (int i = lane; i < HD; i += WAVE) q[i] = f2h(v[i]);
    } else {
        const int64_t slot = (int64_t(g) * a.max_ctx + pos) * HD;
        const int voff = qd + kvd + g * HD;
        const float* vs = a.qkv + int64_t(s) * (qd + 2 * kvd) + voff;
        for (int i = lane; i < HD; i += WAVE) {
            a.kc[slot + i] = v[i];
            a.vc[slot + i] = a.bias ? vs[i] + a.bias[voff + i] : vs[i];
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
    __shared__ __attribute__((aligned(16))) _Float16 Ks[TK][KQ + 8];
    __shared__ __attribute__((aligned(16))) _Float16 Vt[HD][TK + 8];
    __shared__ _Float16 Ps[G][16][TK + 8];
    const int qb = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = tid >> 6;
    const int j = g * G + w;  // query head
    const int s0 = qb * 16;
    // scores in base-2 units (log2(e) / sqrt(hd)), so that each softmax
    // weight is one hardware exp2
    const float scale = 1.4426950408889634f / sqrtf(static_cast<float>(HD));
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
    // With a window, keys before the first query row's window are skipped
    // whole tiles at a time and masked inside the first tile used.
    const int key_lo = a.window > 0 ? max(0, a.p0 + s0 - a.window + 1) : 0;
    for (int kt = key_lo / TK; kt < tiles; ++kt) {
        const int t0 = kt * TK;
        // K tile (row-major, zero-padded depth): 4 halves per 8-byte store,
        // consecutive threads on consecutive addresses.
        for (int e = tid; e < TK * (KQ / 4); e += 64 * G) {
            const int r = e / (KQ / 4);
            const int c = (e % (KQ / 4)) * 4;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (t0 + r < n_keys && c < HD)
                kv = *reinterpret_cast<const float4*>(a.kc + head_base + int64_t(t0 + r) * HD + c);
            *reinterpret_cast<uint2*>(&Ks[r][c]) = make_uint2(pack_h2(kv.x, kv.y), pack_h2(kv.z, kv.w));
        }
        // V tile transposed: a thread takes rows (2i, 2i+1) at 4 dims and
        // writes 4 half pairs; consecutive threads write consecutive pairs
        // of one transposed row (no bank conflicts).
        for (int e = tid; e < (TK / 2) * (HD / 4); e += 64 * G) {
            const int r = (e % (TK / 2)) * 2;
            const int c = (e / (TK / 2)) * 4;
            float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
            if (t0 + r < n_keys) v0 = *reinterpret_cast<const float4*>(a.vc + head_base + int64_t(t0 + r) * HD + c);
            if (t0 + r + 1 < n_keys) v1 = *reinterpret_cast<const float4*>(a.vc + head_base + int64_t(t0 + r + 1) * HD + c);
            *reinterpret_cast<uint32_t*>(&Vt[c][r]) = pack_h2(v0.x, v1.x);
            *reinterpret_cast<uint32_t*>(&Vt[c + 1][r]) = pack_h2(v0.y, v1.y);
            *reinterpret_cast<uint32_t*>(&Vt[c + 2][r]) = pack_h2(v0.z, v1.z);
            *reinterpret_cast<uint32_t*>(&Vt[c + 3][r]) = pack_h2(v0.w, v1.w);
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
            const int kmin = a.window > 0 ? qpos - a.window + 1 : 0;  // first key in the window
            if (t0 + (l & 15) > qpos || t0 + (l & 15) < kmin) x0 = -INFINITY;
            if (t0 + 16 + (l & 15) > qpos || t0 + 16 + (l & 15) < kmin) x1 = -INFINITY;
            const float mt = row16_max(fmaxf(x0, x1));
            const float mn = fmaxf(m[i], mt);
            const float p0v = (x0 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x0 - mn);
            const float p1v = (x1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x1 - mn);
            const float rs = row16_sum(p0v + p1v);
            alpha[i] = (m[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[i] - mn);
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
    case 3: DFK_LAUNCH((attn_prefill_kernel<HD, 3>), grid, dim3(192), 0, s, a); break;
    case 4: DFK_LAUNCH((attn_prefill_kernel<HD, 4>), grid, dim3(256), 0, s, a); break;
    case 5: DFK_LAUNCH((attn_prefill_kernel<HD, 5>), grid, dim3(320), 0, s, a); break;
    case 6: DFK_LAUNCH((attn_prefill_kernel<HD, 6>), grid, dim3(384), 0, s, a); break;
    case 7: DFK_LAUNCH((attn_prefill_kernel<HD, 7>), grid, dim3(448), 0, s, a); break;
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
    switch (mode) {
    case GEMM_STORE_F32: return launch_gemm_t<GBM_, GBN_, GEMM_STORE_F32>(g, s);
    case GEMM_ADD_F32: return launch_gemm_t<GBM_, GBN_, GEMM_ADD_F32>(g, s);
    case GEMM_STORE_F16: return launch_gemm_t<GBM_, GBN_, GEMM_STORE_F16>(g, s);
    case GEMM_SWIGLU_F16: return launch_gemm_t<256, 256, GEMM_SWIGLU_F16>(g, s);
    }
    return hipErrorInvalidValue;
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
    case 256: return launch_attn_prefill_hd<256>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dfk
