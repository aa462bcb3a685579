// prefill.hip — bulk prefill kernels for gfx950: S tokens in one forward.
//
// Bulk prefill runs the same step list over S rows at positions p0..p0+S-1
// and has to agree with S single-token forwards within epsilon (page
// "Execution contract", "Forward phase"). With S rows the four weight
// matmuls are dense contractions, so they run on the CDNA4 matrix cores
// (v_mfma_f32_32x32x16_f16: f16 operands, f32 accumulation); the activation
// operands are rounded to f16 once, by the kernel that produces them.
// Attention is a causal flash attention on v_mfma_f32_16x16x32_f16. At
// head_dim 64 and 128 it reads f16 copies of the KV cache (kept beside the
// f32 cache by every path that writes a cache row) straight into LDS; at
// other head sizes it reads the f32 cache and rounds K and V to f16 in LDS.
#include "kernels.h"

#include <algorithm>
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

// Hand-off between the work-groups of a split GEMM tile, which may run on
// different XCDs (whose L2s are not coherent with each other): partial sums
// are stored and loaded 16 bytes per lane with the cache policy of an
// agent-scope atomic (sc1: at the coherence point, past the XCD's L2), and a
// work-group takes its ticket only after every wave's stores are
// acknowledged. No fence writes back or invalidates a whole L2.
constexpr int CPOL_SC1 = 16;
__device__ inline __amdgpu_buffer_rsrc_t ws_rsrc(float* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, int(bytes), 0x00020000);
}
__device__ inline void st_agent16(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, int(off), 0, CPOL_SC1);
}
__device__ inline f32x4 ld_agent16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, CPOL_SC1));
}
// True in the last of `n` work-groups to call it on `counter` (in all their
// threads), which also resets the counter to 0. Call after every thread
// has issued its hand-off stores.
__device__ inline bool last_of(int* counter, int n, int* flag_lds)
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        typedef __attribute__((address_space(1))) int gint;
        const int prev = __hip_atomic_fetch_add((gint*)counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == n - 1;
        if (last) __hip_atomic_store((gint*)counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag_lds = last;
    }
    __syncthreads();
    return *flag_lds != 0;
}

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
// 8-bit block rows to f16: thread t converts values 8t .. 8t + 7 (one
// 8-byte load, one 16-byte store) of rows blockIdx.y, blockIdx.y +
// gridDim.y, ..., with the same rounding as the 8-bit GEMM's load path (f32
// product, rounded once to f16).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
dequant_q8_kernel(const int8_t* __restrict__ q, const uint16_t* __restrict__ sc, int64_t rows, int64_t cols,
                  uint16_t* __restrict__ out)
{
    const int64_t c = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
    if (c >= cols) return;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const uint2 v = *reinterpret_cast<const uint2*>(q + r * cols + c);
        const float s = h2f(sc[r * (cols / 32) + c / 32]);
        uint4 o;
        o.x = pack_h2(float(int8_t(v.x & 0xff)) * s, float(int8_t((v.x >> 8) & 0xff)) * s);
        o.y = pack_h2(float(int8_t((v.x >> 16) & 0xff)) * s, float(int8_t(v.x >> 24)) * s);
        o.z = pack_h2(float(int8_t(v.y & 0xff)) * s, float(int8_t((v.y >> 8) & 0xff)) * s);
        o.w = pack_h2(float(int8_t((v.y >> 16) & 0xff)) * s, float(int8_t(v.y >> 24)) * s);
        *reinterpret_cast<uint4*>(out + r * cols + c) = o;
    }
}

// ---------------------------------------------------------------------------
// GEMM C[M][N] = A[M][K] B[N][K]^T, f16 operands (both K-contiguous), f32
// accumulation on v_mfma_f32_32x32x16_f16. BM x BN work-group tile, 64-deep
// K stages double-buffered in LDS (rows padded by 16 bytes), 2 x WN waves
// in a grid of (BM/2) x (BN/WN) wave tiles. A wave reads BM/64 A and BN/(32 WN)
// B fragments from LDS per 16-deep step and issues one MFMA per pair, so
// larger wave tiles need less LDS bandwidth per flop; 8 waves (two per SIMD)
// let one wave's LDS traffic and waits overlap the other's MFMAs. A grid of
// 128-row tiles that fills at most half of the compute units may split each
// tile's K loop over 2-4 work-groups (split_reduce: the last adds the
// partial sums in a fixed order).
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
constexpr int GEMM_SPLIT_MAX = 4;  // work-groups per tile along K, at most
// Work-group tile of the prefill GEMMs for small problems (fewer than about
// one 256 x 256 tile per compute unit): 128 x 128 on 4 waves.
constexpr int GBM_ = 128, GBN_ = 128;

template <int BM, int BN>
constexpr size_t gemm_lds_bytes() { return size_t(2) * (BM + BN) * GPAD * sizeof(_Float16); }

// Tile (tm, tn) of block b. Blocks are dispatched to the 8 XCDs in turn
// (block b to XCD b % 8), each XCD running about 32 at a time, one per
// compute unit, and the tiles that run together on an XCD share its L2:
// every stage, each distinct A row block and B row block among them is
// fetched into that L2 once. The tiles are therefore numbered in groups of
// up to 8 row blocks (tm) by all column blocks (tn), tm fastest, so 32
// consecutive tiles cover 8 tm x 4 tn (12 distinct operand blocks; taking
// every tm of one tn pair would need 18), and XCD x takes the x-th eighth
// of that numbering, its blocks in dispatch order.
__device__ inline void gemm_tile_of(int b, int ntm, int ntn, int& tm, int& tn)
{
    const int total = ntm * ntn;
    const int x = b & 7, y = b >> 3;
    const int base = total >> 3, rem = total & 7;
    const int g = x * base + min(x, rem) + y;  // XCD x's tiles are consecutive
    constexpr int GM = 8;
    const int grp = g / (GM * ntn);
    const int gm = min(GM, ntm - grp * GM);    // row blocks in this group
    const int r = g - grp * GM * ntn;
    tn = r / gm;
    tm = grp * GM + r % gm;
}

// Epilogue of a wave's (MI*32) x (NI*32) accumulator tile at rows m0 + wm*WTM,
// columns n0 + wn*WTN (for SwiGLU: output columns of the gate/up block pairs).
template <int MODE, int MI, int NI, int WTM, int WTN>
__device__ inline void gemm_epilogue(const GemmArgs& g, const f32x16 (&acc)[MI][NI], int m0, int n0,
                                     int wm, int wn, int l)
{
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


// Scheduling groups: one MFMA, then RPM LDS reads, until LEFT reads are
// placed.
template <int LEFT, int RPM>
__device__ inline void sched_mfma_reads()
{
    if constexpr (LEFT > 0) {
        constexpr int n = LEFT < RPM ? LEFT : RPM;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, n, 0);
        sched_mfma_reads<LEFT - n, RPM>();
    }
}

// MFMAs of one LDS stage: KS steps of 16 along K over an MI x NI grid of
// 32 x 32 tiles. afrag(kk, mi) / bfrag(kk, ni) give the LDS address of the
// lane's A / B fragment for step kk. The fragments of step kk+1 are read
// into a second register set while the MFMAs of step kk run, one read
// between two MFMAs (fixed by scheduling groups), so each MFMA waits only on
// reads issued a step earlier. PIPE = false: one register set, reads and
// MFMAs left to the compiler's schedule (for kernels with no registers to
// spare).
template <int MI, int NI, int KS, bool PIPE, class FA, class FB>
__device__ inline void mma_stage(f32x16 (&acc)[MI][NI], FA afrag, FB bfrag)
{
    constexpr int NRD = MI + NI;
    if constexpr (!PIPE) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            half8 af[MI], bf[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) af[mi] = *reinterpret_cast<const half8*>(afrag(kk, mi));
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) bf[ni] = *reinterpret_cast<const half8*>(bfrag(kk, ni));
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
        }
        return;
    }
    half8 af[2][MI], bf[2][NI];
    auto rd = [&](int kk, int slot) {
#pragma unroll
        for (int i = 0; i < NRD; ++i) {
            // B fragments first: the first MFMAs need B 0.. and A 0
            if (i < NI) bf[slot][i] = *reinterpret_cast<const half8*>(bfrag(kk, i));
            else af[slot][i - NI] = *reinterpret_cast<const half8*>(afrag(kk, i - NI));
        }
    };
    rd(0, 0);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const int c = kk & 1;
        if (kk + 1 < KS) rd(kk + 1, c ^ 1);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][mi], bf[c][ni], acc[mi][ni], 0, 0, 0);
        if (kk == 0) __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);  // step 0's reads
        if (kk + 1 < KS) {
            // one read after each of the first MFMAs (reading earlier, two
            // per MFMA, measured slower)
            constexpr int NG = NRD < MI * NI ? NRD : MI * NI;
            sched_mfma_reads<NRD, 1>();
            if (MI * NI > NG) __builtin_amdgcn_sched_group_barrier(0x008, MI * NI - NG, 0);
        } else {
            __builtin_amdgcn_sched_group_barrier(0x008, MI * NI, 0);
        }
    }
}

// Byte offset of floats 4q .. 4q+3 of accumulator (mi, ni) of thread tid in
// slot j of a split tile's partial sums: one wave's 16-byte accesses of a
// given (j, mi, ni, q) are 1 KiB contiguous.
template <int MI, int NI, int NT>
__device__ inline uint32_t split_off(int j, int mi, int ni, int q, int tid)
{
    return uint32_t((((j * MI + mi) * NI + ni) * 4 + q) * NT + tid) * 16u;
}

// acc = slot 0 + slot 1 + ... + slot S-1 of a split tile's partial sums,
// added in that order; one accumulator block at a time, all S slots' loads
// issued before the first add (one round trip per block, not per slot).
template <int S, int MI, int NI, int NT>
__device__ inline void split_sum(f32x16 (&acc)[MI][NI], __amdgpu_buffer_rsrc_t rw, int tid)
{
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            f32x4 v[S][4];
#pragma unroll
            for (int j = 0; j < S; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) v[j][q] = ld_agent16(rw, split_off<MI, NI, NT>(j, mi, ni, q, tid));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 sum = v[0][q];
#pragma unroll
                for (int j = 1; j < S; ++j) sum += v[j][q];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[mi][ni][4 * q + e] = sum[e];
            }
        }
}

// A split tile's partial sums: this work-group's into slot `part`; then the
// last of the tile's `split` work-groups sets acc = slot 0 + slot 1 + ...,
// added in that order (its own slot read back like the others), so the
// result does not depend on which one finishes last. Returns false in the
// others.
template <int MI, int NI, int NT>
__device__ inline bool split_reduce(f32x16 (&acc)[MI][NI], float* ws, int* ticket, int split, int part, int tid,
                                    int* flag_lds)
{
    constexpr int SLOT = MI * NI * 16 * NT;  // floats
    const __amdgpu_buffer_rsrc_t rw = ws_rsrc(ws, uint32_t(split) * SLOT * 4);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                st_agent16(rw, split_off<MI, NI, NT>(part, mi, ni, q, tid),
                           f32x4{acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                                 acc[mi][ni][4 * q + 3]});
    if (!last_of(ticket, split, flag_lds)) return false;
    switch (split) {
    case 2: split_sum<2, MI, NI, NT>(acc, rw, tid); break;
    case 3: split_sum<3, MI, NI, NT>(acc, rw, tid); break;
    default: split_sum<GEMM_SPLIT_MAX, MI, NI, NT>(acc, rw, tid); break;
    }
    return true;
}

template <int BM, int BN, int WN, int MODE, bool WQ8>
__global__ void __launch_bounds__(128 * WN)
gemm_kernel(GemmArgs g)
{
    constexpr int NT = 128 * WN;               // 2 x WN waves
    constexpr int WTM = BM / 2, WTN = BN / WN;
    constexpr int MI = WTM / 32, NI = WTN / 32;
    constexpr int CA = BM * 8 / NT, CB = BN * 8 / NT;  // 16-byte chunks per thread per stage
    extern __shared__ _Float16 gsm[];
    _Float16 (*As)[BM][GPAD] = reinterpret_cast<_Float16 (*)[BM][GPAD]>(gsm);
    _Float16 (*Bs)[BN][GPAD] = reinterpret_cast<_Float16 (*)[BN][GPAD]>(gsm + 2 * BM * GPAD);
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    constexpr int ncols = (MODE == GEMM_SWIGLU_F16) ? BN / 2 : BN;  // outputs per tile
    const int ntn = (g.N + ncols - 1) / ncols;
    const int ntm = (g.M + BM - 1) / BM;
    // split > 1 (128-row tiles only): work-group b takes part b % split of
    // tile b / split
    constexpr bool SPLITS = BM == 128;
    const int nsplit = SPLITS ? max(g.split, 1) : 1;
    const int tile = SPLITS ? int(blockIdx.x) / nsplit : int(blockIdx.x);
    const int part = SPLITS ? int(blockIdx.x) - tile * nsplit : 0;
    int tn, tm;
    gemm_tile_of(tile, ntm, ntn, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * ncols;

    // Global rows this thread copies: chunk c of a stage is row c / 8, K
    // offset (c % 8) * 8.
    const uint16_t* aptr[CA];
    const uint16_t* bptr[CB];
    const uint16_t* sptr[WQ8 ? CB : 1];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int c = tid + i * NT;
        const int am = m0 + (c >> 3);
        aptr[i] = am < g.M ? g.A + int64_t(am) * g.lda + (c & 7) * 8 : nullptr;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
        const int c = tid + i * NT;
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
            const bool ok = aptr[i] && k0 + ((tid + i * NT) & 7) * 8 < g.K;
            ra[i] = *reinterpret_cast<const u32x4*>(ok ? aptr[i] + k0 : g.zeros);
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int kc = k0 + ((tid + i * NT) & 7) * 8;
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
            const int c = tid + i * NT;
            *reinterpret_cast<u32x4*>(&As[buf][c >> 3][(c & 7) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = tid + i * NT;
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
        // 8-bit blocks: the dequantising stores already fill the slots between
        // the MFMAs; a second fragment set measured slower there
        mma_stage<MI, NI, GBK / 16, !WQ8>(
            acc,
            [&](int kk, int mi) { return &As[buf][wm * WTM + mi * 32 + (l & 31)][kk * 16 + (l >> 5) * 8]; },
            [&](int kk, int ni) { return &Bs[buf][wn * WTN + ni * 32 + (l & 31)][kk * 16 + (l >> 5) * 8]; });
    };

    // Stage s lives in LDS buffer s & 1. A register set is stored to LDS two
    // stages of compute after its loads were issued: while stage s is
    // computed, the set holding stage s+1 is stored and reloaded with stage
    // s+3, and the other set holds stage s+2 in flight.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    // This work-group's stages: st0 .. st0 + nst - 1 of the K loop's
    // (all of them without a split; the caller keeps nst >= 1).
    const int kst = (g.K + GBK - 1) / GBK;
    const int st0 = SPLITS ? kst * part / nsplit : 0;
    const int nst = SPLITS ? kst * (part + 1) / nsplit - st0 : kst;
    // Loads and stores run unconditionally (past the last stage they repeat
    // the last stage into a buffer nobody reads again), so every path keeps
    // the same loads in flight and the waits stay exact.
    auto kof = [&](int stage) { return (SPLITS ? st0 + min(stage, nst - 1) : min(stage, nst - 1)) * GBK; };
    load_stage(S0{}, kof(0));
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

    if constexpr (SPLITS) {
        if (nsplit > 1) {
            // the flag goes in the operand buffers, no longer read
            if (!split_reduce<MI, NI, NT>(acc, g.ws + int64_t(tile) * nsplit * (MI * NI * 16 * NT),
                                          g.tickets + tile, nsplit, part, tid, reinterpret_cast<int*>(gsm)))
                return;
        }
    }
    gemm_epilogue<MODE, MI, NI, WTM, WTN>(g, acc, m0, n0, wm, wn, l);
}


// ---------------------------------------------------------------------------
// The same GEMM for f16 weights with the operand tiles loaded straight into
// LDS (buffer_load_dwordx4 ... lds: lane i of a wave writes 16 bytes at LDS
// base + 16 i; a per-lane byte offset fixed for the whole K loop plus a
// scalar per-stage offset), no register staging. A stage holds A rows [BM][64] and B rows
// [BN][64] unpadded, each row's 16-byte K chunks permuted (gemm_swz), so a
// load instruction fills 8 whole rows and the fragment reads (32 rows of one
// chunk column per half-wave) fall in distinct banks.
// NB stage buffers (3 where they fit in LDS, else 2): the loads of stage
// s + NB - 1 are issued right after the barrier that opens stage s, and a
// wave waits only for the loads of the stage it is about to read.
// ---------------------------------------------------------------------------
constexpr int GDK = 64;  // K depth of a stage

// Position of K chunk c of tile row r in its 128-byte LDS row: c ^ gemm_swz(r).
// A 16-byte-per-lane LDS read is served 16 lanes at a time from 256 bytes
// of banks (on gfx950 the swizzle c ^ (r & 7), which separates only 8 rows,
// left the bank-conflict counter at half of the LDS-active cycles). The 16
// lanes of a fragment read take 16 consecutive rows of one K chunk; rows 2j
// and 2j+1 lie in different halves of a 256-byte bank line, and
// gemm_swz(r) = (r >> 1) & 7 gives the 8 rows of each half 8 different
// positions, so the 16 reads hit 16 different bank groups.
__device__ inline int gemm_swz(int r) { return (r >> 1) & 7; }

template <int BM, int BN>
constexpr int gemm_dma_stages() { return size_t(3) * (BM + BN) * GDK * 2 <= 160 * 1024 ? 3 : 2; }
template <int BM, int BN>
constexpr size_t gemm_dma_lds_bytes() { return size_t(gemm_dma_stages<BM, BN>()) * (BM + BN) * GDK * 2; }

// s_waitcnt with vmcnt = N (N < 64) and the other counters left alone.
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Buffer descriptors of the direct-to-LDS loads: raw (stride 0) over
// DMA_RANGE bytes from the matrix base; an offset at or past DMA_OOB is out
// of range and reads zeros. Matrices of DMA_RANGE bytes or more take the
// register-staged kernel (gemm_dma_fits).
constexpr int DMA_RANGE = 0x7fffffff;
constexpr uint32_t DMA_OOB = 0x80000000u;
constexpr int BUF_RSRC_W3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t dma_rsrc(const uint16_t* base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, DMA_RANGE, BUF_RSRC_W3);
}

// 16 bytes per lane from byte offset voff + soff of the buffer into LDS at
// dst + 16 * lane.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, _Float16* dst, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst), 16, voff, soff, 0, 0);
}

template <int BM, int BN, int WM, int WN, int MODE>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_dma_kernel(GemmArgs g)
{
    constexpr int NW = WM * WN;                // waves: WM x WN grid
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MI = WTM / 32, NI = WTN / 32;
    constexpr int NB = gemm_dma_stages<BM, BN>();
    constexpr int IA = BM / (8 * NW), IB = BN / (8 * NW);  // 8-row load instructions per wave per stage
    static_assert(IA * 8 * NW == BM && IB * 8 * NW == BN, "tile rows split over the waves");
    constexpr int SA = BM * GDK, SB = BN * GDK;  // halves per stage
    extern __shared__ _Float16 gsm[];
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    constexpr int ncols = (MODE == GEMM_SWIGLU_F16) ? BN / 2 : BN;  // outputs per tile
    const int ntn = (g.N + ncols - 1) / ncols;
    const int ntm = (g.M + BM - 1) / BM;
    int tn, tm;
    gemm_tile_of(blockIdx.x, ntm, ntn, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * ncols;

    // This lane's source rows: load instruction q of the wave fills tile
    // rows r = (wave*I + q)*8 .. +7; lane l takes row r + l/8, position l%8,
    // which holds K chunk (l%8) ^ gemm_swz(row). The loads are buffer loads
    // into LDS: a per-lane byte offset fixed for the whole K loop plus a
    // per-stage scalar offset, one instruction per load. A row past the end
    // gets an offset beyond the buffer's range (DMA_OOB), which reads zeros.
    // g.zeros is not needed here.
    const __amdgpu_buffer_rsrc_t ra = dma_rsrc(g.A);
    const __amdgpu_buffer_rsrc_t rb = dma_rsrc(g.B);
    uint32_t voa[IA], vob[IB];  // byte offsets of this lane's chunks at k = 0
    int kca[IA], kcb[IB];       // K offset of this lane's chunk in a stage
#pragma unroll
    for (int q = 0; q < IA; ++q) {
        const int row = (wave * IA + q) * 8 + (l >> 3);
        kca[q] = ((l & 7) ^ gemm_swz(row)) * 8;
        const int am = m0 + row;
        voa[q] = am < g.M ? uint32_t((int64_t(am) * g.lda + kca[q]) * 2) : DMA_OOB;
    }
#pragma unroll
    for (int q = 0; q < IB; ++q) {
        const int row = (wave * IB + q) * 8 + (l >> 3);
        kcb[q] = ((l & 7) ^ gemm_swz(row)) * 8;
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
        vob[q] = ok ? uint32_t((int64_t(bn) * g.ldb + kcb[q]) * 2) : DMA_OOB;
    }
    const int nst = g.K / GDK;  // K is a multiple of GDK here (gemm_dma_fits)
    // Loads of stage st into buffer buf.
    auto issue = [&](int st, int buf) {
        const uint32_t so = uint32_t(st * GDK) * 2;
        _Float16* a_lds = gsm + buf * (SA + SB);
        _Float16* b_lds = a_lds + SA;
#pragma unroll
        for (int q = 0; q < IA; ++q)
            dma16(ra, a_lds + (wave * IA + q) * 8 * GDK, voa[q], so);
#pragma unroll
        for (int q = 0; q < IB; ++q)
            dma16(rb, b_lds + (wave * IB + q) * 8 * GDK, vob[q], so);
    };

    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;

    // Fragment rows: A rows wm*WTM + mi*32 + l%32, B rows wn*WTN + ni*32 +
    // l%32 (every fragment's first row is a multiple of 32); K chunk
    // kk*2 + l/32 sits at position chunk ^ gemm_swz(row) = chunk ^ ((l/2) & 7).
    auto compute = [&](int buf) {
        const _Float16* a_lds = gsm + buf * (SA + SB);
        const _Float16* b_lds = a_lds + SA;
        auto pos = [&](int kk) { return ((kk * 2 + (l >> 5)) ^ ((l >> 1) & 7)) * 8; };
        __builtin_amdgcn_s_setprio(1);
        mma_stage<MI, NI, GDK / 16, true>(
            acc, [&](int kk, int mi) { return a_lds + (wm * WTM + mi * 32 + (l & 31)) * GDK + pos(kk); },
            [&](int kk, int ni) { return b_lds + (wn * WTN + ni * 32 + (l & 31)) * GDK + pos(kk); });
        __builtin_amdgcn_s_setprio(0);
    };

    // Prologue: stages 0 .. NB-2 in flight.
#pragma unroll
    for (int i = 0; i < NB - 1; ++i)
        if (i < nst) issue(i, i);
    for (int st = 0; st < nst; ++st) {
        // Wait for this wave's loads of stage st; those of the (at most
        // NB-2) later stages already issued may stay in flight.
        if (NB == 3 && st + 1 < nst) wait_vmcnt<(NB == 3 ? IA + IB : 0)>();
        else wait_vmcnt<0>();
        __syncthreads();  // every wave's loads of stage st landed; stage st-1's buffer is free
        if (st + NB - 1 < nst) issue(st + NB - 1, (st + NB - 1) % NB);
        compute(st % NB);
    }
    gemm_epilogue<MODE, MI, NI, WTM, WTN>(g, acc, m0, n0, wm, wn, l);
}

template <int BM, int BN, int WN, int MODE, bool WQ8>
hipError_t launch_gemm_q(const GemmArgs& g, hipStream_t s)
{
    constexpr size_t lds = gemm_lds_bytes<BM, BN>();
    static std::atomic<bool> attr_set{false};  // sessions may launch from several threads
    if (!attr_set.load(std::memory_order_acquire)) {
        const hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<BM, BN, WN, MODE, WQ8>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (r != hipSuccess) return r;
        attr_set.store(true, std::memory_order_release);
    }
    constexpr int ncols = (MODE == GEMM_SWIGLU_F16) ? BN / 2 : BN;
    const int blocks = ((g.N + ncols - 1) / ncols) * ((g.M + BM - 1) / BM) * max(g.split, 1);
    DFK_LAUNCH((gemm_kernel<BM, BN, WN, MODE, WQ8>), dim3(blocks), dim3(128 * WN), lds, s, g);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int MODE>
hipError_t launch_gemm_dma(const GemmArgs& g, hipStream_t s)
{
    constexpr size_t lds = gemm_dma_lds_bytes<BM, BN>();
    static std::atomic<bool> attr_set{false};  // sessions may launch from several threads
    if (!attr_set.load(std::memory_order_acquire)) {
        const hipError_t r = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemm_dma_kernel<BM, BN, WM, WN, MODE>),
            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (r != hipSuccess) return r;
        attr_set.store(true, std::memory_order_release);
    }
    constexpr int ncols = (MODE == GEMM_SWIGLU_F16) ? BN / 2 : BN;
    const int blocks = ((g.N + ncols - 1) / ncols) * ((g.M + BM - 1) / BM);
    DFK_LAUNCH((gemm_dma_kernel<BM, BN, WM, WN, MODE>), dim3(blocks), dim3(64 * WM * WN), lds, s, g);
    return hipGetLastError();
}


// f16 weights on 256-row tiles: operand tiles loaded straight into LDS
// (measured 3% faster there, slower on the smaller tiles); otherwise, and
// for 8-bit blocks (dequantised on the way into LDS), the register-staged
// kernel.
template <int BM, int BN, int WN, int MODE>
hipError_t launch_gemm_t(const GemmArgs& g, bool dma, hipStream_t s)
{
    if (g.Bsc) return launch_gemm_q<BM, BN, WN, MODE, true>(g, s);
    if constexpr (BM == 256) {
        if (dma) return launch_gemm_dma<BM, BN, 2, WN, MODE>(g, s);
    }
    return launch_gemm_q<BM, BN, WN, MODE, false>(g, s);
}

// ---------------------------------------------------------------------------
// Per row s (position p0 + s) and head: bias (qwen2), norm_heads (qwen3),
// RoPE at the position, then q * log2(e)/sqrt(hd) -> Q16[s][head][d] (f16,
// the attention's operand, scores in base 2) and k (after RoPE), v (+ bias)
// -> the f32 KV cache at slot p0 + s.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
qk_post_rows_kernel(QkPostArgs a)
{
    // One block per row; wave w takes heads w, w + 4, ... (query heads, then
    // KV heads). Lane l holds rope pairs l and l + 64 (those below hd/2).
    const int s = blockIdx.x;
    const int lane = threadIdx.x & (WAVE - 1);
    const int w = threadIdx.x >> 6;
    const int HD = a.head_dim, half = HD / 2;
    const int qd = a.n_heads * HD, kvd = a.n_kv * HD;
    const int pos = a.p0 + s;
    const float* row = a.qkv + int64_t(s) * (qd + 2 * kvd);
    const float* cs = a.cos_t + int64_t(pos) * half;
    const float* sn = a.sin_t + int64_t(pos) * half;
    // q for the attention's operand: times log2(e) / sqrt(hd) (the attention
    // takes its softmax in base 2), then rounded to f16 once
    const float qs = 1.4426950408889634f / sqrtf(static_cast<float>(HD));
    for (int h = w; h < a.n_heads + a.n_kv; h += 4) {
        const bool is_q = h < a.n_heads;
        const int g = h - a.n_heads;
        const int off = is_q ? h * HD : qd + g * HD;
        float x0[2], x1[2];
        int i0[2], i1[2];
        float ss = 0.f;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int i = lane + r * WAVE;
            i0[r] = a.adjacent ? 2 * i : i;
            i1[r] = a.adjacent ? 2 * i + 1 : i + half;
            x0[r] = 0.f;
            x1[r] = 0.f;
            if (i < half) {
                x0[r] = row[off + i0[r]];
                x1[r] = row[off + i1[r]];
                if (a.bias) {
                    x0[r] += a.bias[off + i0[r]];
                    x1[r] += a.bias[off + i1[r]];
                }
                ss = fmaf(x0[r], x0[r], fmaf(x1[r], x1[r], ss));
            }
        }
        const float* nw = is_q ? a.q_norm : a.k_norm;
        float rn = 1.f;
        if (nw) rn = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(HD) + a.eps);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int i = lane + r * WAVE;
            if (i >= half) continue;
            float v0 = x0[r], v1 = x1[r];
            if (nw) {
                v0 = nw[i0[r]] * (v0 * rn);
                v1 = nw[i1[r]] * (v1 * rn);
            }
            const float c = cs[i], sv = sn[i];
            const float y0 = fmaf(v0, c, -v1 * sv);
            const float y1 = fmaf(v0, sv, v1 * c);
            if (is_q) {
                uint16_t* q = a.q16 + (int64_t(s) * a.n_heads + h) * HD;
                q[i0[r]] = f2h(y0 * qs);
                q[i1[r]] = f2h(y1 * qs);
            } else {
                float* k = a.kc + (int64_t(g) * a.max_ctx + pos) * HD;
                k[i0[r]] = y0;
                k[i1[r]] = y1;
            }
        }
        if (!is_q) {
            const int voff = qd + kvd + g * HD;
            float* v = a.vc + (int64_t(g) * a.max_ctx + pos) * HD;
            for (int i = lane; i < HD; i += WAVE) v[i] = a.bias ? row[voff + i] + a.bias[voff + i] : row[voff + i];
        }
    }
}

// ---------------------------------------------------------------------------
// Causal flash attention over the cache for QB query rows and one KV head;
// each wave handles 16 * PF_RT rows of one query head of the group, so each
// K/V tile is staged once for every head and row of the block and each K / V
// fragment read from LDS feeds PF_RT MFMAs.
//
// Per tile of 64 (or 32) keys, on v_mfma_f32_16x16x32_f16:
//  * S^T = K Q^T (keys x queries; q arrives pre-scaled by log2(e)/sqrt(hd),
//    so scores are in base 2): per 32 keys lane l holds 8 keys of query
//    l%16, which is the layout P needs as the A operand of P V, so P never
//    leaves the registers; the P V operand pairs keys in the order
//    (l/16)*4 + i, 16 + (l/16)*4 + i, and V is read from LDS in the same
//    order.
//  * Online softmax with a lazy maximum: each lane keeps the running
//    maximum of its query and its own partial sum (the sum over the 4 lanes
//    of a query is taken once, at the end); the maximum moves, with a
//    cross-lane max and a rescale of O, only when some score of the wave's
//    tile exceeds it by more than RESCALE_SLACK, so weights stay below
//    2^slack. O / l is the same either way.
//  * Keys past each row's position (and before its window) are masked only
//    in tiles that reach past the block's first row (or before its last
//    row's window).
// The next tile's K and V rows are loaded into registers while the current
// one is computed (when they fit: 8 float4 per thread, 16 with one wave per
// SIMD). Query blocks
// run latest first: they have the most tiles.
//
// Lane layout of v_mfma_f32_16x16x32_f16 (checked on the device): lane l
// supplies A[l%16][(l/16)*8 + i] and B[(l/16)*8 + i][l%16] for i < 8 and
// receives C[(l/16)*4 + i][l%16] for i < 4.
// ---------------------------------------------------------------------------
// Work split: each wave takes PF_RT row tiles of 16 queries of one head;
// with up to four heads per KV head two waves share a head (the block then
// holds 2G waves, two per SIMD, so one wave's softmax overlaps the other's
// matrix work). Rows per block: 16 * PF_RT * waves per head.
template <int HD>
constexpr int attn_pf_rt() { return HD >= 256 ? 1 : 2; }
template <int G>
constexpr int attn_pf_wph() { return G <= 4 ? 2 : 1; }
template <int HD, int G>
constexpr int attn_pf_rows() { return 16 * attn_pf_rt<HD>() * attn_pf_wph<G>(); }
// Threads of a block: G heads x waves per head (the kernel's launch bound).
template <int G>
constexpr int attn_pf_threads() { return 64 * G * attn_pf_wph<G>(); }

// Float4 registers per thread for the next tile's K and V chunks: 8 with
// two waves per SIMD, 12 where some SIMDs hold one wave (5-7 waves), 16
// where a block has at most one wave per SIMD.
template <int G>
constexpr int attn_pf_prefetch_budget()
{
    return G * attn_pf_wph<G>() <= 4 ? 16 : G * attn_pf_wph<G>() < 8 ? 12 : 8;
}

// Keys per tile of the prefill attention: 64 where the next tile's K and V
// chunks still fit the register prefetch, else 32.
template <int HD, int G>
constexpr bool attn_pf_prefetch_fits(int tk)
{
    constexpr int KQ = HD < 32 ? 32 : HD;
    constexpr int NT = 64 * G * attn_pf_wph<G>();
    const int kpt = (tk * (KQ / 4) + NT - 1) / NT;
    const int vpt = ((tk / 2) * (HD / 4) + NT - 1) / NT;
    return kpt + 2 * vpt <= attn_pf_prefetch_budget<G>();
}
template <int HD, int G>
constexpr int attn_pf_tk() { return attn_pf_prefetch_fits<HD, G>(64) ? 64 : 32; }

// Slack (base-2 units) by which a score may exceed the running maximum
// before the maximum moves: weights stay below 2^8, well inside f16 for P.
constexpr float RESCALE_SLACK = 8.0f;

template <int HD, int G>
__global__ void __launch_bounds__(attn_pf_threads<G>())
attn_prefill_kernel(AttnPrefillArgs a)
{
    constexpr int KQ = HD < 32 ? 32 : HD;  // QK depth, zero padded to 32
    constexpr int TK = attn_pf_tk<HD, G>(); // keys per tile
    constexpr int KB = TK / 16;             // 16-key blocks of a tile
    constexpr int NP = TK / 32;             // 32-key halves: P V steps
    constexpr int DB = HD / 16;             // 16-wide output blocks
    constexpr int QB = attn_pf_rows<HD, G>();  // query rows per block
    constexpr int RT = attn_pf_rt<HD>();    // 16-row tiles per wave
    constexpr int WPH = attn_pf_wph<G>();   // waves per head
    constexpr int NT = 64 * G * WPH;        // threads
    constexpr int KE = TK * (KQ / 4);       // float4 chunks of a K tile (depth padded)
    constexpr int VE = (TK / 2) * (HD / 4); // row-pair chunks of a V tile
    constexpr int KPT = (KE + NT - 1) / NT; // per thread
    constexpr int VPT = (VE + NT - 1) / NT;
    constexpr bool PREF = KPT + 2 * VPT <= attn_pf_prefetch_budget<G>();  // next tile held in registers
    __shared__ __attribute__((aligned(16))) _Float16 Ks[TK][KQ + 8];
    __shared__ __attribute__((aligned(16))) _Float16 Vt[HD][TK + 8];
    const int qb = gridDim.x - 1 - blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int lg = l >> 4;    // lane group: keys lg*4 .. lg*4+3 of each 16
    const int lq = l & 15;    // this lane's query within a row tile
    const int w = tid >> 6;
    const int j = g * G + w % G;  // query head
    const int s0 = qb * QB;
    const int r0 = (w / G) * (16 * RT);  // this wave's first row within the block
    const int64_t head_base = int64_t(g) * a.max_ctx * HD;

    // Q fragments (the B operand of S^T): B[d = kq*32 + (l/16)*8 + i][q = l%16]
    // of row tile rt, 8 consecutive dims per 16-byte load.
    half8 qa[RT][KQ / 32];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int s = s0 + r0 + rt * 16 + lq;
#pragma unroll
        for (int kq = 0; kq < KQ / 32; ++kq) {
            const int d = kq * 32 + lg * 8;
            qa[rt][kq] = (s < a.S && d < HD)
                             ? *reinterpret_cast<const half8*>(a.q16 + (int64_t(s) * a.n_heads + j) * HD + d)
                             : half8{};
        }
    }
    f32x4 o[RT][DB];
    float mq[RT], lsum[RT];  // query rt*16 + l%16: running maximum, this lane's partial sum
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rt][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        mq[rt] = -INFINITY;
        lsum[rt] = 0.f;
    }

    const int s_last = min(a.S, s0 + QB) - 1;
    const int n_keys = a.p0 + s_last + 1;
    const int tiles = (n_keys + TK - 1) / TK;
    // With a window, keys before the first query row's window are skipped
    // whole tiles at a time and masked inside the first tile used.
    const int key_lo = a.window > 0 ? max(0, a.p0 + s0 - a.window + 1) : 0;
    const int kt0 = key_lo / TK;
    // Tiles whose keys all lie at or before the block's first row and, with
    // a window, inside its last row's window, need no mask.
    const int free_hi = a.p0 + s0 - (TK - 1);                            // t0 <= free_hi
    const int free_lo = a.window > 0 ? a.p0 + s0 + QB - a.window : 0;    // t0 >= free_lo

    // Tile loads: K chunk e (row e / (KQ/4), 4 dims), V row pair e (rows
    // 2 (e % (TK/2)) and +1, 4 dims at 4 (e / (TK/2))); rows past n_keys and
    // padded depth read as zero.
    float4 kr[PREF ? KPT : 1], vr0[PREF ? VPT : 1], vr1[PREF ? VPT : 1];
    // Per-thread tile offsets (row within the tile, element offset from the
    // head's row 0), fixed across tiles.
    int krow[PREF ? KPT : 1], vrow[PREF ? VPT : 1];
    const float* kbase[PREF ? KPT : 1];
    const float* vbase[PREF ? VPT : 1];
    if constexpr (PREF) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int e = tid + u * NT;
            const int r = e / (KQ / 4), c = (e % (KQ / 4)) * 4;
            krow[u] = (e < KE && c < HD) ? r : 1 << 30;  // never inside n_keys: reads zero
            kbase[u] = a.kc + head_base + int64_t(r) * HD + c;
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int e = tid + u * NT;
            const int r = (e % (TK / 2)) * 2, c = (e / (TK / 2)) * 4;
            vrow[u] = e < VE ? r : 1 << 30;
            vbase[u] = a.vc + head_base + int64_t(r) * HD + c;
        }
    }
    auto load_tile = [&](int kt) {
        const int t0 = kt * TK;
        const int64_t off = int64_t(t0) * HD;
#pragma unroll
        for (int u = 0; u < KPT; ++u)
            kr[u] = t0 + krow[u] < n_keys ? *reinterpret_cast<const float4*>(kbase[u] + off)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            vr0[u] = t0 + vrow[u] < n_keys ? *reinterpret_cast<const float4*>(vbase[u] + off)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
            vr1[u] = t0 + vrow[u] + 1 < n_keys ? *reinterpret_cast<const float4*>(vbase[u] + off + HD)
                                                : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    // K row-major f16 (4 halves per 8-byte store, consecutive threads on
    // consecutive addresses); V transposed: a thread writes rows (2i, 2i+1)
    // at 4 dims as 4 half pairs, consecutive threads on consecutive pairs of
    // one transposed row (no bank conflicts).
    auto store_k = [&](int r, int c, float4 kv) {
        *reinterpret_cast<uint2*>(&Ks[r][c]) = make_uint2(pack_h2(kv.x, kv.y), pack_h2(kv.z, kv.w));
    };
    auto store_v = [&](int r, int c, float4 v0, float4 v1) {
        *reinterpret_cast<uint32_t*>(&Vt[c][r]) = pack_h2(v0.x, v1.x);
        *reinterpret_cast<uint32_t*>(&Vt[c + 1][r]) = pack_h2(v0.y, v1.y);
        *reinterpret_cast<uint32_t*>(&Vt[c + 2][r]) = pack_h2(v0.z, v1.z);
        *reinterpret_cast<uint32_t*>(&Vt[c + 3][r]) = pack_h2(v0.w, v1.w);
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int e = tid + u * NT;
            if (e < KE) store_k(e / (KQ / 4), (e % (KQ / 4)) * 4, kr[u]);
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int e = tid + u * NT;
            if (e < VE) store_v((e % (TK / 2)) * 2, (e / (TK / 2)) * 4, vr0[u], vr1[u]);
        }
    };
    // Without the register prefetch: each thread converts its chunks one at
    // a time.
    auto stage_direct = [&](int kt) {
        const int t0 = kt * TK;
        for (int e = tid; e < KE; e += NT) {
            const int r = e / (KQ / 4), c = (e % (KQ / 4)) * 4;
            store_k(r, c, (t0 + r < n_keys && c < HD)
                              ? *reinterpret_cast<const float4*>(a.kc + head_base + int64_t(t0 + r) * HD + c)
                              : make_float4(0.f, 0.f, 0.f, 0.f));
        }
        for (int e = tid; e < VE; e += NT) {
            const int r = (e % (TK / 2)) * 2, c = (e / (TK / 2)) * 4;
            float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
            if (t0 + r < n_keys) v0 = *reinterpret_cast<const float4*>(a.vc + head_base + int64_t(t0 + r) * HD + c);
            if (t0 + r + 1 < n_keys) v1 = *reinterpret_cast<const float4*>(a.vc + head_base + int64_t(t0 + r + 1) * HD + c);
            store_v(r, c, v0, v1);
        }
    };

    if constexpr (PREF) {
        if (kt0 < tiles) load_tile(kt0);
    }
    for (int kt = kt0; kt < tiles; ++kt) {
        const int t0 = kt * TK;
        if constexpr (PREF) store_tile();
        else stage_direct(kt);
        __syncthreads();
        if constexpr (PREF) {
            if (kt + 1 < tiles) load_tile(kt + 1);  // in flight during this tile
        }
        // S^T[key = kb*16 + lg*4 + i][query = rt*16 + l%16], with the K
        // fragments as the A operand: A[key = kb*16 + l%16][d = kq*32 + (l/16)*8 + i].
        f32x4 st[RT][KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            half8 kf[KQ / 32];
#pragma unroll
            for (int kq = 0; kq < KQ / 32; ++kq)
                kf[kq] = *reinterpret_cast<const half8*>(&Ks[kb * 16 + lq][kq * 32 + lg * 8]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                st[rt][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kq = 0; kq < KQ / 32; ++kq)
                    st[rt][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[kq], qa[rt][kq], st[rt][kb], 0, 0, 0);
            }
        }
        const bool masked = t0 > free_hi || t0 < free_lo;  // uniform
        bool grow = false;
        float vmax[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (masked) {
                const int qpos = a.p0 + s0 + r0 + rt * 16 + lq;
                const int kmin = a.window > 0 ? qpos - a.window + 1 : 0;  // first key in the window
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = t0 + kb * 16 + lg * 4 + i;
                        if (key > qpos || key < kmin) st[rt][kb][i] = -INFINITY;
                    }
            }
            float vm = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                vm = fmaxf(vm, fmaxf(fmaxf(st[rt][kb][0], st[rt][kb][1]), fmaxf(st[rt][kb][2], st[rt][kb][3])));
            vmax[rt] = vm;
            grow |= vmax[rt] > mq[rt] + RESCALE_SLACK;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            // Move the maxima: the max of each query over its 4 lanes, the
            // partial sums and O's rows scaled by 2^(old - new).
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                float rm = fmaxf(vmax[rt], __shfl_xor(vmax[rt], 16, WAVE));
                rm = fmaxf(rm, __shfl_xor(rm, 32, WAVE));
                const float mn = fmaxf(mq[rt], rm);
                const float alpha = (mq[rt] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mq[rt] - mn);
                lsum[rt] *= alpha;
                mq[rt] = mn;
                // O row (l/16)*4 + i is query (l/16)*4 + i, whose alpha lane (l/16)*4 + i holds
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, lg * 4 + i, WAVE);
#pragma unroll
                    for (int db = 0; db < DB; ++db) o[rt][db][i] *= ai;
                }
            }
        }
        // P = 2^(s - m) in registers, as the A operand of P V: step h takes
        // keys 32h .. 32h + 31 in the slot order lg*8 + i: keys 32h + lg*4 + i,
        // then 32h + 16 + lg*4 + i. A masked score is -inf and gives 0; the
        // maximum is clamped to a finite value so that a row with no key yet
        // (maximum still -inf, all its scores masked) also gives 0 instead of
        // 2^NaN.
        half8 pa[RT][NP];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float mref = fmaxf(mq[rt], -1e30f);
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = __builtin_amdgcn_exp2f(st[rt][kb][i] - mref);
                    ps += pv;
                    pa[rt][kb >> 1][(kb & 1) * 4 + i] = static_cast<_Float16>(pv);
                }
            lsum[rt] += ps;
        }
        // V fragments in the same key order: B[slot][d = db*16 + l%16].
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int h = 0; h < NP; ++h) {
                const uint2 v0 = *reinterpret_cast<const uint2*>(&Vt[db * 16 + lq][32 * h + lg * 4]);
                const uint2 v1 = *reinterpret_cast<const uint2*>(&Vt[db * 16 + lq][32 * h + 16 + lg * 4]);
                const half8 vb = __builtin_bit_cast(half8, u32x4{v0.x, v0.y, v1.x, v1.y});
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    o[rt][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[rt][h], vb, o[rt][db], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    // O / l -> out[s][j*HD + d] in f16 (the o matmul's A operand); l of a
    // query is the sum of its 4 lanes' partial sums.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float lt = lsum[rt] + __shfl_xor(lsum[rt], 16, WAVE);
        lt += __shfl_xor(lt, 32, WAVE);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float li = __shfl(lt, lg * 4 + i, WAVE);
            const int s = s0 + r0 + rt * 16 + lg * 4 + i;
            if (s >= a.S) continue;
            const float inv = 1.0f / li;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = db * 16 + lq;
                a.out16[int64_t(s) * a.n_heads * HD + j * HD + d] = f2h(o[rt][db][i] * inv);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The same causal flash attention for head_dim 64 and 128, reading the f16
// copies of the cache (KvShadowArgs) with loads straight into LDS: no
// conversion, no transposition and no staging registers in the kernel. A
// 64-key tile holds K rows [64][hd] (16-byte chunks permuted by pf_swz_k) and
// V transposed [hd][64] (chunks permuted by (d >> 1) & 7); two tile buffers,
// the next tile's loads issued right after the barrier that opens the
// current tile. Inside S^T = K Q^T the 16 K rows of key block kb are
// permuted (pf_key) so that each lane's 8 P values of a 32-key half are 8
// consecutive keys: the V operand of P V is then one 16-byte read per lane.
// Each wave takes one 16-row query tile, so a block has 16 x (waves per
// head) query rows: twice the blocks of two tiles per wave, which evens out
// the causal imbalance where those would fill the compute units only once
// (2048 rows of 8 KV heads: 512 blocks instead of 256, the latest query
// blocks dispatched first), and four waves per SIMD fit in registers.
// Everything else (lazy maximum, masks, output) is as in attn_prefill_kernel.
// ---------------------------------------------------------------------------
constexpr int PFD_TK = 64;  // keys per tile

// Key (within the tile) of row m of key block kb in S^T: block kb = 2h + b
// takes, for lane group j = m / 4, keys 32h + 8j + 4b .. +3.
__device__ inline int pf_key(int kb, int m)
{
    return 32 * (kb >> 1) + (m >> 2) * 8 + (kb & 1) * 4 + (m & 3);
}

// Position of K chunk c of tile row r in its LDS row: c ^ pf_swz_k(r). The 16
// lanes of a fragment read take the 16 rows pf_key(kb, 0..15) at one chunk;
// a 16-byte-per-lane read is served 16 lanes at a time from 256 bytes of
// banks. hd 128 (one 256-byte row per bank line): the 16 rows get 16
// different positions. hd 64 (two rows per line): the 8 rows of each half
// get 8 different positions.
template <int HD>
__device__ inline int pf_swz_k(int r)
{
    if constexpr (HD == 128) return ((r >> 1) & 12) | (r & 3);
    else return ((r >> 1) & 1) | ((r >> 2) & 6);
}

// Raw buffer descriptor over `bytes` bytes from base (offsets at or past it
// read zeros).
__device__ inline __amdgpu_buffer_rsrc_t dma_rsrc_n(const uint16_t* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, int(bytes), BUF_RSRC_W3);
}

template <int HD, int G>
__global__ void __launch_bounds__(attn_pf_threads<G>()) __attribute__((amdgpu_waves_per_eu(4)))
attn_prefill_dma_kernel(AttnPrefillArgs a)
{
    static_assert(HD == 64 || HD == 128, "head_dim of the f16-copy attention");
    constexpr int TK = PFD_TK;
    constexpr int KB = TK / 16;             // 16-key blocks of a tile
    constexpr int NP = TK / 32;             // 32-key halves: P V steps
    constexpr int DB = HD / 16;             // 16-wide output blocks
    constexpr int RT = 1;                   // 16-row tiles per wave
    constexpr int QB = 16 * attn_pf_wph<G>();  // query rows per block
    constexpr int WPH = attn_pf_wph<G>();   // waves per head
    constexpr int NW = G * WPH;             // waves
    constexpr int CPR = HD / 8;             // 16-byte chunks of a K row
    constexpr int RPI = 64 / CPR;           // K rows one load instruction fills
    constexpr int NK = TK / RPI;            // K load instructions per tile
    constexpr int NV = HD / 8;              // V^T load instructions per tile (8 dims each)
    constexpr int NI = NK + NV;
    constexpr int MI = (NI + NW - 1) / NW;  // per wave, at most
    constexpr int TILE = 2 * TK * HD;       // halves per tile buffer: K, then V^T
    extern __shared__ _Float16 pfs[];
    // Blocks are dispatched to the 8 XCDs in turn (block b to XCD b % 8);
    // XCD x takes the x-th eighth of the (head, query block) pairs in head
    // order, so that its L2 holds one head's copies (2 MiB at 4096 rows and
    // head_dim 128) rather than tiles of every head. Within a head, the
    // latest query blocks (the most tiles) run first.
    const int nqb = gridDim.x;
    int qb, g;
    {
        const int total = nqb * int(gridDim.y);
        const int b = blockIdx.x + blockIdx.y * nqb;
        const int x = b & 7, y = b >> 3;
        const int base = total >> 3, rem = total & 7;
        const int t = x * base + min(x, rem) + y;
        g = t / nqb;
        qb = nqb - 1 - (t - g * nqb);
    }
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int lg = l >> 4;    // lane group: keys 8 lg .. 8 lg + 7 of each 32
    const int lq = l & 15;    // this lane's query within a row tile
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = g * G + w % G;  // query head
    const int s0 = qb * QB;
    const int r0 = (w / G) * (16 * RT);  // this wave's first row within the block
    const uint16_t* khead = a.k16 + int64_t(g) * a.max_ctx * HD;
    const uint16_t* vhead = a.vt16 + int64_t(g) * HD * a.max_ctx;

    // Q fragments (the B operand of S^T), as in attn_prefill_kernel.
    half8 qa[RT][HD / 32];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int s = s0 + r0 + rt * 16 + lq;
#pragma unroll
        for (int kq = 0; kq < HD / 32; ++kq) {
            const int d = kq * 32 + lg * 8;
            qa[rt][kq] = s < a.S ? *reinterpret_cast<const half8*>(a.q16 + (int64_t(s) * a.n_heads + j) * HD + d)
                                 : half8{};
        }
    }
    f32x4 o[RT][DB];
    float mq[RT], lsum[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rt][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        mq[rt] = -INFINITY;
        lsum[rt] = 0.f;
    }

    const int s_last = min(a.S, s0 + QB) - 1;
    const int n_keys = a.p0 + s_last + 1;
    const int tiles = (n_keys + TK - 1) / TK;
    const int key_lo = a.window > 0 ? max(0, a.p0 + s0 - a.window + 1) : 0;
    const int kt0 = key_lo / TK;
    const int free_hi = a.p0 + s0 - (TK - 1);
    const int free_lo = a.window > 0 ? a.p0 + s0 + QB - a.window : 0;

    // This wave's load instructions q = w, w + NW, ...: q < NK fills K rows
    // q*RPI .. +RPI-1 (lane l: row + l / CPR, position l % CPR); the others
    // fill V^T dims 8 (q - NK) .. +7 (lane l: dim + l / 8, position l % 8).
    // Byte offsets from the tile's first key, fixed for every tile.
    uint32_t voff[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int q = w + i * NW;
        if (q < NK) {
            const int row = q * RPI + l / CPR;
            const int c = (l % CPR) ^ pf_swz_k<HD>(row);
            voff[i] = uint32_t(row * HD + c * 8) * 2;
        } else {
            const int d = (q - NK) * 8 + (l >> 3);
            const int c = (l & 7) ^ ((d >> 1) & 7);
            voff[i] = uint32_t(int64_t(d) * a.max_ctx + c * 8) * 2;
        }
    }
    // Loads of tile kt into buffer buf. K rows at or past n_keys read zeros
    // (the descriptor ends there); V^T reads stop at the head's end, so the
    // last tile's V of keys past n_keys is whatever the copies hold there
    // (earlier contents, possibly not finite) and is set to 0 in LDS.
    auto issue = [&](int kt, int buf) {
        const int t0 = kt * TK;
        const __amdgpu_buffer_rsrc_t rk = dma_rsrc_n(khead + int64_t(t0) * HD, uint32_t(n_keys - t0) * HD * 2);
        const __amdgpu_buffer_rsrc_t rv = dma_rsrc_n(vhead + t0, uint32_t(int64_t(HD) * a.max_ctx - t0) * 2);
        _Float16* base = pfs + buf * TILE;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int q = w + i * NW;
            if (q < NK) dma16(rk, base + q * 512, voff[i], 0);
            else if (q < NI) dma16(rv, base + TK * HD + (q - NK) * 512, voff[i], 0);
        }
    };

    if (kt0 < tiles) issue(kt0, kt0 & 1);
    for (int kt = kt0; kt < tiles; ++kt) {
        const int t0 = kt * TK;
        wait_vmcnt<0>();  // this wave's loads of tile kt
        __syncthreads();  // every wave's: tile kt in LDS, and tile kt-1's buffer no longer read
        if (kt + 1 < tiles) {
            issue(kt + 1, (kt + 1) & 1);
        } else if (t0 + TK > n_keys) {  // uniform
            // The last tile's V of keys at or past n_keys: their P is 0, but
            // 0 times a stale infinity is not, so they are set to 0 first.
            _Float16* vz = pfs + (kt & 1) * TILE + TK * HD;
            const int k0 = n_keys - t0;
            for (int e = tid; e < HD * TK; e += NW * 64) {
                const int d = e / TK, k = e % TK;
                if (k >= k0) vz[d * TK + (((k >> 3) ^ ((d >> 1) & 7)) * 8) + (k & 7)] = static_cast<_Float16>(0.f);
            }
            __syncthreads();
        }
        const _Float16* Kl = pfs + (kt & 1) * TILE;
        const _Float16* Vl = Kl + TK * HD;
        // S^T[key = pf_key(kb, lg*4 + i)][query = rt*16 + l%16]. Depth step
        // kq outermost: the KB * RT accumulators in flight are independent,
        // so no MFMA waits for the previous one's result.
        f32x4 st[RT][KB];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) st[rt][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Each K fragment feeds one MFMA (one row tile per wave), so they
        // are read one depth step at a time: 16 registers rather than the
        // tile's 64, which keeps four waves per SIMD in registers. The
        // matrix sections run at raised wave priority: of the waves of a
        // SIMD, the one that reaches its MFMAs first keeps the matrix unit,
        // and the others' softmax overlaps them.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kq = 0; kq < HD / 32; ++kq) {
            half8 kf[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int row = pf_key(kb, lq);
                kf[kb] = *reinterpret_cast<const half8*>(Kl + row * HD + (((kq * 4 + lg) ^ pf_swz_k<HD>(row)) * 8));
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    st[rt][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[kb], qa[rt][kq], st[rt][kb], 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        const bool masked = t0 > free_hi || t0 < free_lo;  // uniform
        bool grow = false;
        float vmax[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (masked) {
                const int qpos = a.p0 + s0 + r0 + rt * 16 + lq;
                const int kmin = a.window > 0 ? qpos - a.window + 1 : 0;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = t0 + pf_key(kb, lg * 4 + i);
                        if (key > qpos || key < kmin) st[rt][kb][i] = -INFINITY;
                    }
            }
            float vm = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                vm = fmaxf(vm, fmaxf(fmaxf(st[rt][kb][0], st[rt][kb][1]), fmaxf(st[rt][kb][2], st[rt][kb][3])));
            vmax[rt] = vm;
            grow |= vmax[rt] > mq[rt] + RESCALE_SLACK;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                float rm = fmaxf(vmax[rt], __shfl_xor(vmax[rt], 16, WAVE));
                rm = fmaxf(rm, __shfl_xor(rm, 32, WAVE));
                const float mn = fmaxf(mq[rt], rm);
                const float alpha = (mq[rt] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mq[rt] - mn);
                lsum[rt] *= alpha;
                mq[rt] = mn;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, lg * 4 + i, WAVE);
#pragma unroll
                    for (int db = 0; db < DB; ++db) o[rt][db][i] *= ai;
                }
            }
        }
        // P in registers as the A operand of P V: step h, slot 4b + i holds
        // key 32h + 8 lg + 4b + i, which is row lg*4 + i of key block 2h + b.
        half8 pa[RT][NP];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float mref = fmaxf(mq[rt], -1e30f);
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = __builtin_amdgcn_exp2f(st[rt][kb][i] - mref);
                    ps += pv;
                    pa[rt][kb >> 1][(kb & 1) * 4 + i] = static_cast<_Float16>(pv);
                }
            lsum[rt] += ps;
        }
        // V fragments: B[slot][d = db*16 + l%16] = V^T[d][32h + 8 lg .. +7].
        // Half h outermost: consecutive MFMAs update different accumulators.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int h = 0; h < NP; ++h) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = db * 16 + lq;
                const half8 vb = *reinterpret_cast<const half8*>(Vl + d * TK + (((h * 4 + lg) ^ ((d >> 1) & 7)) * 8));
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    o[rt][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[rt][h], vb, o[rt][db], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float lt = lsum[rt] + __shfl_xor(lsum[rt], 16, WAVE);
        lt += __shfl_xor(lt, 32, WAVE);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float li = __shfl(lt, lg * 4 + i, WAVE);
            const int s = s0 + r0 + rt * 16 + lg * 4 + i;
            if (s >= a.S) continue;
            const float inv = 1.0f / li;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = db * 16 + lq;
                a.out16[int64_t(s) * a.n_heads * HD + j * HD + d] = f2h(o[rt][db][i] * inv);
            }
        }
    }
}

// f16 copies of cache rows (KvShadowArgs): block (tile, g) takes 64 rows of
// KV head g. K rows are converted in place, coalesced; V rows are converted
// into LDS and written out transposed, 64 consecutive positions per dim (one
// 128-byte run per wave store).
constexpr int KVS_ROWS = 64;
__global__ void __launch_bounds__(256)
kv_shadow_kernel(KvShadowArgs a)
{
    __shared__ uint16_t vs[KVS_ROWS][256 + 2];  // [row][dim]; the pad puts a column's rows in distinct banks
    const int g = blockIdx.y;
    const int hd = a.head_dim;
    const int r0 = a.pos0 + blockIdx.x * KVS_ROWS;
    const int nr = min(KVS_ROWS, a.pos0 + a.n - r0);
    const int64_t head = int64_t(g) * a.max_ctx * hd;
    const int tid = threadIdx.x;
    const int q4 = hd / 4;
    for (int e = tid; e < nr * q4; e += 256) {
        const int r = e / q4, c = (e % q4) * 4;
        const int64_t off = head + int64_t(r0 + r) * hd + c;
        if (a.do_k) {
            const float4 k = *reinterpret_cast<const float4*>(a.kc + off);
            *reinterpret_cast<uint2*>(a.k16 + off) = make_uint2(pack_h2(k.x, k.y), pack_h2(k.z, k.w));
        }
        if (a.do_v) {
            const float4 v = *reinterpret_cast<const float4*>(a.vc + off);
            *reinterpret_cast<uint32_t*>(&vs[r][c]) = pack_h2(v.x, v.y);
            *reinterpret_cast<uint32_t*>(&vs[r][c + 2]) = pack_h2(v.z, v.w);
        }
    }
    if (!a.do_v) return;  // uniform
    __syncthreads();
    const int lane = tid & 63, wv = tid >> 6;
    if (lane < nr) {
        uint16_t* vt = a.vt16 + int64_t(g) * hd * a.max_ctx + r0 + lane;
        for (int d = wv; d < hd; d += 4) vt[int64_t(d) * a.max_ctx] = vs[lane][d];
    }
}

template <int HD, int G>
dim3 pf_grid(const AttnPrefillArgs& a)
{
    return dim3((a.S + attn_pf_rows<HD, G>() - 1) / attn_pf_rows<HD, G>(), a.n_kv);
}

template <int HD, int G>
hipError_t launch_attn_prefill_dma(const AttnPrefillArgs& a, hipStream_t s)
{
    constexpr size_t lds = size_t(2) * 2 * PFD_TK * HD * 2;
    constexpr int QB = 16 * attn_pf_wph<G>();
    static std::atomic<bool> attr_set{false};  // sessions may launch from several threads
    if (!attr_set.load(std::memory_order_acquire)) {
        const hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_prefill_dma_kernel<HD, G>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (r != hipSuccess) return r;
        attr_set.store(true, std::memory_order_release);
    }
    DFK_LAUNCH((attn_prefill_dma_kernel<HD, G>), dim3((a.S + QB - 1) / QB, a.n_kv), dim3(attn_pf_threads<G>()), lds,
               s, a);
    return hipGetLastError();
}

template <int HD>
hipError_t launch_attn_prefill_hd(const AttnPrefillArgs& a, hipStream_t s)
{
    if constexpr (HD == 64 || HD == 128) {
        if (a.k16 && a.vt16) {
            switch (a.n_heads / a.n_kv) {
            case 1: return launch_attn_prefill_dma<HD, 1>(a, s);
            case 2: return launch_attn_prefill_dma<HD, 2>(a, s);
            case 3: return launch_attn_prefill_dma<HD, 3>(a, s);
            case 4: return launch_attn_prefill_dma<HD, 4>(a, s);
            case 5: return launch_attn_prefill_dma<HD, 5>(a, s);
            case 6: return launch_attn_prefill_dma<HD, 6>(a, s);
            case 7: return launch_attn_prefill_dma<HD, 7>(a, s);
            case 8: return launch_attn_prefill_dma<HD, 8>(a, s);
            default: return hipErrorInvalidValue;
            }
        }
    }
    switch (a.n_heads / a.n_kv) {
    case 1: DFK_LAUNCH((attn_prefill_kernel<HD, 1>), (pf_grid<HD, 1>(a)), dim3(attn_pf_threads<1>()), 0, s, a); break;
    case 2: DFK_LAUNCH((attn_prefill_kernel<HD, 2>), (pf_grid<HD, 2>(a)), dim3(attn_pf_threads<2>()), 0, s, a); break;
    case 3: DFK_LAUNCH((attn_prefill_kernel<HD, 3>), (pf_grid<HD, 3>(a)), dim3(attn_pf_threads<3>()), 0, s, a); break;
    case 4: DFK_LAUNCH((attn_prefill_kernel<HD, 4>), (pf_grid<HD, 4>(a)), dim3(attn_pf_threads<4>()), 0, s, a); break;
    case 5: DFK_LAUNCH((attn_prefill_kernel<HD, 5>), (pf_grid<HD, 5>(a)), dim3(attn_pf_threads<5>()), 0, s, a); break;
    case 6: DFK_LAUNCH((attn_prefill_kernel<HD, 6>), (pf_grid<HD, 6>(a)), dim3(attn_pf_threads<6>()), 0, s, a); break;
    case 7: DFK_LAUNCH((attn_prefill_kernel<HD, 7>), (pf_grid<HD, 7>(a)), dim3(attn_pf_threads<7>()), 0, s, a); break;
    case 8: DFK_LAUNCH((attn_prefill_kernel<HD, 8>), (pf_grid<HD, 8>(a)), dim3(attn_pf_threads<8>()), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant_q8(const void* values, const uint16_t* scales, int64_t rows, int64_t cols,
                             uint16_t* out, hipStream_t s)
{
    if (rows <= 0 || cols <= 0) return hipSuccess;
    if (cols % 32 != 0) return hipErrorInvalidValue;
    const int64_t per_row = cols / 8;  // 8 values per thread
    const dim3 grid(unsigned((per_row + 255) / 256), unsigned(rows < 65535 ? rows : 65535));
    DFK_LAUNCH(dequant_q8_kernel, grid, dim3(256), 0, s, static_cast<const int8_t*>(values), scales, rows, cols,
               out);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const float* x, const float* w, int rows, int d, float eps,
                               uint16_t* out, hipStream_t s)
{
    if (rows <= 0) return hipSuccess;
    DFK_LAUNCH(rmsnorm_rows_kernel, dim3(rows), dim3(256), 0, s, x, w, d, eps, out);
    return hipGetLastError();
}

// Compute units of the current device (once; 256 on MI355X).
int gemm_cu_count()
{
    static std::atomic<int> n{0};
    int v = n.load(std::memory_order_relaxed);
    if (v == 0) {
        int dev = 0, c = 0;
        v = (hipGetDevice(&dev) == hipSuccess &&
             hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
                ? c
                : 256;
        n.store(v, std::memory_order_relaxed);
    }
    return v;
}

// The direct-to-LDS kernel runs whole 64-deep stages and addresses each
// operand with 32-bit byte offsets below DMA_RANGE; A is [M][lda],
// B [N (+ up_rows)][ldb], f16.
static bool gemm_dma_fits(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t up_rows, int mode)
{
    const int64_t brows = N + (mode == GEMM_SWIGLU_F16 ? up_rows : 0);
    return K % GDK == 0 && M * lda * 2 < DMA_RANGE && brows * ldb * 2 < DMA_RANGE;
}

// Tile code and K split of an M x N x K problem.
static int gemm_tile_plan(int64_t M, int64_t N, int64_t K, int64_t up_rows, int mode, bool q8, int* split)
{
    *split = 1;
    if (M <= 0 || N <= 0) return 0;
    // Every large tile runs one block per compute unit, so a GEMM takes
    // ceil(tiles / units) rounds of its tile's time. Tile times relative to
    // a 256 x 256 tile (8 waves of 128 x 64), measured on the 8B shapes:
    // 128 x 256 (8 waves of 64 x 64) 0.68, 256 x 192 (8 waves of 64 x 96,
    // operands loaded straight into LDS; not with the SwiGLU epilogue) 0.88.
    // The fewest estimated tile-times win, 256 x 256 unless another is 5%
    // faster; 128 x 128 on 4 waves for small problems. E.g. q/k/v of the 8B
    // shapes (N 6144) at 4096 rows: 384 tiles of 256 x 256 in 2 rounds (2),
    // 768 of 128 x 256 in 3 (2.04), 512 of 256 x 192 in 2 full rounds (1.76).
    const int64_t cols = mode == GEMM_SWIGLU_F16 ? 128 : 256;  // output columns of a 256-wide B tile
    const int64_t nt = (N + cols - 1) / cols;
    const int64_t cu = gemm_cu_count();
    const int64_t t2 = ((M + 255) / 256) * nt, t1 = ((M + 127) / 128) * nt;
    // f16 weights on 256-row tiles load straight into LDS (where K is a
    // multiple of 64 and the operands fit its 32-bit offsets; the operands
    // are contiguous, K elements per row); 8-bit blocks (dequantised on their way into LDS)
    // and the smaller tiles use the register-staged kernel.
    const bool dma = !q8 && gemm_dma_fits(M, N, K, K, K, up_rows, mode);
    int tile = GEMM_PLAN_128x128;
    if (t1 >= 64) {
        const double r2 = double((t2 + cu - 1) / cu);
        const double r1 = double((t1 + cu - 1) / cu) * 0.68;
        double r3 = 1e30;
        if (dma && mode != GEMM_SWIGLU_F16) {
            const int64_t t3 = ((M + 255) / 256) * ((N + 191) / 192);
            r3 = double((t3 + cu - 1) / cu) * 0.88;
        }
        if (std::min(r1, r3) >= r2 * 0.95) tile = dma ? GEMM_PLAN_256x256_LDS : GEMM_PLAN_256x256;
        else tile = r3 < r1 ? GEMM_PLAN_256x192_LDS : GEMM_PLAN_128x256;
    }
    // A grid of the register-staged 128-row tiles that fills at most half of
    // the compute units splits each tile's K loop over up to GEMM_SPLIT_MAX
    // work-groups; their partial sums (64 or 128 KiB per work-group) are
    // stored and added by the last one, which costs about 25 us whatever
    // the split (measured), against a tile's 1.0 us (128 x 128) or 1.7 us
    // (128 x 256) per 64-deep stage: split where that saves over a tenth.
    // E.g. the 8B shapes at 1024 rows (8-bit blocks): o and down on 128
    // tiles of 128 x 256 in 2 (o 109 -> 84 us, down 327 -> 201); qwen3-0.6B
    // at 512 rows: down (K 3072) in 4 (51 -> 39 us), o (K 2048) not (4
    // measured 32 -> 36 us).
    if (tile == GEMM_PLAN_128x128 || tile == GEMM_PLAN_128x256) {
        const int64_t tiles = tile == GEMM_PLAN_128x256 ? t1 : ((M + 127) / 128) * ((N + (cols / 2) - 1) / (cols / 2));
        const int64_t nst = (K + GBK - 1) / GBK;
        if (tiles > 0 && tiles * 2 <= cu && tiles <= GEMM_SPLIT_TICKETS) {
            const double t = double(nst) * (tile == GEMM_PLAN_128x256 ? 1.7 : 1.0);
            double best = 0.1 * t;
            for (int sp = 2; sp <= GEMM_SPLIT_MAX && sp <= cu / tiles && nst / sp >= 8; ++sp) {
                const double save = t * (1.0 - 1.0 / sp) - 25.0;
                if (save > best) {
                    best = save;
                    *split = sp;
                }
            }
        }
    }
    return tile;
}

int gemm_plan(int64_t M, int64_t N, int64_t K, int64_t up_rows, int mode, bool q8)
{
    int split;
    const int tile = gemm_tile_plan(M, N, K, up_rows, mode, q8, &split);
    if (!tile) return 0;
    return tile | (q8 ? GEMM_PLAN_Q8_IN_GEMM : 0) | (split << GEMM_PLAN_SPLIT_SHIFT);
}

size_t gemm_split_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t up_rows, int mode, bool q8)
{
    int split;
    const int tile = gemm_tile_plan(M, N, K, up_rows, mode, q8, &split);
    if (split <= 1) return 0;
    const int64_t bn = tile == GEMM_PLAN_128x256 ? 256 : 128;
    const int64_t ncols = mode == GEMM_SWIGLU_F16 ? bn / 2 : bn;
    const int64_t tiles = ((M + 127) / 128) * ((N + ncols - 1) / ncols);
    return size_t(tiles) * size_t(split) * 128 * size_t(bn) * sizeof(float);
}

hipError_t launch_gemm(const GemmArgs& g, int mode, hipStream_t s)
{
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    int split;
    const int plan = gemm_tile_plan(g.M, g.N, g.K, g.up_rows, mode, g.Bsc != nullptr, &split);
    const int shape = plan == GEMM_PLAN_128x128 ? 0 : plan == GEMM_PLAN_128x256 ? 1 : 2;
    // the split needs the caller's partial-sum space and tickets
    GemmArgs ga = g;
    ga.split = split > 1 && g.ws && g.tickets ? split : 1;
    // the plan assumes contiguous f16 operands; other strides, and 8-bit
    // weights (g.Bsc: an int8 plane half the size an f16 load would read),
    // never take the direct-to-LDS kernels
    const bool fits = g.Bsc == nullptr && gemm_dma_fits(g.M, g.N, g.K, g.lda, g.ldb, g.up_rows, mode);
    const bool dma = plan == GEMM_PLAN_256x256_LDS && fits;
    if (plan == GEMM_PLAN_256x192_LDS && mode != GEMM_SWIGLU_F16) {
        switch (mode) {
        case GEMM_STORE_F32:
            return fits ? launch_gemm_dma<256, 192, 4, 2, GEMM_STORE_F32>(ga, s)
                        : launch_gemm_t<128, 256, 4, GEMM_STORE_F32>(ga, false, s);
        case GEMM_ADD_F32:
            return fits ? launch_gemm_dma<256, 192, 4, 2, GEMM_ADD_F32>(ga, s)
                        : launch_gemm_t<128, 256, 4, GEMM_ADD_F32>(ga, false, s);
        case GEMM_STORE_F16:
            return fits ? launch_gemm_dma<256, 192, 4, 2, GEMM_STORE_F16>(ga, s)
                        : launch_gemm_t<128, 256, 4, GEMM_STORE_F16>(ga, false, s);
        }
    }
#define DF_GEMM_BY_SHAPE(MODE_)                                                  \
    return shape == 2   ? launch_gemm_t<256, 256, 4, MODE_>(ga, dma, s)          \
           : shape == 1 ? launch_gemm_t<128, 256, 4, MODE_>(ga, false, s)        \
                        : launch_gemm_t<GBM_, GBN_, 2, MODE_>(ga, false, s);
    switch (mode) {
    case GEMM_STORE_F32: DF_GEMM_BY_SHAPE(GEMM_STORE_F32)
    case GEMM_ADD_F32: DF_GEMM_BY_SHAPE(GEMM_ADD_F32)
    case GEMM_STORE_F16: DF_GEMM_BY_SHAPE(GEMM_STORE_F16)
    case GEMM_SWIGLU_F16: DF_GEMM_BY_SHAPE(GEMM_SWIGLU_F16)
    }
#undef DF_GEMM_BY_SHAPE
    return hipErrorInvalidValue;
}

hipError_t launch_qk_post_rows(const QkPostArgs& a, hipStream_t s)
{
    if (a.S <= 0) return hipSuccess;
    if (a.head_dim > 4 * WAVE) return hipErrorInvalidValue;  // two rope pairs per lane at most
    DFK_LAUNCH(qk_post_rows_kernel, dim3(a.S), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_kv_shadow(const KvShadowArgs& a, hipStream_t s)
{
    if (a.n <= 0) return hipSuccess;
    if (a.head_dim > 256 || a.head_dim % 4 != 0) return hipErrorInvalidValue;
    DFK_LAUNCH(kv_shadow_kernel, dim3((a.n + KVS_ROWS - 1) / KVS_ROWS, a.n_kv), dim3(256), 0, s, a);
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
