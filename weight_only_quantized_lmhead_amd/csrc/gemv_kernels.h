// Lane-per-row GEMV for one to four activation rows (the decode case):
// y[m,v] = sum_k x[m,k] * q[v,k] * s[v,k/G] (+ bias[v]).
//
// vLLM PR #48870, review comment, point 1: at one activation row the time is
// set by the bytes read from HBM, so this kernel is built to look like a plain
// read stream: every weight load of a wave is issued before its first
// arithmetic instruction, the activation needs no staging barrier, and the
// launch has many short waves (measured on the 151936 x 1024 int4 g64 head:
// the same load pattern with the arithmetic removed reads 83 MB in 13.8 us,
// as fast as a bare read-only kernel).
//
// Work layout.  A workgroup is 8 waves.  A 64-row block of the vocabulary is
// split along K over KS waves (KS = 8, 4, 2 or 1, chosen per head at run
// time): wave ks of the block takes the NCs = NC / KS superchunks
// [ks NCs, (ks + 1) NCs), and a lane owns one vocabulary row of the block and
// reads its 16-byte slots (64 lanes = 1 KiB contiguous per load instruction).
// The KS partial results meet in LDS and are added in wave order, so the
// result does not depend on timing.  A wave with one or two superchunks
// (NCB = 1, 2) requests all of them up front; with more, either two register
// buffers alternate, the next superchunk in flight while one is computed
// (NCB = 0), or (NCB = -1, the forced 3- and 4-row variants, whose registers
// would not hold two buffers) each superchunk is loaded and then computed.
//
// Activations (XM).  One fp16 row is read with wave-uniform loads (XM = 0:
// the scalar unit; each 16-byte piece of x is the same for all 64 lanes), so
// no staging barrier precedes the arithmetic.  Several fp16 rows are staged
// once per workgroup in LDS (XM = 1; read back as 16-byte broadcasts), which
// keeps them out of the scalar registers.  bf16 rows (XM = 2) are staged in
// LDS as fp16 x * 2^-e with a power-of-two row exponent e that puts max|x| in
// [2^14, 2^15), computed here; the result is scaled back by 2^e (exact; values
// below 2^-17 after scaling lose bits).
//
// Groups.  When a wave's superchunks cover whole scale groups, the wave
// scales them itself (one fp32 FMA per group on the group's fp32 partial
// sum); when a group spans several waves (FRAC, e.g. one scale per row), each
// wave passes its unscaled partial sum and the reduction adds the partials
// of a group before its scale is applied.
//
// TK (top-K epilogue, fp32 logits, one activation row): the wave that holds a
// block's final 64 logits also writes that block's T largest as a sorted list
// of order codes (value descending, then index ascending; see topk_code),
// entry j at lists[(m*T + j)*NB + blk] (entry-major, so that the merge reads
// the lists' heads as one contiguous run): each lane ranks its own code
// against the 64 codes of the wave (staged in LDS and read back as broadcasts,
// two per read), and the lanes of rank < T store.  Rows past V take codes below every real
// entry.  y may then be null (logits not stored).
#pragma once

#include "logits_common.h"

namespace lmh {
namespace {

constexpr int kGemvWaves = 8;

// (a & mask) | orv as one v_and_or_b32, like and_or(), but not volatile: a
// volatile statement keeps its place among the others, which made the
// scheduler unpack every code of a wave's superchunks before the first dot
// product and spill them.
__device__ __forceinline__ uint32_t and_or_free(uint32_t a, uint32_t mask, uint32_t orv) {
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask), "v"(orv));
    return d;
}

// unpack_i4 with the freely scheduled AND-OR.
__device__ __forceinline__ void unpack_i4_free(uint32_t w, uint32_t magic, const ZC& zc, h2& p0,
                                               h2& p1, h2& p2, h2& p3) {
    const uint32_t hi = w >> 8;
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    p0 = __builtin_bit_cast(h2, and_or_free(w, 0x000F000Fu, magic)) + zc.lo;
    p1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or_free(w, 0x00F000F0u, magic)),
                                   sixteenth, zc.hi);
    p2 = __builtin_bit_cast(h2, and_or_free(hi, 0x000F000Fu, magic)) + zc.lo;
    p3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or_free(hi, 0x00F000F0u, magic)),
                                   sixteenth, zc.hi);
}

// Ordering points for the scheduler (empty volatile statements keep their
// order among themselves): order_after makes `r` count as rewritten after
// `dep` is available, so nothing computed from r moves above it; used_here
// makes `v` count as read at this point, so its computation cannot sink below
// it.  Together they run one 32-column chunk at a time -- its code words
// unpacked after the previous chunk's dot products, its dot products before
// the next chunk's unpacking (the scheduler otherwise unpacks every code of a
// superchunk first, or sinks the dot products, and keeps everything live).
__device__ __forceinline__ void order_after(uint32_t& r, float dep) {
    asm volatile("" : "+v"(r) : "v"(dep));
}
__device__ __forceinline__ void used_here(float v) { asm volatile("" ::"v"(v)); }

// Largest |x| of eight bf16 values, as bits (the order of non-negative bf16
// bit patterns is the order of their values).
__device__ __forceinline__ uint32_t bf16x8_absmax(const uint4& v) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w = word_of(v, j);
        m = max(m, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
    }
    return m;
}

// One superchunk of one lane's row as loaded: its 4 slots, the scales of its
// groups and (ZP) their zero points.
template <int GPS>
struct GemvBuf {
    uint4 w[4];
    uint16_t s[GPS];
    uint32_t z[GPS];
};

// Register budget: the waves per SIMD the compiler must leave room for.  The
// one-superchunk, one-row variant (the decode case) fits 8 (64 VGPRs;
// measured 3 % faster than 7); the others keep what they need (capped, they
// spill).
template <int MM, int XM, int NCB>
constexpr int gemv_occupancy() { return XM == 0 && NCB == 1 ? 8 : 1; }

template <int BITS, int MM, int GPS, int NCB, int OUT, bool ZP, bool TK, int XM>
__global__ __launch_bounds__(64 * kGemvWaves)
__attribute__((amdgpu_waves_per_eu(gemv_occupancy<MM, XM, NCB>()))) void gemv_kernel(
    const uint4* __restrict__ wq, const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zq,
    const uint16_t* __restrict__ xg, const float* __restrict__ bias, void* __restrict__ y,
    int64_t ldy, int V, int K, int NB, int NC, int NG, int SPG, int sbf16, int lks, int frac,
    u64* __restrict__ lists, int T) {
    constexpr int SPAN = span_of(BITS);
    constexpr int CPS = SPAN / 32;    // 32-column chunks per superchunk
    constexpr int CPG = CPS / GPS;    // chunks per group
    constexpr int NA = MM == 1 ? 4 : (MM == 2 ? 2 : 1);  // independent partial sums per group
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KS = 1 << lks;
    const int blk_raw = (blockIdx.x << (3 - lks)) + (wv >> lks);
    const int ks = wv & (KS - 1);
    const bool live = blk_raw < NB;
    const int blk = live ? blk_raw : NB - 1;  // dead waves read a real block, store nothing
    const int NCs = NC >> lks;
    const int c0 = ks * NCs, cend = c0 + NCs;
    const bool fr = GPS == 1 && frac != 0;
    const uint4* wp = wq + (int64_t)blk * NC * 256 + lane;
    const uint16_t* sp = sc + (int64_t)blk * NG * 64 + lane;
    // zero point of row `lane` in group g: byte (blk*NG + g)*64 + 4*(lane%16) + lane/16
    const uint8_t* zp = ZP ? zq + (int64_t)blk * NG * 64 + 4 * (lane & 15) + (lane >> 4) : nullptr;
    const int Kh = K >> 1;
    const uint32_t magic = 0x64006400u;

    auto load = [&](GemvBuf<GPS>& d, int c) {
#pragma unroll
        for (int t = 0; t < 4; ++t) d.w[t] = wp[((int64_t)c * 4 + t) * 64];
#pragma unroll
        for (int g = 0; g < GPS; ++g) {
            const int64_t gi = GPS > 1 ? (int64_t)c * GPS + g : (int64_t)(c / SPG);
            d.s[g] = sp[gi * 64];
            if constexpr (ZP) d.z[g] = zp[gi * 64];
        }
    };

    constexpr bool XL = XM == 2;       // bf16 rows, converted here
    extern __shared__ uint4 xs_raw[];  // XM = 1, 2: the rows as fp16, MM x K
    const h2* xl = (const h2*)xs_raw;
    const h2* xh = (const h2*)xg;
    int xe[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) xe[m] = 0;
    // the rows into LDS (every wave of the workgroup takes part): fp16 rows as
    // they are, bf16 rows as fp16 x * 2^-e
    __shared__ uint32_t mx_s[kGemvWaves][MM];
    auto stage_x = [&]() {
        const uint4* src = (const uint4*)xg;
        const int P = K >> 3;
        if constexpr (XM == 1) {
            for (int i = threadIdx.x; i < MM * P; i += 64 * kGemvWaves) xs_raw[i] = src[i];
            __syncthreads();
            return;
        }
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            uint32_t mx = 0;
            for (int i = threadIdx.x; i < P; i += 64 * kGemvWaves) mx = max(mx, bf16x8_absmax(src[m * P + i]));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
            if (lane == 0) mx_s[wv][m] = mx;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            uint32_t mx = 0;
#pragma unroll
            for (int w = 0; w < kGemvWaves; ++w) mx = max(mx, mx_s[w][m]);
            const float amax = __uint_as_float(mx << 16);
            int e = 0;
            if (amax > 0.0f) {
                int E;
                frexpf(amax, &E);  // amax = f * 2^E, f in [0.5, 1)
                e = E - 15;        // amax * 2^-e in [2^14, 2^15)
            }
            xe[m] = e;
            for (int i = threadIdx.x; i < P; i += 64 * kGemvWaves) {
                const uint4 v = src[m * P + i];
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w = word_of(v, j);
                    const _Float16 lo = (_Float16)ldexpf(__uint_as_float(w << 16), -e);
                    const _Float16 hi = (_Float16)ldexpf(__uint_as_float(w & 0xFFFF0000u), -e);
                    o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                xs_raw[m * P + i] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
        __syncthreads();
    };

    float acc[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[m] = 0.0f;
    auto compute = [&](const GemvBuf<GPS>& d, int c) {
        float part[MM][GPS][NA];
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int g = 0; g < GPS; ++g)
#pragma unroll
                for (int a = 0; a < NA; ++a) part[m][g][a] = 0.0f;
        ZC zc[GPS];
#pragma unroll
        for (int g = 0; g < GPS; ++g) zc[g] = ZP ? zc_byte(d.z[g], 0) : zc_sym<BITS>();
        const int xc = c * (SPAN / 2);  // half2 index of the superchunk's first column
        // The 32-column chunks are unpacked one after the other: a chunk's
        // code words pass an ordering point after the previous chunk's last
        // unpacked pair (for the first chunk, after the running result), so
        // one chunk's codes are live at a time.  (Requesting x a chunk ahead
        // as well was measured slower.)
        float dep = acc[0];
#pragma unroll
        for (int j = 0; j < CPS; ++j) {
            // LDS-staged x: its reads for this chunk pass the same ordering
            // point (the scalar loads of XM = 0 need none)
            uint32_t xo = (uint32_t)(xc + 16 * j) * 4u;  // byte offset of the chunk's x
            if constexpr (XM != 0) order_after(xo, dep);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                h2 p0, p1, p2, p3;
                if constexpr (BITS == 4) {
                    uint32_t w = word_of(d.w[t], j);
                    order_after(w, dep);
                    unpack_i4_free(w, magic, zc[j / CPG], p0, p1, p2, p3);
                } else {
                    uint32_t w0 = word_of(d.w[t], 2 * j), w1 = word_of(d.w[t], 2 * j + 1);
                    order_after(w0, dep);
                    order_after(w1, dep);
                    unpack_i8(w0, zc[j / CPG], p0, p1);
                    unpack_i8(w1, zc[j / CPG], p2, p3);
                }
                if (t == 3) dep = __builtin_bit_cast(float, p3);
                const int xi = xc + 16 * j + 4 * t;  // columns span*c + 32j + 8t
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    const uint4 xv =
                        XM == 0 ? *(const uint4*)(xh + m * Kh + xi)
                                : *(const uint4*)((const char*)xl + xo + 16u * t + 2u * (uint32_t)(m * K));
                    float a = part[m][j / CPG][t % NA];
                    a = __builtin_amdgcn_fdot2(p0, __builtin_bit_cast(h2, xv.x), a, false);
                    a = __builtin_amdgcn_fdot2(p1, __builtin_bit_cast(h2, xv.y), a, false);
                    a = __builtin_amdgcn_fdot2(p2, __builtin_bit_cast(h2, xv.z), a, false);
                    a = __builtin_amdgcn_fdot2(p3, __builtin_bit_cast(h2, xv.w), a, false);
                    part[m][j / CPG][t % NA] = a;
                }
            }
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int a = 0; a < NA; ++a) used_here(part[m][j / CPG][a]);
        }
#pragma unroll
        for (int g = 0; g < GPS; ++g) {
            const float sv = scale_to_f32(d.s[g], sbf16);
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float q = part[m][g][0];
#pragma unroll
                for (int a = 1; a < NA; ++a) q += part[m][g][a];
                acc[m] = fr ? acc[m] + q : fmaf(sv, q, acc[m]);
            }
        }
    };

    float gs = 0.0f;  // FRAC: the scale of the wave's group
    if constexpr (NCB > 0) {
        GemvBuf<GPS> b[NCB];
#pragma unroll
        for (int i = 0; i < NCB; ++i) load(b[i], c0 + i);
        if constexpr (XM != 0) stage_x();
#pragma unroll
        for (int i = 0; i < NCB; ++i) {
            compute(b[i], c0 + i);
            __builtin_amdgcn_sched_barrier(0);
        }
        gs = scale_to_f32(b[0].s[0], sbf16);
    } else if constexpr (NCB < 0) {
        GemvBuf<GPS> A;
        load(A, c0);
        if constexpr (XM != 0) stage_x();
        gs = scale_to_f32(A.s[0], sbf16);
#pragma unroll 1
        for (int c = c0; c < cend; ++c) {
            if (c > c0) load(A, c);
            compute(A, c);
        }
    } else {
        GemvBuf<GPS> A, B;
        load(A, c0);
        if constexpr (XM != 0) stage_x();
        gs = scale_to_f32(A.s[0], sbf16);
        int c = c0;
#pragma unroll 1
        for (; c + 1 < cend; c += 2) {
            load(B, c + 1);
            compute(A, c);
            __builtin_amdgcn_sched_barrier(0);
            if (c + 2 < cend) load(A, c + 2);
            compute(B, c + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (c < cend) compute(A, c);
    }

    if (KS > 1) {
        __shared__ float red[kGemvWaves][MM][64];
        __shared__ float gsc[kGemvWaves][64];
#pragma unroll
        for (int m = 0; m < MM; ++m) red[wv][m][lane] = acc[m];
        if (fr) gsc[wv][lane] = gs;
        __syncthreads();
        if (ks != 0) return;
        if (!fr) {
            // all partials read at once (unrolled over the largest split, the
            // unused ones masked), then added in wave order
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float pk[kGemvWaves];
#pragma unroll
                for (int k = 0; k < kGemvWaves; ++k) pk[k] = red[(wv + k) & (kGemvWaves - 1)][m][lane];
                float r = pk[0];
#pragma unroll
                for (int k = 1; k < kGemvWaves; ++k)
                    if (k < KS) r += pk[k];
                acc[m] = r;
            }
        } else {
            // W waves per group: add a group's partials, then scale it
            const int W = SPG / NCs;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float r = 0.0f;
                for (int k0 = 0; k0 < KS; k0 += W) {
                    float p = red[wv + k0][m][lane];
                    for (int k = 1; k < W; ++k) p += red[wv + k0 + k][m][lane];
                    r = fmaf(gsc[wv + k0][lane], p, r);
                }
                acc[m] = r;
            }
        }
    }
    const int v = blk * 64 + lane;
    if constexpr (!TK) {
        if (live && v < V) {
            const float b = bias ? bias[v] : 0.0f;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float r = acc[m];
                if constexpr (XL) r = ldexpf(r, xe[m]);
                ((YT<OUT>*)y)[(int64_t)m * ldy + v] = to_out<OUT>(r + b);
            }
        }
    } else {
        static_assert(OUT == F32, "the top-K epilogue ranks fp32 logits");
        if (!live) return;  // wave-uniform: every lane of the wave takes part below
        const float b = (bias && v < V) ? bias[v] : 0.0f;
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            float r = acc[m];
            if constexpr (XL) r = ldexpf(r, xe[m]);
            r = r + b;
            if (y && v < V) ((float*)y)[(int64_t)m * ldy + v] = r;
            const u64 c = v < V ? topk_code(r, v) : (u64)(64 - lane);
            // the wave's 64 codes through LDS, read back two at a time as
            // broadcasts (one wave's LDS operations are done in order), so
            // each code costs one 64-bit compare and one add
            __shared__ __attribute__((aligned(16))) u64 tkc[kGemvWaves][64];
            tkc[wv][lane] = c;
            int rank = 0;
#pragma unroll
            for (int j = 0; j < 64; j += 2) {
                const uint4 two = *(const uint4*)&tkc[wv][j];
                const u64 c0 = ((u64)two.y << 32) | two.x, c1 = ((u64)two.w << 32) | two.z;
                rank += (int)(c0 > c) + (int)(c1 > c);
            }
            if (rank < T) lists[((int64_t)m * T + rank) * NB + blk] = c;
        }
    }
}

// K split of a head: the largest KS <= 8 (a power of two dividing the
// superchunk count) whose per-wave range covers whole groups or lies inside
// one group; KS = 1 always qualifies.
inline void gemv_split(int NC, int SPG, int& lks, int& frac) {
    for (int l = 3; l >= 0; --l) {
        const int ks = 1 << l;
        if (NC % ks != 0) continue;
        const int ncs = NC / ks;
        if (ncs % SPG == 0) {
            lks = l;
            frac = 0;
            return;
        }
        if (SPG % ncs == 0) {
            lks = l;
            frac = 1;
            return;
        }
    }
    lks = 0;
    frac = 0;
}

template <int BITS, int MM, int GPS, int OUT, bool ZP>
hipError_t gemv_launch(const LogitsArgs& a, hipStream_t st) {
    const int NB = (int)((a.V + 63) / 64);
    const int NC = (int)(a.K / span_of(BITS));
    const int NG = (int)(a.K / a.G);
    const int SPG = GPS == 1 ? (int)(a.G / span_of(BITS)) : 1;
    const Regions<BITS> rg(a, ZP);
    int lks, frac;
    gemv_split(NC, SPG, lks, frac);
    const int ncs = NC >> lks;
    // x: bf16 rows converted in LDS; one fp16 row through the scalar unit;
    // several fp16 rows staged in LDS
    const int xm = a.x_bf16 ? 2 : (MM == 1 ? 0 : 1);
    const size_t lds = xm != 0 ? (size_t)MM * a.K * 2 : 0;
    const int64_t nwaves = (int64_t)NB << lks;  // KS waves per row block
    const dim3 grid((unsigned)((nwaves + kGemvWaves - 1) / kGemvWaves));
    // the top-K epilogue: fp32 logits, one activation row (its only user)
    constexpr bool kTK = OUT == F32 && MM == 1;
    const bool tk = kTK && a.lists != nullptr;
#define LMH_GEMV_GO(NCB_, TK_, XM_)                                                                \
    hipLaunchKernelGGL((gemv_kernel<BITS, MM, GPS, NCB_, OUT, ZP, TK_, XM_>), grid,                 \
                       dim3(64 * kGemvWaves), lds, st, rg.wq, rg.sc, rg.zq, (const uint16_t*)a.x,   \
                       a.bias, a.y, a.ldy, (int)a.V, (int)a.K, NB, NC, NG, SPG, a.scale_bf16, lks, \
                       frac, a.lists, a.list_T)
#define LMH_GEMV_XL(NCB_, TK_)                                                                     \
    do {                                                                                           \
        if (xm == 2) LMH_GEMV_GO(NCB_, TK_, 2);                                                    \
        else if constexpr (MM == 1) LMH_GEMV_GO(NCB_, TK_, 0);                                     \
        else LMH_GEMV_GO(NCB_, TK_, 1);                                                            \
    } while (0)
#define LMH_GEMV_TK(NCB_)                                                                          \
    do {                                                                                           \
        if constexpr (kTK) {                                                                       \
            if (tk) LMH_GEMV_XL(NCB_, true);                                                       \
            else LMH_GEMV_XL(NCB_, false);                                                         \
        } else {                                                                                   \
            LMH_GEMV_XL(NCB_, false);                                                              \
        }                                                                                          \
    } while (0)
    // one or two superchunks per wave: all requested up front; more: the
    // two-buffer ring (the forced 3- and 4-row variants: one at a time)
    if (ncs == 1) {
        LMH_GEMV_TK(1);
    } else if constexpr (MM <= 2) {
        if (ncs == 2) LMH_GEMV_TK(2);
        else LMH_GEMV_TK(0);
    } else {
        LMH_GEMV_TK(-1);
    }
#undef LMH_GEMV_TK
#undef LMH_GEMV_XL
#undef LMH_GEMV_GO
    return hipGetLastError();
}

template <int BITS, int MM, int OUT, bool ZP>
hipError_t gemv_dispatch_mm(const LogitsArgs& a, hipStream_t st) {
    const int gps = gps_of(BITS, a.G);
    if (gps == 1) return gemv_launch<BITS, MM, 1, OUT, ZP>(a, st);
    if constexpr (BITS == 8) return gemv_launch<BITS, MM, 2, OUT, ZP>(a, st);
    else if (gps == 2) return gemv_launch<BITS, MM, 2, OUT, ZP>(a, st);
    else return gemv_launch<BITS, MM, 4, OUT, ZP>(a, st);
}

template <bool ZP>
hipError_t gemv_run(const LogitsArgs& a, hipStream_t st) {
#define LMH_GEMV_MM(BITS_, OUT_)                                                                   \
    switch (a.M) {                                                                                 \
    case 1: return gemv_dispatch_mm<BITS_, 1, OUT_, ZP>(a, st);                                    \
    case 2: return gemv_dispatch_mm<BITS_, 2, OUT_, ZP>(a, st);                                    \
    case 3: return gemv_dispatch_mm<BITS_, 3, OUT_, ZP>(a, st);                                    \
    default: return gemv_dispatch_mm<BITS_, 4, OUT_, ZP>(a, st);                                   \
    }
#define LMH_GEMV_OUT(BITS_)                                                                        \
    switch (a.y_dtype) {                                                                           \
    case F32: LMH_GEMV_MM(BITS_, F32)                                                              \
    case F16: LMH_GEMV_MM(BITS_, F16)                                                              \
    default: LMH_GEMV_MM(BITS_, BF16)                                                              \
    }
    if (a.bits == 4) {
        LMH_GEMV_OUT(4)
    } else {
        LMH_GEMV_OUT(8)
    }
#undef LMH_GEMV_OUT
#undef LMH_GEMV_MM
}

}  // namespace
}  // namespace lmh
