// Split-K MFMA kernel for up to 16 activation rows (the automatic choice for
// 3..16 rows of heads with K <= 2048):
// y[m,v] = sum_k x[m,k] * q[v,k] * s[v,k/G] (+ bias[v]).
//
// vLLM PR #48870, Perf evals table: between one and a few hundred activation
// rows the call stays bound by the weight bytes, so this kernel reads them
// the way the GEMV does (gemv_kernels.h) and does the arithmetic the way the
// MFMA kernels do (logits_kernels.h).
//
// Work layout.  A workgroup is 8 waves.  A 64-row block of the vocabulary is
// split along K over KS waves (KS = 8, 4, 2 or 1: the largest power of two
// <= 8 dividing the superchunk count); wave ks takes the NCs = NC / KS
// superchunks [ks NCs, (ks + 1) NCs).  Lane (r = lane & 15, t = lane >> 4)
// reads slot t of rows 16 nt + r, nt = 0..3 (the four 16-row column tiles of
// the block), which are exactly the B operands of v_mfma_f32_16x16x32_f16 per
// 32-bit word, and the A operands x[16 mt + r][chunk + 8t .. +8] of the MT
// activation tiles straight from global memory (the activation rows are a
// few KiB and stay in the caches).  Every load of a wave's superchunks is
// issued before its first MFMA (one or two superchunks; more: two register
// buffers alternate), so the kernel is a stream of short read bursts like
// the GEMV.
//
// Arithmetic.  Per superchunk and scale group: the group's code words of
// each column tile unpacked exactly into fp16 (logits_common.h), a CPG-long
// MFMA chain per (activation tile, column tile) started from zero, and the
// chain's fp32 result folded into the wave's accumulator with one fp32 FMA by
// the group scale of the lane's vocabulary row -- the per-group arithmetic of
// the other MFMA kernels.  The KS waves' partial tiles meet in LDS and are
// added in wave order by all the block's threads, four columns each, which
// then store 16-byte row segments.  So the result does not depend on timing;
// it differs from the other MFMA kernels' only in how the KS partial sums
// associate (those add every group into one accumulator in K order).
#pragma once

#include "logits_common.h"

namespace lmh {
namespace {

constexpr int kSkWaves = 8;

// K split of the split-K kernel: the largest power of two <= 8 dividing the
// superchunk count (each superchunk's chains are scaled on their own, so any
// split keeps whole groups per chain).
inline int splitk_lks(int NC) {
    for (int l = 3; l > 0; --l)
        if (NC % (1 << l) == 0) return l;
    return 0;
}

// One superchunk as loaded by a lane: the slots of its four column tiles, the
// group scales of its rows, (ZP) the zero-point words of its groups, and the
// activation A operands of its chunks.
template <int BITS, int MT, int GPS>
struct SkBuf {
    static constexpr int CPS = span_of(BITS) / 32;
    uint4 w[4];
    uint16_t s[GPS][4];
    uint32_t z[GPS];
    uint4 a[MT][CPS];
};

template <int BITS, int MT, int GPS, int NCB, int OUT, bool ZP>
__global__ __launch_bounds__(64 * kSkWaves) void mfma_splitk_kernel(
    const uint4* __restrict__ wq, const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zq,
    const _Float16* __restrict__ x, const int* __restrict__ xexp, const float* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int V, int K, int M, int NB, int NC, int NG, int SPG,
    int sbf16, int lks) {
    constexpr int NT = 4, ROWS = 16 * MT;
    constexpr int SPAN = span_of(BITS), CPS = SPAN / 32, CPG = CPS / GPS;
    constexpr int WPG = BITS == 4 ? CPG : 2 * CPG;  // 32-bit code words per group and slot
    constexpr int RP = 68;  // row pitch of the partial tiles in LDS (floats; 16-byte rows, no bank conflicts)
    __shared__ float red[kSkWaves][ROWS][RP];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, t = lane >> 4;
    const int KS = 1 << lks;
    const int blk_raw = (blockIdx.x << (3 - lks)) + (wv >> lks);
    const int ks = wv & (KS - 1);
    const bool live = blk_raw < NB;
    const int blk = live ? blk_raw : NB - 1;  // dead waves read a real block, store nothing
    const int NCs = NC >> lks;
    const int c0 = ks * NCs, cend = c0 + NCs;

    const uint4* wp = wq + (int64_t)blk * NC * 256 + t * 64 + r;
    const uint16_t* sp = sc + (int64_t)blk * NG * 64 + r;
    const uint32_t* zp = ZP ? (const uint32_t*)zq + (int64_t)blk * NG * 16 + r : nullptr;
    const _Float16* xr[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xr[mt] = x + (int64_t)min(16 * mt + r, M - 1) * K + 8 * t;  // rows past M: any valid row

    using Buf = SkBuf<BITS, MT, GPS>;
    auto load = [&](Buf& b, int c) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) b.w[nt] = wp[(int64_t)c * 256 + 16 * nt];
#pragma unroll
        for (int g = 0; g < GPS; ++g) {
            const int64_t gi = GPS > 1 ? (int64_t)c * GPS + g : (int64_t)(c / SPG);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) b.s[g][nt] = sp[gi * 64 + 16 * nt];
            if constexpr (ZP) b.z[g] = zp[gi * 16];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ch = 0; ch < CPS; ++ch)
                b.a[mt][ch] = *(const uint4*)(xr[mt] + (int64_t)c * SPAN + 32 * ch);
    };

    f4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
    const uint32_t magic = 0x64006400u;
    auto compute = [&](const Buf& b) {
#pragma unroll
        for (int g = 0; g < GPS; ++g) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const ZC zc = ZP ? zc_byte(b.z[g], nt) : zc_sym<BITS>();
                h8 bop[CPG];
#pragma unroll
                for (int jj = 0; jj < CPG; ++jj) {
                    h2 p0, p1, p2, p3;
                    if constexpr (BITS == 4) {
                        unpack_i4(word_of(b.w[nt], g * WPG + jj), magic, zc, p0, p1, p2, p3);
                    } else {
                        unpack_i8(word_of(b.w[nt], g * WPG + 2 * jj), zc, p0, p1);
                        unpack_i8(word_of(b.w[nt], g * WPG + 2 * jj + 1), zc, p2, p3);
                    }
                    bop[jj] = (h8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
                }
                const float sv = scale_to_f32(b.s[g][nt], sbf16);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    // D[4t + e][r]: activation row 16 mt + 4 t + e, vocabulary row 16 nt + r
                    f4 q = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(h8, b.a[mt][g * CPG]), bop[0], (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int jj = 1; jj < CPG; ++jj)
                        q = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(h8, b.a[mt][g * CPG + jj]), bop[jj], q, 0, 0, 0);
                    acc[mt][nt] += sv * q;
                }
            }
        }
    };

    if constexpr (NCB > 0) {
        Buf b[NCB];
#pragma unroll
        for (int i = 0; i < NCB; ++i) load(b[i], c0 + i);
#pragma unroll
        for (int i = 0; i < NCB; ++i) {
            compute(b[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        Buf A, B;
        load(A, c0);
        int c = c0;
#pragma unroll 1
        for (; c + 1 < cend; c += 2) {
            load(B, c + 1);
            compute(A);
            __builtin_amdgcn_sched_barrier(0);
            if (c + 2 < cend) load(A, c + 2);
            compute(B);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (c < cend) compute(A);
    }

    // the partial tiles meet in LDS: element (row 16 mt + 4 t + e, column
    // 16 nt + r) of wave wv
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wv][16 * mt + 4 * t + e][16 * nt + r] = acc[mt][nt][e];
    __syncthreads();
    if (!live) return;

    // the block's KS waves add the partials in wave order, each thread four
    // contiguous columns of a row, and store them
    const int wb = wv & ~(KS - 1);
    const int u = ks * 64 + lane;  // 0 .. 64 KS - 1
    const int q4 = u & 15;
    const int v0 = blk * 64 + 4 * q4;
    constexpr int OSZ = OUT == F32 ? 4 : 2;
    const bool vec16 = ((uintptr_t)y & (4 * OSZ - 1)) == 0 && (ldy & 3) == 0 && v0 + 3 < V;
    f4 bv = (f4){0.f, 0.f, 0.f, 0.f};
    if (bias) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = v0 + e < V ? bias[v0 + e] : 0.0f;
    }
    for (int row = u >> 4; row < ROWS && row < M; row += 4 * KS) {
        f4 s = *(const f4*)&red[wb][row][4 * q4];
#pragma unroll
        for (int k = 1; k < kSkWaves; ++k)
            if (k < KS) s += *(const f4*)&red[wb + k][row][4 * q4];
        if (xexp) {
            const int xe = xexp[row];
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] = ldexpf(s[e], xe);
        }
        s = s + bv;
        YT<OUT>* yrow = (YT<OUT>*)y + (int64_t)row * ldy + v0;
        if (vec16) {
            store4<OUT>(yrow, s);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (v0 + e < V) yrow[e] = to_out<OUT>(s[e]);
        }
    }
}

template <int BITS, int MT, int GPS, int OUT, bool ZP>
hipError_t splitk_launch(const LogitsArgs& a, hipStream_t st) {
    const int NB = (int)((a.V + 63) / 64);
    const int NC = (int)(a.K / span_of(BITS));
    const int NG = (int)(a.K / a.G);
    const int SPG = GPS == 1 ? (int)(a.G / span_of(BITS)) : 1;
    const Regions<BITS> rg(a, ZP);
    const int lks = splitk_lks(NC);
    const int ncs = NC >> lks;
    const int64_t nwaves = (int64_t)NB << lks;
    const dim3 grid((unsigned)((nwaves + kSkWaves - 1) / kSkWaves));
#define LMH_SK(NCB_)                                                                               \
    hipLaunchKernelGGL((mfma_splitk_kernel<BITS, MT, GPS, NCB_, OUT, ZP>), grid,                   \
                       dim3(64 * kSkWaves), 0, st, rg.wq, rg.sc, rg.zq, (const _Float16*)a.x,      \
                       a.xexp, a.bias, a.y, a.ldy, (int)a.V, (int)a.K, a.M, NB, NC, NG, SPG,       \
                       a.scale_bf16, lks)
    if (ncs == 1) LMH_SK(1);
    else if (ncs == 2) LMH_SK(2);
    else LMH_SK(0);
#undef LMH_SK
    return hipGetLastError();
}

template <int BITS, int MT, int OUT, bool ZP>
hipError_t splitk_dispatch_mt(const LogitsArgs& a, hipStream_t st) {
    const int gps = gps_of(BITS, a.G);
    if (gps == 1) return splitk_launch<BITS, MT, 1, OUT, ZP>(a, st);
    if constexpr (BITS == 8) return splitk_launch<BITS, MT, 2, OUT, ZP>(a, st);
    else if (gps == 2) return splitk_launch<BITS, MT, 2, OUT, ZP>(a, st);
    else return splitk_launch<BITS, MT, 4, OUT, ZP>(a, st);
}

// One 16-row activation tile (M <= 16).  A 32-row tile (MT = 2) needs 104
// registers and 70 KiB of LDS per workgroup, half the waves of the 16-row
// one, and was measured slower than the activation-resident and LDS-staged
// kernels at 17..32 rows (as were two 16-row tiles, which read the weights
// twice), so it is not instantiated.
template <bool ZP>
hipError_t splitk_run(const LogitsArgs& a, hipStream_t st) {
#define LMH_SK_MT(BITS_, OUT_) return splitk_dispatch_mt<BITS_, 1, OUT_, ZP>(a, st);
#define LMH_SK_OUT(BITS_)                                                                          \
    switch (a.y_dtype) {                                                                           \
    case F32: LMH_SK_MT(BITS_, F32)                                                                \
    case F16: LMH_SK_MT(BITS_, F16)                                                                \
    default: LMH_SK_MT(BITS_, BF16)                                                                \
    }
    if (a.bits == 4) {
        LMH_SK_OUT(4)
    } else {
        LMH_SK_OUT(8)
    }
#undef LMH_SK_OUT
#undef LMH_SK_MT
}

}  // namespace
}  // namespace lmh
