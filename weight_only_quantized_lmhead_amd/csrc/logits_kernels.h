// Fused weight-only-quantized logits, the MFMA kernels for many activation rows:
// y[m,v] = sum_k x[m,k] * q[v,k] * s[v,k/G].
//
// vLLM PR #48870 ("Fused WNA16 GEMM for tied quantized lm_head logits",
// Purpose and perf table): the logits come straight from the packed codes and
// scales; the dense weight is never formed.  The codes enter the MFMA
// operands exactly (fp16 integers, logits_common.h), each group's MFMA chain
// starts from zero and is scaled in fp32, so the three kernels below give the
// same bits as each other.
//
// Kernels (which one runs for which M and head is decided in api.hip; the
// lane-per-row GEMV for one to four rows is in gemv_kernels.h, the split-K
// MFMA kernel for up to 16 rows in splitk_kernels.h)
//   mfma         register-fed MFMA.  A wave owns one row block (4 MFMA column
//                tiles of 16 rows) and MT row tiles of 16 activations; each
//                16-byte slot load is one 16x16x32 B operand per 32-column
//                word.
//   mfma_lds     the same tiles, every operand staged in LDS by direct
//                global-to-LDS loads; 32- or 64-row activation tiles.
//   mfma_xres    a 64-row (or, for M <= 32, 32-row) activation tile resident
//                in LDS, weights streamed through a register ring (K <= 1024).
//
// Each kernel takes ZP (zero-point heads) as a template flag; the symmetric
// instantiations are unchanged.  logits.hip instantiates the symmetric
// kernels and logits_zp.hip the zero-point ones (two translation units so
// that they compile in parallel).
#pragma once

#include "logits_common.h"

namespace lmh {
namespace {
// ---------------------------------------------------------------------------
// MFMA kernel.  A workgroup = 4 waves = 4 row blocks (256 vocabulary rows) x
// MT*16 activation rows (grid.y tiles M).  For each superchunk the workgroup
// stages the activation tile x[m0 .. m0+16MT, span columns] in LDS (double
// buffered; rows padded to span+8 halves so the 16-row A-operand reads hit 16
// distinct bank groups), while each wave streams its own row block's 16-byte
// slots: the current superchunk in registers, the next one in flight.
// Lane (r = lane & 15, t = lane >> 4) reads slot t of vocabulary row 16*nt + r:
// word j is the 8-value B operand (k = 8t .. 8t+7 of 32-column chunk j) of one
// v_mfma_f32_16x16x32_f16, and the A operand is x[16*mt + r][chunk + 8t .. +8]
// from LDS.  The 16x16 result lands as D[4t + e][r]: activation row 4t + e,
// vocabulary row r.  Per scale group: the B operands of the 4 column tiles are
// unpacked once, then per row tile a CPG-long MFMA chain is started from zero
// and folded into the fp32 accumulator with the group scale of the lane's row.
// With ZP the lane reads one 32-bit word per group: the zero points of its
// rows 16 nt + r, nt = 0..3, in bytes nt.
template <int BITS, int MT, int GPS, int OUT, bool ZP>
__global__ __launch_bounds__(256, MT >= 4 ? 1 : 2) void mfma_kernel(
    const uint4* __restrict__ wq, const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zq,
    const _Float16* __restrict__ x,
    const int* __restrict__ xexp, const float* __restrict__ bias, void* __restrict__ y,
    int64_t ldy, int V, int K, int M, int NB, int NC, int NG, int SPG, int sbf16) {
    // grid (row groups, activation tiles): all row groups of one activation
    // tile run before the next tile's; the last-level cache serves the
    // re-read weights (an XCD-grouped order, which reads them from HBM once,
    // measured slower on the 151936 x 1024 head at M = 256)
    const int rg = blockIdx.x, mtile = blockIdx.y;
    constexpr int NT = 4;
    constexpr int SPAN = BITS == 4 ? 128 : 64;
    constexpr int CPS = SPAN / 32;
    constexpr int CPG = CPS / GPS;
    constexpr int ROWH = SPAN + 8;        // padded LDS row, in halves
    constexpr int ROWS = MT * 16;
    constexpr int STAGE = ROWS * ROWH;    // halves per LDS stage
    constexpr int XV = ROWS * SPAN / 8;   // 16-byte pieces of one x tile
    constexpr int XPT = (XV + 255) / 256; // pieces per thread
    constexpr int P8 = SPAN / 8;          // 16-byte pieces per tile row
    constexpr int RPU = 256 / P8;         // rows between one thread's pieces
    __shared__ __attribute__((aligned(16))) _Float16 xs[2 * STAGE];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int blk = rg * 4 + wv;
    const bool live = blk < NB;
    const int blkc = live ? blk : NB - 1;
    const int r = lane & 15, t = lane >> 4;
    const int m0 = mtile * ROWS;
    const uint4* wp = wq + (int64_t)blkc * NC * 256 + t * 64 + r;
    const uint16_t* sp = sc + (int64_t)blkc * NG * 64 + r;
    const uint32_t* zp = ZP ? (const uint32_t*)zq + (int64_t)blkc * NG * 16 + r : nullptr;
    const uint32_t magic = 0x64006400u;

    // x tile staging: thread i copies the 16-byte pieces (row i / P8 + u*RPU,
    // 8-column group i % P8), u < XPT; rows past M are staged as zeros
    const int xrow0 = threadIdx.x / P8, xcol8 = threadIdx.x % P8;
    const _Float16* xsrc = x + (int64_t)(m0 + xrow0) * K + 8 * xcol8;
    _Float16* xdst = xs + xrow0 * ROWH + 8 * xcol8;
    uint32_t xvalid = 0;
#pragma unroll
    for (int u = 0; u < XPT; ++u)
        if (xrow0 + u * RPU < ROWS && m0 + xrow0 + u * RPU < M) xvalid |= 1u << u;
    uint4 xr[XPT];
    auto xload = [&](int c) {
#pragma unroll
        for (int u = 0; u < XPT; ++u)
            xr[u] = (xvalid >> u) & 1u
                        ? *(const uint4*)(xsrc + (int64_t)u * RPU * K + (int64_t)c * SPAN)
                        : make_uint4(0, 0, 0, 0);
    };
    auto xstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < XPT; ++u)
            if (xrow0 + u * RPU < ROWS) *(uint4*)(xdst + buf * STAGE + u * RPU * ROWH) = xr[u];
    };

    // weights: loads past the end are clamped so every load is unconditional
    uint4 wcur[NT], wnxt[NT];
    uint16_t scur[GPS][NT], snxt[GPS][NT];
    uint32_t zcur[GPS], znxt[GPS];
    int pf_g = 0, pf_left = SPG;
    auto wload = [&](uint4 (&wd)[NT], uint16_t (&sd)[GPS][NT], uint32_t (&zd)[GPS], int c) {
        const int cc = c < NC ? c : NC - 1;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) wd[nt] = wp[(int64_t)cc * 256 + 16 * nt];
        if constexpr (GPS > 1) {
#pragma unroll
            for (int g = 0; g < GPS; ++g) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    sd[g][nt] = sp[((int64_t)cc * GPS + g) * 64 + 16 * nt];
                if constexpr (ZP) zd[g] = zp[((int64_t)cc * GPS + g) * 16];
            }
        } else {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) sd[0][nt] = sp[(int64_t)pf_g * 64 + 16 * nt];
            if constexpr (ZP) zd[0] = zp[(int64_t)pf_g * 16];
            if (--pf_left == 0 && pf_g + 1 < NG) {
                ++pf_g;
                pf_left = SPG;
            }
        }
    };

    f4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};

    xload(0);
    wload(wcur, scur, zcur, 0);
    xstore(0);
    __syncthreads();
    for (int c = 0; c < NC; ++c) {
        wload(wnxt, snxt, znxt, c + 1);
        xload(c + 1 < NC ? c + 1 : NC - 1);
        const _Float16* xb = xs + (c & 1) * STAGE;
#pragma unroll
        for (int g = 0; g < GPS; ++g) {
            h8 bop[NT][CPG];
            float sv[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const ZC zc = ZP ? zc_byte(zcur[g], nt) : zc_sym<BITS>();
#pragma unroll
                for (int jj = 0; jj < CPG; ++jj) {
                    const int j = g * CPG + jj;
                    h2 p0, p1, p2, p3;
                    if constexpr (BITS == 4) {
                        unpack_i4(word_of(wcur[nt], j), magic, zc, p0, p1, p2, p3);
                    } else {
                        unpack_i8(word_of(wcur[nt], 2 * j), zc, p0, p1);
                        unpack_i8(word_of(wcur[nt], 2 * j + 1), zc, p2, p3);
                    }
                    bop[nt][jj] = (h8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
                }
                sv[nt] = scale_to_f32(scur[g][nt], sbf16);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                h8 a[CPG];
#pragma unroll
                for (int jj = 0; jj < CPG; ++jj)
                    a[jj] = *(const h8*)(xb + (16 * mt + r) * ROWH + 32 * (g * CPG + jj) + 8 * t);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f4 pt = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], bop[nt][0],
                                                                    (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int jj = 1; jj < CPG; ++jj)
                        pt = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[jj], bop[nt][jj], pt, 0, 0, 0);
                    acc[mt][nt] += sv[nt] * pt;
                }
            }
        }
        xstore((c + 1) & 1);
        __syncthreads();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            wcur[nt] = wnxt[nt];
#pragma unroll
            for (int g = 0; g < GPS; ++g) scur[g][nt] = snxt[g][nt];
        }
#pragma unroll
        for (int g = 0; g < GPS; ++g) zcur[g] = znxt[g];
    }
    if (!live) return;
    // write D[4t + e][r] of each tile
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int v = blk * 64 + 16 * nt + r;
        if (v >= V) continue;
        const float b = bias ? bias[v] : 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + 16 * mt + 4 * t + e;
                if (m < M) {
                    float o = acc[mt][nt][e];
                    if (xexp) o = ldexpf(o, xexp[m]);
                    ((YT<OUT>*)y)[(int64_t)m * ldy + v] = to_out<OUT>(o + b);
                }
            }
    }
}

// One direct global->LDS load of 16 bytes per active lane: lane i writes
// LDS bytes [lds + 16i, lds + 16i + 16) from its own global address `g`
// (global_load_lds_dwordx4; `lds` must be wave-uniform).  Issued through asm
// so that the compiler does not track it: its conservative wait analysis
// would otherwise wait for every stage in flight before any LDS read.  The
// caller waits with s_waitcnt vmcnt before reading the stage.  M0 is written
// here and by nothing else in the kernels that use this helper.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ---------------------------------------------------------------------------
// LDS-staged MFMA kernel (larger M).  A tile is WPB row blocks (one per wave;
// 64*WPB vocabulary rows) x 16*MT activation rows with the same lane roles as
// mfma_kernel (lane (r, t) of wave w owns row block WPB*rg + w), but every
// operand goes through LDS by direct global->LDS loads, so no registers hold
// data in flight and the activation tile can be 64-128 rows, which shares each
// unpacked B operand among 4-8 MFMAs.
// Per superchunk a stage holds:
//   W  the WPB row blocks' packed superchunks as stored (WPB x 4 KiB);
//   S  their scales for the superchunk's groups (WPB x GPS x 128 B), and
//      with ZP after them the groups' zero points (WPB x GPS x 64 B, moved by
//      the same load instruction);
//   X  the activation tile, row-major, 16-byte piece p of row m stored at
//      piece (p ^ (m mod P8)) of that row (P8 = pieces per row), so the 16
//      rows of one A-operand read fall in distinct banks.
// A workgroup runs one or more tiles back to back as one stream of (tile,
// superchunk) steps, with the loads of the next STAGES-1 steps in flight
// (across tile boundaries too).  Tiles are numbered rg*NMT + mtile (the
// activation tiles of a row group are adjacent); XCD x (workgroups b with
// b % 8 == x) owns a contiguous eighth of them, dealt round-robin to its
// workgroups, so the activation tiles of one row group run at the same time
// on one XCD and read its weights through that XCD's L2 once.  With WPB = 8
// the 8 waves (two per SIMD) share one activation tile.
// Bytes of one stage, and the workgroups per CU the kernel is built for: 3
// for 32-row tiles (2 with zero points, whose extra registers would spill at
// 3), 2 for 64-row ones, 1 with 8 waves, fewer if the stages do not fit that
// many times in the CU's 160 KiB of LDS.
template <int BITS, int MT, int GPS, int WPB, bool ZP>
constexpr int lds_stage_bytes() {
    return WPB * 4096 + WPB * GPS * (ZP ? 192 : 128) + MT * 16 * span_of(BITS) * 2;
}
template <int BITS, int MT, int GPS, int STAGES, int WPB, bool ZP>
constexpr int lds_wg_per_cu() {
    const int want = WPB == 8 ? 1 : (MT <= 2 ? (ZP ? 2 : 3) : (MT <= 4 ? 2 : 1));
    const int fit = 160 * 1024 / (STAGES * lds_stage_bytes<BITS, MT, GPS, WPB, ZP>());
    return want < fit ? want : fit;
}

template <int BITS, int MT, int GPS, int STAGES, int WPB, int OUT, bool ZP>
__global__ __launch_bounds__(64 * WPB, (lds_wg_per_cu<BITS, MT, GPS, STAGES, WPB, ZP>()))
void mfma_lds_kernel(
    const uint4* __restrict__ wq, const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zq,
    const _Float16* __restrict__ x,
    const int* __restrict__ xexp, const float* __restrict__ bias, void* __restrict__ y,
    int64_t ldy, int V, int K, int M, int NB, int NC, int NG, int SPG, int sbf16, int NMT,
    int total) {
    constexpr int NT = 4;
    constexpr int SPAN = BITS == 4 ? 128 : 64;
    constexpr int CPS = SPAN / 32;
    constexpr int CPG = CPS / GPS;
    constexpr int P8 = SPAN / 8;           // 16-byte pieces per activation row
    constexpr int ROWS = MT * 16;
    constexpr int WB = WPB * 4096;         // packed weights per stage
    constexpr int SGB = GPS * (ZP ? 192 : 128);  // scales (+ zero points) per wave and stage
    constexpr int SB = WPB * SGB;
    constexpr int XB = ROWS * SPAN * 2;    // activation tile per stage
    constexpr int STB = WB + SB + XB;
    static_assert(STB == lds_stage_bytes<BITS, MT, GPS, WPB, ZP>(), "stage size");
    constexpr int NXW = ROWS * P8 / 64 / WPB;  // activation loads per wave per stage
    static_assert(WPB == 4 || WPB == 8, "4 or 8 waves per workgroup");
    static_assert(ROWS * P8 % (64 * WPB) == 0, "activation tile must split evenly over the waves");
    constexpr int NPS = 4 + 1 + NXW;  // loads per wave per stage
    static_assert(STAGES == 2 || STAGES == 3, "two or three stages");
    static_assert(NPS < 64, "vmcnt holds 6 bits");
    __shared__ __attribute__((aligned(16))) unsigned char lds[STAGES * STB];
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));

    // this workgroup's tiles: xt0 + l, xt0 + l + L, ... < xt1
    const int L = gridDim.x >> 3, xcd = blockIdx.x & 7, l = blockIdx.x >> 3;
    const int perx = (total + 7) / 8;
    const int xt0 = xcd * perx;
    const int xt1 = min(xt0 + perx, total);
    const int ntile = xt1 - xt0 > l ? (xt1 - xt0 - l + L - 1) / L : 0;
    const int nsteps = ntile * NC;
    if (nsteps == 0) return;

    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, t = lane >> 4;
    // fixed parts of this lane's activation loads: wave instruction q = wv + 4i
    // fills LDS pieces [64q, 64q+64); piece P = row*P8 + sp holds global piece
    // sp ^ (row % P8); rows past M read row M-1 (never stored)
    int xrc[NXW];  // row | column << 16 (one register each)
#pragma unroll
    for (int i = 0; i < NXW; ++i) {
        const int P = (wv + WPB * i) * 64 + lane;
        xrc[i] = P / P8 | (8 * ((P % P8) ^ ((P / P8) % P8))) << 16;
    }

    auto tile_of = [&](int i, int& rg, int& mtile) {
        const int tt = xt0 + l + i * L;
        rg = tt / NMT;
        mtile = tt - rg * NMT;
    };
    auto issue = [&](int stage, int s) {
        const int i = s / NC, c = s - i * NC;
        int rg, mtile;
        tile_of(i, rg, mtile);
        const int blk = min(rg * WPB + wv, NB - 1);
        const int m0 = mtile * ROWS;
        const uint32_t sb = lds0 + stage * STB;
        const uint4* wc = wq + ((int64_t)blk * NC + c) * 256 + lane;
#pragma unroll
        for (int k = 0; k < 4; ++k) lds_dma16(wc + k * 64, sb + wv * 4096 + k * 1024);
        const int g0 = GPS > 1 ? c * GPS : c / SPG;
        // lanes 0 .. 8 GPS - 1: the scales; with ZP lanes 8 GPS .. 12 GPS - 1:
        // the zero points (the groups' 64-byte runs are adjacent)
        if (lane < SGB / 16) {
            const uint4* src =
                !ZP || lane < GPS * 8
                    ? (const uint4*)(sc + ((int64_t)blk * NG + g0) * 64) + lane
                    : (const uint4*)(zq + ((int64_t)blk * NG + g0) * 64) + (lane - GPS * 8);
            lds_dma16(src, sb + WB + wv * SGB);
        }
        const _Float16* xc = x + (int64_t)m0 * K + c * SPAN;
#pragma unroll
        for (int k = 0; k < NXW; ++k) {
            const int row = xrc[k] & 0xFFFF, col = xrc[k] >> 16;
            const int rr = m0 + row < M ? row : M - 1 - m0;
            lds_dma16(xc + rr * K + col, sb + WB + SB + (wv + WPB * k) * 1024);
        }
    };

    f4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
    const uint32_t magic = 0x64006400u;

    auto compute = [&](const unsigned char* s) {
        const unsigned char* W = s + wv * 4096 + (t * 64 + r) * 16;  // + nt*256: slot t, row 16nt + r
        const uint16_t* S = (const uint16_t*)(s + WB + wv * SGB);
        const uint32_t* Z = (const uint32_t*)(s + WB + wv * SGB + GPS * 128) + r;
        const unsigned char* X = s + WB + SB;
        constexpr int WPG = BITS == 4 ? CPG : 2 * CPG;  // 32-bit code words per group
#pragma unroll
        for (int g = 0; g < GPS; ++g) {
            // only this group's words of each slot are read (fewer live registers)
            uint32_t wg[NT][WPG];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int u = 0; u < WPG; ++u)
                    wg[nt][u] = *(const uint32_t*)(W + nt * 256 + 4 * (g * WPG + u));
            h8 bop[NT][CPG];
            float sv[NT];
            const uint32_t zw = ZP ? Z[g * 16] : 0u;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const ZC zc = ZP ? zc_byte(zw, nt) : zc_sym<BITS>();
#pragma unroll
                for (int jj = 0; jj < CPG; ++jj) {
                    h2 p0, p1, p2, p3;
                    if constexpr (BITS == 4) {
                        unpack_i4(wg[nt][jj], magic, zc, p0, p1, p2, p3);
                    } else {
                        unpack_i8(wg[nt][2 * jj], zc, p0, p1);
                        unpack_i8(wg[nt][2 * jj + 1], zc, p2, p3);
                    }
                    bop[nt][jj] = (h8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
                }
                sv[nt] = scale_to_f32(S[g * 64 + 16 * nt + r], sbf16);
            }
            // software pipeline over the activation tiles: the A operands of
            // tile mt+1 are read from LDS and the scale FMAs of tile mt-1 are
            // issued while the MFMA chains of tile mt run
            auto load_a = [&](int mt, h8 (&a)[CPG]) {
                const int m = 16 * mt + r;
#pragma unroll
                for (int jj = 0; jj < CPG; ++jj) {
                    const int pc = 4 * (g * CPG + jj) + t;
                    a[jj] = *(const h8*)(X + (m * P8 + (pc ^ (m % P8))) * 16);
                }
            };
            h8 a0[CPG], a1[CPG];
            f4 p0[NT], p1[NT];
            load_a(0, a0);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                h8 (&acur)[CPG] = (mt & 1) ? a1 : a0;
                h8 (&anxt)[CPG] = (mt & 1) ? a0 : a1;
                f4 (&pcur)[NT] = (mt & 1) ? p1 : p0;
                f4 (&pprv)[NT] = (mt & 1) ? p0 : p1;
                if (mt + 1 < MT) load_a(mt + 1, anxt);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f4 q = __builtin_amdgcn_mfma_f32_16x16x32_f16(acur[0], bop[nt][0],
                                                                   (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int jj = 1; jj < CPG; ++jj)
                        q = __builtin_amdgcn_mfma_f32_16x16x32_f16(acur[jj], bop[nt][jj], q, 0, 0, 0);
                    pcur[nt] = q;
                }
                if (mt > 0) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) acc[mt - 1][nt] += sv[nt] * pprv[nt];
                }
            }
            {
                f4 (&plast)[NT] = ((MT - 1) & 1) ? p1 : p0;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[MT - 1][nt] += sv[nt] * plast[nt];
            }
        }
    };

    // results of tile i when more tiles follow on this workgroup: y[m, v] =
    // acc * 2^xexp[m] + bias[v]; plain stores, left to drain while the next
    // tile computes (its stages are in use, so no transpose through LDS)
    auto epilogue = [&](int i) {
        int rg, mtile;
        tile_of(i, rg, mtile);
        const int blk = rg * WPB + wv;
        const int m0 = mtile * ROWS;
        if (blk < NB) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int v = blk * 64 + 16 * nt + r;
                const float b = (bias && v < V) ? bias[v] : 0.0f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = m0 + 16 * mt + 4 * t + e;
                        if (m < M && v < V) {
                            float o = acc[mt][nt][e];
                            if (xexp) o = ldexpf(o, xexp[m]);
                            ((YT<OUT>*)y)[(int64_t)m * ldy + v] = to_out<OUT>(o + b);
                        }
                    }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
    };

    // results of the workgroup's last tile, transposed through LDS (every
    // stage has landed and no further load is issued then): each wave writes
    // its 64 columns x 32 activation rows at a time into its own padded
    // region, and each lane then stores 4 contiguous columns of one row (16
    // bytes for fp32), 4 rows x 256 contiguous bytes per store instruction --
    // a quarter of the store instructions of one element per lane (measured
    // on the 151936 x 1024 int4 g64 head: M = 32 28.0 -> 26.8 us, M = 256
    // 136.6 -> 119.7 us on this kernel)
    constexpr int OSZ = OUT == F32 ? 4 : 2;
    const bool vec16 = ((uintptr_t)y & (4 * OSZ - 1)) == 0 && (ldy & 3) == 0;
    auto epilogue_tr = [&](int i) {
        int rg, mtile;
        tile_of(i, rg, mtile);
        const int blk = rg * WPB + wv;
        const int m0 = mtile * ROWS;
        constexpr int RS = 68;  // padded row stride (floats): 4 rows x 16 columns hit 64 banks
        float* T = (float*)lds + wv * 32 * RS;
        const int vc = 4 * (lane & 15);
        const int vb = blk * 64 + vc;
        float bb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) bb[q] = (bias && vb + q < V) ? bias[vb + q] : 0.0f;
        const bool full = vec16 && vb + 3 < V;
#pragma unroll
        for (int h = 0; h < MT; h += 2) {
            __syncthreads();  // the previous readers of this LDS are done
#pragma unroll
            for (int mh = 0; mh < 2 && h + mh < MT; ++mh)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        T[(16 * mh + 4 * t + e) * RS + 16 * nt + r] = acc[h + mh][nt][e];
            __syncthreads();
            if (blk < NB) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int row = (lane >> 4) + 4 * j;
                    const int m = m0 + 16 * h + row;
                    if (row < 16 * (MT - h) && m < M) {
                        f4 o = *(const f4*)&T[row * RS + vc];
                        const int xe = xexp ? xexp[m] : 0;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            if (xexp) o[q] = ldexpf(o[q], xe);
                            o[q] = o[q] + bb[q];
                        }
                        YT<OUT>* yp = (YT<OUT>*)y + (int64_t)m * ldy + vb;
                        if (full) {
                            store4<OUT>(yp, o);
                        } else {
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (vb + q < V) yp[q] = to_out<OUT>(o[q]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
    };

    // Step s: wait for this wave's loads of stage s (loads of later stages,
    // issued after them, may still be in flight) and for its LDS reads, then
    // meet the other waves at a bare s_barrier (a __syncthreads() fence would
    // also wait for the later stages' loads; the empty asm statements keep
    // the compiler from moving memory accesses across it); refill the stage
    // read in step s-1, which every wave finished before the barrier.
    constexpr int kWaitNewer = (NPS & 15) | ((NPS >> 4) << 14) | (7 << 4);
    constexpr int kWaitAll = 7 << 4;
    constexpr int AHEAD = STAGES - 1;
    for (int s = 0; s < AHEAD && s < nsteps; ++s) issue(s, s);
    int stage = 0, s = 0;
    for (int i = 0; i < ntile; ++i) {
        for (int c = 0; c < NC; ++c, ++s) {
            if (STAGES == 3 && s + 1 < nsteps)
                __builtin_amdgcn_s_waitcnt(kWaitNewer);
            else
                __builtin_amdgcn_s_waitcnt(kWaitAll);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (s + AHEAD < nsteps) issue(stage == 0 ? STAGES - 1 : stage - 1, s + AHEAD);
            compute(lds + stage * STB);
            stage = stage + 1 == STAGES ? 0 : stage + 1;
        }
        if (i + 1 < ntile) epilogue(i);
    }
    // (after the loop, so that its registers do not compete with the steps')
    __builtin_amdgcn_sched_barrier(0);
    epilogue_tr(ntile - 1);
}

// ---------------------------------------------------------------------------
// Activation-resident MFMA kernel (M > 32, K <= kXresMaxK).  A workgroup of
// 16 waves (8 with NT = 4) loads one 64-row activation tile
// x[m0 .. m0+63, 0 .. K) into LDS once (16-byte pieces swizzled as in
// mfma_lds_kernel) and then sweeps a contiguous range of row blocks with no
// further barrier.  A wave's unit of work is 16 NT columns of a row block
// (NT = 2: half a block, so 32 accumulator registers and 4 waves per SIMD to
// hide each other's latency); each wave streams its units' weight slots and
// scales through a D-deep register ring (loads past its last step are clamped
// to that step, so every load is unconditional and the wait counts stay
// exact; what those steps add is never stored), reads its A operands from
// the resident tile, and stores a unit's 64 x 16 NT results as soon as its
// last superchunk is done.  The workgroups of one XCD cover NMT activation
// tiles times VRX vocabulary ranges with the NMT tiles of a range side by
// side, so a weight slot comes from HBM once and from that XCD's L2 for the
// other tiles.
constexpr int kXresMaxK = 1024;

// Wait for every outstanding vector-memory operation of the wave.  Issued
// right after the epilogue's bias loads, so that no path leaves a load in
// flight into a register that another path of the loop reuses: the compiler's
// wait insertion cannot tell the paths apart, and would otherwise make the
// no-bias stores wait for the ring loads too.
__device__ __forceinline__ void wait_vm_all() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt untouched
}

template <int NT_>
constexpr int xres_waves() { return NT_ == 4 ? 8 : 16; }

// SB: the scale type as a template flag (0 fp16, 1 bf16), so that the per-step
// scale conversion is one instruction per scale and carries no select.
// MT_: activation tiles of 16 rows resident in LDS (4: a 64-row tile, 2: a
// 32-row tile for M <= 32, half the LDS).
template <int BITS, int GPS, int D, bool TR, int OUT, bool ZP, int NT_, int SB, int MT_>
__global__ __launch_bounds__(64 * xres_waves<NT_>(), 1) void mfma_xres_kernel(
    const uint4* __restrict__ wq, const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zq,
    const _Float16* __restrict__ x,
    const int* __restrict__ xexp, const float* __restrict__ bias, void* __restrict__ y,
    int64_t ldy, int V, int K, int M, int NB, int NC, int NG, int SPG, int NMT, int VRX) {
    constexpr int MT = MT_, NT = NT_, ROWS = 16 * MT_;
    constexpr int WAVES = xres_waves<NT_>(), NTH = 64 * WAVES;
    constexpr int PARTS = 4 / NT;  // a row block's 64 columns in PARTS units of 16 NT
    constexpr int SPAN = BITS == 4 ? 128 : 64;
    constexpr int CPS = SPAN / 32;
    constexpr int CPG = CPS / GPS;
    constexpr int WPG = BITS == 4 ? CPG : 2 * CPG;  // 32-bit code words per group and slot
    __shared__ uint4 xs[ROWS * kXresMaxK / 8];
    __shared__ int xe_s[ROWS];  // power-of-two row exponents of the tile (bf16 x)

    const int xcd = blockIdx.x & 7, l = blockIdx.x >> 3;
    const int mtile = l % NMT, vr = xcd * VRX + l / NMT;
    const int NV = 8 * VRX;
    const int rb0 = (int)((int64_t)NB * vr / NV), rb1 = (int)((int64_t)NB * (vr + 1) / NV);
    const int m0 = mtile * ROWS;
    // rows at a fixed pitch of kXresMaxK / 8 pieces (2 KiB), whatever K is, so
    // that a lane's read addresses differ between tiles and steps by constants;
    // piece p of row m sits at p ^ (m & 15)
    constexpr int PP = kXresMaxK / 8;
    const int P = K / 8;                       // 16-byte pieces per row

    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, t = lane >> 4;
    // the lane's A operand of chunk ch of superchunk cc, activation tile mt:
    // row 16 mt + r, piece cc * CPS * 4 + 4 ch + t, stored at that piece ^ r;
    // when a superchunk spans 16 pieces (int4) the XOR touches only the
    // 4 ch + t part, so the address is aoff[ch] + cc * 256 + mt * 16 * PP * 16
    // bytes
    constexpr bool kFixedA = CPS * 4 == 16;
    uint32_t aoff[CPS];
#pragma unroll
    for (int ch = 0; ch < CPS; ++ch) aoff[ch] = (uint32_t)(r * PP + ((4 * ch + t) ^ r)) * 16u;
    // 4-element output stores need rows aligned to 4 elements
    constexpr int OSZ = OUT == F32 ? 4 : 2;
    const bool vec16 = ((uintptr_t)y & (4 * OSZ - 1)) == 0 && (ldy & 3) == 0;
    // the wave's units: u = wv + WAVES i, row block rb0 + u / PARTS, columns
    // from 16 nb on; WAVES is a multiple of PARTS, so nb is the wave's own
    static_assert(WAVES % PARTS == 0, "each wave keeps one column range");
    const int nb = (wv % PARTS) * NT;
    const int nunit = (rb1 - rb0) * PARTS;
    const int nblk = nunit > wv ? (nunit - wv + WAVES - 1) / WAVES : 0;
    const int nsteps = nblk * NC;

    // ring stage: the NT slots, and per group and column tile the scales of the
    // lane's vocabulary rows: row 16 nt + r (one 2-byte load), or with TR the
    // 4 rows 16 nt + 4 t .. + 3 (one 8-byte load); with ZP per group the zero
    // points of the rows the lane unpacks, 16 nt + r (one 4-byte load)
    using SW = typename std::conditional<TR, uint2, uint16_t>::type;
    uint4 wbuf[D][NT];
    SW sbuf[D][GPS][NT];
    uint32_t zbuf[D][GPS];
    auto load = [&](int p, int s) {
        const int sl = min(s, nsteps - 1);
        const int i = sl / NC, c = sl - i * NC;
        const int blk = rb0 + wv / PARTS + (WAVES / PARTS) * i;
        const uint4* wp = wq + ((int64_t)blk * NC + c) * 256 + t * 64 + r + 16 * nb;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) wbuf[p][nt] = wp[16 * nt];
        const int g0 = GPS > 1 ? c * GPS : c / SPG;
        const uint16_t* sp = sc + ((int64_t)blk * NG + g0) * 64 + (TR ? 4 * t : r) + 16 * nb;
#pragma unroll
        for (int g = 0; g < GPS; ++g)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) sbuf[p][g][nt] = *(const SW*)(sp + g * 64 + 16 * nt);
        if constexpr (ZP) {
            const uint32_t* zp = (const uint32_t*)zq + ((int64_t)blk * NG + g0) * 16 + r;
#pragma unroll
            for (int g = 0; g < GPS; ++g) zbuf[p][g] = zp[g * 16];
        }
    };

    // the ring's first steps are requested before the activation tile is
    // staged, so that their latency overlaps the staging (where the ring's
    // registers fit beside the staging loop's without spilling: the 32-row
    // tile, and the symmetric int4 fp32-output kernels)
    constexpr bool kEarly = MT_ == 2 || (BITS == 4 && !ZP && OUT == F32);
    if (kEarly && nsteps > 0) {
#pragma unroll
        for (int p = 0; p < D; ++p) load(p, p);
    }
    for (int i = threadIdx.x; i < ROWS * P; i += NTH) {
        const int m = i / P, p = i - m * P;
        const int mr = min(m0 + m, M - 1);     // rows past M: any valid row, never stored
        xs[m * PP + (p ^ (m & 15))] = *(const uint4*)(x + (int64_t)mr * K + p * 8);
    }
    if (xexp && threadIdx.x < ROWS) xe_s[threadIdx.x] = xexp[min(m0 + (int)threadIdx.x, M - 1)];
    __syncthreads();
    if (nsteps == 0) return;

    f4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
    const uint32_t magic = 0x64006400u;

    if constexpr (!kEarly) {
#pragma unroll
        for (int p = 0; p < D; ++p) load(p, p);
    }
    int ci = 0, cc = 0;  // block index within the wave's list, superchunk of step s
    for (int sb = 0; sb < nsteps; sb += D) {
#pragma unroll
        for (int p = 0; p < D; ++p) {
            const int s = sb + p;
            const bool real = s < nsteps;
#pragma unroll
            for (int g = 0; g < GPS; ++g) {
                h8 bop[NT][CPG];
                f4 sv[NT];  // the scale of each of the lane's 4 result elements
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const ZC zc = ZP ? zc_byte(zbuf[p][g], nb + nt) : zc_sym<BITS>();
#pragma unroll
                    for (int jj = 0; jj < CPG; ++jj) {
                        h2 p0, p1, p2, p3;
                        if constexpr (BITS == 4) {
                            unpack_i4(word_of(wbuf[p][nt], g * WPG + jj), magic, zc, p0, p1, p2, p3);
                        } else {
                            unpack_i8(word_of(wbuf[p][nt], g * WPG + 2 * jj), zc, p0, p1);
                            unpack_i8(word_of(wbuf[p][nt], g * WPG + 2 * jj + 1), zc, p2, p3);
                        }
                        bop[nt][jj] = (h8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
                    }
                    // (a step past the wave's last is not masked: the last
                    // real step ends a unit, whose results are stored and
                    // whose accumulators are cleared, so what such a step
                    // adds is never stored)
                    if constexpr (TR) {
                        const uint2 sw = sbuf[p][g][nt];
                        sv[nt] = (f4){scale_to_f32((uint16_t)sw.x, SB),
                                      scale_to_f32((uint16_t)(sw.x >> 16), SB),
                                      scale_to_f32((uint16_t)sw.y, SB),
                                      scale_to_f32((uint16_t)(sw.y >> 16), SB)};
                    } else {
                        const float v1 = scale_to_f32(sbuf[p][g][nt], SB);
                        sv[nt] = (f4){v1, v1, v1, v1};
                    }
                }
                // activation tiles in a software pipeline: the MFMA chains of
                // tile mt are issued before the scale FMAs of tile mt - 1 read
                // their results, so the chains' latency is hidden
                auto read_a = [&](int mt, h8 (&a)[CPG]) {
#pragma unroll
                    for (int jj = 0; jj < CPG; ++jj) {
                        if constexpr (kFixedA) {
                            const uint32_t off = aoff[g * CPG + jj] + (uint32_t)cc * 256u +
                                                 (uint32_t)mt * (16 * PP * 16);
                            a[jj] = __builtin_bit_cast(h8, *(const uint4*)((const char*)xs + off));
                        } else {
                            const int m = 16 * mt + r;
                            const int pc = cc * (SPAN / 8) + 4 * (g * CPG + jj) + t;
                            a[jj] = __builtin_bit_cast(h8, xs[m * PP + (pc ^ r)]);
                        }
                    }
                };
                f4 pq[2][NT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    h8 a[CPG];
                    read_a(mt, a);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        // D[4t + e][r] holds activation row 16 mt + 4 t + e and
                        // vocabulary row 16 nt + r; with TR (weights as the A
                        // operand) vocabulary row 16 nt + 4 t + e and activation
                        // row 16 mt + r.  Same products, same sums, either way.
                        f4 q = TR ? __builtin_amdgcn_mfma_f32_16x16x32_f16(bop[nt][0], a[0],
                                                                            (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0)
                                  : __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], bop[nt][0],
                                                                            (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                        for (int jj = 1; jj < CPG; ++jj)
                            q = TR ? __builtin_amdgcn_mfma_f32_16x16x32_f16(bop[nt][jj], a[jj], q, 0, 0, 0)
                                   : __builtin_amdgcn_mfma_f32_16x16x32_f16(a[jj], bop[nt][jj], q, 0, 0, 0);
                        pq[mt & 1][nt] = q;
                    }
                    if (mt > 0) {
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) acc[mt - 1][nt] += sv[nt] * pq[(mt - 1) & 1][nt];
                    }
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[MT - 1][nt] += sv[nt] * pq[(MT - 1) & 1][nt];
            }
            load(p, s + D);
            if (real && cc == NC - 1) {
                if constexpr (TR) {
                // the unit's results: y[m, v] = acc * 2^xexp[m] + bias[v] for
                // row m = m0 + 16 mt + r and the 4 columns v = cb + 16 nt +
                // 4 t + e, e = 0..3, contiguous: one 16-byte store each (when
                // y's rows are 16-byte aligned and all 4 columns exist)
                const int blk = rb0 + wv / PARTS + (WAVES / PARTS) * ci;
                const int cb = blk * 64 + 16 * nb;  // the unit's first column
                const int vlim = V - cb - 4 * t;  // 16 nt + e < vlim: column inside V
                int mlim = M - m0 - r;                  // 16 mt < mlim: row inside M
                // (kept opaque so the row tests stay here instead of being
                // hoisted out of the loop)
                asm volatile("" : "+v"(mlim));
                f4 bv[NT];
                if (bias) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            bv[nt][e] = 16 * nt + e < vlim ? bias[cb + 16 * nt + 4 * t + e] : 0.0f;
                    wait_vm_all();
                } else {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) bv[nt] = (f4){0.f, 0.f, 0.f, 0.f};
                }
                YT<OUT>* yrow = (YT<OUT>*)y + (int64_t)(m0 + r) * ldy + (int64_t)cb + 4 * t;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (16 * mt < mlim) {
                        const int xe = xexp ? xe_s[16 * mt + r] : 0;
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            f4 o = acc[mt][nt];
                            if (xexp) {
#pragma unroll
                                for (int e = 0; e < 4; ++e) o[e] = ldexpf(o[e], xe);
                            }
                            o = o + bv[nt];
                            if (vec16 && 16 * nt + 3 < vlim) {
                                store4<OUT>(yrow + 16 * nt, o);
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (16 * nt + e < vlim) yrow[16 * nt + e] = to_out<OUT>(o[e]);
                            }
                        }
                    }
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
                    yrow += 16 * ldy;
                }
                } else {
                // the unit's results: y[m, v] = acc * 2^xexp[m] + bias[v] for
                // rows m = m0 + 16 mt + 4 t + e and columns v = cb + 16 nt + r,
                // through one row pointer that steps down the lane's rows
                const int blk = rb0 + wv / PARTS + (WAVES / PARTS) * ci;
                const int cb = blk * 64 + 16 * nb;  // the unit's first column
                if (xexp == nullptr && V - cb >= 16 * NT) {
                    // every column of the unit inside V, fp16 x: no column
                    // tests, and row tests only in a tile that extends past M
                    // (one per row of NT stores)
                    float bv[NT];
                    if (bias) {
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) bv[nt] = bias[cb + 16 * nt + r];
                        wait_vm_all();
                    } else {
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) bv[nt] = 0.0f;
                    }
                    YT<OUT>* yrow = (YT<OUT>*)y + (int64_t)(m0 + 4 * t) * ldy + (int64_t)cb + r;
                    auto row_out = [&](int mt, int e) {
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            yrow[16 * nt] = to_out<OUT>(acc[mt][nt][e] + bv[nt]);
                    };
                    if (M - m0 >= ROWS) {
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                row_out(mt, e);
                                yrow += ldy;
                            }
                            yrow += 12 * ldy;
                        }
                    } else {
                        int mlim = M - m0 - 4 * t;  // 16 mt + e < mlim: row inside M
                        asm volatile("" : "+v"(mlim));
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                if (16 * mt + e < mlim) row_out(mt, e);
                                yrow += ldy;
                            }
                            yrow += 12 * ldy;
                        }
                    }
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
                } else {
                const int vlim = V - cb - r;  // 16 nt < vlim: column inside V
                int mlim = M - m0 - 4 * t;          // 16 mt + e < mlim: row inside M
                // (kept opaque so the row tests stay here instead of being
                // hoisted out of the loop, where they would pin 32 SGPRs)
                asm volatile("" : "+v"(mlim));
                float bv[NT];
                if (bias) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) bv[nt] = 16 * nt < vlim ? bias[cb + 16 * nt + r] : 0.0f;
                    wait_vm_all();
                } else {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) bv[nt] = 0.0f;
                }
                YT<OUT>* yrow = (YT<OUT>*)y + (int64_t)(m0 + 4 * t) * ldy + (int64_t)cb + r;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool rowok = 16 * mt + e < mlim;
                        const int xe = xexp ? xe_s[16 * mt + 4 * t + e] : 0;
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            if (rowok && 16 * nt < vlim) {
                                float o = acc[mt][nt][e];
                                if (xexp) o = ldexpf(o, xe);
                                yrow[16 * nt] = to_out<OUT>(o + bv[nt]);
                            }
                            acc[mt][nt][e] = 0.0f;
                        }
                        yrow += ldy;
                    }
                    yrow += 12 * ldy;  // the lane's next rows are 16 further on
                }
                }
                }
            }
            if (++cc == NC) {
                cc = 0;
                ++ci;
            }
        }
    }
}


template <int BITS, int MT, int OUT, bool ZP>
hipError_t mfma_dispatch_mt(const LogitsArgs& a, hipStream_t st) {
    const int NB = (int)((a.V + 63) / 64);
    const int NC = (int)(a.K / span_of(BITS));
    const int NG = (int)(a.K / a.G);
    const int gps = gps_of(BITS, a.G);
    const int SPG = gps == 1 ? (int)(a.G / span_of(BITS)) : 1;
    const Regions<BITS> rg(a, ZP);
    const dim3 grid((NB + 3) / 4, (a.M + MT * 16 - 1) / (MT * 16));
#define LMH_MFMA(G_)                                                                               \
    hipLaunchKernelGGL((mfma_kernel<BITS, MT, G_, OUT, ZP>), grid, dim3(256), 0, st, rg.wq, rg.sc, \
                       rg.zq,                                                                     \
                       (const _Float16*)a.x, a.xexp, a.bias, a.y, a.ldy, (int)a.V, (int)a.K, a.M, \
                       NB, NC, NG, SPG, a.scale_bf16)
    if (gps == 1) LMH_MFMA(1);
    else if constexpr (BITS == 8) LMH_MFMA(2);
    else if (gps == 2) LMH_MFMA(2);
    else LMH_MFMA(4);
#undef LMH_MFMA
    return hipGetLastError();
}

template <int BITS, int MT, int STAGES, int WPB, int OUT, bool ZP>
hipError_t mfma_lds_dispatch_mt(const LogitsArgs& a, hipStream_t st) {
    const int NB = (int)((a.V + 63) / 64);
    const int NC = (int)(a.K / span_of(BITS));
    const int NG = (int)(a.K / a.G);
    const int gps = gps_of(BITS, a.G);
    const int SPG = gps == 1 ? (int)(a.G / span_of(BITS)) : 1;
    const Regions<BITS> rg(a, ZP);
    const int NMT = (a.M + MT * 16 - 1) / (MT * 16);
    const int total = (NB + WPB - 1) / WPB * NMT;
    // one tile per workgroup (the kernel also runs several tiles per
    // workgroup, back to back, when the grid is smaller: measured slower on
    // the 151936 x 1024 head, whose output stores then stall the next tile)
    const dim3 grid((unsigned)((total + 7) / 8 * 8));
#define LMH_MFMA_LDS(G_)                                                                           \
    hipLaunchKernelGGL((mfma_lds_kernel<BITS, MT, G_, STAGES, WPB, OUT, ZP>), grid,               \
                       dim3(64 * WPB), 0, st, rg.wq, rg.sc, rg.zq,                                \
                       (const _Float16*)a.x, a.xexp, a.bias, a.y, a.ldy, (int)a.V, (int)a.K, a.M, \
                       NB, NC, NG, SPG, a.scale_bf16, NMT, total)
    if (gps == 1) LMH_MFMA_LDS(1);
    else if constexpr (BITS == 8) LMH_MFMA_LDS(2);
    else if (gps == 2) LMH_MFMA_LDS(2);
    else LMH_MFMA_LDS(4);
#undef LMH_MFMA_LDS
    return hipGetLastError();
}

template <int BITS, int OUT, bool ZP>
hipError_t mfma_lds_dispatch(const LogitsArgs& a, hipStream_t st) {
    // 32-row tiles for M <= 32 (3 workgroups of 4 waves per CU), else 64-row
    // tiles (2 per CU).  Measured on the 151936 x 1024 int4 head, M = 128 and
    // 256: 128-row tiles, with one workgroup of 4 or 8 waves per CU, lose more
    // to the waves meeting at one barrier than they gain from sharing each
    // unpacked operand among more MFMAs.
    if (a.M <= 32) return mfma_lds_dispatch_mt<BITS, 2, 2, 4, OUT, ZP>(a, st);
    return mfma_lds_dispatch_mt<BITS, 4, 2, 4, OUT, ZP>(a, st);
}

template <int BITS, int D, bool TR, int OUT, bool ZP, int NT_, int MT_>
hipError_t mfma_xres_dispatch_d(const LogitsArgs& a, hipStream_t st) {
    const int NB = (int)((a.V + 63) / 64);
    const int NC = (int)(a.K / span_of(BITS));
    const int NG = (int)(a.K / a.G);
    const int gps = gps_of(BITS, a.G);
    const int SPG = gps == 1 ? (int)(a.G / span_of(BITS)) : 1;
    const Regions<BITS> rg(a, ZP);
    const int NMT = (a.M + 16 * MT_ - 1) / (16 * MT_);
    // one workgroup per CU: per XCD, NMT activation tiles x VRX vocabulary ranges
    const int VRX = NMT >= 32 ? 1 : 32 / NMT;
    const dim3 grid((unsigned)(8 * NMT * VRX));
#define LMH_XRES_SB(G_, SB_)                                                                      \
    hipLaunchKernelGGL((mfma_xres_kernel<BITS, G_, D, TR, OUT, ZP, NT_, SB_, MT_>), grid,        \
                       dim3(64 * xres_waves<NT_>()), 0, st,                                       \
                       rg.wq, rg.sc, rg.zq,                                                       \
                       (const _Float16*)a.x, a.xexp, a.bias, a.y, a.ldy, (int)a.V, (int)a.K, a.M, \
                       NB, NC, NG, SPG, NMT, VRX)
#define LMH_XRES(G_)                                                                              \
    do {                                                                                          \
        if (a.scale_bf16) LMH_XRES_SB(G_, 1);                                                     \
        else LMH_XRES_SB(G_, 0);                                                                  \
    } while (0)
    if (gps == 1) LMH_XRES(1);
    else if constexpr (BITS == 8) LMH_XRES(2);
    else if (gps == 2) LMH_XRES(2);
    else LMH_XRES(4);
#undef LMH_XRES
#undef LMH_XRES_SB
    return hipGetLastError();
}

template <int BITS, int OUT, bool ZP>
hipError_t mfma_dispatch(const LogitsArgs& a, hipStream_t st) {
    // one 16-row activation tile for M <= 16; two (32 rows) otherwise: the
    // 64-row tile needs one wave per SIMD and loses more to latency than it
    // saves in unpacking (measured on the 151936 x 1024 head, M = 64..256)
    if (a.M <= 16) return mfma_dispatch_mt<BITS, 1, OUT, ZP>(a, st);
    return mfma_dispatch_mt<BITS, 2, OUT, ZP>(a, st);
}

// int4: results as activation rows x single vocabulary columns; int8:
// transposed results (4 contiguous vocabulary columns per lane, one 4-element
// store); both with a 2-deep ring -- the fastest of the variants that fit in
// 128 VGPRs (16 waves) on the 151936 x 1024 heads.  Up to 32 activation rows:
// a 32-row tile and 16-column units (NT = 1), which spread a head's columns
// over the 16 waves of a CU in 2-3 units each instead of 1-2.
template <int BITS, int OUT, bool ZP>
hipError_t xres_dispatch(const LogitsArgs& a, hipStream_t st) {
    if (a.M <= 32) {
        if constexpr (BITS == 4) return mfma_xres_dispatch_d<4, 2, false, OUT, ZP, 1, 2>(a, st);
        else return mfma_xres_dispatch_d<8, 2, true, OUT, ZP, 1, 2>(a, st);
    }
    if constexpr (BITS == 4) return mfma_xres_dispatch_d<4, 2, false, OUT, ZP, 2, 4>(a, st);
    else return mfma_xres_dispatch_d<8, 2, true, OUT, ZP, 2, 4>(a, st);
}

// The kernel family `f` for the head's code width and the output type.
template <bool ZP>
hipError_t run_family(int f, const LogitsArgs& a, hipStream_t st) {
#define LMH_BY_BITS_OUT(FN)                                                                       \
    switch (a.y_dtype) {                                                                          \
    case F32: return a.bits == 4 ? FN<4, F32, ZP>(a, st) : FN<8, F32, ZP>(a, st);                 \
    case F16: return a.bits == 4 ? FN<4, F16, ZP>(a, st) : FN<8, F16, ZP>(a, st);                 \
    default: return a.bits == 4 ? FN<4, BF16, ZP>(a, st) : FN<8, BF16, ZP>(a, st);                \
    }
    switch (f) {
    case kFamMfma: LMH_BY_BITS_OUT(mfma_dispatch)
    case kFamMfmaLds: LMH_BY_BITS_OUT(mfma_lds_dispatch)
    default: LMH_BY_BITS_OUT(xres_dispatch)
    }
#undef LMH_BY_BITS_OUT
}

}  // namespace
}  // namespace lmh

