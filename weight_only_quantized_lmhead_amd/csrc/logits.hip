// Fused weight-only-quantized logits: y[m,v] = sum_k x[m,k] * q[v,k] * s[v,k/G].
//
// vLLM PR #48870 ("Fused WNA16 GEMM for tied quantized lm_head logits",
// Purpose and perf table): the logits come straight from the packed codes and
// scales; the dense weight is never formed.  Its review comment (point 1)
// notes that M = 1 is purely bandwidth-bound: the only lever is bytes moved.
//
// Codes are unpacked exactly into fp16 in registers with the exponent trick:
// OR-ing a nibble n into the fp16 pattern 0x6400 gives 1024 + n, so one
// AND-OR per pair of codes plus one packed subtract yields q = n - 8 exactly
// (int8: a byte permute into 0x64xx gives 1024 + b, minus 1152).  Products
// with fp16 x are exact in fp32; each group's partial sum is accumulated in
// fp32 and multiplied by the group scale in fp32 (the scale never touches a
// 16-bit product).
//
// Kernels
//   x_to_f16     bf16 x -> fp16 x * 2^-e per row (exact power-of-two scale,
//                e chosen so max|x| lands in [2^14, 2^15)); y is scaled back.
//   gemv         M <= 4.  A wave owns 64 vocabulary rows (one row block, one
//                lane per row: no cross-lane reduction); the 4 waves of a
//                workgroup split K and add their partials through LDS in a
//                fixed order.  x is wave-uniform and is read through the
//                scalar unit straight into v_dot2 operands.
//   mfma         larger M.  A wave owns one row block (4 MFMA column tiles of
//                16 rows) and MT row tiles of 16 activations; each 16-byte
//                slot load is one 16x16x32 B operand per 32-column word.
//   dense        unquantized 16-bit control GEMV (the fp16 logits of the
//                review comment, point 1).
#include "lmh_internal.h"

#include <math.h>

namespace lmh {
namespace {

__device__ __forceinline__ float scale_to_f32(uint16_t b, int sbf16) {
    return sbf16 ? __uint_as_float((uint32_t)b << 16) : (float)__builtin_bit_cast(_Float16, b);
}

// int4 word (8 codes; even columns in the low nibbles of each half-word) ->
// four fp16 pairs (cols 0,1), (2,3), (4,5), (6,7), exact.
__device__ __forceinline__ void unpack_i4(uint32_t w, h2& p0, h2& p1, h2& p2, h2& p3) {
    const uint32_t hi = w >> 8;
    const h2 b1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 b72 = {(_Float16)-72.0f, (_Float16)-72.0f};
    p0 = __builtin_bit_cast(h2, (w & 0x000F000Fu) | 0x64006400u) + b1032;
    p1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (w & 0x00F000F0u) | 0x64006400u), sixteenth, b72);
    p2 = __builtin_bit_cast(h2, (hi & 0x000F000Fu) | 0x64006400u) + b1032;
    p3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (hi & 0x00F000F0u) | 0x64006400u), sixteenth, b72);
}

// int8 word (4 codes, byte i = column i, biased by 128) -> two fp16 pairs.
__device__ __forceinline__ void unpack_i8(uint32_t w, h2& p0, h2& p1) {
    const h2 b1152 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    p0 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, w, 0x04010400u)) + b1152;
    p1 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, w, 0x04030402u)) + b1152;
}

__device__ __forceinline__ uint32_t word_of(const uint4& u, int j) {
    return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
}

// ---------------------------------------------------------------------------
// bf16 x -> fp16 x * 2^-e, one workgroup per row.
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t* __restrict__ xb, int K,
                                                       _Float16* __restrict__ xh,
                                                       int* __restrict__ xexp) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    const uint16_t* row = xb + (int64_t)m * K;
    float amax = 0.0f;
    for (int k = threadIdx.x; k < K; k += 256) amax = fmaxf(amax, fabsf(__uint_as_float((uint32_t)row[k] << 16)));
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    if (amax > 0.0f) {
        int E;
        frexpf(amax, &E);  // amax = f * 2^E, f in [0.5, 1)
        e = E - 15;        // amax * 2^-e in [2^14, 2^15)
    }
    for (int k = threadIdx.x; k < K; k += 256)
        xh[(int64_t)m * K + k] = (_Float16)ldexpf(__uint_as_float((uint32_t)row[k] << 16), -e);
    if (threadIdx.x == 0) xexp[m] = e;
}

// ---------------------------------------------------------------------------
// GEMV: 4 waves per 64-row block, K split in 4 contiguous superchunk ranges.
// GPS = groups per superchunk (1 when a group spans >= 1 superchunk).
template <int BITS, int MM, int GPS>
__global__ __launch_bounds__(256) void gemv_kernel(const uint4* __restrict__ wq,
                                                   const uint16_t* __restrict__ sc,
                                                   const h2* __restrict__ x,
                                                   const int* __restrict__ xexp,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ y, int64_t ldy, int V, int K,
                                                   int NC, int NG, int SPG, int sbf16) {
    constexpr int SPAN = BITS == 4 ? 128 : 64;
    constexpr int CPS = SPAN / 32;    // 32-column chunks per superchunk
    constexpr int CPG = CPS / GPS;    // chunks per group when GPS > 1
    __shared__ float red[4][MM][64];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int blk = blockIdx.x;
    const int c0 = (NC * wv) / 4, c1 = (NC * (wv + 1)) / 4;
    const uint4* wp = wq + (int64_t)blk * NC * 256 + lane;
    const uint16_t* sp = sc + (int64_t)blk * NG * 64 + lane;
    const int Kh = K >> 1;

    float acc[MM];
    float part[MM][GPS];
#pragma unroll
    for (int m = 0; m < MM; ++m) {
        acc[m] = 0.0f;
#pragma unroll
        for (int g = 0; g < GPS; ++g) part[m][g] = 0.0f;
    }
    // group bookkeeping for GPS == 1
    int g_cur = (GPS == 1) ? c0 / SPG : 0;
    int left = (GPS == 1) ? SPG - (c0 - g_cur * SPG) : 0;
    float sv = 0.0f;
    if (GPS == 1 && c0 < c1) sv = scale_to_f32(sp[(int64_t)g_cur * 64], sbf16);

    uint4 cur[4], nxt[4];
    if (c0 < c1) {
#pragma unroll
        for (int t = 0; t < 4; ++t) cur[t] = wp[((int64_t)c0 * 4 + t) * 64];
    }
    for (int c = c0; c < c1; ++c) {
        if (c + 1 < c1) {
#pragma unroll
            for (int t = 0; t < 4; ++t) nxt[t] = wp[((int64_t)(c + 1) * 4 + t) * 64];
        }
        float sg[GPS];
        if constexpr (GPS > 1) {
#pragma unroll
            for (int g = 0; g < GPS; ++g) sg[g] = scale_to_f32(sp[((int64_t)c * GPS + g) * 64], sbf16);
        }
        const int xc = c * (SPAN / 2);  // half2 index of the superchunk's first column
#pragma unroll
        for (int j = 0; j < CPS; ++j) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if constexpr (BITS == 4) {
                    h2 p0, p1, p2, p3;
                    unpack_i4(word_of(cur[t], j), p0, p1, p2, p3);
                    const int xi = xc + 16 * j + 4 * t;  // cols 128c + 32j + 8t
#pragma unroll
                    for (int m = 0; m < MM; ++m) {
                        const h2* xm = x + (int64_t)m * Kh + xi;
                        float a = part[m][j / CPG];
                        a = __builtin_amdgcn_fdot2(p0, xm[0], a, false);
                        a = __builtin_amdgcn_fdot2(p1, xm[1], a, false);
                        a = __builtin_amdgcn_fdot2(p2, xm[2], a, false);
                        a = __builtin_amdgcn_fdot2(p3, xm[3], a, false);
                        part[m][j / CPG] = a;
                    }
                } else {
                    h2 p0, p1, p2, p3;
                    unpack_i8(word_of(cur[t], 2 * j), p0, p1);
                    unpack_i8(word_of(cur[t], 2 * j + 1), p2, p3);
                    const int xi = xc + 16 * j + 4 * t;  // cols 64c + 32j + 8t
#pragma unroll
                    for (int m = 0; m < MM; ++m) {
                        const h2* xm = x + (int64_t)m * Kh + xi;
                        float a = part[m][j / CPG];
                        a = __builtin_amdgcn_fdot2(p0, xm[0], a, false);
                        a = __builtin_amdgcn_fdot2(p1, xm[1], a, false);
                        a = __builtin_amdgcn_fdot2(p2, xm[2], a, false);
                        a = __builtin_amdgcn_fdot2(p3, xm[3], a, false);
                        part[m][j / CPG] = a;
                    }
                }
            }
        }
        if constexpr (GPS > 1) {
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int g = 0; g < GPS; ++g) {
                    acc[m] = fmaf(sg[g], part[m][g], acc[m]);
                    part[m][g] = 0.0f;
                }
        } else {
            if (--left == 0 || c + 1 == c1) {
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    acc[m] = fmaf(sv, part[m][0], acc[m]);
                    part[m][0] = 0.0f;
                }
                if (left == 0 && c + 1 < c1) {
                    ++g_cur;
                    left = SPG;
                    sv = scale_to_f32(sp[(int64_t)g_cur * 64], sbf16);
                }
            }
        }
        if (c + 1 < c1) {
#pragma unroll
            for (int t = 0; t < 4; ++t) cur[t] = nxt[t];
        }
    }
#pragma unroll
    for (int m = 0; m < MM; ++m) red[wv][m][lane] = acc[m];
    __syncthreads();
    if (wv == 0) {
        const int v = blk * 64 + lane;
        if (v < V) {
            const float b = bias ? bias[v] : 0.0f;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float r = ((red[0][m][lane] + red[1][m][lane]) + red[2][m][lane]) + red[3][m][lane];
                if (xexp) r = ldexpf(r, xexp[m]);
                y[(int64_t)m * ldy + v] = r + b;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// MFMA kernel.  Grid: x = row blocks (one per wave, 4 per workgroup), y = row
// tiles of MT*16 activations.  Lane (r = lane & 15, t = lane >> 4) reads slot
// t of vocabulary row 16*nt + r; word j of that slot is the 8-value B operand
// (k = 8t .. 8t+7 of the 32-column chunk) of one v_mfma_f32_16x16x32_f16, and
// the A operand is x[m0 + 16*mt + r][chunk + 8t .. +8].  The 16x16 result
// lands as D[4t + e][r]: activation row 4t + e, vocabulary row r.
template <int BITS, int MT, int GPS>
__global__ __launch_bounds__(256) void mfma_kernel(const uint4* __restrict__ wq,
                                                   const uint16_t* __restrict__ sc,
                                                   const _Float16* __restrict__ x,
                                                   const int* __restrict__ xexp,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ y, int64_t ldy, int V, int K,
                                                   int M, int NB, int NC, int NG, int SPG,
                                                   int sbf16) {
    constexpr int NT = 4;
    constexpr int SPAN = BITS == 4 ? 128 : 64;
    constexpr int CPS = SPAN / 32;
    constexpr int CPG = CPS / GPS;
    const int lane = threadIdx.x & 63;
    const int blk = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= NB) return;  // wave-uniform; this kernel has no barriers
    const int r = lane & 15, t = lane >> 4;
    const int m0 = blockIdx.y * MT * 16;
    const uint4* wp = wq + (int64_t)blk * NC * 256 + t * 64 + r;
    const uint16_t* sp = sc + (int64_t)blk * NG * 64 + r;

    // activation row pointers (rows past M read row 0 and are zeroed)
    const _Float16* xr[MT];
    bool xok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + 16 * mt + r;
        xok[mt] = m < M;
        xr[mt] = x + (int64_t)(xok[mt] ? m : 0) * K + 8 * t;
    }

    f4 acc[MT][NT], part[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            acc[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
            part[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
        }
    int g_cur = 0, left = SPG;
    float sv[NT];
    if (GPS == 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sv[nt] = scale_to_f32(sp[16 * nt], sbf16);
    }

    for (int c = 0; c < NC; ++c) {
        uint4 wv[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) wv[nt] = wp[(int64_t)c * 256 + 16 * nt];
        float sg[GPS][NT];
        if constexpr (GPS > 1) {
#pragma unroll
            for (int g = 0; g < GPS; ++g)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    sg[g][nt] = scale_to_f32(sp[((int64_t)c * GPS + g) * 64 + 16 * nt], sbf16);
        }
#pragma unroll
        for (int j = 0; j < CPS; ++j) {
            h8 a[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                h8 v = *(const h8*)(xr[mt] + (int64_t)c * SPAN + 32 * j);
                a[mt] = xok[mt] ? v : (h8){0, 0, 0, 0, 0, 0, 0, 0};
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                h2 p0, p1, p2, p3;
                if constexpr (BITS == 4) {
                    unpack_i4(word_of(wv[nt], j), p0, p1, p2, p3);
                } else {
                    unpack_i8(word_of(wv[nt], 2 * j), p0, p1);
                    unpack_i8(word_of(wv[nt], 2 * j + 1), p2, p3);
                }
                const h8 b = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    part[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt], b, part[mt][nt], 0, 0, 0);
            }
            if constexpr (GPS > 1) {
                if ((j + 1) % CPG == 0) {
                    const int g = j / CPG;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            acc[mt][nt] += sg[g][nt] * part[mt][nt];
                            part[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
                        }
                }
            }
        }
        if constexpr (GPS == 1) {
            if (--left == 0) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        acc[mt][nt] += sv[nt] * part[mt][nt];
                        part[mt][nt] = (f4){0.f, 0.f, 0.f, 0.f};
                    }
                left = SPG;
                if (++g_cur < NG) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        sv[nt] = scale_to_f32(sp[(int64_t)g_cur * 64 + 16 * nt], sbf16);
                }
            }
        }
    }
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
                    y[(int64_t)m * ldy + v] = o + b;
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Dense 16-bit control GEMV: a wave computes 4 rows at a time; lane l covers
// columns 8l + 512i; partial sums meet in a fixed xor-shuffle tree.
template <int DT, int MM>
__global__ __launch_bounds__(256) void dense_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ w,
                                                    float* __restrict__ y, int64_t ldy, int64_t V,
                                                    int K) {
    constexpr int R = 4;
    const int lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    if (row0 >= V) return;
    const int nk = (K + 511) / 512;
    float acc[R][MM];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[i][m] = 0.0f;
    for (int i = 0; i < nk; ++i) {
        const int k = 8 * lane + 512 * i;
        if (k >= K) break;
        uint4 xv[MM];
#pragma unroll
        for (int m = 0; m < MM; ++m) xv[m] = *(const uint4*)(x + (int64_t)m * K + k);
        uint4 wv[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int64_t v = row0 + rr < V ? row0 + rr : V - 1;
            wv[rr] = *(const uint4*)(w + v * K + k);
        }
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t a = word_of(wv[rr], q), b = word_of(xv[m], q);
                    if constexpr (DT == F16)
                        acc[rr][m] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), acc[rr][m], false);
                    else {
                        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                        acc[rr][m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a), __builtin_bit_cast(bf2, b), acc[rr][m], false);
                    }
                }
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            float a = acc[rr][m];
            for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o);
            acc[rr][m] = a;
        }
    if (lane < R * MM) {
        const int rr = lane / MM, m = lane % MM;
        const int64_t v = row0 + rr;
        float val = 0.0f;
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int mm = 0; mm < MM; ++mm)
                if (i == rr && mm == m) val = acc[i][mm];
        if (v < V) y[(int64_t)m * ldy + v] = val;
    }
}

inline int gps_of(int bits, int64_t G) {
    const int span = span_of(bits);
    return G >= span ? 1 : span / (int)G;
}

template <int BITS, int MM>
hipError_t gemv_dispatch_gps(const LogitsArgs& a, int gps, hipStream_t st) {
    const int NB = (int)((a.V + 63) / 64);
    const int NC = (int)(a.K / span_of(BITS));
    const int NG = (int)(a.K / a.G);
    const int SPG = gps == 1 ? (int)(a.G / span_of(BITS)) : 1;
    const uint4* wq = (const uint4*)a.packed;
    const uint16_t* sc = (const uint16_t*)(a.packed + (int64_t)NB * 64 * a.K * BITS / 8);
#define LMH_GEMV(G_)                                                                           \
    hipLaunchKernelGGL((gemv_kernel<BITS, MM, G_>), dim3(NB), dim3(256), 0, st, wq, sc,        \
                       (const h2*)a.x, a.xexp, a.bias, a.y, a.ldy, (int)a.V, (int)a.K, NC, NG, \
                       SPG, a.scale_bf16)
    if (gps == 1) LMH_GEMV(1);
    else if constexpr (BITS == 8) LMH_GEMV(2);
    else if (gps == 2) LMH_GEMV(2);
    else LMH_GEMV(4);
#undef LMH_GEMV
    return hipGetLastError();
}

template <int BITS>
hipError_t gemv_dispatch(const LogitsArgs& a, hipStream_t st) {
    const int gps = gps_of(BITS, a.G);
    switch (a.M) {
    case 1: return gemv_dispatch_gps<BITS, 1>(a, gps, st);
    case 2: return gemv_dispatch_gps<BITS, 2>(a, gps, st);
    case 3: return gemv_dispatch_gps<BITS, 3>(a, gps, st);
    default: return gemv_dispatch_gps<BITS, 4>(a, gps, st);
    }
}

template <int BITS, int MT>
hipError_t mfma_dispatch_mt(const LogitsArgs& a, hipStream_t st) {
    const int NB = (int)((a.V + 63) / 64);
    const int NC = (int)(a.K / span_of(BITS));
    const int NG = (int)(a.K / a.G);
    const int gps = gps_of(BITS, a.G);
    const int SPG = gps == 1 ? (int)(a.G / span_of(BITS)) : 1;
    const uint4* wq = (const uint4*)a.packed;
    const uint16_t* sc = (const uint16_t*)(a.packed + (int64_t)NB * 64 * a.K * BITS / 8);
    const dim3 grid((NB + 3) / 4, (a.M + MT * 16 - 1) / (MT * 16));
#define LMH_MFMA(G_)                                                                              \
    hipLaunchKernelGGL((mfma_kernel<BITS, MT, G_>), grid, dim3(256), 0, st, wq, sc,              \
                       (const _Float16*)a.x, a.xexp, a.bias, a.y, a.ldy, (int)a.V, (int)a.K, a.M, \
                       NB, NC, NG, SPG, a.scale_bf16)
    if (gps == 1) LMH_MFMA(1);
    else if constexpr (BITS == 8) LMH_MFMA(2);
    else if (gps == 2) LMH_MFMA(2);
    else LMH_MFMA(4);
#undef LMH_MFMA
    return hipGetLastError();
}

template <int BITS>
hipError_t mfma_dispatch(const LogitsArgs& a, hipStream_t st) {
    if (a.M <= 16) return mfma_dispatch_mt<BITS, 1>(a, st);
    if (a.M <= 32) return mfma_dispatch_mt<BITS, 2>(a, st);
    return mfma_dispatch_mt<BITS, 4>(a, st);
}

}  // namespace

hipError_t launch_x_to_f16(const uint16_t* x_bf16, int M, int K, _Float16* xh, int* xexp,
                           hipStream_t st) {
    hipLaunchKernelGGL(x_to_f16_kernel, dim3(M), dim3(256), 0, st, x_bf16, K, xh, xexp);
    return hipGetLastError();
}

hipError_t launch_gemv(const LogitsArgs& a, hipStream_t st) {
    return a.bits == 4 ? gemv_dispatch<4>(a, st) : gemv_dispatch<8>(a, st);
}

hipError_t launch_mfma(const LogitsArgs& a, hipStream_t st) {
    return a.bits == 4 ? mfma_dispatch<4>(a, st) : mfma_dispatch<8>(a, st);
}

hipError_t launch_dense(const void* x, int dtype, int M, const void* w, int64_t V, int64_t K,
                        float* y, int64_t ldy, hipStream_t st) {
    const int64_t nwaves = (V + 3) / 4;
    const dim3 grid((unsigned)((nwaves + 3) / 4)), block(256);
#define LMH_DENSE(DT, MM)                                                                        \
    hipLaunchKernelGGL((dense_kernel<DT, MM>), grid, block, 0, st, (const uint16_t*)x,          \
                       (const uint16_t*)w, y, ldy, V, (int)K)
    if (dtype == F16) {
        switch (M) {
        case 1: LMH_DENSE(F16, 1); break;
        case 2: LMH_DENSE(F16, 2); break;
        case 3: LMH_DENSE(F16, 3); break;
        default: LMH_DENSE(F16, 4); break;
        }
    } else {
        switch (M) {
        case 1: LMH_DENSE(BF16, 1); break;
        case 2: LMH_DENSE(BF16, 2); break;
        case 3: LMH_DENSE(BF16, 3); break;
        default: LMH_DENSE(BF16, 4); break;
        }
    }
#undef LMH_DENSE
    return hipGetLastError();
}

}  // namespace lmh
