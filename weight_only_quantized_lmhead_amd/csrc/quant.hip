// Load-time quantizer and packer kernels.
//
// Quantizer: page "radiance_lmhead_int4.py" (docstring "How" paragraph,
// module constants CLIP_RATIOS / QMAX / ZP_BIAS, quantize_int4_rows): per group
// of G columns one 16-bit scale, symmetric codes, scale rounded to the 16-bit
// type before the codes are chosen, optional least-squared-error search over
// the clip ratios 1.0 .. 0.8.  The results are bit-exact with a plain CPU
// implementation: IEEE-rounded fp32 division, ties-to-even everywhere, and the
// squared error summed in fp64 in ascending column order with one fused
// multiply-add per element.
//
// Packer: writes the blob layout documented in include/lmhead.h.
//
// Both kernels are load-time work (run once per head), VALU-bound rather than
// HBM-bound; they favour simple, obviously-exact code over speed.
#include "lmh_internal.h"

#include <math.h>

namespace lmh {
namespace {

// fp32 -> bfloat16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
    _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round-to-nearest-even mode
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

template <int WDT>
__device__ __forceinline__ float load_w(const void* w, int64_t i) {
    if constexpr (WDT == F32) return ((const float*)w)[i];
    else if constexpr (WDT == F16) return f16_to_f32(((const uint16_t*)w)[i]);
    else return bf16_to_f32(((const uint16_t*)w)[i]);
}

struct QuantConsts {
    float c[5];  // fl32(r / qmax) for each clip ratio, rounded on the host from doubles
};

// One thread per (row, group); the flat group f covers w[f*G, f*G + G).
template <int WDT>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ w, int64_t ngroups,
                                                       int G, int qmin, int qmax, int sbf16,
                                                       int nratios, QuantConsts cs,
                                                       int8_t* __restrict__ q,
                                                       uint16_t* __restrict__ s) {
#pragma clang fp contract(off)
    const int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (f >= ngroups) return;
    const int64_t base = f * (int64_t)G;
    float amax = 0.0f;
    for (int k = 0; k < G; ++k) amax = fmaxf(amax, fabsf(load_w<WDT>(w, base + k)));
    int8_t* qd = q + base;
    if (amax == 0.0f) {
        for (int k = 0; k < G; ++k) qd[k] = 0;
        s[f] = 0;
        return;
    }
    const float floor_s = sbf16 ? 1e-8f : 5.9604644775390625e-8f;  // 2^-24
    const float fqmin = (float)qmin, fqmax = (float)qmax;
    float best_s = 0.0f;
    double best_err = 0.0;
    for (int i = 0; i < nratios; ++i) {
        float s32 = amax * cs.c[i];
        s32 = s32 < floor_s ? floor_s : s32;
        const float sv = sbf16 ? bf16_to_f32(f32_to_bf16_rne(s32)) : f16_to_f32(f32_to_f16_rne(s32));
        if (nratios == 1) {
            best_s = sv;
            break;
        }
        double err = 0.0;
        const double sd = (double)sv;
        for (int k = 0; k < G; ++k) {
            const float wk = load_w<WDT>(w, base + k);
            float r = rintf(__fdiv_rn(wk, sv));
            r = fminf(fmaxf(r, fqmin), fqmax);
            const double d = (double)r * sd - (double)wk;  // exact: product and difference fit in 53 bits
            err = __builtin_fma(d, d, err);
        }
        if (i == 0 || err < best_err) {
            best_err = err;
            best_s = sv;
        }
    }
    for (int k = 0; k < G; ++k) {
        const float wk = load_w<WDT>(w, base + k);
        float r = rintf(__fdiv_rn(wk, best_s));
        r = fminf(fmaxf(r, fqmin), fqmax);
        qd[k] = (int8_t)(int)r;
    }
    s[f] = sbf16 ? f32_to_bf16_rne(best_s) : f32_to_f16_rne(best_s);
}

// One thread per 16-byte weight slot of the blob.
template <int BITS>
__global__ __launch_bounds__(256) void pack_weights_kernel(const int8_t* __restrict__ q, int64_t V,
                                                           int64_t K, int64_t nslots, int NC,
                                                           uint4* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nslots) return;
    const int r = (int)(i & 63);
    const int t = (int)((i >> 6) & 3);
    const int64_t bc = i >> 8;  // b * NC + c
    const int c = (int)(bc % NC);
    const int64_t b = bc / NC;
    const int64_t v = b * 64 + r;
    uint32_t word[4];
    if (v >= V) {
        const uint32_t pad = BITS == 4 ? 0x88888888u : 0x80808080u;
        for (int j = 0; j < 4; ++j) word[j] = pad;
    } else if constexpr (BITS == 4) {
        for (int j = 0; j < 4; ++j) {
            const int8_t* src = q + v * K + (int64_t)c * 128 + 32 * j + 8 * t;
            uint32_t wd = 0;
            for (int i8 = 0; i8 < 8; ++i8) {
                // column i8 goes to nibble position p: even columns 0,2,4,6 -> p 0..3,
                // odd columns 1,3,5,7 -> p 4..7
                const int p = (i8 & 1) ? 4 + (i8 >> 1) : (i8 >> 1);
                wd |= (uint32_t)((src[i8] + 8) & 0xF) << (4 * p);
            }
            word[j] = wd;
        }
    } else {
        for (int j = 0; j < 4; ++j) {
            const int8_t* src = q + v * K + (int64_t)c * 64 + 32 * (j >> 1) + 8 * t + 4 * (j & 1);
            uint32_t wd = 0;
            for (int i4 = 0; i4 < 4; ++i4) wd |= (uint32_t)(uint8_t)(src[i4] + 128) << (8 * i4);
            word[j] = wd;
        }
    }
    out[i] = make_uint4(word[0], word[1], word[2], word[3]);
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint16_t* __restrict__ s, int64_t V,
                                                          int NG, int64_t n,
                                                          uint16_t* __restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n) return;
    const int r = (int)(e & 63);
    const int64_t bg = e >> 6;
    const int g = (int)(bg % NG);
    const int64_t b = bg / NG;
    const int64_t v = b * 64 + r;
    out[e] = v < V ? s[v * NG + g] : (uint16_t)0;
}

inline unsigned grid_for(int64_t n, int block) { return (unsigned)((n + block - 1) / block); }

}  // namespace

hipError_t launch_quantize(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t G,
                           int scale_dtype, int nratios, int8_t* q, uint16_t* s, hipStream_t st) {
    static const double kRatios[5] = {1.0, 0.95, 0.9, 0.85, 0.8};
    const int qmax = bits == 4 ? 7 : 127;
    const int qmin = bits == 4 ? -8 : -128;
    QuantConsts cs;
    for (int i = 0; i < 5; ++i) cs.c[i] = (float)(kRatios[i] / (double)qmax);
    const int64_t ngroups = V * (K / G);
    const dim3 grid(grid_for(ngroups, 256)), block(256);
    const int sbf = scale_dtype == BF16;
    switch (w_dtype) {
    case F32:
        hipLaunchKernelGGL(quantize_kernel<F32>, grid, block, 0, st, w, ngroups, (int)G, qmin, qmax,
                           sbf, nratios, cs, q, s);
        break;
    case F16:
        hipLaunchKernelGGL(quantize_kernel<F16>, grid, block, 0, st, w, ngroups, (int)G, qmin, qmax,
                           sbf, nratios, cs, q, s);
        break;
    default:
        hipLaunchKernelGGL(quantize_kernel<BF16>, grid, block, 0, st, w, ngroups, (int)G, qmin,
                           qmax, sbf, nratios, cs, q, s);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_pack(const int8_t* q, const uint16_t* s, int64_t V, int64_t K, int bits,
                       int64_t G, uint8_t* out, hipStream_t st) {
    const int64_t NB = (V + 63) / 64;
    const int NC = (int)(K / span_of(bits));
    const int NG = (int)(K / G);
    const int64_t nslots = NB * NC * 256;
    if (bits == 4)
        hipLaunchKernelGGL(pack_weights_kernel<4>, dim3(grid_for(nslots, 256)), dim3(256), 0, st, q,
                           V, K, nslots, NC, (uint4*)out);
    else
        hipLaunchKernelGGL(pack_weights_kernel<8>, dim3(grid_for(nslots, 256)), dim3(256), 0, st, q,
                           V, K, nslots, NC, (uint4*)out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nsc = NB * NG * 64;
    uint16_t* sout = (uint16_t*)(out + NB * 64 * K * bits / 8);
    hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(nsc, 256)), dim3(256), 0, st, s, V, NG, nsc,
                       sout);
    return hipGetLastError();
}

}  // namespace lmh
