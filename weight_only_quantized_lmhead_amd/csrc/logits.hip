// Fused weight-only-quantized logits: the symmetric instantiations of the
// MFMA kernels in logits_kernels.h, the bf16 -> fp16 activation conversion
// they take, the dense control GEMV and the MFMA launch entry points (which
// hand zero-point heads to logits_zp.hip).
#include "logits_kernels.h"

namespace lmh {
namespace {

// ---------------------------------------------------------------------------
// bf16 x -> fp16 x * 2^-e, one workgroup per row: max |x| of the row (16-byte
// loads; the order of non-negative bf16 bit patterns is the order of their
// values), e such that max |x| * 2^-e lies in [2^14, 2^15), then every
// element rounded once to fp16 (the same conversion the GEMV does in LDS).
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t* __restrict__ xb, int K,
                                                       _Float16* __restrict__ xh,
                                                       int* __restrict__ xexp) {
    __shared__ uint32_t red[4];
    const int m = blockIdx.x;
    const int P = K >> 3;  // 16-byte pieces per row (K is a multiple of 64)
    const uint4* row = (const uint4*)(xb + (int64_t)m * K);
    uint32_t mx = 0;
    for (int i = threadIdx.x; i < P; i += 256) {
        const uint4 v = row[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = word_of(v, j);
            mx = max(mx, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    const float amax = __uint_as_float(mx << 16);
    int e = 0;
    if (amax > 0.0f) {
        int E;
        frexpf(amax, &E);  // amax = f * 2^E, f in [0.5, 1)
        e = E - 15;        // amax * 2^-e in [2^14, 2^15)
    }
    uint4* out = (uint4*)(xh + (int64_t)m * K);
    for (int i = threadIdx.x; i < P; i += 256) {
        const uint4 v = row[i];
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = word_of(v, j);
            const _Float16 lo = (_Float16)ldexpf(__uint_as_float(w << 16), -e);
            const _Float16 hi = (_Float16)ldexpf(__uint_as_float(w & 0xFFFF0000u), -e);
            o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        out[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (threadIdx.x == 0) xexp[m] = e;
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

}  // namespace

hipError_t launch_x_to_f16(const uint16_t* x_bf16, int M, int K, _Float16* xh, int* xexp,
                           hipStream_t st) {
    hipLaunchKernelGGL(x_to_f16_kernel, dim3(M), dim3(256), 0, st, x_bf16, K, xh, xexp);
    return hipGetLastError();
}

namespace {
hipError_t run(int f, const LogitsArgs& a, hipStream_t st) {
    return a.zp ? run_family_zp(f, a, st) : run_family<false>(f, a, st);
}
}  // namespace

hipError_t launch_mfma(const LogitsArgs& a, hipStream_t st) { return run(kFamMfma, a, st); }

hipError_t launch_mfma_lds(const LogitsArgs& a, hipStream_t st) { return run(kFamMfmaLds, a, st); }

hipError_t launch_mfma_xres(const LogitsArgs& a, hipStream_t st) { return run(kFamXres, a, st); }

bool xres_fits(int64_t K) { return K <= kXresMaxK; }

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
