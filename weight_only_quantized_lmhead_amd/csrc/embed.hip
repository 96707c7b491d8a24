// Embedding gather from the packed blob.
//
// A tied head's quantized table is also the model's input-embedding table
// (vLLM PR #48870, Purpose: the packed embedding that serves the input lookup
// is the one reused as the tied lm_head, and that PR keeps a second,
// gather-format copy for the lookup).  Here the lookup reads the same blob the
// logits kernels read, so one copy serves both:
//
//     out[t, k] = q[id, k] * s[id, k / G],   id = ids[t],
//
// (zero-point heads: (n[id, k] - z[id, k / G]) * s[id, k / G]),
// the product exact in fp32 (at most 8 + 11 significant bits) and rounded once
// to the output type.  An id outside [0, V) yields a row of zeros.
//
// Work mapping: one thread per (token, 16-byte weight slot).  A slot holds 32
// columns of one row (int4: four runs of 8 contiguous columns, one per 32-bit
// word; int8: four runs of 4, 16 columns), so the thread issues one 16-byte
// load, up to four 2-byte scale loads, and four stores of contiguous output
// runs.  Decode-size gathers are latency-bound; prefill-size ones are bound by
// the output writes (2-4 bytes per element against 0.5-1 byte read).
#include "lmh_internal.h"

namespace lmh {
namespace {

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t to_f16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int OUT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    // the products stay opaque here: otherwise the backend folds multiply and
    // fp16 conversion into one mixed fma with a +0 addend, which turns the -0
    // of a negative code times a zero scale into +0
    asm("" : "+v"(a), "+v"(b));
    if constexpr (OUT == F16) return (uint32_t)to_f16_rne(a) | ((uint32_t)to_f16_rne(b) << 16);
    else return (uint32_t)to_bf16_rne(a) | ((uint32_t)to_bf16_rne(b) << 16);
}

// Store n (8 or 4) consecutive values of a row.
template <int OUT, int N>
__device__ __forceinline__ void store_run(char* dst, const float* v) {
    if constexpr (OUT == F32) {
        if constexpr (N == 8) {
            *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
            *(float4*)(dst + 16) = make_float4(v[4], v[5], v[6], v[7]);
        } else {
            *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
        }
    } else {
        if constexpr (N == 8)
            *(uint4*)dst = make_uint4(pack2<OUT>(v[0], v[1]), pack2<OUT>(v[2], v[3]),
                                      pack2<OUT>(v[4], v[5]), pack2<OUT>(v[6], v[7]));
        else
            *(uint2*)dst = make_uint2(pack2<OUT>(v[0], v[1]), pack2<OUT>(v[2], v[3]));
    }
}

__device__ __forceinline__ float scale_f32(uint16_t b, bool sbf16) {
    return sbf16 ? __uint_as_float((uint32_t)b << 16) : (float)__builtin_bit_cast(_Float16, b);
}

template <int BITS, int OUT, bool ZP>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ ids, int64_t nthreads,
                                                    const uint8_t* __restrict__ blob,
                                                    const uint16_t* __restrict__ sblob,
                                                    const uint8_t* __restrict__ zblob, int64_t V,
                                                    int K, int G, int NC, int NG, int sbf16,
                                                    char* __restrict__ out, int64_t ldo_bytes) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= nthreads) return;
    const int spr = NC * 4;  // slots per row
    const int64_t t = gid / spr;
    const int sl = (int)(gid - t * spr);
    const int c = sl >> 2, tt = sl & 3;
    const int id = ids[t];
    const bool valid = id >= 0 && (int64_t)id < V;
    constexpr int span = span_of(BITS);
    constexpr int esz = OUT == F32 ? 4 : 2;
    char* orow = out + t * ldo_bytes;
    // an id outside the table reads as code 0 everywhere: a row of +0
    constexpr uint32_t kZero = ZP ? 0u : (BITS == 4 ? 0x88888888u : 0x80808080u);
    uint4 slot = make_uint4(kZero, kZero, kZero, kZero);
    int64_t b = 0;
    int r = 0;
    if (valid) {
        b = id >> 6;
        r = id & 63;
        slot = *(const uint4*)(blob + ((((b * NC + c) * 4 + tt) * 64 + r) * 16));
    }
    const uint32_t wd[4] = {slot.x, slot.y, slot.z, slot.w};
    // the code offset of a column's group: 8 / 128, or the row's zero point
    // (byte (b*NG + g)*64 + 4*(r%16) + r/16 of the zero-point region)
    auto zero_of = [&](int col) -> int {
        if constexpr (ZP) return valid ? (int)zblob[(b * NG + col / G) * 64 + 4 * (r & 15) + (r >> 4)] : 0;
        else return BITS == 4 ? 8 : 128;
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (BITS == 4) {
            const int col = c * span + 32 * j + 8 * tt;
            const float s = valid ? scale_f32(sblob[(b * NG + col / G) * 64 + r], sbf16) : 0.0f;
            const int z = zero_of(col);
            float v[8];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                // nibble p: even column 2p, nibble p + 4: odd column 2p + 1
                v[2 * p] = (float)((int)((wd[j] >> (4 * p)) & 15u) - z) * s;
                v[2 * p + 1] = (float)((int)((wd[j] >> (4 * p + 16)) & 15u) - z) * s;
            }
            store_run<OUT, 8>(orow + (int64_t)col * esz, v);
        } else {
            const int col = c * span + 32 * (j >> 1) + 8 * tt + 4 * (j & 1);
            const float s = valid ? scale_f32(sblob[(b * NG + col / G) * 64 + r], sbf16) : 0.0f;
            const int z = zero_of(col);
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (float)((int)((wd[j] >> (8 * i)) & 255u) - z) * s;
            store_run<OUT, 4>(orow + (int64_t)col * esz, v);
        }
    }
}

template <int BITS, bool ZP>
void launch_b(int out_dtype, dim3 grid, hipStream_t st, const int32_t* ids, int64_t n,
              const uint8_t* blob, const uint16_t* sblob, const uint8_t* zblob, int64_t V, int K,
              int G, int NC, int NG, int sbf16, char* out, int64_t ldo_bytes) {
    switch (out_dtype) {
    case F32:
        hipLaunchKernelGGL((embed_kernel<BITS, F32, ZP>), grid, dim3(256), 0, st, ids, n, blob,
                           sblob, zblob, V, K, G, NC, NG, sbf16, out, ldo_bytes);
        break;
    case F16:
        hipLaunchKernelGGL((embed_kernel<BITS, F16, ZP>), grid, dim3(256), 0, st, ids, n, blob,
                           sblob, zblob, V, K, G, NC, NG, sbf16, out, ldo_bytes);
        break;
    default:
        hipLaunchKernelGGL((embed_kernel<BITS, BF16, ZP>), grid, dim3(256), 0, st, ids, n, blob,
                           sblob, zblob, V, K, G, NC, NG, sbf16, out, ldo_bytes);
        break;
    }
}

}  // namespace

hipError_t launch_embed(const int32_t* ids, int64_t T, const uint8_t* blob, int64_t V, int64_t K,
                        int bits, int64_t G, int scale_dtype, bool zp, void* out, int out_dtype,
                        int64_t ldo, hipStream_t st) {
    const int NC = (int)(K / span_of(bits));
    const int NG = (int)(K / G);
    const int64_t vpad = (V + 63) / 64 * 64;
    const uint16_t* sblob = (const uint16_t*)(blob + vpad * K * bits / 8);
    const uint8_t* zblob = zp ? blob + vpad * K * bits / 8 + vpad * NG * 2 : nullptr;
    const int64_t n = T * NC * 4;
    const dim3 grid((unsigned)((n + 255) / 256));
    const int64_t ldo_bytes = ldo * (out_dtype == F32 ? 4 : 2);
#define LMH_EMB(B_, Z_)                                                                         \
    launch_b<B_, Z_>(out_dtype, grid, st, ids, n, blob, sblob, zblob, V, (int)K, (int)G, NC, NG, \
                     scale_dtype == BF16, (char*)out, ldo_bytes)
    if (bits == 4) {
        if (zp) LMH_EMB(4, true); else LMH_EMB(4, false);
    } else {
        if (zp) LMH_EMB(8, true); else LMH_EMB(8, false);
    }
#undef LMH_EMB
    return hipGetLastError();
}

}  // namespace lmh
