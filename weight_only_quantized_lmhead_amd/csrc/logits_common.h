// Helpers shared by the logits kernels (gemv_kernels.h, logits_kernels.h):
// exact unpacking of the packed codes into fp16 pairs, the scale and output
// conversions, and the regions of the packed blob.
//
// Codes are unpacked exactly into fp16 in registers with the exponent trick:
// OR-ing a nibble n into the fp16 pattern 0x6400 gives 1024 + n, so one
// AND-OR per pair of codes plus one packed subtract yields q = n - 8 exactly
// (int8: a byte permute into 0x64xx gives 1024 + b, minus 1152).  Products
// with fp16 x are exact in fp32; each group's partial sum is accumulated in
// fp32 and multiplied by the group scale in fp32 (the scale never touches a
// 16-bit product).
//
// Zero-point heads (the asymmetric layout: unsigned codes n and one 8-bit
// zero point z per row and group, w = (n - z) * s) use the same unpacking
// with the fixed offset 8 / 128 replaced by the row's z: the fp16 pattern
// 0xE400 | z is -(1024 + z), so the same single packed add yields n - z
// exactly.
#pragma once

#include "lmh_internal.h"

#include <type_traits>

#include <math.h>

namespace lmh {
namespace {

__device__ __forceinline__ float scale_to_f32(uint16_t b, int sbf16) {
    return sbf16 ? __uint_as_float((uint32_t)b << 16) : (float)__builtin_bit_cast(_Float16, b);
}

// (a & mask) | orv in one v_and_or_b32.  Written out because the compiler
// otherwise splits it into v_and + v_or (gfx9 VOP3 cannot take two literals);
// the mask comes from an SGPR and orv from a VGPR (one constant-bus read).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t orv) {
    uint32_t d;
    asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask), "v"(orv));
    return d;
}

// Offsets that turn the biased fp16 patterns of the unpacking into signed
// codes: lo = -(1024 + z) for low nibbles and int8 bytes (1024 + n -> n - z),
// hi = -(64 + z) for high nibbles ((1024 + 16 n) / 16 -> n - z).  Symmetric
// heads have the fixed z = 8 (int4) / 128 (int8).
struct ZC {
    h2 lo, hi;
};

template <int BITS>
__device__ __forceinline__ ZC zc_sym() {
    constexpr float z = BITS == 4 ? 8.0f : 128.0f;
    return {{(_Float16)(-1024.0f - z), (_Float16)(-1024.0f - z)},
            {(_Float16)(-64.0f - z), (_Float16)(-64.0f - z)}};
}

// Zero point z = byte i of zw (i a compile-time constant after unrolling):
// the fp16 pattern 0xE400 | z is -(1024 + z) exactly (z < 1024), and adding
// 960 gives -(64 + z), also exactly.
__device__ __forceinline__ ZC zc_byte(uint32_t zw, int i) {
    const h2 lo = __builtin_bit_cast(
        h2, __builtin_amdgcn_perm(0xE4E4E4E4u, zw, 0x04000400u + (uint32_t)i * 0x00010001u));
    const h2 k960 = {(_Float16)960.0f, (_Float16)960.0f};
    return {lo, lo + k960};
}

// int4 word (8 codes; even columns in the low nibbles of each half-word) ->
// four fp16 pairs (cols 0,1), (2,3), (4,5), (6,7), exact.  `magic` must hold
// 0x64006400 (fp16 1024.0 in both halves).
__device__ __forceinline__ void unpack_i4(uint32_t w, uint32_t magic, const ZC& zc, h2& p0, h2& p1,
                                          h2& p2, h2& p3) {
    const uint32_t hi = w >> 8;
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    p0 = __builtin_bit_cast(h2, and_or(w, 0x000F000Fu, magic)) + zc.lo;          // 1024+n -> n-z
    p1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(w, 0x00F000F0u, magic)), sixteenth,
                                   zc.hi);                                        // (1024+16n)/16-64-z
    p2 = __builtin_bit_cast(h2, and_or(hi, 0x000F000Fu, magic)) + zc.lo;
    p3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(hi, 0x00F000F0u, magic)), sixteenth,
                                   zc.hi);
}

// int8 word (4 codes, byte i = column i) -> two fp16 pairs, exact.
__device__ __forceinline__ void unpack_i8(uint32_t w, const ZC& zc, h2& p0, h2& p1) {
    p0 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, w, 0x04010400u)) + zc.lo;
    p1 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, w, 0x04030402u)) + zc.lo;
}

__device__ __forceinline__ uint32_t word_of(const uint4& u, int j) {
    return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
}

// Logits storage type: fp32, or the 16-bit pattern of fp16 / bf16.
template <int OUT>
using YT = typename std::conditional<OUT == F32, float, uint16_t>::type;

// fp32 -> the output type, rounded to nearest even once, from the final fp32
// value (bias and row exponent already applied).  The value passes through an
// empty asm first: otherwise the backend may fold the last fp32 add into a
// mixed-precision fma that rounds only once, which differs from rounding the
// fp32 result.
template <int OUT>
__device__ __forceinline__ YT<OUT> to_out(float v) {
    if constexpr (OUT == F32) {
        return v;
    } else {
        asm("" : "+v"(v));
        if constexpr (OUT == F16) {
            return __builtin_bit_cast(uint16_t, (_Float16)v);
        } else {
            uint32_t u = __float_as_uint(v);
            u += 0x7FFFu + ((u >> 16) & 1u);  // nearest even (finite values)
            return (uint16_t)(u >> 16);
        }
    }
}

// Four consecutive logits at p (aligned to four elements).
template <int OUT>
__device__ __forceinline__ void store4(YT<OUT>* p, f4 v) {
    if constexpr (OUT == F32) {
        *(f4*)p = v;
    } else {
        const uint32_t lo = (uint32_t)to_out<OUT>(v[0]) | ((uint32_t)to_out<OUT>(v[1]) << 16);
        const uint32_t hi = (uint32_t)to_out<OUT>(v[2]) | ((uint32_t)to_out<OUT>(v[3]) << 16);
        *(uint2*)p = make_uint2(lo, hi);
    }
}



inline int gps_of(int bits, int64_t G) {
    const int span = span_of(bits);
    return G >= span ? 1 : span / (int)G;
}

// Regions of the blob: codes, then scales, then (zero-point heads) zero points.
template <int BITS>
struct Regions {
    const uint4* wq;
    const uint16_t* sc;
    const uint8_t* zq;
    Regions(const LogitsArgs& a, bool zp) {
        const int64_t vpad = (a.V + 63) / 64 * 64;
        const int64_t wbytes = vpad * a.K * BITS / 8;
        wq = (const uint4*)a.packed;
        sc = (const uint16_t*)(a.packed + wbytes);
        zq = zp ? a.packed + wbytes + vpad * (a.K / a.G) * 2 : nullptr;
    }
};

}  // namespace
}  // namespace lmh
