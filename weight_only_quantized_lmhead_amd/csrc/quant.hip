// Load-time quantizer and packer kernels.
//
// Quantizer: page "radiance_lmhead_int4.py" (docstring "How" paragraph,
// module constants CLIP_RATIOS / QMAX / ZP_BIAS, quantize_int4_rows): per group
// of G columns one 16-bit scale, symmetric codes, the scale rounded to the
// 16-bit type before the codes are chosen, and an optional least-squared-error
// search over the clip ratios 1.0 .. 0.8.  Results are bit-exact with a plain
// CPU implementation: IEEE-rounded fp32 quotients, ties-to-even everywhere,
// and the squared error summed in fp64 in ascending column order with one
// fused multiply-add per element.
//
// Work mapping.  One wavefront owns one 64-row block of the head and one unit
// of columns; lane r owns row 64b + r.  A group of up to 128 columns stays in
// the lane's registers for every pass (amax, each clip ratio, the final
// codes); a longer group is streamed from memory once per pass.  Either way
// the weights arrive through the wave's own LDS region: coalesced loads (each
// covering a few rows) in, one row per lane out.  Two outputs:
//   * codes mode: q int8 [V, K] and s [V, K/G] row-major (lmhead_quantize);
//   * packed mode: the blob itself (lmhead_quantize_pack).  The unit is one
//     superchunk of the packed layout (or one group, when a group is longer),
//     so a lane assembles its row's four 16-byte slots in registers and the 64
//     lanes store each slot as one contiguous 1 KiB run; no int8 copy of the
//     codes ever reaches memory.  A launch may cover any run of whole 64-row
//     blocks, which is what lets a caller quantize a head chunk by chunk.
//
// Zero-point heads (ASYM): unsigned codes n in [0, qr] (qr = 15 / 255) and a
// per-group zero point z, w ~ (n - z) * s, in place of the symmetric module's
// fixed offset 8.  The pages give no quantizer for that form; this one is the
// plain min/max round-to-nearest over the group's range widened to include
// zero (so zero is exactly representable): lo = min(0, min w), hi = max(0,
// max w), s = round16(max(fl32(fl32(hi - lo) * fl32(1 / qr)), floor)),
// z = clamp(rint(fl32(-lo / s)), 0, qr), n = clamp(rint(fl32(w / s)) + z, 0,
// qr); an all-zero group gets s = z = n = 0.  No clip search.
//
// Quotient rounding.  q = rint(fl32(w / s)) is computed without a division
// and without any data-dependent branch: fl32(w / s) == RN32(RN64(w * r))
// with r = RN64(1 / s) (once per group and ratio).  Proof sketch: write the
// scale's odd significand as S < 2^11 (fp16; < 2^8 for bf16) and the weight's
// significand as W < 2^24.  An fp32 rounding midpoint is m = (2M + 1) 2^g with
// 2^24 <= 2M + 1 < 2^25; w / s = m would need W 2^j = S (2M + 1), an odd
// number of at least 2^24, so w / s is never a midpoint, and when nonzero its
// distance to one is at least 2^g / S, i.e. a relative 1 / (S (2M + 1)) >
// 2^-36.  The fp64 product is within 2^-52 (relative) of w / s, so it lies on
// the same side of every fp32 midpoint and rounds to the same fp32 value;
// exactly representable quotients (half-integers included) come back
// unchanged, so ties still go to even.
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

struct QCfg {
    float c[5];     // fl32(ratio / qmax) per clip ratio, rounded on the host from doubles
    float floor_s;  // smallest scale before rounding: 1e-8 (bf16 scales) or 2^-24 (fp16)
    int nratios;    // 1 (round-to-nearest) or 5 (clip search)
    int sbf16;      // scale type: 1 bf16, 0 fp16
};

struct QuantArgs {
    int asym;            // zero-point form (informational; the kernels take ASYM)
    const void* w;       // row `row0` of the head
    int64_t ldw;         // row stride of w in elements
    int64_t row0, rows;  // rows present in w: [row0, row0 + rows)
    int64_t blk0;        // first 64-row block of the launch
    int64_t nunits;      // wavefronts with work: blocks * upb
    int upb;             // units per 64-row block
    int K, G, NG, NC;
    QCfg cf;
    uint8_t* wout;   // packed mode: weight region of the blob
    uint16_t* sout;  //              scale region of the blob
    uint8_t* zout;   //              zero-point region of the blob (ASYM)
    int8_t* q;       // codes mode: q [V, K] (ASYM: the unsigned codes n)
    uint16_t* s;     //             s [V, NG]
    uint8_t* z;      //             z [V, NG] (ASYM)
};

template <int BITS>
struct QRange {
    static constexpr float lo = BITS == 4 ? -8.0f : -128.0f;
    static constexpr float hi = BITS == 4 ? 7.0f : 127.0f;
    static constexpr float qr = BITS == 4 ? 15.0f : 255.0f;  // unsigned code range (ASYM)
};

__device__ __forceinline__ float round_scale(float s32, int sbf16) {
    return sbf16 ? bf16_to_f32(f32_to_bf16_rne(s32)) : f16_to_f32(f32_to_f16_rne(s32));
}

// The candidate scale of one clip ratio: round16(max(fl32(amax * c), floor)).
__device__ __forceinline__ float ratio_scale(float amax, float c, const QCfg& cf) {
#pragma clang fp contract(off)
    float s32 = amax * c;
    s32 = s32 < cf.floor_s ? cf.floor_s : s32;
    return round_scale(s32, cf.sbf16);
}

// q = clamp(rint(fl32(w / s)), lo, hi) for N weights, r = RN64(1 / s) (see
// the header).
template <int BITS, int N>
__device__ __forceinline__ void codes(const float* w, double r, float* q) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float x = (float)((double)w[i] * r);
        q[i] = __builtin_amdgcn_fmed3f(rintf(x), QRange<BITS>::lo, QRange<BITS>::hi);
    }
}

// Zero-point codes: n = clamp(rint(fl32(w / s)) + z, 0, qr), the sum of two
// small integers exact.
template <int BITS, int N>
__device__ __forceinline__ void codes_asym(const float* w, double r, float zf, float* n) {
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float x = (float)((double)w[i] * r);
        n[i] = __builtin_amdgcn_fmed3f(rintf(x) + zf, 0.0f, QRange<BITS>::qr);
    }
}

// err += sum_i (q_i * s - w_i)^2, i ascending, one fp64 fma each.  d = q*s - w
// is exact in fp32: q*s has at most 8 + 11 significant bits, and for q != 0 it
// lies within a factor of two of w (|w/s - q| <= 1/2 + 2^-16, or the clamp,
// which leaves w/s within 1.25 q), so the difference is representable
// (Sterbenz) and the single rounding of fmaf returns it unchanged.
template <int N>
__device__ __forceinline__ double errN(const float* w, const float* q, float sv, double err) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const double d = (double)__builtin_fmaf(q[i], sv, -w[i]);
        err = __builtin_fma(d, d, err);
    }
    return err;
}

// Staging of a wave's 64 rows through LDS, so that its global loads are
// coalesced: a piece of up to 256 bytes of every row is read with 16-byte
// loads whose consecutive lanes take consecutive 16 bytes of one row (a load
// instruction covers 64 / P rows, P = piece bytes / 16), written to the
// wave's own LDS region, rows padded by 16 bytes, and read back one row per
// lane.  The padding makes the row stride (P + 1 words of 16 bytes) odd, so
// the 64 lanes' reads of word p of their rows fall in distinct banks.
constexpr int kStagePiece = 256;  // most bytes of a row staged at once

// Stage 16 P bytes of each of the wave's 64 rows (block b), from column colp
// on, into st with a row stride of P + 1 words; rows past the launch's input
// as zeros.
template <int WDT, int P>
__device__ __forceinline__ void stage_piece(const QuantArgs& a, int64_t b, int colp, uint4* st) {
    constexpr int esz = WDT == F32 ? 4 : 2;
    constexpr int RPI = 64 / P;  // rows per load instruction
    const int lane = threadIdx.x & 63;
    const int rq = lane / P, pw = lane % P;  // this lane's row (of each RPI) and word
    const int64_t lr0 = b * 64 - a.row0 + rq;
    const char* wb = (const char*)a.w + (size_t)colp * esz + pw * 16;
    uint4 u[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int64_t lr = lr0 + i * RPI;
        u[i] = lr < a.rows ? *(const uint4*)(wb + lr * a.ldw * esz) : make_uint4(0, 0, 0, 0);
    }
    // every lane's reads of the previous piece are done before its words are
    // overwritten (LDS operations of a wave run in order); the empty asm
    // statements keep the compiler from moving accesses across
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < P; ++i) st[(i * RPI + rq) * (P + 1) + pw] = u[i];
    asm volatile("" ::: "memory");
}

// A group of NE <= 128 weights of one row held in registers: fp32 as is,
// 16-bit weights as their raw bit patterns two to a register (widened on use).
template <int WDT, int NE>
struct Held {
    static constexpr int kWords = WDT == F32 ? NE : NE / 2;
    static constexpr int kRowBytes = kWords * 4;
    static constexpr int kPiece = kRowBytes < kStagePiece ? kRowBytes : kStagePiece;
    static constexpr int P = kPiece / 16;  // 16-byte words per row and piece
    static constexpr int kStageWords = 64 * (P + 1);  // a wave's LDS region, 16-byte words
    uint32_t v[kWords];
    // Columns [col0, col0 + NE) of the wave's 64 rows (block b; rows past the
    // launch's input read as zeros), lane r receiving row 64b + r.  `st` is
    // the wave's LDS region (kStageWords words).
    __device__ __forceinline__ void load(const QuantArgs& a, int64_t b, int col0, uint4* st) {
        constexpr int esz = WDT == F32 ? 4 : 2;
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int pc = 0; pc < kRowBytes / kPiece; ++pc) {
            stage_piece<WDT, P>(a, b, col0 + pc * (kPiece / esz), st);
#pragma unroll
            for (int w = 0; w < P; ++w) {
                const uint4 x = st[lane * (P + 1) + w];
                const int o = pc * (kPiece / 4) + 4 * w;
                v[o] = x.x, v[o + 1] = x.y, v[o + 2] = x.z, v[o + 3] = x.w;
            }
        }
    }
    // N weights starting at element k (a multiple of N), as fp32
    template <int N>
    __device__ __forceinline__ void get(int k, float* o) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if constexpr (WDT == F32) {
                o[i] = __uint_as_float(v[k + i]);
            } else {
                const uint32_t x = v[(k + i) / 2];
                if constexpr (WDT == BF16)
                    o[i] = __uint_as_float((i & 1) ? (x & 0xFFFF0000u) : (x << 16));
                else
                    o[i] = f16_to_f32((uint16_t)((i & 1) ? (x >> 16) : x));
            }
        }
    }
};

template <int WDT, int NE>
struct HeldGet {
    const Held<WDT, NE>& h;
    template <int N>
    __device__ __forceinline__ void operator()(int k, float* o) const {
        h.template get<N>(k, o);
    }
};

// A longer group's columns [col0 + k, col0 + k + N) of each lane's row for a
// pass that walks k upwards from 0 in steps of N <= 32: every 64 columns
// (which divide the group) the wave stages the next 64 columns of its 64
// rows through its LDS region as above, so the pass's loads are coalesced.
template <int WDT>
struct StageGet {
    static constexpr int esz = WDT == F32 ? 4 : 2;
    static constexpr int P = 64 * esz / 16;  // 16-byte words per row of a 64-column piece
    static constexpr int kStageWords = 64 * (P + 1);
    const QuantArgs& a;
    int64_t b;
    int col0;
    uint4* st;
    template <int N>
    __device__ __forceinline__ void operator()(int k, float* o) const {
        if (k % 64 == 0) stage_piece<WDT, P>(a, b, col0 + k, st);
        const uint4* row = st + (threadIdx.x & 63) * (P + 1) + (k % 64) * esz / 16;
#pragma unroll
        for (int j = 0; j < N * esz / 16; ++j) {
            const uint4 x = row[j];
            const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (WDT == F32) {
                    o[4 * j + e] = __uint_as_float(wd[e]);
                } else if constexpr (WDT == BF16) {
                    o[8 * j + 2 * e] = __uint_as_float(wd[e] << 16);
                    o[8 * j + 2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
                } else {
                    o[8 * j + 2 * e] = f16_to_f32((uint16_t)wd[e]);
                    o[8 * j + 2 * e + 1] = f16_to_f32((uint16_t)(wd[e] >> 16));
                }
            }
        }
    }
};

constexpr int kRatios = 5;  // the clip search's ratios: 1.0, 0.95, 0.9, 0.85, 0.8
constexpr int kSearchN = 16;  // columns per step of the search

// Chosen scale of a group; zero = the group is all zeros (its stored scale is
// then 0 and every code 0).  `get(k, w)` yields the group's columns
// [k, k + N) as fp32 for any multiple k of N.  The clip search walks the group
// once with the five candidate scales side by side: each ratio's error is
// still summed in ascending column order, but the five independent fp64
// chains interleave instead of running one after another.
template <int BITS, bool UNROLL, class Get>
__device__ __forceinline__ float pick_scale(const Get& get, int G, const QCfg& cf, bool& zero) {
    constexpr int kU = UNROLL ? 16 : 1;  // held groups: fully unrolled; streamed: rolled
    float amax = 0.0f;
#pragma unroll kU
    for (int k = 0; k < G; k += 32) {
        float w[32];
        get.template operator()<32>(k, w);
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(w[i]));
    }
    zero = amax == 0.0f;
    if (cf.nratios == 1) return ratio_scale(amax, cf.c[0], cf);
    float sv[kRatios];
    double rr[kRatios], err[kRatios];
#pragma unroll
    for (int i = 0; i < kRatios; ++i) {
        sv[i] = ratio_scale(amax, cf.c[i], cf);
        rr[i] = 1.0 / (double)sv[i];
        err[i] = 0.0;
    }
#pragma unroll kU
    for (int k = 0; k < G; k += kSearchN) {
        float w[kSearchN];
        get.template operator()<kSearchN>(k, w);
#pragma unroll
        for (int i = 0; i < kRatios; ++i) {
            float q[kSearchN];
            codes<BITS, kSearchN>(w, rr[i], q);
            err[i] = errN<kSearchN>(w, q, sv[i], err[i]);
        }
    }
    // the first ratio whose error is strictly below every earlier one
    float best = sv[0];
    double best_err = err[0];
#pragma unroll
    for (int i = 1; i < kRatios; ++i) {
        if (err[i] < best_err) {
            best_err = err[i];
            best = sv[i];
        }
    }
    return best;
}

// Scale and zero point of a zero-point group (the header's ASYM rules):
// returns s, sets zf = z and zero = the group is all zeros.
template <int BITS, bool UNROLL, class Get>
__device__ __forceinline__ float pick_asym(const Get& get, int G, const QCfg& cf, bool& zero,
                                           float& zf) {
#pragma clang fp contract(off)
    constexpr int kU = UNROLL ? 16 : 1;
    float lo = 0.0f, hi = 0.0f;
#pragma unroll kU
    for (int k = 0; k < G; k += 32) {
        float w[32];
        get.template operator()<32>(k, w);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            lo = fminf(lo, w[i]);
            hi = fmaxf(hi, w[i]);
        }
    }
    zero = hi == lo;
    const float sv = ratio_scale(hi - lo, cf.c[0], cf);
    const double rr = 1.0 / (double)sv;
    zf = __builtin_amdgcn_fmed3f(rintf((float)((double)(-lo) * rr)), 0.0f, QRange<BITS>::qr);
    return sv;
}

__device__ __forceinline__ uint16_t scale_bits(float sv, bool zero, int sbf16) {
    if (zero) return 0;
    return sbf16 ? f32_to_bf16_rne(sv) : f32_to_f16_rne(sv);
}

// Packed-layout words of one 32-column chunk (codes q[0..31], already
// clamped) into slot words sw[t][j]: int4 chunk jj fills word j = jj of the
// four slots (nibble q + 8; even columns in the low half-word, odd columns in
// the high one); int8 chunk jj fills words 2jj and 2jj + 1 (byte q + 128).
// ASYM codes are stored as they are (nibble n, byte n).
template <int BITS, bool ASYM>
__device__ __forceinline__ void put_chunk(const float* q, int jj, uint32_t (&sw)[4][4]) {
    constexpr float off = ASYM ? 0.0f : (BITS == 4 ? 8.0f : 128.0f);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float* q8 = q + 8 * t;
        if constexpr (BITS == 4) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                lo |= (uint32_t)(int)(q8[2 * p] + off) << (4 * p);
                hi |= (uint32_t)(int)(q8[2 * p + 1] + off) << (4 * p);
            }
            sw[t][jj] = lo | (hi << 16);
        } else {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                uint32_t wd = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) wd |= (uint32_t)(int)(q8[4 * e + i] + off) << (8 * i);
                sw[t][2 * jj + e] = wd;
            }
        }
    }
}

// The four slots of superchunk c of a lane's row: 64 lanes store 1 KiB runs.
__device__ __forceinline__ void store_slots(uint8_t* wout, int64_t b, int NC, int c, int r,
                                            const uint32_t (&sw)[4][4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
        *(uint4*)(wout + ((((b * NC + c) * 4 + t) * 64 + r) * 16)) =
            make_uint4(sw[t][0], sw[t][1], sw[t][2], sw[t][3]);
}

// 32 codes of a row in codes mode: int8 two's complement, row-major.
__device__ __forceinline__ void store_codes32(int8_t* dst, const float* q) {
    uint32_t wd[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        uint32_t x = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) x |= ((uint32_t)(int)q[4 * m + i] & 0xFFu) << (8 * i);
        wd[m] = x;
    }
    *(uint4*)dst = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    *(uint4*)(dst + 16) = make_uint4(wd[4], wd[5], wd[6], wd[7]);
}

// Whether head row v lies in the launch's input (the padding rows of the last
// block do not: they read as zeros and store nothing of their own).
__device__ __forceinline__ bool row_present(const QuantArgs& a, int64_t v) {
    return v - a.row0 < a.rows;
}

// Groups of GT <= 128 columns, held in registers.  Unit: one superchunk (or
// one group when GT exceeds the span) in packed mode, one group in codes mode.
// Byte offset of the zero point of row r (of a 64-row block) in group g of
// block b, within the blob's zero-point region.
__device__ __forceinline__ int64_t zp_offset(int64_t b, int NG, int g, int r) {
    return (b * NG + g) * 64 + 4 * (r & 15) + (r >> 4);
}

// The unit (one wave's work) of this thread.  The launch's workgroups are
// dealt round-robin to the 8 XCDs, so the work is numbered for XCD x to take
// the contiguous run of workgroups [x per, (x + 1) per), per = grid / 8 (the
// grid is a multiple of 8; workgroups past the work find unit >= nunits).  In
// codes mode a workgroup writes 4 groups' scales of each of its 64 rows, only
// part of the row's scale line; its neighbour writes the next part.  On one
// XCD the parts meet in that XCD's L2 and go to HBM as whole lines; dealt to
// two XCDs they would leave two L2s as two partial lines.
__device__ __forceinline__ int64_t quant_unit() {
    const int64_t per = gridDim.x >> 3;
    const int64_t wg = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    return wg * 4 + (threadIdx.x >> 6);
}

template <int WDT, int BITS, int GT, bool PACKED, bool ASYM>
__global__ __launch_bounds__(256, 2) void
quant_held_kernel(
    const QuantArgs a) {
#pragma clang fp contract(off)
    const int64_t unit = quant_unit();
    if (unit >= a.nunits) return;
    const int r = threadIdx.x & 63;
    const int64_t b = a.blk0 + unit / a.upb;
    const int u = (int)(unit % a.upb);
    const int64_t v = b * 64 + r;
    const bool present = row_present(a, v);
    constexpr int span = span_of(BITS);
    constexpr int UC = PACKED ? (GT > span ? GT : span) : GT;  // unit columns
    constexpr int CPS = span / 32;                             // chunks per superchunk
    const int col_u = u * UC;
    __shared__ uint4 stage[4][Held<WDT, GT>::kStageWords];  // one region per wave
    uint4* st = stage[threadIdx.x >> 6];
    uint32_t sw[4][4];
#pragma unroll
    for (int gi = 0; gi < UC / GT; ++gi) {
        const int col0 = col_u + gi * GT;
        Held<WDT, GT> h;
        h.load(a, b, col0, st);
        bool zero;
        float zf = 0.0f;
        const float sv = ASYM ? pick_asym<BITS, true>(HeldGet<WDT, GT>{h}, GT, a.cf, zero, zf)
                              : pick_scale<BITS, true>(HeldGet<WDT, GT>{h}, GT, a.cf, zero);
        const uint16_t sb = scale_bits(sv, zero, a.cf.sbf16);
        const double rr = 1.0 / (double)sv;
        if constexpr (PACKED) {
            a.sout[(b * a.NG + col0 / GT) * 64 + r] = sb;
            if constexpr (ASYM) a.zout[zp_offset(b, a.NG, col0 / GT, r)] = (uint8_t)(int)zf;
#pragma unroll
            for (int ch = 0; ch < GT / 32; ++ch) {
                float w[32], q[32];
                h.template get<32>(32 * ch, w);
                if constexpr (ASYM) codes_asym<BITS, 32>(w, rr, zf, q);
                else codes<BITS, 32>(w, rr, q);
                const int cu = gi * (GT / 32) + ch;  // chunk index within the unit
                put_chunk<BITS, ASYM>(q, cu % CPS, sw);
                if (cu % CPS == CPS - 1) store_slots(a.wout, b, a.NC, (col_u + 32 * cu) / span, r, sw);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if (present) {
            a.s[v * a.NG + col0 / GT] = sb;
            if constexpr (ASYM) a.z[v * a.NG + col0 / GT] = (uint8_t)(int)zf;
#pragma unroll
            for (int ch = 0; ch < GT / 32; ++ch) {
                float w[32], q[32];
                h.template get<32>(32 * ch, w);
                if constexpr (ASYM) codes_asym<BITS, 32>(w, rr, zf, q);
                else codes<BITS, 32>(w, rr, q);
                store_codes32(a.q + v * a.K + col0 + 32 * ch, q);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// Longer groups, streamed once per pass.  Unit: one group.
template <int WDT, int BITS, bool PACKED, bool ASYM>
__global__ __launch_bounds__(256, 2) void quant_stream_kernel(const QuantArgs a) {
#pragma clang fp contract(off)
    const int64_t unit = quant_unit();
    if (unit >= a.nunits) return;
    const int r = threadIdx.x & 63;
    const int64_t b = a.blk0 + unit / a.upb;
    const int g = (int)(unit % a.upb);
    const int64_t v = b * 64 + r;
    const bool present = row_present(a, v);
    const int col0 = g * a.G;
    __shared__ uint4 stage[4][StageGet<WDT>::kStageWords];  // one region per wave
    const StageGet<WDT> get{a, b, col0, stage[threadIdx.x >> 6]};
    bool zero;
    float zf = 0.0f;
    const float sv = ASYM ? pick_asym<BITS, false>(get, a.G, a.cf, zero, zf)
                          : pick_scale<BITS, false>(get, a.G, a.cf, zero);
    const uint16_t sb = scale_bits(sv, zero, a.cf.sbf16);
    const double rr = 1.0 / (double)sv;
    if constexpr (PACKED) {
        constexpr int span = span_of(BITS);
        a.sout[(b * a.NG + g) * 64 + r] = sb;
        if constexpr (ASYM) a.zout[zp_offset(b, a.NG, g, r)] = (uint8_t)(int)zf;
#pragma unroll 1
        for (int c = col0 / span; c < (col0 + a.G) / span; ++c) {
            uint32_t sw[4][4];
#pragma unroll
            for (int ch = 0; ch < span / 32; ++ch) {
                float w[32], q[32];
                get.template operator()<32>(c * span + 32 * ch - col0, w);
                if constexpr (ASYM) codes_asym<BITS, 32>(w, rr, zf, q);
                else codes<BITS, 32>(w, rr, q);
                put_chunk<BITS, ASYM>(q, ch, sw);
            }
            store_slots(a.wout, b, a.NC, c, r, sw);
        }
    } else {
        // every lane takes part in the staging; rows past the head store nothing
        if (present) {
            a.s[v * a.NG + g] = sb;
            if constexpr (ASYM) a.z[v * a.NG + g] = (uint8_t)(int)zf;
        }
#pragma unroll 1
        for (int col = col0; col < col0 + a.G; col += 32) {
            float w[32], q[32];
            get.template operator()<32>(col - col0, w);
            if constexpr (ASYM) codes_asym<BITS, 32>(w, rr, zf, q);
            else codes<BITS, 32>(w, rr, q);
            if (present) store_codes32(a.q + v * a.K + col, q);
        }
    }
}

template <int WDT, int BITS, bool PACKED, bool ASYM>
void launch_q3(const QuantArgs& a, dim3 grid, hipStream_t st) {
    switch (a.G) {
    case 32:
        hipLaunchKernelGGL((quant_held_kernel<WDT, BITS, 32, PACKED, ASYM>), grid, dim3(256), 0, st, a);
        break;
    case 64:
        hipLaunchKernelGGL((quant_held_kernel<WDT, BITS, 64, PACKED, ASYM>), grid, dim3(256), 0, st, a);
        break;
    case 128:
        hipLaunchKernelGGL((quant_held_kernel<WDT, BITS, 128, PACKED, ASYM>), grid, dim3(256), 0, st,
                           a);
        break;
    default:
        hipLaunchKernelGGL((quant_stream_kernel<WDT, BITS, PACKED, ASYM>), grid, dim3(256), 0, st, a);
        break;
    }
}

template <bool PACKED>
hipError_t launch_q(const QuantArgs& a, int w_dtype, int bits, hipStream_t st) {
    if (a.nunits <= 0) return hipSuccess;
    const dim3 grid((unsigned)(((a.nunits + 3) / 4 + 7) / 8 * 8));  // a multiple of 8: quant_unit
#define LMH_Q_CASE(WDT)                                                                 \
    if (a.asym) {                                                                       \
        if (bits == 4) launch_q3<WDT, 4, PACKED, true>(a, grid, st);                    \
        else launch_q3<WDT, 8, PACKED, true>(a, grid, st);                              \
    } else {                                                                            \
        if (bits == 4) launch_q3<WDT, 4, PACKED, false>(a, grid, st);                   \
        else launch_q3<WDT, 8, PACKED, false>(a, grid, st);                             \
    }
    switch (w_dtype) {
    case F32: LMH_Q_CASE(F32) break;
    case F16: LMH_Q_CASE(F16) break;
    default: LMH_Q_CASE(BF16) break;
    }
#undef LMH_Q_CASE
    return hipGetLastError();
}

QCfg make_cfg(int bits, int scale_dtype, int nratios, bool asym) {
    static const double kRatios[5] = {1.0, 0.95, 0.9, 0.85, 0.8};
    // symmetric: c_i = fl32(ratio_i / qmax); zero-point: c_0 = fl32(1 / qr)
    const int qmax = asym ? (bits == 4 ? 15 : 255) : (bits == 4 ? 7 : 127);
    QCfg cf;
    for (int i = 0; i < 5; ++i) cf.c[i] = (float)(kRatios[i] / (double)qmax);
    cf.sbf16 = scale_dtype == BF16;
    cf.floor_s = cf.sbf16 ? 1e-8f : 5.9604644775390625e-8f;  // 2^-24
    cf.nratios = nratios;
    return cf;
}

// One thread per 16-byte weight slot of the blob, one workgroup per (64-row
// block, superchunk).  ZP: the codes are the unsigned n (stored as they are;
// padding rows 0), else the signed q (stored biased by 8 / 128; padding rows
// q = 0).  The superchunk's codes (64 rows x 128 or 64 bytes) are first
// staged in LDS with coalesced 16-byte loads (consecutive threads take
// consecutive pieces of one row; rows padded by 8 bytes), then each thread
// builds its slot from its row there.
template <int BITS, bool ZP>
__global__ __launch_bounds__(256) void pack_weights_kernel(const int8_t* __restrict__ q, int64_t V,
                                                           int64_t K, int64_t nslots, int NC,
                                                           uint4* __restrict__ out) {
    constexpr int RB = BITS == 4 ? 128 : 64;  // code bytes of a row in one superchunk
    constexpr int RS = RB + 8;                // LDS row stride
    constexpr int PPR = RB / 16;              // 16-byte pieces per row
    __shared__ __attribute__((aligned(16))) uint8_t cs[64 * RS];
    const int64_t bc = blockIdx.x;  // b * NC + c
    if (bc * 256 >= nslots) return;
    const int c = (int)(bc % NC);
    const int64_t b = bc / NC;
    for (int e = threadIdx.x; e < 64 * PPR; e += 256) {
        const int rr = e / PPR, pc = e % PPR;
        const int64_t vr = b * 64 + rr;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (vr < V) u = *(const uint4*)(q + vr * K + (int64_t)c * RB + 16 * pc);
        uint2* d = (uint2*)(cs + rr * RS + 16 * pc);
        d[0] = make_uint2(u.x, u.y);
        d[1] = make_uint2(u.z, u.w);
    }
    __syncthreads();
    const int r = threadIdx.x & 63;
    const int t = threadIdx.x >> 6;
    const int64_t v = b * 64 + r;
    const uint8_t* row = cs + r * RS;
    uint32_t word[4];
    if (v >= V) {
        const uint32_t pad = ZP ? 0u : (BITS == 4 ? 0x88888888u : 0x80808080u);
        for (int j = 0; j < 4; ++j) word[j] = pad;
    } else if constexpr (BITS == 4) {
        for (int j = 0; j < 4; ++j) {
            const uint2 w8 = *(const uint2*)(row + 32 * j + 8 * t);
            uint32_t wd = 0;
            for (int i8 = 0; i8 < 8; ++i8) {
                const int code = (int8_t)((i8 < 4 ? w8.x >> (8 * i8) : w8.y >> (8 * (i8 - 4))) & 0xFFu);
                // column i8 goes to nibble position p: even columns 0,2,4,6 -> p 0..3,
                // odd columns 1,3,5,7 -> p 4..7
                const int p = (i8 & 1) ? 4 + (i8 >> 1) : (i8 >> 1);
                wd |= (uint32_t)((code + (ZP ? 0 : 8)) & 0xF) << (4 * p);
            }
            word[j] = wd;
        }
    } else {
        for (int j = 0; j < 4; ++j) {
            const uint32_t w4 = *(const uint32_t*)(row + 32 * (j >> 1) + 8 * t + 4 * (j & 1));
            uint32_t wd = 0;
            for (int i4 = 0; i4 < 4; ++i4) {
                const int code = (int8_t)((w4 >> (8 * i4)) & 0xFFu);
                wd |= (uint32_t)(uint8_t)(code + (ZP ? 0 : 128)) << (8 * i4);
            }
            word[j] = wd;
        }
    }
    out[bc * 256 + threadIdx.x] = make_uint4(word[0], word[1], word[2], word[3]);
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

// One thread per byte of the zero-point region: byte e holds, for block b and
// group g ((b*NG + g) = e / 64), row r = (e%64)/4 + 16 ((e%64) % 4).
__global__ __launch_bounds__(256) void pack_zeros_kernel(const uint8_t* __restrict__ z, int64_t V,
                                                         int NG, int64_t n,
                                                         uint8_t* __restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n) return;
    const int pos = (int)(e & 63);
    const int r = (pos >> 2) + 16 * (pos & 3);
    const int64_t bg = e >> 6;
    const int g = (int)(bg % NG);
    const int64_t b = bg / NG;
    const int64_t v = b * 64 + r;
    out[e] = v < V ? z[v * NG + g] : (uint8_t)0;
}

inline unsigned grid_for(int64_t n, int block) { return (unsigned)((n + block - 1) / block); }

}  // namespace

hipError_t launch_quantize(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t G,
                           int scale_dtype, int nratios, int8_t* q, uint16_t* s, uint8_t* z,
                           hipStream_t st) {
    QuantArgs a{};
    a.asym = z != nullptr;
    a.z = z;
    a.w = w;
    a.ldw = K;
    a.row0 = 0;
    a.rows = V;
    a.blk0 = 0;
    a.K = (int)K;
    a.G = (int)G;
    a.NG = (int)(K / G);
    a.NC = 0;
    a.upb = a.NG;  // codes mode: one unit per group
    a.nunits = (V + 63) / 64 * a.upb;
    a.cf = make_cfg(bits, scale_dtype, nratios, a.asym);
    a.q = q;
    a.s = s;
    return launch_q<false>(a, w_dtype, bits, st);
}

hipError_t launch_quantize_pack(const void* w, int w_dtype, int64_t ldw, int64_t V, int64_t K,
                                int bits, int64_t G, int scale_dtype, int nratios, bool asym,
                                int64_t row0, int64_t rows, uint8_t* blob, hipStream_t st) {
    const int span = span_of(bits);
    const int64_t vpad = (V + 63) / 64 * 64;
    QuantArgs a{};
    a.asym = asym;
    a.w = w;
    a.ldw = ldw;
    a.row0 = row0;
    a.rows = rows;
    a.blk0 = row0 / 64;
    a.K = (int)K;
    a.G = (int)G;
    a.NG = (int)(K / G);
    a.NC = (int)(K / span);
    // unit: a superchunk, or a whole group when the group is longer
    a.upb = (int)(K / (G > span ? G : span));
    a.nunits = (rows + 63) / 64 * a.upb;
    a.cf = make_cfg(bits, scale_dtype, nratios, asym);
    a.wout = blob;
    a.sout = (uint16_t*)(blob + vpad * K * bits / 8);
    a.zout = asym ? blob + vpad * K * bits / 8 + vpad * a.NG * 2 : nullptr;
    return launch_q<true>(a, w_dtype, bits, st);
}

hipError_t launch_pack(const int8_t* q, const uint16_t* s, const uint8_t* z, int64_t V, int64_t K,
                       int bits, int64_t G, uint8_t* out, hipStream_t st) {
    const int64_t NB = (V + 63) / 64;
    const int NC = (int)(K / span_of(bits));
    const int NG = (int)(K / G);
    const int64_t nslots = NB * NC * 256;
#define LMH_PACKW(B_, Z_)                                                                        \
    hipLaunchKernelGGL((pack_weights_kernel<B_, Z_>), dim3(grid_for(nslots, 256)), dim3(256), 0, st, \
                       q, V, K, nslots, NC, (uint4*)out)
    if (bits == 4) {
        if (z) LMH_PACKW(4, true); else LMH_PACKW(4, false);
    } else {
        if (z) LMH_PACKW(8, true); else LMH_PACKW(8, false);
    }
#undef LMH_PACKW
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nsc = NB * NG * 64;
    uint16_t* sout = (uint16_t*)(out + NB * 64 * K * bits / 8);
    hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(nsc, 256)), dim3(256), 0, st, s, V, NG, nsc,
                       sout);
    if (z) {
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(pack_zeros_kernel, dim3(grid_for(nsc, 256)), dim3(256), 0, st, z, V, NG,
                           nsc, out + NB * 64 * K * bits / 8 + nsc * 2);
    }
    return hipGetLastError();
}

}  // namespace lmh
