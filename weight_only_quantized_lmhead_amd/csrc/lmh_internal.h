// Internal declarations shared by the HIP translation units of liblmhead.so.
// Not part of the public ABI (that is include/lmhead.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lmh {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

enum Dtype { F32 = 0, F16 = 1, BF16 = 2 };

typedef unsigned long long u64;

// Top-K order codes: unsigned order of the code = value descending, then index
// ascending (-0 and +0 tie; NaN ranks below every number).  High word: the
// value's bits mapped to an order-preserving integer; low word: 0x7FFFFFFF -
// index.  Code 0 is never a real entry's code (it marks "no list").
__device__ __forceinline__ u64 topk_code(float v, int idx) {
    const float f = v == 0.0f ? 0.0f : v;  // -0 -> +0
    const int b = __float_as_int(f);
    const int key = (f != f) ? (int)0x80000000 : (b >= 0 ? b : b ^ 0x7FFFFFFF);
    return ((u64)((uint32_t)key ^ 0x80000000u) << 32) | (uint32_t)(0x7FFFFFFF - idx);
}

__device__ __forceinline__ int topk_code_idx(u64 c) { return 0x7FFFFFFF - (int)(uint32_t)c; }

__device__ __forceinline__ float topk_code_val(u64 c) {
    const int key = (int)((uint32_t)(c >> 32) ^ 0x80000000u);
    return __int_as_float(key >= 0 ? key : key ^ 0x7FFFFFFF);
}

// Columns covered by one 4-slot superchunk of the packed layout.
constexpr int span_of(int bits) { return bits == 4 ? 128 : 64; }

// Launch helpers (defined in the .hip files).  All return hipError_t of the
// launch; arguments are already validated by the API layer.
// Codes mode; z non-null selects the zero-point form (q then holds the
// unsigned codes n and z [V, K/G] the zero points).
hipError_t launch_quantize(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t G,
                           int scale_dtype, int nratios, int8_t* q, uint16_t* s, uint8_t* z,
                           hipStream_t st);
// Fused quantize + pack of rows [row0, row0 + rows) (w points at row row0,
// row stride ldw elements) straight into the blob of a V-row head.
hipError_t launch_quantize_pack(const void* w, int w_dtype, int64_t ldw, int64_t V, int64_t K,
                                int bits, int64_t G, int scale_dtype, int nratios, bool asym,
                                int64_t row0, int64_t rows, uint8_t* blob, hipStream_t st);
// Embedding rows of ids[0..T) from the blob into out (row stride ldo elements).
hipError_t launch_embed(const int32_t* ids, int64_t T, const uint8_t* blob, int64_t V, int64_t K,
                        int bits, int64_t G, int scale_dtype, bool zp, void* out, int out_dtype,
                        int64_t ldo, hipStream_t st);
// z non-null: the zero-point layout (q holds the unsigned codes n).
hipError_t launch_pack(const int8_t* q, const uint16_t* s, const uint8_t* z, int64_t V, int64_t K,
                       int bits, int64_t G, uint8_t* out, hipStream_t st);

struct LogitsArgs {
    const void* x;         // [M, K] row-major: fp16, or bf16 when x_bf16 (GEMV only)
    int x_bf16;            // the GEMV converts bf16 rows itself (other kernels take fp16)
    const int* xexp;       // [M] power-of-two row exponents of converted bf16 rows, or nullptr
    const uint8_t* packed; // blob
    const float* bias;     // [V] or nullptr
    void* y;               // [M, ldy] in y_dtype (F32, F16 or BF16)
    int y_dtype;
    int64_t ldy;
    int64_t V, K, G;
    int M, bits, scale_bf16;
    int zp;                // zero-point head: a zero-point region follows the scales
    u64* lists;            // GEMV top-K epilogue (M = 1, fp32 y): per-block sorted lists, or nullptr
    int list_T;            //   entries per list
};

hipError_t launch_x_to_f16(const uint16_t* x_bf16, int M, int K, _Float16* xh, int* xexp,
                           hipStream_t st);
// Lane-per-row GEMV (gemv.hip; zero-point heads in gemv_zp.hip).
hipError_t launch_gemv(const LogitsArgs& a, hipStream_t st);
hipError_t launch_gemv_zp(const LogitsArgs& a, hipStream_t st);
hipError_t launch_mfma(const LogitsArgs& a, hipStream_t st);
// Activation-resident MFMA kernel for large M; needs K <= xres max (xres_fits).
bool xres_fits(int64_t K);
hipError_t launch_mfma_xres(const LogitsArgs& a, hipStream_t st);
hipError_t launch_mfma_lds(const LogitsArgs& a, hipStream_t st);
// Split-K MFMA kernel for M <= 16 (splitk.hip; zero-point heads in splitk_zp.hip).
constexpr int kSplitkMaxM = 16;
hipError_t launch_mfma_splitk(const LogitsArgs& a, hipStream_t st);
hipError_t launch_mfma_splitk_zp(const LogitsArgs& a, hipStream_t st);
// Logits kernel families (gemv, register MFMA, LDS-staged MFMA, activation
// resident) and the zero-point instantiations of the MFMA ones (logits_zp.hip).
enum { kFamGemv = 0, kFamMfma = 1, kFamMfmaLds = 2, kFamXres = 3 };
hipError_t run_family_zp(int family, const LogitsArgs& a, hipStream_t st);
hipError_t launch_dense(const void* x, int dtype, int M, const void* w, int64_t V, int64_t K,
                        float* y, int64_t ldy, hipStream_t st);
hipError_t launch_topk_rescore(const void* x, int x_dtype, int M, const void* w, int w_dtype,
                               int64_t V, int64_t K, float* y, int64_t ldy, int topk,
                               int32_t* idx, float* val, int32_t* top1, void* ws,
                               hipStream_t st);
size_t topk_ws_bytes(int64_t M, int64_t V, int topk);
// Fused top-K (GEMV epilogue lists + merge): whether it serves (V, topk), the
// bytes of its lists, and the merge + rescoring launch.
bool topk_fused_ok(int64_t V, int topk);
size_t topk_fused_lists_bytes(int64_t M, int64_t V, int topk);
hipError_t launch_topk_merge_rescore(const u64* lists, const void* x, int x_dtype, int M,
                                     const void* w, int w_dtype, int64_t V, int64_t K, float* y,
                                     int64_t ldy, int topk, int T, int32_t* idx, float* val,
                                     int32_t* top1, hipStream_t st);
int64_t topk_max_v();  // largest row length lmhead_topk_rescore supports
// Read-only stream over `bytes` (a multiple of 16) at src; sink >= 1 KiB.
hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t st);
// read+write stream: its workgroup count and words written per thread
void stream_mix_shape(int64_t read_bytes, int64_t write_bytes, int64_t* grid, int64_t* words);
hipError_t launch_stream_mix(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                             hipStream_t st);
// MFMA ceiling: mfma_ceiling_grid() workgroups of 16 waves, `rounds` rounds of
// 8 MFMAs per wave, valu_per_mfma (0, 2 or 4) fp32 FMAs per MFMA; sink holds
// one float per thread.
int mfma_ceiling_grid();
hipError_t launch_mfma_ceiling(int rounds, int valu_per_mfma, float* sink, hipStream_t st);

// Largest M the lane-per-row GEMV accepts when forced, the largest it runs by
// default (from M = 3 on an MFMA kernel is faster, its unpacking being shared
// by all rows), and the largest M*K it stages in LDS (64 KiB of fp16).
constexpr int kGemvMaxM = 4;
constexpr int kGemvAutoMaxM = 2;
constexpr int64_t kGemvMaxMK = 32768;

}  // namespace lmh
