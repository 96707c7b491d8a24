// Top-K selection of the quantized logits and exact rescoring of those rows.
//
// vLLM PR #48870, review comment, point 2: take the top-K of the quantized
// logits, recompute those K rows exactly from the unquantized weight, and
// scatter the exact values back (K = 8 costs 32 KB of weight reads next to a
// 311 MB int8 head).
//
// Order: value descending, then index ascending (a total order, so the
// selection is unique and deterministic).  -0 and +0 count as equal, as in a
// float comparison; a NaN logit ranks below every number (the oracle leaves
// NaN inputs unspecified; here they only have to stay memory-safe).  Each
// entry becomes one 64-bit code whose unsigned order is that order: the high
// word is the value's bits mapped to an order-preserving integer, the low word
// 0x7FFFFFFF - index.  All codes of a row are distinct, so "the entries with
// rank < T" is a set of exactly T entries and every comparison is one 64-bit
// integer compare.
//
// The top-1 after rescoring is the first maximum of the updated row: every
// unselected entry is at most the (K+1)-th largest quantized value, so it is
// found among the K rescored values and that one extra candidate.
//
// Neither pass runs arg-max rounds (their serial latency dominated): each
// takes a threshold that at least T entries reach, keeps the few entries at or
// above it, and places each kept entry by its rank among them.
//
// Pass 1 (grid: blocks of 2048 entries x rows, 256 threads, 8 entries each):
//   thread maxima -> each wave's T-th largest thread maximum (rank among the
//   wave's 64) -> threshold = the largest of those (T <= 64; for T = 65 the
//   T-th largest of all 256 thread maxima) -> entries >= threshold into LDS
//   -> rank among them -> the block's top T, sorted, into the workspace.
// Pass 2 (grid: rows, 256 threads): the T-th largest list head is the
//   threshold; only the T lists whose heads reach it can hold a top-T entry;
//   their entries >= threshold are ranked as in pass 1.  Then the exact fp32
//   dot products of the selected rows (all rows at once), the scatter into y,
//   idx/val and the top-1.
#include "lmh_internal.h"

#include <limits.h>
#include <math.h>

namespace lmh {
namespace {

typedef unsigned long long u64;

constexpr int kPer = 8;                // entries per thread in pass 1
constexpr int kBlockN = 256 * kPer;    // entries per pass-1 block (2048)
constexpr int kMaxT = 65;              // topk <= 64, plus the top-1 candidate
constexpr int kMaxLists = 1024;        // pass-2 lists per row: V <= 2^21
constexpr int kPass2Cand = kMaxT * kMaxT;

__device__ __forceinline__ u64 make_code(float v, int idx) {
    const float f = v == 0.0f ? 0.0f : v;  // -0 -> +0
    const int b = __float_as_int(f);
    const int key = (f != f) ? INT_MIN : (b >= 0 ? b : b ^ 0x7FFFFFFF);
    return ((u64)((uint32_t)key ^ 0x80000000u) << 32) | (uint32_t)(0x7FFFFFFF - idx);
}

__device__ __forceinline__ int code_idx(u64 c) { return 0x7FFFFFFF - (int)(uint32_t)c; }

__device__ __forceinline__ float code_val(u64 c) {
    const int key = (int)((uint32_t)(c >> 32) ^ 0x80000000u);
    return __int_as_float(key >= 0 ? key : key ^ 0x7FFFFFFF);
}

// Pass 1.  A position past the end of the row gets a code below every real
// entry (high word 0, low word < 2048, distinct within the block), so a block
// with fewer than T real entries still yields T distinct codes; they never
// reach the final top T because T <= V.
__global__ __launch_bounds__(256) void topk_block_kernel(const float* __restrict__ y, int64_t ldy,
                                                         int64_t V, int T, u64* __restrict__ out) {
    __shared__ u64 tmax[256];
    __shared__ u64 wthr[4];
    __shared__ u64 cs[kBlockN];
    __shared__ int cnt;
    const int tid = threadIdx.x, wv = tid >> 6;
    const int64_t m = blockIdx.y;
    const int64_t base = (int64_t)blockIdx.x * kBlockN;
    u64 c[kPer];
    u64 best = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int loc = i * 256 + tid;
        const int64_t e = base + loc;
        const bool in = e < V;
        const float val = y[m * ldy + (in ? e : V - 1)];  // unconditional load, clamped
        c[i] = in ? make_code(val, (int)e) : (u64)(kBlockN - 1 - loc);
        best = c[i] > best ? c[i] : best;
    }
    tmax[tid] = best;
    if (tid == 0) cnt = 0;
    __syncthreads();
    // threshold: at least T entries of the block are >= it
    if (T <= 64) {
        int r = 0;
#pragma unroll 16
        for (int j = 0; j < 64; ++j) r += tmax[wv * 64 + j] > best;
        if (r == T - 1) wthr[wv] = best;
        __syncthreads();
        if (tid == 0) {
            u64 t = wthr[0];
#pragma unroll
            for (int k = 1; k < 4; ++k) t = wthr[k] > t ? wthr[k] : t;
            wthr[0] = t;
        }
    } else {
        int r = 0;
#pragma unroll 16
        for (int j = 0; j < 256; ++j) r += tmax[j] > best;
        if (r == T - 1) wthr[0] = best;
    }
    __syncthreads();
    const u64 thr = wthr[0];
    // keep the entries >= thr: only threads whose maximum reaches thr have any
    if (best >= thr) {
        int nc = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) nc += c[i] >= thr;
        int off = atomicAdd(&cnt, nc);
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (c[i] >= thr) cs[off++] = c[i];
    }
    __syncthreads();
    const int S = cnt;  // T <= S <= 2048
    u64* o = out + (m * gridDim.x + blockIdx.x) * T;
    for (int k = tid; k < S; k += 256) {
        const u64 me = cs[k];
        int r = 0;
        for (int j = 0; j < S; ++j) r += cs[j] > me;
        if (r < T) o[r] = me;
    }
}

__device__ __forceinline__ float ld16(const uint16_t* p, int64_t i, int dt) {
    const uint16_t b = p[i];
    return dt == BF16 ? __uint_as_float((uint32_t)b << 16) : (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ void to_f32x8(uint4 q, int dt, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t u = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
        f[2 * j] = dt == BF16 ? __uint_as_float(u << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)u);
        f[2 * j + 1] = dt == BF16 ? __uint_as_float(u & 0xFFFF0000u)
                                  : (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
    }
}

__device__ __forceinline__ void load_w8(const void* w, int w_dtype, int64_t off, float* f) {
    if (w_dtype == F32) {
        const float4 a = *(const float4*)((const float*)w + off);
        const float4 b = *(const float4*)((const float*)w + off + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
        to_f32x8(*(const uint4*)((const uint16_t*)w + off), w_dtype, f);
    }
}

// Exact fp32 dot products of x row m with the reference rows idx[t], t < topk.
// All rows at once, so their loads are in flight together: row t goes to a
// group of G = 256/P consecutive threads (P = topk rounded up to a power of
// two, at least 4, so a group never spans two waves).  Each thread takes 8
// consecutive columns per 16-byte load when `vec` (K % 8 == 0 and 16-byte
// aligned rows), else one column at a time, strided by the group; its partial
// sum is sequential and the group's partials meet in a fixed xor-shuffle tree,
// so the result does not depend on timing.  An index outside [0, V) is never
// dereferenced.
__device__ void rescore_rows(const int* idx, int topk, int64_t m, int64_t V, const void* __restrict__ x,
                             int x_dtype, const void* __restrict__ w, int w_dtype, int64_t K, int vec,
                             float* rv) {
    int P = 4;
    while (P < topk) P *= 2;
    const int G = 256 / P;  // 64, 32, 16, 8 or 4
    const int t = threadIdx.x / G, sub = threadIdx.x % G;
    const int64_t v0 = t < topk ? idx[t] : 0;
    const bool on = t < topk && v0 >= 0 && v0 < V;
    const int64_t v = on ? v0 : 0;
    const int64_t kend = on ? K : 0;
    float acc = 0.0f;
    if (vec) {
#pragma unroll 4
        for (int64_t k = 8 * sub; k < kend; k += 8 * G) {
            float xf[8], wf[8];
            to_f32x8(*(const uint4*)((const uint16_t*)x + m * K + k), x_dtype, xf);
            load_w8(w, w_dtype, v * K + k, wf);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc = fmaf(xf[q], wf[q], acc);
        }
    } else {
#pragma unroll 4
        for (int64_t k = sub; k < kend; k += G) {
            const float xv = ld16((const uint16_t*)x, m * K + k, x_dtype);
            const float wv = w_dtype == F32 ? ((const float*)w)[v * K + k]
                                            : ld16((const uint16_t*)w, v * K + k, w_dtype);
            acc = fmaf(xv, wv, acc);
        }
    }
    for (int o = G / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (t < topk && sub == 0) rv[t] = on ? acc : NAN;
}

// Pass 2: one workgroup per row over the C sorted lists of T codes that
// pass 1 wrote; then rescoring, scatter, idx/val and top-1.
__global__ __launch_bounds__(256) void topk_select_rescore_kernel(
    const u64* __restrict__ lists, int C, int T, int topk, const void* __restrict__ x, int x_dtype,
    const void* __restrict__ w, int w_dtype, int64_t V, int64_t K, int vec, float* __restrict__ y,
    int64_t ldy, int32_t* __restrict__ idx_out, float* __restrict__ val_out,
    int32_t* __restrict__ top1_out) {
    __shared__ u64 heads[kMaxLists];
    __shared__ u64 cs[kPass2Cand];
    __shared__ int qual[kMaxT];
    __shared__ u64 sel[kMaxT];
    __shared__ int ti[kMaxT];
    __shared__ float rv[64];
    __shared__ u64 thr_s;
    __shared__ int nq, cnt;
    const int tid = threadIdx.x;
    const int64_t m = blockIdx.x;
    const u64* L = lists + m * (int64_t)C * T;
    for (int l = tid; l < C; l += 256) heads[l] = L[(int64_t)l * T];
    if (tid == 0) {
        nq = 0;
        cnt = 0;
        thr_s = 0;  // C < T: every entry of every list
    }
    __syncthreads();
    // threshold: the T-th largest head (then exactly T lists reach it)
    if (C >= T) {
        for (int l = tid; l < C; l += 256) {
            const u64 h = heads[l];
            int r = 0;
            for (int j = 0; j < C; ++j) r += heads[j] > h;
            if (r == T - 1) thr_s = h;
        }
    }
    __syncthreads();
    const u64 thr = thr_s;
    for (int l = tid; l < C; l += 256)
        if (heads[l] >= thr) qual[atomicAdd(&nq, 1)] = l;
    __syncthreads();
    // entries >= thr of the qualifying lists (at most T*T)
    const int ne = nq * T;
    for (int e = tid; e < ne; e += 256) {
        const int l = qual[e / T];
        const u64 c = L[(int64_t)l * T + e % T];
        if (c >= thr) cs[atomicAdd(&cnt, 1)] = c;
    }
    __syncthreads();
    const int S = cnt;  // T <= S <= T*T
    for (int k = tid; k < S; k += 256) {
        const u64 me = cs[k];
        int r = 0;
        for (int j = 0; j < S; ++j) r += cs[j] > me;
        if (r < T) sel[r] = me;
    }
    __syncthreads();
    if (tid < T) ti[tid] = code_idx(sel[tid]);
    __syncthreads();
    rescore_rows(ti, topk, m, V, x, x_dtype, w, w_dtype, K, vec, rv);
    __syncthreads();
    if (tid < topk) {
        if (ti[tid] >= 0 && ti[tid] < V) y[m * ldy + ti[tid]] = rv[tid];
        if (idx_out) idx_out[m * topk + tid] = ti[tid];
        if (val_out) val_out[m * topk + tid] = rv[tid];
    }
    if (tid == 0 && top1_out) {
        // first maximum among the rescored values and the (K+1)-th candidate,
        // compared as floats (value descending, then index ascending)
        float bv = rv[0];
        int bi = ti[0];
        for (int t = 1; t < topk; ++t)
            if ((rv[t] > bv) | ((rv[t] == bv) & (ti[t] < bi))) {
                bv = rv[t];
                bi = ti[t];
            }
        if (T > topk) {
            const float cv = code_val(sel[topk]);
            const int ci = ti[topk];
            if ((cv > bv) | ((cv == bv) & (ci < bi))) bi = ci;
        }
        top1_out[m] = bi;
    }
}

}  // namespace

int64_t topk_max_v() { return (int64_t)kBlockN * kMaxLists; }

size_t topk_ws_bytes(int64_t M, int64_t V, int topk) {
    const int64_t C = (V + kBlockN - 1) / kBlockN;
    const int64_t T = topk + 1;
    return (size_t)(M * C * T * 8 + 256);
}

hipError_t launch_topk_rescore(const void* x, int x_dtype, int M, const void* w, int w_dtype,
                               int64_t V, int64_t K, float* y, int64_t ldy, int topk,
                               int32_t* idx, float* val, int32_t* top1, void* ws,
                               hipStream_t st) {
    const int C = (int)((V + kBlockN - 1) / kBlockN);
    const int T = (int)(topk + 1 <= V ? topk + 1 : V);
    u64* lists = (u64*)ws;
    hipLaunchKernelGGL(topk_block_kernel, dim3(C, M), dim3(256), 0, st, y, ldy, V, T, lists);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int esz = w_dtype == F32 ? 4 : 2;
    const int vec = K % 8 == 0 && ((uintptr_t)x & 15u) == 0 && ((uintptr_t)w & 15u) == 0 &&
                    (K * esz) % 16 == 0;
    hipLaunchKernelGGL(topk_select_rescore_kernel, dim3(M), dim3(256), 0, st, lists, C, T, topk, x,
                       x_dtype, w, w_dtype, V, K, vec, y, ldy, idx, val, top1);
    return hipGetLastError();
}

}  // namespace lmh
