// Top-K selection of the quantized logits and exact rescoring of those rows.
//
// vLLM PR #48870, review comment, point 2: take the top-K of the quantized
// logits, recompute those K rows exactly from the unquantized weight, and
// scatter the exact values back (K = 8 costs 32 KB of weight reads next to a
// 311 MB int8 head).
//
// Order: value descending, then index ascending (a total order, so the
// selection is unique and deterministic).  The top-1 after rescoring is the
// first maximum of the updated row; because every unselected entry is at most
// the (K+1)-th largest quantized value, it is found among the K rescored
// values and that one extra candidate, without another pass over the row.
//
// Pass 1 (grid: chunks x rows): each workgroup reads a 4096-entry chunk of a
//   row and extracts its T = K+1 best entries by T rounds of a workgroup
//   arg-max restricted to entries that come after the previous winner.
// Pass 2 (grid: rows): the same selection over the chunk winners, then one
//   wave per selected row computes the exact fp32 dot product (per-lane
//   sequential FMA, then a fixed xor-shuffle tree) and the results are
//   scattered into y.
#include "lmh_internal.h"

#include <math.h>

namespace lmh {
namespace {

constexpr int kChunk = 4096;  // entries per pass-1 workgroup (256 threads x 16)
constexpr int kNone = 0x7FFFFFFF;

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
    return av > bv || (av == bv && ai < bi);
}

// Workgroup arg-max of (v, i) pairs under `better`; every thread gets the winner.
__device__ __forceinline__ void wg_best(float& v, int& i, float* sv, int* si) {
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(v, o);
        const int oi = __shfl_xor(i, o);
        if (better(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sv[w] = v;
        si[w] = i;
    }
    __syncthreads();
    v = sv[0];
    i = si[0];
    for (int k = 1; k < 4; ++k)
        if (better(sv[k], si[k], v, i)) {
            v = sv[k];
            i = si[k];
        }
    __syncthreads();
}

__global__ __launch_bounds__(256) void topk_chunk_kernel(const float* __restrict__ y, int64_t ldy,
                                                         int64_t V, int T, float* __restrict__ cval,
                                                         int* __restrict__ cidx) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int64_t m = blockIdx.y;
    const int C = gridDim.x;
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    float v[16];
    int id[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t e = base + i * 256 + threadIdx.x;
        v[i] = e < V ? y[m * ldy + e] : -INFINITY;
        id[i] = e < V ? (int)e : kNone;
    }
    float lv = INFINITY;
    int li = -1;
    for (int r = 0; r < T; ++r) {
        float bv = -INFINITY;
        int bi = kNone;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bool after = r == 0 || better(lv, li, v[i], id[i]);
            if (after && better(v[i], id[i], bv, bi)) {
                bv = v[i];
                bi = id[i];
            }
        }
        wg_best(bv, bi, sv, si);
        if (threadIdx.x == 0) {
            const int64_t o = (m * C + blockIdx.x) * T + r;
            cval[o] = bv;
            cidx[o] = bi;
        }
        lv = bv;
        li = bi;
    }
}

__device__ __forceinline__ float ld16(const uint16_t* p, int64_t i, int dt) {
    const uint16_t b = p[i];
    return dt == BF16 ? __uint_as_float((uint32_t)b << 16) : (float)__builtin_bit_cast(_Float16, b);
}

__global__ __launch_bounds__(256) void topk_merge_rescore_kernel(
    const float* __restrict__ cval, const int* __restrict__ cidx, int C, int T, int topk,
    const void* __restrict__ x, int x_dtype, const void* __restrict__ w, int w_dtype, int64_t K,
    float* __restrict__ y, int64_t ldy, int32_t* __restrict__ idx_out,
    float* __restrict__ val_out, int32_t* __restrict__ top1_out) {
    __shared__ float sv[4];
    __shared__ int si[4];
    __shared__ float tv[65];
    __shared__ int ti[65];
    __shared__ float rv[64];
    const int64_t m = blockIdx.x;
    const int64_t n = (int64_t)C * T;
    const float* cv = cval + m * n;
    const int* ci = cidx + m * n;
    float lv = INFINITY;
    int li = -1;
    for (int r = 0; r < T; ++r) {
        float bv = -INFINITY;
        int bi = kNone;
        for (int64_t e = threadIdx.x; e < n; e += 256) {
            const float ev = cv[e];
            const int ei = ci[e];
            const bool after = r == 0 || better(lv, li, ev, ei);
            if (after && better(ev, ei, bv, bi)) {
                bv = ev;
                bi = ei;
            }
        }
        wg_best(bv, bi, sv, si);
        if (threadIdx.x == 0) {
            tv[r] = bv;
            ti[r] = bi;
        }
        lv = bv;
        li = bi;
    }
    __syncthreads();
    // exact rescoring: wave wv handles selected rows wv, wv+4, ...
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int t = wv; t < topk; t += 4) {
        const int64_t v = ti[t];
        float acc = 0.0f;
        for (int64_t k = lane; k < K; k += 64) {
            const float xv = ld16((const uint16_t*)x, m * K + k, x_dtype);
            const float wvv = w_dtype == F32 ? ((const float*)w)[v * K + k]
                                             : ld16((const uint16_t*)w, v * K + k, w_dtype);
            acc = fmaf(xv, wvv, acc);
        }
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        if (lane == 0) rv[t] = acc;
    }
    __syncthreads();
    if (threadIdx.x < topk) {
        const int t = threadIdx.x;
        y[m * ldy + ti[t]] = rv[t];
        if (idx_out) idx_out[m * topk + t] = ti[t];
        if (val_out) val_out[m * topk + t] = rv[t];
    }
    if (threadIdx.x == 0 && top1_out) {
        float bv = rv[0];
        int bi = ti[0];
        for (int t = 1; t < topk; ++t)
            if (better(rv[t], ti[t], bv, bi)) {
                bv = rv[t];
                bi = ti[t];
            }
        if (T > topk && ti[topk] != kNone && better(tv[topk], ti[topk], bv, bi)) bi = ti[topk];
        top1_out[m] = bi;
    }
}

}  // namespace

size_t topk_ws_bytes(int64_t M, int64_t V, int topk) {
    const int64_t C = (V + kChunk - 1) / kChunk;
    const int64_t T = topk + 1;
    return (size_t)(M * C * T * 8 + 256);
}

hipError_t launch_topk_rescore(const void* x, int x_dtype, int M, const void* w, int w_dtype,
                               int64_t V, int64_t K, float* y, int64_t ldy, int topk,
                               int32_t* idx, float* val, int32_t* top1, void* ws,
                               hipStream_t st) {
    const int C = (int)((V + kChunk - 1) / kChunk);
    const int T = (int)(topk + 1 <= V ? topk + 1 : V);
    float* cval = (float*)ws;
    int* cidx = (int*)((char*)ws + (((size_t)M * C * T * 4 + 255) / 256) * 256);
    hipLaunchKernelGGL(topk_chunk_kernel, dim3(C, M), dim3(256), 0, st, y, ldy, V, T, cval, cidx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_rescore_kernel, dim3(M), dim3(256), 0, st, cval, cidx, C, T, topk,
                       x, x_dtype, w, w_dtype, K, y, ldy, idx, val, top1);
    return hipGetLastError();
}

}  // namespace lmh
