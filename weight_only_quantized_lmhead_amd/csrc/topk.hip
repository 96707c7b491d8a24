// Top-K selection of the quantized logits and exact rescoring of those rows.
//
// vLLM PR #48870, review comment, point 2: the K best quantized logits of a
// row are replaced by exact dot products with the 16-bit weight rows they
// index; with K = 8 those rows are 32 KB against the 311 MB int8 head.
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
// Pass 1 (grid: blocks of 256*kPer entries x rows, 256 threads, kPer = 8, 16
//   or 32 entries each, so that a row has at most 256 blocks):
//   thread maxima -> each wave's T-th largest thread maximum (rank among the
//   wave's 64) -> threshold = the largest of those (T <= 64; for T = 65 the
//   T-th largest of all 256 thread maxima) -> entries >= threshold into LDS
//   -> rank among them -> the block's top T, sorted, into the workspace.
// Pass 2 (grid: rows, 256 threads, one list per thread): the T-th largest
//   list head is the threshold; the entries at or above it of the T lists
//   that reach it are ranked as in pass 1.  Then the exact fp32 dot products
//   of the selected rows (all rows at once), the scatter into y, idx/val and
//   the top-1.
//
// Fused form (one activation row, topk <= 16): the GEMV itself writes one
// sorted list of T codes per 64-row block, so pass 1 (and its read of y)
// disappears; the merge (1024 threads: a few list heads per thread, so that
// they arrive in one short burst; 16 per thread took 1.9 us longer) takes up
// to 4096 lists: in each of four runs of 64 groups of 4 threads, the T-th
// largest group maximum bounds the row's T-th largest from below (that run
// alone has T entries at or above it), the largest of the four is the first
// threshold, the lists whose heads reach it (at most 4T groups' worth) give
// the second threshold (their T-th largest
// head: exactly T lists reach it), and the entries at or above it of those T
// lists are ranked as above.  The rescoring keeps the 256-thread grouping of
// pass 2, so both paths add the same products in the same order.
#include "lmh_internal.h"

#include <math.h>

namespace lmh {
namespace {

constexpr int kMaxT = 65;              // topk <= 64, plus the top-1 candidate
constexpr int kMaxLists = 256;         // pass-2 lists per row (one per pass-1 block)

// Entries per thread in pass 1 (a block takes 256 times as many): the
// smallest of 8, 16, 32 that keeps the row to at most kMaxLists blocks.
inline int pass1_per(int64_t V) { return V <= 2048 * kMaxLists ? 8 : V <= 4096 * kMaxLists ? 16 : 32; }
constexpr int kPass2Cand = kMaxT * kMaxT;

// Pass 1.  A position past the end of the row gets a code below every real
// entry (high word 0, low word in [1, 256*kPer], distinct within the block; 0
// means "no list" in pass 2), so a block with fewer than T real entries still
// yields T distinct codes; they never reach the final top T because T <= V.
template <int kPer>
__global__ __launch_bounds__(256) void topk_block_kernel(const float* __restrict__ y, int64_t ldy,
                                                         int64_t V, int T, u64* __restrict__ out) {
    constexpr int kBlockN = 256 * kPer;
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
        c[i] = in ? topk_code(val, (int)e) : (u64)(kBlockN - loc);
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
#pragma unroll 8
        for (int j = 0; j < S; ++j) r += cs[j] > me;
        if (r < T) o[r] = me;
    }
}

template <int DT>
__device__ __forceinline__ float ld16(const uint16_t* p, int64_t i) {
    const uint16_t b = p[i];
    return DT == BF16 ? __uint_as_float((uint32_t)b << 16) : (float)__builtin_bit_cast(_Float16, b);
}

template <int DT>
__device__ __forceinline__ void to_f32x8(uint4 q, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t u = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
        f[2 * j] = DT == BF16 ? __uint_as_float(u << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)u);
        f[2 * j + 1] = DT == BF16 ? __uint_as_float(u & 0xFFFF0000u)
                                  : (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
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
// dereferenced.  XD / WD are the dtypes of x and of the reference weight.
template <int XD, int WD>
__device__ __forceinline__ void rescore_rows_t(const int* idx, int topk, int64_t m, int64_t V,
                                               const void* __restrict__ x,
                                               const void* __restrict__ w, int64_t K, int vec,
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
        // batches of kB chunks: all their loads are issued before the first
        // multiply, so a long row costs a few round trips to memory, not one
        // per chunk; the sum still runs over the chunks in order
        constexpr int kB = 8;
        constexpr int WU = WD == F32 ? 2 : 1;  // 16-byte loads per 8 weights
        for (int64_t k0 = 8 * sub; k0 < kend; k0 += (int64_t)8 * G * kB) {
            uint4 xr[kB], wr[kB][WU];
#pragma unroll
            for (int b = 0; b < kB; ++b) {
                const int64_t k = k0 + (int64_t)8 * G * b;
                if (k < kend) {
                    xr[b] = *(const uint4*)((const uint16_t*)x + m * K + k);
#pragma unroll
                    for (int u = 0; u < WU; ++u)
                        wr[b][u] = WD == F32 ? *(const uint4*)((const float*)w + v * K + k + 4 * u)
                                             : *(const uint4*)((const uint16_t*)w + v * K + k);
                }
            }
#pragma unroll
            for (int b = 0; b < kB; ++b) {
                const int64_t k = k0 + (int64_t)8 * G * b;
                if (k < kend) {
                    float xf[8], wf[8];
                    to_f32x8<XD>(xr[b], xf);
                    if constexpr (WD == F32) {
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            wf[4 * u] = __uint_as_float(wr[b][u].x);
                            wf[4 * u + 1] = __uint_as_float(wr[b][u].y);
                            wf[4 * u + 2] = __uint_as_float(wr[b][u].z);
                            wf[4 * u + 3] = __uint_as_float(wr[b][u].w);
                        }
                    } else {
                        to_f32x8<WD>(wr[b][0], wf);
                    }
#pragma unroll
                    for (int q = 0; q < 8; ++q) acc = fmaf(xf[q], wf[q], acc);
                }
            }
        }
    } else {
#pragma unroll 4
        for (int64_t k = sub; k < kend; k += G) {
            const float xv = ld16<XD>((const uint16_t*)x, m * K + k);
            const float wv = WD == F32 ? ((const float*)w)[v * K + k] : ld16<WD>((const uint16_t*)w, v * K + k);
            acc = fmaf(xv, wv, acc);
        }
    }
    for (int o = G / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (t < topk && sub == 0) rv[t] = on ? acc : NAN;
}

__device__ __forceinline__ void rescore_rows(const int* idx, int topk, int64_t m, int64_t V,
                                             const void* __restrict__ x, int x_dtype,
                                             const void* __restrict__ w, int w_dtype, int64_t K,
                                             int vec, float* rv) {
    if (x_dtype == BF16) {
        if (w_dtype == BF16) rescore_rows_t<BF16, BF16>(idx, topk, m, V, x, w, K, vec, rv);
        else if (w_dtype == F32) rescore_rows_t<BF16, F32>(idx, topk, m, V, x, w, K, vec, rv);
        else rescore_rows_t<BF16, F16>(idx, topk, m, V, x, w, K, vec, rv);
    } else {
        if (w_dtype == BF16) rescore_rows_t<F16, BF16>(idx, topk, m, V, x, w, K, vec, rv);
        else if (w_dtype == F32) rescore_rows_t<F16, F32>(idx, topk, m, V, x, w, K, vec, rv);
        else rescore_rows_t<F16, F16>(idx, topk, m, V, x, w, K, vec, rv);
    }
}

// Workgroup barrier for kernels whose threads share data only through LDS:
// waits for this thread's LDS operations, not for its global loads (a
// __syncthreads() fence would also wait for global loads still in flight).
// The empty asm statements keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct SelectShared {
    u64 heads[256];
    int qual[kMaxT];
    u64 cs[kPass2Cand];
    u64 sel[kMaxT];
    int ti[kMaxT];
    float rv[64];
    u64 thr;
    int nq, cnt;
};

// The top T of C <= 256 sorted lists of T codes (code 0: none) into sh.sel,
// sorted: the T-th largest head is the threshold (then exactly T lists reach
// it; all lists when C < T), and the entries of those lists at or above it
// (at most T*T) are placed by rank.  Thread i owns list i; with T <= 16 it
// loads the whole list at once, so the candidates come from its registers
// (one round trip to memory instead of two).  Ends with a barrier.
__device__ __forceinline__ void select_lists(const u64* __restrict__ L, int C, int T,
                                             SelectShared& sh) {
    constexpr int kRegT = 16;
    const int tid = threadIdx.x;
    const bool own = tid < C;
    const int64_t lb = (int64_t)(own ? tid : C - 1) * T;  // clamped: loads are unconditional
    u64 e[kRegT];
    const bool inreg = T <= kRegT;
    if (inreg) {
#pragma unroll
        for (int i = 0; i < kRegT; ++i) e[i] = L[lb + (i < T ? i : 0)];
    } else {
        e[0] = L[lb];
    }
    const u64 h = e[0];
    sh.heads[tid] = own ? h : 0;
    if (tid == 0) {
        sh.nq = sh.cnt = 0;
        sh.thr = 0;
    }
    lds_barrier();
    if (own && C >= T) {
        int r = 0;
#pragma unroll 8
        for (int j = 0; j < C; ++j) r += sh.heads[j] > h;
        if (r == T - 1) sh.thr = h;
    }
    lds_barrier();
    const u64 thr = sh.thr;
    if (inreg) {
        if (own && h >= thr) {
#pragma unroll
            for (int i = 0; i < kRegT; ++i)
                if (i < T && e[i] != 0 && e[i] >= thr) sh.cs[atomicAdd(&sh.cnt, 1)] = e[i];
        }
    } else {
        if (own && h >= thr) sh.qual[atomicAdd(&sh.nq, 1)] = tid;
        lds_barrier();
        const int ne = sh.nq * T;  // at most T*T entries
        for (int q = tid; q < ne; q += 256) {
            const int l = sh.qual[q / T];
            const u64 c = L[(int64_t)l * T + q % T];
            if (c != 0 && c >= thr) sh.cs[atomicAdd(&sh.cnt, 1)] = c;
        }
    }
    lds_barrier();
    const int S = sh.cnt;  // T <= S <= T*T
    for (int k = tid; k < S; k += 256) {
        const u64 me = sh.cs[k];
        int r = 0;
#pragma unroll 8
        for (int j = 0; j < S; ++j) r += sh.cs[j] > me;
        if (r < T) sh.sel[r] = me;
    }
    lds_barrier();
}

// Rescore the selected rows, scatter into y (if given), write idx/val and
// the top-1: the first maximum among the rescored values and the (K+1)-th
// candidate, compared as floats (value descending, then index ascending).
__device__ __forceinline__ void finish_row(SelectShared& sh, int T, int topk, int64_t m, int64_t V,
                                           const void* __restrict__ x, int x_dtype,
                                           const void* __restrict__ w, int w_dtype, int64_t K,
                                           int vec, float* __restrict__ y, int64_t ldy,
                                           int32_t* __restrict__ idx_out,
                                           float* __restrict__ val_out,
                                           int32_t* __restrict__ top1_out) {
    const int tid = threadIdx.x;
    if (tid < T) sh.ti[tid] = topk_code_idx(sh.sel[tid]);
    lds_barrier();
    rescore_rows(sh.ti, topk, m, V, x, x_dtype, w, w_dtype, K, vec, sh.rv);
    lds_barrier();
    if (tid < topk) {
        const int v = sh.ti[tid];
        if (y && v >= 0 && v < V) y[m * ldy + v] = sh.rv[tid];
        if (idx_out) idx_out[m * topk + tid] = v;
        if (val_out) val_out[m * topk + tid] = sh.rv[tid];
    }
    if (tid == 0 && top1_out) {
        float bv = sh.rv[0];
        int bi = sh.ti[0];
        for (int t = 1; t < topk; ++t)
            if ((sh.rv[t] > bv) | ((sh.rv[t] == bv) & (sh.ti[t] < bi))) {
                bv = sh.rv[t];
                bi = sh.ti[t];
            }
        if (T > topk) {
            const float cv = topk_code_val(sh.sel[topk]);
            const int ci = sh.ti[topk];
            if ((cv > bv) | ((cv == bv) & (ci < bi))) bi = ci;
        }
        top1_out[m] = bi;
    }
}

// Pass 2: one workgroup per row over the C <= 256 lists of pass 1.
__global__ __launch_bounds__(256) void topk_select_rescore_kernel(
    const u64* __restrict__ lists, int C, int T, int topk, const void* __restrict__ x, int x_dtype,
    const void* __restrict__ w, int w_dtype, int64_t V, int64_t K, int vec, float* __restrict__ y,
    int64_t ldy, int32_t* __restrict__ idx_out, float* __restrict__ val_out,
    int32_t* __restrict__ top1_out) {
    __shared__ SelectShared sh;
    const int64_t m = blockIdx.x;
    select_lists(lists + m * (int64_t)C * T, C, T, sh);
    finish_row(sh, T, topk, m, V, x, x_dtype, w, w_dtype, K, vec, y, ldy, idx_out, val_out,
               top1_out);
}

constexpr int kMergeMaxT = 17;     // topk <= 16, plus the top-1 candidate
constexpr int kMergeThreads = 1024;
constexpr int kMergeLPT = 4;       // lists per thread: up to 4096 lists (64-row blocks) per row
constexpr int kMergeMaxQual = 4 * kMergeMaxT * 4 * kMergeLPT;  // 4T groups of 4 threads

struct MergeShared {
    SelectShared s;
    u64 wthr[4];
    u64 thr2;
    u64 qh[kMergeMaxQual];  // heads of the lists that reach the first threshold
    int ql[kMergeMaxQual];  // and their list numbers
};

// The top T of C <= 4096 sorted lists of T codes into sh.s.sel, sorted (see
// the header).  The lists are stored entry-major: entry j of list l at
// L[j*C + l].  1024 threads; thread i owns lists i, i + 1024, ... (a few
// loads per thread: the heads arrive in one short burst), and the 4 threads
// 4g .. 4g+3 form group g (up to 16 lists), whose largest head takes part in
// the first threshold as one of 256.  Ends with a barrier.
__device__ __forceinline__ void merge_lists(const u64* __restrict__ L, int C, int T,
                                            MergeShared& sh) {
    const int tid = threadIdx.x;
    u64 hd[kMergeLPT];
    u64 tmax = 0;
#pragma unroll
    for (int i = 0; i < kMergeLPT; ++i) {
        const int l = tid + kMergeThreads * i;
        hd[i] = l < C ? L[l] : 0;
        tmax = hd[i] > tmax ? hd[i] : tmax;
    }
    // the group's largest head: lanes 4g .. 4g+3 of the wave
    u64 gmax = tmax;
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
        const u64 other = ((u64)(uint32_t)__shfl_xor((int)(uint32_t)(gmax >> 32), o) << 32) |
                          (uint32_t)__shfl_xor((int)(uint32_t)gmax, o);
        gmax = other > gmax ? other : gmax;
    }
    if ((tid & 3) == 0) sh.s.heads[tid >> 2] = gmax;
    if (tid < 4) sh.wthr[tid] = 0;
    if (tid == 0) {
        sh.s.nq = sh.s.cnt = 0;
        sh.thr2 = 0;
    }
    lds_barrier();
    // first threshold: the largest of the T-th largest group maxima of the
    // four runs of 64 groups (0 when no run has T lists: then every list
    // takes part)
    if (tid < 256) {
        const u64 h = sh.s.heads[tid];
        if (h != 0) {
            const int run = tid >> 6;
            int r = 0;
#pragma unroll 16
            for (int j = 0; j < 64; ++j) r += sh.s.heads[run * 64 + j] > h;
            if (r == T - 1) sh.wthr[run] = h;
        }
    }
    lds_barrier();
    u64 thr1 = sh.wthr[0];
#pragma unroll
    for (int k = 1; k < 4; ++k) thr1 = sh.wthr[k] > thr1 ? sh.wthr[k] : thr1;
    if (tmax != 0 && tmax >= thr1) {
#pragma unroll
        for (int i = 0; i < kMergeLPT; ++i) {
            if (hd[i] != 0 && hd[i] >= thr1) {
                const int q = atomicAdd(&sh.s.nq, 1);
                sh.qh[q] = hd[i];
                sh.ql[q] = tid + kMergeThreads * i;
            }
        }
    }
    lds_barrier();
    // at most T groups of the run that sets the threshold and T - 1 of each
    // other run reach it, with up to 16 lists each
    const int nq = sh.s.nq;
    // second threshold: the T-th largest qualifying head (0 when fewer than T)
    for (int q = tid; q < nq; q += kMergeThreads) {
        const u64 me = sh.qh[q];
        int r = 0;
        for (int j = 0; j < nq; ++j) r += sh.qh[j] > me;
        if (r == T - 1) sh.thr2 = me;
    }
    lds_barrier();
    const u64 thr2 = sh.thr2;
    // the entries at or above it of the (at most T) lists whose heads reach it
    for (int e = tid; e < nq * T; e += kMergeThreads) {
        const int q = e / T;
        if (sh.qh[q] >= thr2) {
            const u64 c = L[(int64_t)(e - q * T) * C + sh.ql[q]];
            if (c != 0 && c >= thr2) sh.s.cs[atomicAdd(&sh.s.cnt, 1)] = c;
        }
    }
    lds_barrier();
    const int S = sh.s.cnt;  // T <= S <= T*T
    for (int k = tid; k < S; k += kMergeThreads) {
        const u64 me = sh.s.cs[k];
        int r = 0;
#pragma unroll 8
        for (int j = 0; j < S; ++j) r += sh.s.cs[j] > me;
        if (r < T) sh.s.sel[r] = me;
    }
    lds_barrier();
}

// Merge of the GEMV's per-block lists, then rescoring as in pass 2.
__global__ __launch_bounds__(kMergeThreads) void topk_merge_rescore_kernel(
    const u64* __restrict__ lists, int C, int T, int topk, const void* __restrict__ x, int x_dtype,
    const void* __restrict__ w, int w_dtype, int64_t V, int64_t K, int vec, float* __restrict__ y,
    int64_t ldy, int32_t* __restrict__ idx_out, float* __restrict__ val_out,
    int32_t* __restrict__ top1_out) {
    __shared__ MergeShared sh;
    const int64_t m = blockIdx.x;
    merge_lists(lists + m * (int64_t)C * T, C, T, sh);
    finish_row(sh.s, T, topk, m, V, x, x_dtype, w, w_dtype, K, vec, y, ldy, idx_out, val_out,
               top1_out);
}

inline int rescore_vec(const void* x, const void* w, int w_dtype, int64_t K) {
    const int esz = w_dtype == F32 ? 4 : 2;
    return K % 8 == 0 && ((uintptr_t)x & 15u) == 0 && ((uintptr_t)w & 15u) == 0 &&
           (K * esz) % 16 == 0;
}

}  // namespace

bool topk_fused_ok(int64_t V, int topk) {
    return topk + 1 <= kMergeMaxT && (V + 63) / 64 <= kMergeThreads * kMergeLPT;
}

size_t topk_fused_lists_bytes(int64_t M, int64_t V, int topk) {
    const int64_t T = topk + 1 <= V ? topk + 1 : V;
    return (size_t)(M * ((V + 63) / 64) * T * 8);
}

hipError_t launch_topk_merge_rescore(const u64* lists, const void* x, int x_dtype, int M,
                                     const void* w, int w_dtype, int64_t V, int64_t K, float* y,
                                     int64_t ldy, int topk, int T, int32_t* idx, float* val,
                                     int32_t* top1, hipStream_t st) {
    const int C = (int)((V + 63) / 64);
    hipLaunchKernelGGL(topk_merge_rescore_kernel, dim3(M), dim3(kMergeThreads), 0, st, lists, C, T, topk, x,
                       x_dtype, w, w_dtype, V, K, rescore_vec(x, w, w_dtype, K), y, ldy, idx, val,
                       top1);
    return hipGetLastError();
}

int64_t topk_max_v() { return (int64_t)256 * 32 * kMaxLists; }

size_t topk_ws_bytes(int64_t M, int64_t V, int topk) {
    const int64_t bn = 256 * pass1_per(V);
    const int64_t C = (V + bn - 1) / bn;
    const int64_t T = topk + 1;
    return (size_t)(M * C * T * 8 + 256);
}

hipError_t launch_topk_rescore(const void* x, int x_dtype, int M, const void* w, int w_dtype,
                               int64_t V, int64_t K, float* y, int64_t ldy, int topk,
                               int32_t* idx, float* val, int32_t* top1, void* ws,
                               hipStream_t st) {
    const int per = pass1_per(V);
    const int C = (int)((V + 256 * per - 1) / (256 * per));
    if (C > kMaxLists) return hipErrorInvalidValue;  // V <= topk_max_v(), checked by the API
    const int T = (int)(topk + 1 <= V ? topk + 1 : V);
    u64* lists = (u64*)ws;
    if (per == 8)
        hipLaunchKernelGGL(topk_block_kernel<8>, dim3(C, M), dim3(256), 0, st, y, ldy, V, T, lists);
    else if (per == 16)
        hipLaunchKernelGGL(topk_block_kernel<16>, dim3(C, M), dim3(256), 0, st, y, ldy, V, T, lists);
    else
        hipLaunchKernelGGL(topk_block_kernel<32>, dim3(C, M), dim3(256), 0, st, y, ldy, V, T, lists);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int vec = rescore_vec(x, w, w_dtype, K);
    hipLaunchKernelGGL(topk_select_rescore_kernel, dim3(M), dim3(256), 0, st, lists, C, T, topk, x,
                       x_dtype, w, w_dtype, V, K, vec, y, ldy, idx, val, top1);
    return hipGetLastError();
}

}  // namespace lmh
