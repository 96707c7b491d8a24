// Measurement aids, not part of the logits path: the practical ceilings the
// logits kernels are measured against.
//
// Read-only HBM stream.  Each workgroup reads one contiguous run of 768
// 16-byte words (12 KiB), one load per thread per step; the best of the
// shapes measured on MI355X for a cold 83 MB buffer (5.9 TB/s, against
// 5.3-5.7 for fewer, longer-lived workgroups or a grid-stride loop).
//
// Read+write HBM stream.  Each 256-thread workgroup reads a run of 4
// 16-byte words per thread (16 KiB) and then writes its share of the output,
// ceil(written / read) words per thread; the reads cover the source once and
// the writes the destination once.  The best of the shapes measured on MI355X
// for the byte mixes of the logits calls beyond one activation row (83 MB
// read with 19 or 156 MB written, source and destination both rotating over
// 13 copies: 5.1-5.4 TB/s combined, against 4.4-4.8 for 8- or 17-word runs).
//
// MFMA issue.  One workgroup of 16 waves per CU (the activation-resident
// kernel's shape); every wave runs `rounds` rounds of 8 independent
// v_mfma_f32_16x16x32_f16 chains on register operands, and with NV > 0 also
// NV independent fp32 FMAs per MFMA (the scale FMAs of a G-column group cost
// 128 / G per MFMA), so that the time of MFMA work alone and of MFMA work
// with a given VALU share is measured on the same grid.
#include "lmh_internal.h"

namespace lmh {
namespace {

constexpr int kStreamThreads = 256;
constexpr int64_t kStreamRun = 3 * kStreamThreads;  // 16-byte words per workgroup

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* __restrict__ p,
                                                                     int64_t n16,
                                                                     uint32_t* __restrict__ sink) {
    const int64_t beg = (int64_t)blockIdx.x * kStreamRun;
    const int64_t end = beg + kStreamRun < n16 ? beg + kStreamRun : n16;
    uint32_t acc = 0;
    for (int64_t i = beg + threadIdx.x; i < end; i += kStreamThreads) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // keeps the loads alive; stores only when the folded word hits this value
    if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

constexpr int kMixRun = 4;  // 16-byte words read per thread

// Thread t of workgroup b reads words b * 1024 + 256 i + t (i < 4) and writes
// words b * W * 256 + 256 i + t (i < W), each access only below its end:
// word i of the output is the XOR of the words read, its first 32-bit lane
// plus i (so that every written word depends on the reads).
__global__ __launch_bounds__(kStreamThreads) void stream_mix_kernel(const uint4* __restrict__ src,
                                                                    int64_t nsrc,
                                                                    uint4* __restrict__ dst,
                                                                    int64_t ndst, int W) {
    const int64_t br = (int64_t)blockIdx.x * kMixRun * kStreamThreads + threadIdx.x;
    uint4 a = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kMixRun; ++i) {
        const int64_t p = br + (int64_t)i * kStreamThreads;
        if (p < nsrc) {
            const uint4 v = src[p];
            a.x ^= v.x;
            a.y ^= v.y;
            a.z ^= v.z;
            a.w ^= v.w;
        }
    }
    const int64_t bw = (int64_t)blockIdx.x * W * kStreamThreads + threadIdx.x;
    for (int i = 0; i < W; ++i) {
        const int64_t p = bw + (int64_t)i * kStreamThreads;
        if (p < ndst) dst[p] = make_uint4(a.x + (uint32_t)i, a.y, a.z, a.w);
    }
}

constexpr int kCeilWaves = 16;

template <int NV>
__global__ __launch_bounds__(64 * kCeilWaves, 1) void mfma_ceiling_kernel(int rounds,
                                                                          float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    h8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(float)((lane + i) & 7);
        b[i] = (_Float16)(float)((3 * lane + i) & 7);
    }
    f4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (f4){0.f, 0.f, 0.f, 0.f};
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (float)(lane + i);
    const float c = 0.5f + (float)(lane & 1), d = 1.0f;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[i], 0, 0, 0);
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                float& r = v[(i * NV + k) & 15];
                r = __builtin_fmaf(r, c, d);
            }
        }
    }
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
#pragma unroll
    for (int i = 0; i < 16; ++i) t += v[i];
    sink[(int64_t)blockIdx.x * 64 * kCeilWaves + threadIdx.x] = t;
}

}  // namespace

int mfma_ceiling_grid() { return 256; }

hipError_t launch_mfma_ceiling(int rounds, int valu_per_mfma, float* sink, hipStream_t st) {
    const dim3 grid((unsigned)mfma_ceiling_grid()), block(64 * kCeilWaves);
    switch (valu_per_mfma) {
    case 0: hipLaunchKernelGGL(mfma_ceiling_kernel<0>, grid, block, 0, st, rounds, sink); break;
    case 2: hipLaunchKernelGGL(mfma_ceiling_kernel<2>, grid, block, 0, st, rounds, sink); break;
    default: hipLaunchKernelGGL(mfma_ceiling_kernel<4>, grid, block, 0, st, rounds, sink); break;
    }
    return hipGetLastError();
}

void stream_mix_shape(int64_t read_bytes, int64_t write_bytes, int64_t* grid, int64_t* words) {
    const int64_t nsrc = read_bytes / 16, ndst = write_bytes / 16;
    int64_t g = (nsrc + kMixRun * kStreamThreads - 1) / (kMixRun * kStreamThreads);
    if (g == 0) g = 1;
    *grid = g;
    *words = (ndst + g * kStreamThreads - 1) / (g * kStreamThreads);
}

hipError_t launch_stream_mix(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                             hipStream_t st) {
    int64_t grid, words;
    stream_mix_shape(read_bytes, write_bytes, &grid, &words);
    hipLaunchKernelGGL(stream_mix_kernel, dim3((unsigned)grid), dim3(kStreamThreads), 0, st,
                       (const uint4*)src, read_bytes / 16, (uint4*)dst, write_bytes / 16, (int)words);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t st) {
    const int64_t n16 = bytes / 16;
    const int64_t blocks = (n16 + kStreamRun - 1) / kStreamRun;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kStreamThreads), 0, st,
                       (const uint4*)src, n16, (uint32_t*)sink);
    return hipGetLastError();
}

}  // namespace lmh
