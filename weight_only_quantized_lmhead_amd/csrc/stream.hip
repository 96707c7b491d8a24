// Read-only HBM stream: the practical read ceiling the logits kernels are
// measured against (a measurement aid, not part of the logits path).  Each
// workgroup reads one contiguous run of 768 16-byte words (12 KiB), one load
// per thread per step; the best of the shapes measured on MI355X for a cold
// 83 MB buffer (5.9 TB/s, against 5.3-5.7 for fewer, longer-lived
// workgroups or a grid-stride loop).
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

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t st) {
    const int64_t n16 = bytes / 16;
    const int64_t blocks = (n16 + kStreamRun - 1) / kStreamRun;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kStreamThreads), 0, st,
                       (const uint4*)src, n16, (uint32_t*)sink);
    return hipGetLastError();
}

}  // namespace lmh
