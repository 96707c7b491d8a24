// Lane-per-row GEMV (gemv_kernels.h), symmetric heads; zero-point heads are
// instantiated in gemv_zp.hip (a translation unit of its own, compiled in
// parallel).
#include "gemv_kernels.h"

namespace lmh {

hipError_t launch_gemv(const LogitsArgs& a, hipStream_t st) {
    return a.zp ? launch_gemv_zp(a, st) : gemv_run<false>(a, st);
}

}  // namespace lmh
