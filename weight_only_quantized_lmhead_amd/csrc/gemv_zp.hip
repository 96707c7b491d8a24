// Lane-per-row GEMV (gemv_kernels.h) for zero-point heads.
#include "gemv_kernels.h"

namespace lmh {

hipError_t launch_gemv_zp(const LogitsArgs& a, hipStream_t st) { return gemv_run<true>(a, st); }

}  // namespace lmh
