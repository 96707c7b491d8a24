// Split-K MFMA kernel (splitk_kernels.h): the symmetric instantiations and
// the launch entry point (zero-point heads go to splitk_zp.hip).
#include "splitk_kernels.h"

namespace lmh {

hipError_t launch_mfma_splitk(const LogitsArgs& a, hipStream_t st) {
    return a.zp ? launch_mfma_splitk_zp(a, st) : splitk_run<false>(a, st);
}

}  // namespace lmh
