// Split-K MFMA kernel, zero-point instantiations (a translation unit of its
// own so that they compile in parallel with the symmetric ones).
#include "splitk_kernels.h"

namespace lmh {

hipError_t launch_mfma_splitk_zp(const LogitsArgs& a, hipStream_t st) { return splitk_run<true>(a, st); }

}  // namespace lmh
