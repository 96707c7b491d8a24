// Fused logits of zero-point heads: the ZP instantiations of the kernels in
// logits_kernels.h (w = (n - z) * s with a per-row, per-group zero point z in
// place of the symmetric layout's fixed offset).  Compiled as a translation
// unit of its own so that it builds in parallel with logits.hip.
#include "logits_kernels.h"

namespace lmh {

hipError_t run_family_zp(int f, const LogitsArgs& a, hipStream_t st) {
    return run_family<true>(f, a, st);
}

}  // namespace lmh
