// Instances handling CB4 and CB8 projections in one launch (a layer stack and its 8-bit head),
// for the vector-ALU instances only (M < WQD_MFMA_MIN_M).  Inlined together, the two matrix-core
// bodies need about 150 VGPRs against 97 for either alone, which would halve the waves per CU;
// at those M the stack runs one launch per format instead.
#include "gemv_impl.h"

namespace wqd {
GemvFn gemv_fn_cb48(int M, bool epi) {
    switch (M) {
    case 1: return epi ? gemv_kernel<kMaskCB48, 1, true> : gemv_kernel<kMaskCB48, 1, false>;
#if WQD_MFMA_MIN_M > 2
    case 2: return epi ? gemv_kernel<kMaskCB48, 2, true> : gemv_kernel<kMaskCB48, 2, false>;
#endif
    }
    static_assert(WQD_MFMA_MIN_M >= 2 && WQD_MFMA_MIN_M <= 3, "instances listed for M < WQD_MFMA_MIN_M");
    return nullptr;
}
}  // namespace wqd
