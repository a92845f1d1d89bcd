// Instances of the dequantize-and-multiply kernel for TQ2 weights times int8 activations (see
// gemv_impl.h, tq2i8_chunks).
#include "gemv_impl.h"

namespace wqd {
GemvFn gemv_fn_tq2i8(int M, bool epi, bool bi) { return gemv_fn<fmt_bit(TQ2I8), false>(M, epi, bi); }
}  // namespace wqd
