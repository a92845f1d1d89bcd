// TQ2 instances of the dequantize-and-multiply kernel (see gemv_impl.h).
#include "gemv_impl.h"

namespace wqd {
GemvFn gemv_fn_tq2(int M, bool epi, bool bi) { return gemv_fn<fmt_bit(TQ2)>(M, epi, bi); }
}  // namespace wqd
