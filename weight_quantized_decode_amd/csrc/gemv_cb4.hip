// CB4 instances of the dequantize-and-multiply kernel (see gemv_impl.h).
#include "gemv_impl.h"

namespace wqd {
GemvFn gemv_fn_cb4(int M, bool epi, bool bi) { return gemv_fn<fmt_bit(CB4)>(M, epi, bi); }
}  // namespace wqd
