// Q4_0 instances of the dequantize-and-multiply kernel (see gemv_impl.h).
#include "gemv_impl.h"

namespace wqd {
GemvFn gemv_fn_q4_0(int M, bool epi, bool bi) { return gemv_fn<fmt_bit(Q4_0)>(M, epi, bi); }
}  // namespace wqd
