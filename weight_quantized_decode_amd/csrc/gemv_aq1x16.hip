// AQ1X16 instances of the dequantize-and-multiply kernel (see gemv_impl.h, aq16_chunks).
#include "gemv_impl.h"

namespace wqd {
GemvFn gemv_fn_aq1x16(int M, bool epi, bool bi) { return gemv_fn<fmt_bit(AQ1X16)>(M, epi, bi); }
}  // namespace wqd
