// Instances handling CB4 and CB8 projections in one launch (a layer stack and its 8-bit head).
#include "gemv_impl.h"

namespace wqd {
GemvFn gemv_fn_cb48(int M) { return gemv_fn<kMaskCB48>(M); }
}  // namespace wqd
