// Types shared by the kernel translation units and the host launch code of libwqd.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace wqd {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef const uint32_t __attribute__((address_space(4))) *cu32p;  // scalar-loadable pointer

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kU = 4;                     // chunks per load group (double buffered)
constexpr int kTableCopies = 64;          // LDS table copies (one per lane slot)

struct Desc {
    const uint8_t *codes;
    const uint8_t *scales;
    const uint16_t *cbk;
    const uint16_t *x;
    float *y;
    float *part;        // split-K partials [M][S][Npad], or null when S == 1
    int64_t ldx, ldy;
    int32_t N, K, C, C_full, S, CS, Q, RG, Npad;
    int32_t wgu_begin;  // first workgroup-unit of this projection
    int32_t wu_count;   // wave units = RG * S
    int32_t pad_;
};

struct GemvParams {
    Desc d0;             // used when descs == nullptr
    const Desc *descs;   // device array (stack)
    int32_t ndesc;
    int32_t total_wgu;
};

struct RedDesc {
    const float *part;
    float *y;
    int64_t ldy;
    int32_t N, Npad, S, M;
    int64_t begin;       // first flattened (m, n) element
};

struct RedParams {
    RedDesc d0;
    const RedDesc *descs;
    int32_t ndesc;
    int64_t total;
};

typedef void (*GemvFn)(GemvParams);

// Kernel instances of one format for M = 1..8 (each defined in its own translation unit).
GemvFn gemv_fn_q4_0(int M);
GemvFn gemv_fn_cb4(int M);
GemvFn gemv_fn_cb8(int M);
GemvFn gemv_fn_tq2(int M);
GemvFn gemv_fn_aq2x8(int M);

}  // namespace wqd
