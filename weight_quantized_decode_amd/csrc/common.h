// Types shared by the kernel translation units and the host launch code of libwqd.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace wqd {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef const uint32_t __attribute__((address_space(4))) *cu32p;  // scalar-loadable pointer

#ifndef WQD_WAVES
#define WQD_WAVES 8
#endif
#ifndef WQD_U
#define WQD_U 4
#endif
#ifndef WQD_TABLE_COPIES
#define WQD_TABLE_COPIES 64
#endif
#ifndef WQD_STACK_MIN_CS
#define WQD_STACK_MIN_CS 64
#endif
#ifndef WQD_UNITS_PER_WAVE
#define WQD_UNITS_PER_WAVE 4
#endif
#ifndef WQD_STACK_UNITS
#define WQD_STACK_UNITS 1
#endif
#ifndef WQD_NT_CODES
#define WQD_NT_CODES 1
#endif
#ifndef WQD_POOL_PERCENT
#define WQD_POOL_PERCENT 0
#endif
#ifndef WQD_WG_PER_CU
#define WQD_WG_PER_CU 2
#endif
constexpr int kMaxM = 8;                  // largest M (activation rows) per call
constexpr int kWaves = WQD_WAVES;         // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kU = WQD_U;                 // chunks per load group (double buffered)
constexpr int kTableCopies = WQD_TABLE_COPIES;  // LDS table copies (one per lane slot)

struct Desc {
    const uint8_t *codes;
    const uint8_t *scales;
    const uint16_t *cbk;
    const uint16_t *x;
    float *y;
    float *part;        // split-K partials [M][S][Npad], or null when S == 1
    int *cnt;           // per row group: K-slices finished (zero between calls), or null
    int64_t ldx, ldy;
    int32_t N, K, C, C_full, S, CS, Q, RG, Npad;
    int32_t wgu_begin;  // first workgroup-unit of this projection
    int32_t wu_count;   // wave units = RG * S
    int32_t fmt;        // wqd format id of this projection
};

struct GemvParams {
    Desc d0;             // used when descs == nullptr
    const Desc *descs;   // device array (stack)
    int32_t ndesc;
    int32_t total_wgu;
    // Dynamic tail: workgroup units [pool_begin, total_wgu) are taken one at a time from the
    // counter ctr[0] (ctr[1] counts finished workgroups; the last one resets both to 0).
    // ctr == nullptr: static assignment of every unit.
    int *ctr;
    int32_t pool_begin;
    int32_t pad_;
};


typedef void (*GemvFn)(GemvParams);

// Format sets a kernel instance handles (bit 1 << fmt per format).
constexpr int fmt_bit(int fmt) { return 1 << fmt; }
constexpr int kMaskCB48 = (1 << CB4) | (1 << CB8);

// Kernel instances for M = 1..8 of one format, or of the CB4+CB8 pair (the layer stack with its
// 8-bit head), each defined in its own translation unit.
GemvFn gemv_fn_q4_0(int M);
GemvFn gemv_fn_cb4(int M);
GemvFn gemv_fn_cb8(int M);
GemvFn gemv_fn_tq2(int M);
GemvFn gemv_fn_aq2x8(int M);
GemvFn gemv_fn_cb48(int M);

}  // namespace wqd
