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
#ifndef WQD_STACK_MAX_CS
#define WQD_STACK_MAX_CS 128  // largest stack K-slice (chunks) of the vector-ALU instances
#endif
#ifndef WQD_MIN_CS
#define WQD_MIN_CS 16  // shortest K-slice (chunks) a launch is cut into
#endif
#ifndef WQD_UNITS_PER_WAVE
#define WQD_UNITS_PER_WAVE 1
#endif
#ifndef WQD_STACK_UNITS
#define WQD_STACK_UNITS 1
#endif
#ifndef WQD_NT_CODES
#define WQD_NT_CODES 1
#endif
#ifndef WQD_POOL_PERCENT
#define WQD_POOL_PERCENT 15  // share of workgroup units handed out dynamically (the tail)
#endif
#ifndef WQD_POOL_MIN_CS
#define WQD_POOL_MIN_CS 64  // smallest K-slice (chunks) of a launch that uses the dynamic tail
#endif
#ifndef WQD_WG_PER_CU
#define WQD_WG_PER_CU 2  // resident workgroups per CU of the row kernels (they are compiled for it)
#endif
// Smallest M whose codebook-format kernels multiply on the matrix cores (v_mfma_f32_4x4x4_16b_f16)
// instead of v_dot2; below it the VALU path stays (it is HBM-bound there).
#ifndef WQD_MFMA_MIN_M
#define WQD_MFMA_MIN_M 2
#endif
#ifndef WQD_MF_U
#define WQD_MF_U 4       // chunks per load group of the matrix-core instances
#endif
#ifndef WQD_MF_U_WIDE
#define WQD_MF_U_WIDE 4  // the same for CB4 at M > 4
#endif
// Launch groups whose work per resident wave is below WQD_WSPLIT_BELOW chunks use workgroup-split
// units of at least WQD_WSPLIT_MIN chunks per wave (fewer, longer units: a row group's slices
// then mostly stay inside one workgroup instead of going through memory).
#ifndef WQD_WSPLIT_BELOW
#define WQD_WSPLIT_BELOW 64
#endif
#ifndef WQD_WSPLIT_MIN
#define WQD_WSPLIT_MIN 16
#endif
#ifndef WQD_M1_MF_SHORT
#define WQD_M1_MF_SHORT 1  // M = 1 launches under WQD_WSPLIT_MIN chunks per wave use the matrix cores
#endif
#ifndef WQD_BI_CW
#define WQD_BI_CW 16   // chunks per wave of the workgroup-split slices of a batch-invariant list
#endif
#ifndef WQD_BI_CS
#define WQD_BI_CS 128  // K-slice (chunks) of a batch-invariant list when WQD_BI_CW is 0
#endif
#ifndef WQD_STACK_MF_CS
#define WQD_STACK_MF_CS 128  // largest stack K-slice (chunks) of the matrix-core instances
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
    float *part;        // split-K partials [M][S_all][Npad], or null when S_all == 1
    int *cnt;           // per row group: K-slices finished (zero between calls), or null
    int64_t ldx, ldy;
    int32_t N, K, C, C_full, S, CS, Q, RG, Npad;
    int32_t wgu_begin;  // first workgroup-unit of this projection
    int32_t wu_count;   // wave units = RG * S
    int32_t fmt;        // wqd format id of this projection
    // Epilogue and split-K slots.  Partial sums live at part[m][slot][Npad] with S_all slots per
    // activation row; this projection's K-slice s writes slot slot0 + s, and the row group is
    // done when S_all slices have arrived.  A gate/up pair (kEpiSiluPair) shares cnt, part and y:
    // gate slots [0, S_first), up slots [S_first, S_all).  S_all == 1: no split, y written directly.
    int32_t epi;        // kEpiNone, kEpiAdd or kEpiSiluPair
    int32_t slot0, S_all, S_first;
    // Workgroup split (launches too small to give every wave a long slice): a workgroup unit is
    // row group g times one K-slice of CS chunks, cut into kWaves consecutive pieces of CS/kWaves
    // chunks, one per wave, added through LDS; wu_count = RG * S * kWaves.  Otherwise a wave
    // unit is one slice of CS chunks and wu_count = RG * S.
    int32_t wsplit;
    int32_t pad_;
};

constexpr int kEpiNone = 0;      // y = x W^T
constexpr int kEpiAdd = 1;       // y += x W^T (the residual add of the o and down projections)
constexpr int kEpiSiluPair = 2;  // y = SiLU(x Wg^T) * (x Wu^T), both descriptors of a gate/up pair

// Descriptors a launch carries in its kernel arguments (a fused group of projections: q/k/v, a
// gate/up pair); larger lists use a table in device memory.
constexpr int kInlineDescs = 4;

struct GemvParams {
    Desc d[kInlineDescs]; // the descriptors when descs == nullptr
    const Desc *descs;   // device array (stack)
    int32_t ndesc;
    int32_t total_wgu;
    // first workgroup unit of each inline descriptor (d[i].wgu_begin, here too so that a
    // workgroup finds its descriptor without a load that depends on another)
    int32_t wgu_begin[kInlineDescs];
    // Dynamic tail: workgroup units [pool_begin, total_wgu) are taken one at a time from the
    // counter ctr[0] (ctr[1] counts finished workgroups; the last one resets both to 0).
    // ctr == nullptr: static assignment of every unit.
    int *ctr;
    int32_t pool_begin;
    int32_t pad_;
    // Launches from a descriptor table: the table's stamp and the fingerprint of the list this
    // launch was planned for; on a mismatch the launch exits without writing y and sets *stale.
    // stamp == nullptr: no check (descriptors in the kernel arguments).
    const uint64_t *stamp;
    uint64_t fp;
    int *stale;
};


typedef void (*GemvFn)(GemvParams);

// Format sets a kernel instance handles (bit 1 << fmt per format).
constexpr int fmt_bit(int fmt) { return 1 << fmt; }
constexpr int kMaskCB48 = (1 << CB4) | (1 << CB8);

// ------------------------------------------------------------------------------------------
// AQ2X8 (kernels of their own, on the 16-row x 32-group tile layout of layout.h).  A projection's
// (16-row block x 32-group slice) tiles are cut into a x b rectangular pieces: a row chunks of
// nrb blocks times b K-splits of ns slices.  Piece j = split * a + chunk runs on workgroup
// wb + (j mod nw) of the launch, where wb = off and nw of the projection say which workgroups
// serve it.  Wave w of a workgroup owns row blocks w, w + 16, .. (RW of them) of every piece.
// With b > 1 each piece stores fp32 partial sums per row and counts itself done on its row chunk
// (one counter per chunk, each on a 128-byte line of its own); the workgroup that arrives last
// adds the b partials in split order.
// ------------------------------------------------------------------------------------------
constexpr int kAqWaves = 16;        // waves per AQ2X8 workgroup (one workgroup per CU)
constexpr int kAqLutMaxSplits = 32; // most K-splits of a lookup-table (M = 1) projection
constexpr int kAqMmaMaxSplits = 8;  // most K-splits of a matrix-core projection
constexpr int kAqLutRW = 4;         // row blocks per wave per slice, lookup-table kernel (M = 1)
#ifndef WQD_AQ_LUT2_RW
#define WQD_AQ_LUT2_RW 2
#endif
constexpr int kAqLut2RW = WQD_AQ_LUT2_RW;  // the same at M = 2 (two rows' accumulators)
constexpr int kAqMmaRW = 2;         // row blocks per wave per slice, matrix-core kernel
constexpr int kAqCntStride = 32;    // ints between the arrival counters of two row chunks
constexpr int kAqMaxMmaM = 8;       // activation rows of one matrix-core launch
constexpr int kAqLutRecs = 64;      // most pieces per workgroup kept as LDS records, lookup-table kernel
constexpr int kAqMmaRecs = 40;      // the same, matrix-core kernel (its LDS holds the codebook copies)
#ifndef WQD_AQ_BUILD_CHARGE
#define WQD_AQ_BUILD_CHARGE 8       // planner charge of a slice's table build, in tile loads
#endif
#ifndef WQD_AQ_SPLIT_CHARGE
#define WQD_AQ_SPLIT_CHARGE 32      // planner charge of a K-split (partial round trip), in tiles
#endif

struct AqDesc {
    const uint8_t *codes;     // tile plane
    const uint16_t *rscale;   // row scales s[Npad], fp16
    const uint16_t *cbk;      // codebooks C[2][256][8], fp16
    const uint16_t *x;        // activations, M rows of ldx fp16
    float *y;                 // output, M rows of ldy fp32
    float *part;              // [M][b][Npad] partial sums when b > 1
    int *cnt;                 // arrival counter of chunk c at cnt[c * kAqCntStride] when b > 1
                              // (zero between calls)
    int64_t ldx, ldy;
    int32_t N, G, KS, RB;     // rows, groups, 32-group slices, 16-row blocks holding rows < N
    int32_t Npad;
    int32_t a, b, nrb, ns;    // pieces: a row chunks of nrb blocks x b splits of ns slices
    int32_t npieces;          // a * b
    int32_t off, nw;          // workgroups off .. off + nw - 1 (mod the launch's) serve the pieces
};

struct AqParams {
    AqDesc d0;                // the projection when descs == nullptr
    const AqDesc *descs;      // device array (stack)
    int32_t ndesc;
    int32_t nwg;              // workgroups of the launch
    const uint64_t *stamp;    // as in GemvParams
    uint64_t fp;
    int *stale;
};

typedef void (*AqFn)(AqParams);
// AQ2X8 kernel instance: the lookup-table kernel (lut: M = 1 or 2) or the matrix-core kernel for M
// activation rows (1 <= M <= 8; every batch-invariant call takes it).  rec: the form that keeps
// each workgroup's pieces as LDS records, valid when no workgroup serves more than kAqLutRecs
// (lut) or kAqMmaRecs pieces; the other form walks the descriptors.
AqFn aq_fn(int M, bool lut, bool rec);

// Kernel instances for M = 1..8 of one format, or of the CB4+CB8 pair (the layer stack with its
// 8-bit head), each defined in its own translation unit; `epi` selects the instance that applies
// epilogues (residual add, SiLU pair), `bi` the batch-invariant one (single formats only; these
// also exist for M = 9..16, a verify of up to 16 rows in one pass).
GemvFn gemv_fn_q4_0(int M, bool epi, bool bi);
GemvFn gemv_fn_cb4(int M, bool epi, bool bi);
GemvFn gemv_fn_cb8(int M, bool epi, bool bi);
GemvFn gemv_fn_tq2(int M, bool epi, bool bi);
GemvFn gemv_fn_aq1x16(int M, bool epi, bool bi);
GemvFn gemv_fn_tq2i8(int M, bool epi, bool bi);
GemvFn gemv_fn_cb48(int M, bool epi);

}  // namespace wqd
