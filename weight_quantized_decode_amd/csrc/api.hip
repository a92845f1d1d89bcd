// Host launch code and C entry points of libwqd, plus the debug dequantize kernel.  The
// dequantize-and-multiply kernels live in gemv_<format>.hip (instances of gemv_impl.h).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/wqd.h"
#include "common.h"

namespace wqd {

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Debug decode of the prepared layout to dense fp32, one thread per (row, chunk).
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *w, const uint8_t *scales, const uint16_t *cbk,
                                                      Layout L, float *out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= L.N * L.C) return;
    const int64_t n = i / L.C, c = i - n * L.C;
    const int64_t g = n / 64, r = n % 64;
    const uint4 v = *reinterpret_cast<const uint4 *>(w + ((g * L.C + c) * 64 + r) * 16);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    float *orow = out + n * L.K;
    if constexpr (FMT == Q4_0 || FMT == TQ2) {
        const int64_t b = (FMT == Q4_0) ? c : c / 2;
        const uint16_t dh = reinterpret_cast<const uint16_t *>(scales)[((g * L.Q + b / 4) * 64 + r) * 4 + b % 4];
        const float d = half_bits_to_float(dh);
        for (int t = 0; t < 4; t++) {
            if constexpr (FMT == Q4_0) {
                for (int i2 = 0; i2 < 8; i2++) {
                    const int p = i2 / 2 + 4 * (i2 % 2);
                    const int code = (w4[t] >> (4 * p)) & 0xF;
                    orow[c * 32 + 8 * t + i2] = float(code - 8) * d;
                }
            } else {
                for (int i2 = 0; i2 < 16; i2++) {
                    const int p = i2 / 2 + 8 * (i2 % 2);
                    const int code = (w4[t] >> (2 * p)) & 3;
                    orow[c * 64 + 16 * t + i2] = float(code - 1) * d;
                }
            }
        }
    } else if constexpr (FMT == CB4) {
        for (int b = 0; b < 16; b++) {
            const uint32_t byte = (w4[b / 4] >> (8 * (b % 4))) & 0xFF;
            const int64_t k = c * 32 + 2 * b;
            if (k < L.K) orow[k] = half_bits_to_float(cbk[byte & 0xF]);
            if (k + 1 < L.K) orow[k + 1] = half_bits_to_float(cbk[byte >> 4]);
        }
    } else if constexpr (FMT == CB8) {
        for (int b = 0; b < 16; b++) {
            const uint32_t byte = (w4[b / 4] >> (8 * (b % 4))) & 0xFF;
            const int64_t k = c * 16 + b;
            if (k < L.K) orow[k] = half_bits_to_float(cbk[byte]);
        }
    }
}

// Debug decode of AQ1X16, one thread per (row, group of 8 weights): fp16 scale times fp16 entry
// (exact in fp32).
__global__ __launch_bounds__(256) void dequant_aq1x16_kernel(const uint8_t *w, const uint16_t *rscale,
                                                             const uint16_t *cbk, Layout L, float *out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= L.N * (L.K / 8)) return;
    const int64_t G = L.K / 8;
    const int64_t n = i / G, g = i - n * G;
    const int64_t g64 = n / 64, r = n % 64, c = g / 8;
    const uint16_t code = reinterpret_cast<const uint16_t *>(w + ((g64 * L.C + c) * 64 + r) * 16)[g % 8];
    const float s = half_bits_to_float(rscale[n]);
    float *o = out + n * L.K + g * 8;
    for (int j = 0; j < 8; j++) o[j] = __fmul_rn(half_bits_to_float(cbk[(int64_t)code * 8 + j]), s);
}

// Debug decode of the AQ2X8 tile layout, one thread per (row, group of 8 weights).
__global__ __launch_bounds__(256) void dequant_aq2x8_kernel(const uint8_t *w, const uint16_t *rscale,
                                                            const uint16_t *cbk, Layout L, float *out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= L.N * L.G) return;
    const int64_t n = i / L.G, g = i - n * L.G;
    const int64_t lane = ((n % 16) / 8) * 32 + g % 32;
    const uint8_t *t = w + ((g / 32 * (L.Npad / 16) + n / 16) * 64 + lane) * 16 + 2 * (n % 8);
    const uint32_t c0 = t[0], c1 = t[1];
    const float s = half_bits_to_float(rscale[n]);
    float *o = out + n * L.K + g * 8;
    for (int j = 0; j < 8; j++) {
        const float e0 = half_bits_to_float(cbk[(0 * 256 + c0) * 8 + j]);
        const float e1 = half_bits_to_float(cbk[(1 * 256 + c1) * 8 + j]);
        o[j] = __fmul_rn(__fadd_rn(e0, e1), s);
    }
}

// Int8 activations for the TQ2 int8 path: one wave per (row m, 128-element block b).  PERM = false
// stores q in natural order (the inspection entry point).  a = max|x|
// / 127 and q = x / a rounded to nearest even, both in fp32 (q = 0 when a == 0); q is stored in
// the field order of the TQ2 chunk words (layout.h): within each 16-weight word, dword j holds the
// activations of weights 2j, 2j+8, 2j+1, 2j+9.  Also writes a and the block's sum of q.
template <bool PERM>
__device__ __forceinline__ void quantize_block(const uint16_t *x, int64_t ldx, int m, int b, int nb, int8_t *q,
                                               int64_t ldq, float *a, int32_t *qs) {
    const int lane = threadIdx.x & 63;
    const uint32_t pair = *reinterpret_cast<const uint32_t *>(x + (int64_t)m * ldx + (int64_t)b * 128 + 2 * lane);
    const float x0 = half_bits_to_float(pair & 0xFFFFu), x1 = half_bits_to_float(pair >> 16);
    float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float sc = __fdiv_rn(amax, 127.0f);
    int q0 = 0, q1 = 0;
    if (sc > 0.f) {
        q0 = (int)rintf(__fdiv_rn(x0, sc));
        q1 = (int)rintf(__fdiv_rn(x1, sc));
        q0 = min(127, max(-127, q0));
        q1 = min(127, max(-127, q1));
    }
    int sum = q0 + q1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o);
    int8_t *qrow = q + (int64_t)m * ldq + (int64_t)b * 128;
    for (int e = 0; e < 2; e++) {
        const int k = 2 * lane + e;                 // element of the block
        const int base = k & ~15, i = k & 15;       // word start, weight in the word
        const int j = (i & 1) ? ((i >= 9) ? (i - 9) >> 1 : (i - 1) >> 1) : ((i >= 8) ? (i - 8) >> 1 : i >> 1);
        const int f = (i & 1) ? ((i >= 9) ? 3 : 2) : ((i >= 8) ? 1 : 0);
        qrow[PERM ? base + 4 * j + f : k] = (int8_t)(e ? q1 : q0);
    }
    if (lane == 0) {
        a[(int64_t)m * nb + b] = sc;
        qs[(int64_t)m * nb + b] = sum;
    }
}

template <bool PERM>
__global__ __launch_bounds__(256) void quantize_i8_kernel(const uint16_t *x, int64_t ldx, int M, int nb, int8_t *q,
                                                          int64_t ldq, float *a, int32_t *qs) {
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= M * nb) return;
    const int m = wv / nb, b = wv - m * nb;
    quantize_block<PERM>(x, ldx, m, b, nb, q, ldq, a, qs);
}

// Several activations quantized by one launch (the int8 activations a list segment is the first
// to read): job j takes waves [wave0, wave0 + M * nb) of the grid.
constexpr int kMaxQuantJobs = 8;
struct QuantJob {
    const uint16_t *x;
    int64_t ldx;
    int8_t *q;
    int64_t ldq;
    float *a;
    int32_t *qs;
    int32_t M, nb, wave0, pad_;
};
struct QuantJobs {
    QuantJob j[kMaxQuantJobs];
    int32_t n, waves;
};
__global__ __launch_bounds__(256) void quantize_i8_jobs_kernel(QuantJobs J) {
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= J.waves) return;
    int k = 0;
#pragma unroll
    for (int i = 1; i < kMaxQuantJobs; i++) k += (i < J.n && J.j[i].wave0 <= wv) ? 1 : 0;
    // (the job's fields by a switch on k: indexing the argument array with a variable would copy
    // it to scratch memory)
    QuantJob jb = J.j[0];
#pragma unroll
    for (int i = 1; i < kMaxQuantJobs; i++)
        if (k == i) jb = J.j[i];
    const int local = wv - jb.wave0, m = local / jb.nb, b = local - m * jb.nb;
    quantize_block<true>(jb.x, jb.ldx, m, b, jb.nb, jb.q, jb.ldq, jb.a, jb.qs);
}

// ------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------

thread_local int g_last_hip_error = 0;

static int hip_fail(hipError_t e) {
    g_last_hip_error = int(e);
    return WQD_EHIP;
}

static int device_cus() {
    static thread_local int cached_dev = -1;
    static thread_local int cached_cus = 256;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            cached_cus = cus;
        cached_dev = dev;
    }
    return cached_cus;
}

static GemvFn pick_gemv(int mask, int M, bool epi = false, bool bi = false) {
    switch (mask) {
    case 1 << Q4_0: return gemv_fn_q4_0(M, epi, bi);
    case 1 << CB4: return gemv_fn_cb4(M, epi, bi);
    case 1 << CB8: return gemv_fn_cb8(M, epi, bi);
    case 1 << TQ2: return gemv_fn_tq2(M, epi, bi);
    case 1 << AQ1X16: return gemv_fn_aq1x16(M, epi, bi);
    case 1 << TQ2I8: return gemv_fn_tq2i8(M, epi, bi);
    case kMaskCB48: return bi ? nullptr : gemv_fn_cb48(M, epi);
    }
    return nullptr;
}

// The row kernels are compiled for WQD_WG_PER_CU resident workgroups per CU (see gemv_impl.h).
static int resident_per_cu(GemvFn fn, int64_t M) { return fn ? (M > kMaxM ? 1 : WQD_WG_PER_CU) : 1; }

// Wave slots resident at once for a kernel instance (the persistent grid's capacity).
static int64_t resident_waves(int mask, int64_t M, int cus) {
    GemvFn fn = pick_gemv(mask, int(M));
    return int64_t(cus) * resident_per_cu(fn, M) * kWaves;
}

// Chunks per wave unit for a launch covering `total_cc` chunk-columns (one 1 KiB wave load
// each): about WQD_UNITS_PER_WAVE units per resident wave, between WQD_MIN_CS and the cap chunks.
static int64_t target_cs(int64_t total_cc, int64_t waves, int64_t M) {
    const int64_t cap = M >= WQD_MFMA_MIN_M ? WQD_STACK_MF_CS : WQD_STACK_MAX_CS;
    int64_t cs = total_cc / (waves * WQD_UNITS_PER_WAVE);
    if (cs < WQD_MIN_CS) cs = WQD_MIN_CS;
    if (cs > cap) cs = cap;
    return cs;
}

// Chunks per K-slice.  `splits_wanted` slices per row are asked for (at least min_cs chunks
// each); the slices are then made as equal as the format's alignment allows.
static int64_t choose_cs(const Layout &L, int64_t splits_wanted, int64_t min_cs) {
    int64_t mult = (L.fmt == TQ2) ? 8 : (L.fmt == Q4_0) ? 4 : 1;
    int64_t cap = (L.fmt == Q4_0) ? 64 : (L.fmt == TQ2) ? 128 : (int64_t(1) << 30);
    int64_t splits = splits_wanted < 1 ? 1 : splits_wanted;
    int64_t cs = (L.C + splits - 1) / splits;
    if (cs < min_cs) cs = min_cs;
    if (cs > cap) cs = cap;
    if (cs >= L.C) return L.C;  // one slice: the whole row
    const int64_t S = (L.C + cs - 1) / cs;
    cs = align_up((L.C + S - 1) / S, mult);  // equalize the slices
    if (cs > cap) cs = cap;
    return cs;
}

// Slice counters live in a region of their own that partial sums never overlap, so a
// workspace stays valid across calls of different shapes: the first kCntRegion bytes of a
// wqd_gemm workspace, or the counter region of a stack workspace.
constexpr int64_t kCntRegion = 65536;
constexpr int64_t kMaxSplitRG = kCntRegion / 4;  // row groups one split call can count

struct Plan {
    Layout L;
    int64_t CS = 0, S = 1;
    bool wsplit = false;     // workgroup-split units (CS = kWaves pieces of CS / kWaves chunks)
    bool tiny = false;       // (plan_single) under WQD_WSPLIT_MIN chunks per resident wave
    int64_t cnt_bytes = 0;   // one int per row group when S > 1 (256-byte aligned)
    int64_t part_bytes = 0;  // M * S * Npad * 4 when S > 1 (256-byte aligned)
    // wqd_gemm workspace: [kCntRegion bytes of counters][partials]
    int64_t ws_bytes() const { return S > 1 ? kCntRegion + part_bytes : 0; }
};

static Plan finish_plan(Plan P, int64_t M) {
    if (P.L.RG > kMaxSplitRG) P.CS = P.L.C;  // too many row groups to count: no split
    P.S = (P.L.C + P.CS - 1) / P.CS;
    P.cnt_bytes = (P.S > 1) ? align_up(P.L.RG * 4, 256) : 0;
    P.part_bytes = (P.S > 1) ? align_up(M * P.S * P.L.Npad * 4, 256) : 0;
    return P;
}

// A projection split into K-slices of about `cs_target` chunks (equal slices).
static Plan plan_cs(int fmt, int64_t N, int64_t K, int64_t M, int64_t cs_target) {
    Plan P;
    P.L = make_layout(fmt, N, K);
    if (!P.L.ok) return P;
    int64_t splits = (P.L.C + cs_target / 2) / cs_target;
    P.CS = choose_cs(P.L, splits, 1);
    return finish_plan(P, M);
}

// A projection in workgroup-split units of about `cw_target` chunks per wave: slices of
// kWaves * cw chunks, made as equal as the format's alignment allows.  (Falls back to plan_cs
// when the row groups are too many to count and one slice cannot cover a row.)
static Plan plan_ws(int fmt, int64_t N, int64_t K, int64_t M, int64_t cw_target) {
    Plan P;
    P.L = make_layout(fmt, N, K);
    if (!P.L.ok) return P;
    const int64_t mult = (fmt == TQ2) ? 8 : (fmt == Q4_0) ? 4 : 1;
    const int64_t cap = (fmt == Q4_0) ? 64 : (fmt == TQ2) ? 128 : (int64_t(1) << 30);
    const int64_t C = P.L.C;
    int64_t cw = align_up(cw_target < 1 ? 1 : cw_target, mult);
    if (cw > cap) cw = cap;
    int64_t S = (C + kWaves * cw - 1) / (kWaves * cw);
    if (P.L.RG > kMaxSplitRG) S = 1;
    cw = align_up((C + kWaves * S - 1) / (kWaves * S), mult);
    if (cw > cap) {
        if (P.L.RG > kMaxSplitRG) return plan_cs(fmt, N, K, M, C);
        cw = cap;
    }
    P.wsplit = true;
    P.CS = kWaves * cw;
    P.S = (C + P.CS - 1) / P.CS;
    P.cnt_bytes = (P.S > 1) ? align_up(P.L.RG * 4, 256) : 0;
    P.part_bytes = (P.S > 1) ? align_up(M * P.S * P.L.Npad * 4, 256) : 0;
    return P;
}

// K-slicing of a launch group: chunks per wave and whether units are workgroup-split.  A group
// whose work per resident wave is short splits each slice over a workgroup's waves, so all
// waves get work without cutting rows into many slices whose partial sums go through memory.
struct SliceTarget {
    int64_t cs = 0;
    bool ws = false;
    bool tiny = false;  // under WQD_WSPLIT_MIN chunks per resident wave
};
static SliceTarget slice_target(int mask, int64_t total_cc, int64_t waves, int64_t M) {
    SliceTarget t;
    const int64_t per = total_cc / waves;
    // (TQ2 slices move in 8-chunk scale quads, too coarse to share a row between 8 waves)
    if (per < WQD_WSPLIT_BELOW && !(mask & (fmt_bit(TQ2) | fmt_bit(TQ2I8)))) {
        t.ws = true;
        t.tiny = per < WQD_WSPLIT_MIN;
        t.cs = t.tiny ? WQD_WSPLIT_MIN : per;
    } else {
        t.cs = target_cs(total_cc, waves, M);
    }
    return t;
}
static Plan plan_target(int fmt, int64_t N, int64_t K, int64_t M, const SliceTarget &t) {
    return t.ws ? plan_ws(fmt, N, K, M, t.cs) : plan_cs(fmt, N, K, M, t.cs);
}

// One projection alone.
static Plan plan_single(int fmt, int64_t N, int64_t K, int64_t M, int cus) {
    Layout L = make_layout(fmt, N, K);
    if (!L.ok) {
        Plan P;
        P.L = L;
        return P;
    }
    const SliceTarget t = slice_target(fmt_bit(fmt), L.RG * L.C, resident_waves(fmt_bit(fmt), M, cus), M);
    Plan P = plan_target(fmt, N, K, M, t);
    P.tiny = t.tiny;
    return P;
}

static Desc make_desc(const Plan &P, const wqd_weight *w, const void *x, int64_t ldx, float *y, int64_t ldy,
                      float *part, int *cnt) {
    Desc D;
    memset(&D, 0, sizeof(D));
    D.codes = static_cast<const uint8_t *>(w->codes);
    D.scales = static_cast<const uint8_t *>(w->scales);
    D.cbk = static_cast<const uint16_t *>(w->codebooks);
    D.x = static_cast<const uint16_t *>(x);
    D.y = y;
    D.part = P.S > 1 ? part : nullptr;
    D.cnt = P.S > 1 ? cnt : nullptr;
    D.ldx = ldx;
    D.ldy = ldy;
    D.N = int32_t(P.L.N);
    D.K = int32_t(P.L.K);
    D.C = int32_t(P.L.C);
    D.C_full = int32_t(P.L.C_full);
    D.S = int32_t(P.S);
    D.CS = int32_t(P.CS);
    D.Q = int32_t(P.L.Q);
    D.RG = int32_t(P.L.RG);
    D.Npad = int32_t(P.L.Npad);
    D.wsplit = P.wsplit ? 1 : 0;
    D.wu_count = int32_t(P.L.RG * P.S * (P.wsplit ? kWaves : 1));
    D.wgu_begin = 0;
    D.fmt = P.L.fmt;
    D.epi = kEpiNone;
    D.slot0 = 0;
    D.S_all = int32_t(P.S);
    D.S_first = int32_t(P.S);
    return D;
}

static int launch_gemv(int mask, int M, const GemvParams &GP, hipStream_t st, int cus, bool epi = false,
                       bool bi = false) {
    GemvFn fn = pick_gemv(mask, M, epi, bi);
    if (!fn) return WQD_EINVAL;
    int64_t grid = int64_t(cus) * resident_per_cu(fn, M);
    if (grid > GP.total_wgu) grid = GP.total_wgu;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(fn, dim3(unsigned(grid)), dim3(kThreads), 0, st, GP);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

// ------------------------------------------------------------------------------------------
// AQ2X8 planning.  A projection's RB x KS tiles (16-row blocks x 32-group slices) are cut into
// a x b pieces (row chunks of nrb <= 16*RW blocks, K-splits of ns slices), dealt over the nw
// workgroups that serve the projection.  Cost model per piece, in tile loads (KiB): ns * (nrb +
// slice setup) plus a fixed charge for a K-split (its partial round trip); the shape whose
// busiest workgroup is cheapest wins.  M = 1 and 2 run the lookup-table kernel; M > 2 and every
// batch-invariant call run the matrix-core kernel.
// ------------------------------------------------------------------------------------------
static bool aq_lut(int64_t M, bool bi) { return M <= 2 && !bi; }

struct AqPlan {
    Layout L;
    bool lut = false;
    int64_t RB = 0, a = 1, b = 1, nrb = 1, ns = 1;
    int64_t cnt_bytes = 0;   // a arrival counters, kAqCntStride ints apart, when b > 1 (256-byte aligned)
    int64_t part_bytes = 0;  // M * b * Npad fp32 partials when b > 1 (256-byte aligned)
    int64_t tiles() const { return RB * L.KS; }
    // wqd_gemm workspace: [kCntRegion bytes of counters][partials]
    int64_t ws_bytes() const { return b > 1 ? kCntRegion + part_bytes : 0; }
};

static AqPlan plan_aq(int64_t N, int64_t K, int64_t M, int64_t nw, bool lut) {
    AqPlan A;
    A.L = make_layout(AQ2X8, N, K);
    if (!A.L.ok) return A;
    A.lut = lut;
    const int64_t RB = (N + 15) / 16, KS = A.L.KS;
    const int64_t per = int64_t(kAqWaves) * (lut ? (M == 1 ? kAqLutRW : kAqLut2RW) : kAqMmaRW);  // most row blocks per piece
    const int64_t bmax = lut ? kAqLutMaxSplits : kAqMmaMaxSplits;
    const int64_t setup = lut ? WQD_AQ_BUILD_CHARGE : 2;  // table build / activation staging
    if (nw < 1) nw = 1;
    double best = 1e300;
    // The matrix-core kernel's waves take the row blocks of a slice in turn and meet at a barrier
    // after each slice, so a slice costs its busiest wave: nrb rounded up to whole passes of the
    // kAqWaves waves.  It also tries row chunks of exactly one or two such passes.
    const int64_t gran = lut ? 1 : kAqWaves;
    for (int64_t b = 1; b <= KS && b <= bmax; b++) {
        const int64_t ns = (KS + b - 1) / b;
        if ((KS + ns - 1) / ns != b) continue;  // same split as a smaller b
        const int64_t cand[3] = {nw / b, (RB + kAqWaves - 1) / kAqWaves, (RB + 2 * kAqWaves - 1) / (2 * kAqWaves)};
        for (int ci = 0; ci < (lut ? 1 : 3); ci++) {
            int64_t a = cand[ci];
            if (a < (RB + per - 1) / per) a = (RB + per - 1) / per;
            if (a > RB) a = RB;
            if (a < 1) a = 1;
            const int64_t nrb = (RB + a - 1) / a;
            a = (RB + nrb - 1) / nrb;
            if (b > 1 && a * kAqCntStride * 4 > kCntRegion) continue;  // the counters fit their region
            const int64_t rounds = (a * b + nw - 1) / nw;
            const int64_t nrb_cost = (nrb + gran - 1) / gran * gran;
            const double cost =
                double(rounds) * double(ns * (nrb_cost + setup) + (b > 1 ? WQD_AQ_SPLIT_CHARGE : 0));
            if (cost < best) {
                best = cost;
                A.a = a;
                A.b = b;
                A.nrb = nrb;
                A.ns = ns;
            }
        }
    }
    A.RB = RB;
    A.cnt_bytes = A.b > 1 ? align_up(A.a * kAqCntStride * 4, 256) : 0;
    A.part_bytes = A.b > 1 ? align_up(M * A.b * A.L.Npad * 4, 256) : 0;
    return A;
}

static AqDesc make_aq_desc(const AqPlan &A, const wqd_weight *w, const void *x, int64_t ldx, float *y, int64_t ldy,
                           void *part, void *cnt, int64_t off, int64_t nw) {
    AqDesc D;
    memset(&D, 0, sizeof(D));
    D.codes = static_cast<const uint8_t *>(w->codes);
    D.rscale = static_cast<const uint16_t *>(w->scales);
    D.cbk = static_cast<const uint16_t *>(w->codebooks);
    D.x = static_cast<const uint16_t *>(x);
    D.y = y;
    D.part = A.b > 1 ? static_cast<float *>(part) : nullptr;
    D.cnt = A.b > 1 ? static_cast<int *>(cnt) : nullptr;
    D.ldx = ldx;
    D.ldy = ldy;
    D.N = int32_t(A.L.N);
    D.G = int32_t(A.L.G);
    D.KS = int32_t(A.L.KS);
    D.RB = int32_t(A.RB);
    D.Npad = int32_t(A.L.Npad);
    D.a = int32_t(A.a);
    D.b = int32_t(A.b);
    D.nrb = int32_t(A.nrb);
    D.ns = int32_t(A.ns);
    D.npieces = int32_t(A.a * A.b);
    D.off = int32_t(off);
    D.nw = int32_t(nw);
    return D;
}

// Whether the record form of the AQ2X8 kernels may run these descriptors: a bound on the pieces
// one workgroup serves (the sum over projections of ceil(npieces / nw)) within the record count.
static bool aq_rec(const AqDesc *d, int64_t n, bool lut) {
    int64_t pieces = 0;
    for (int64_t i = 0; i < n; i++) pieces += (int64_t(d[i].npieces) + d[i].nw - 1) / d[i].nw;
    return pieces <= (lut ? kAqLutRecs : kAqMmaRecs);
}

static int launch_aq(int64_t M, bool lut, bool rec, const AqParams &AP, hipStream_t st) {
    AqFn fn = aq_fn(int(M), lut, rec);
    if (!fn) return WQD_EINVAL;
    hipLaunchKernelGGL(fn, dim3(unsigned(AP.nwg)), dim3(kAqWaves * 64), 0, st, AP);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

// Workgroups of an AQ2X8 launch over projections with these plans (one per CU at most, none idle)
// and the share of each projection: the lookup-table kernel deals every projection's pieces over
// all workgroups (each starting where the previous one stopped); the matrix-core kernel gives
// each projection a contiguous range of workgroups in proportion to its tiles, so a workgroup
// loads the 16 LDS copies of one projection's codebooks once.
struct AqShare {
    int64_t off = 0, nw = 1;
};
static int64_t aq_assign(const std::vector<AqPlan> &plans, int cus, bool lut, std::vector<AqShare> &share) {
    share.assign(plans.size(), AqShare());
    int64_t pieces = 0, tiles = 0;
    for (const AqPlan &A : plans) {
        pieces += A.a * A.b;
        tiles += A.tiles();
    }
    int64_t nwg = pieces < cus ? pieces : cus;
    if (nwg < 1) nwg = 1;
    if (lut) {
        int64_t off = 0;
        for (size_t k = 0; k < plans.size(); k++) {
            share[k].off = off % nwg;
            share[k].nw = nwg;
            off += plans[k].a * plans[k].b;
        }
        return nwg;
    }
    int64_t start = 0;
    for (size_t k = 0; k < plans.size(); k++) {
        int64_t nw = tiles > 0 ? (plans[k].tiles() * nwg + tiles / 2) / tiles : 1;
        if (nw < 1) nw = 1;
        if (nw > nwg) nw = nwg;
        if (nw > plans[k].a * plans[k].b) nw = plans[k].a * plans[k].b;
        share[k].off = start % nwg;
        share[k].nw = nw;
        start += nw;
    }
    return nwg;
}

// One AQ2X8 projection alone, on a workspace of counters then partials.
static int aq_gemm_launch(int64_t N, int64_t K, const wqd_weight *w, const void *x, int64_t M, int64_t ldx, float *y,
                          int64_t ldy, uint8_t *ws, int64_t ws_bytes, hipStream_t st, int cus) {
    const bool lut = aq_lut(M, false);
    std::vector<AqPlan> plans(1, plan_aq(N, K, M, cus, lut));
    if (plans[0].ws_bytes() > 0 && (!ws || ws_bytes < plans[0].ws_bytes())) return WQD_ESPACE;
    std::vector<AqShare> share;
    const int64_t nwg = aq_assign(plans, cus, lut, share);
    AqParams AP;
    memset(&AP, 0, sizeof(AP));
    AP.d0 = make_aq_desc(plans[0], w, x, ldx, y, ldy, ws ? ws + kCntRegion : nullptr, ws, share[0].off, share[0].nw);
    AP.descs = nullptr;
    AP.ndesc = 1;
    AP.nwg = int32_t(nwg);
    return launch_aq(M, lut, aq_rec(&AP.d0, 1, lut), AP, st);
}

// Scales per row of each format's prepared scale plane (0: none) and its plane alignment.
static int64_t scale_row_elems(int fmt, int64_t K) {
    switch (fmt) {
    case Q4_0: return K / 32;
    case TQ2: return K / 128;
    case AQ2X8:
    case AQ1X16: return 1;
    default: return 0;
    }
}

// A bound weight view: known format, shape inside the limits, the planes this format reads
// present and aligned for the kernels' loads, and row sizes that agree with the shape.
static int check_weight(const wqd_weight *w) {
    if (!w || k_multiple(w->fmt) == 0) return WQD_EINVAL;
    const int fmt = w->fmt;
    Layout L = make_layout(fmt, w->N, w->K);
    if (!L.ok) return WQD_ESHAPE;
    if (w->code_row_bytes != L.row_code_bytes || w->scale_row_elems != scale_row_elems(fmt, w->K)) return WQD_ESHAPE;
    const bool has_scales = fmt == Q4_0 || fmt == TQ2 || fmt == AQ2X8 || fmt == AQ1X16;
    const bool has_cbk = fmt == CB4 || fmt == CB8 || fmt == AQ2X8 || fmt == AQ1X16;
    if (!w->codes || (has_scales && !w->scales) || (has_cbk && !w->codebooks)) return WQD_EINVAL;
    const uintptr_t c = reinterpret_cast<uintptr_t>(w->codes), sc = reinterpret_cast<uintptr_t>(w->scales),
                    cb = reinterpret_cast<uintptr_t>(w->codebooks);
    if (c & 15) return WQD_EALIGN;
    if (has_scales && (sc & ((fmt == Q4_0 || fmt == TQ2) ? 7 : 1))) return WQD_EALIGN;
    if (has_cbk && (cb & ((fmt == AQ2X8 || fmt == AQ1X16) ? 15 : 1))) return WQD_EALIGN;
    return WQD_OK;
}

static int check_proj(const wqd_weight *w, const void *x, int64_t M, int64_t ldx, const float *y, int64_t ldy,
                      int64_t mmax = WQD_MAX_M) {
    int rc = check_weight(w);
    if (rc != WQD_OK) return rc;
    if (!x || !y) return WQD_EINVAL;
    if (M < 1 || M > mmax || ldx < w->K || ldy < w->N) return WQD_ESHAPE;
    if ((reinterpret_cast<uintptr_t>(x) & 3) || (reinterpret_cast<uintptr_t>(y) & 3) || (ldx & 1)) return WQD_EALIGN;
    return WQD_OK;
}

// One projection onto the stream, with its slice counters and partials.
static int gemm_launch(const Plan &P, const wqd_weight *w, const void *x, int64_t M, int64_t ldx, float *y,
                       int64_t ldy, int *cnt, float *part, hipStream_t st, int cus) {
    GemvParams GP;
    memset(&GP, 0, sizeof(GP));
    GP.d[0] = make_desc(P, w, x, ldx, y, ldy, part, cnt);
    GP.descs = nullptr;
    GP.ndesc = 1;
    GP.total_wgu = int32_t((GP.d[0].wu_count + kWaves - 1) / kWaves);
    // the shortest M = 1 launches run the matrix-core instance, as in the list launches
    return launch_gemv(fmt_bit(P.L.fmt), int(M), GP, st, cus, false, WQD_M1_MF_SHORT && M == 1 && P.tiny);
}

// ------------------------------------------------------------------------------------------
// Projection lists.  A list is cut into segments, run one after another in stream order:
//   WQD_PERSISTENT  one segment, the whole list;
//   WQD_ORDERED     one entry per segment (a gate/up pair is one entry);
//   WQD_FUSED       runs of consecutive entries of one row format that read the same x (q/k/v,
//                   a gate/up pair), at most kInlineDescs descriptors, a pair never split.
// Within a segment the row-format projections are grouped into launches (all CB4/CB8 together
// when both appear, in WQD_PERSISTENT mode at M < WQD_MFMA_MIN_M, otherwise one launch per
// format; descriptors in format order), then one AQ2X8 launch.
//
// Workspace (the same layout in every mode): [Desc table, count entries][AqDesc table, count
// entries][launch-group counters, 256 B][slice counters][partials], each region 256-byte
// aligned.  The slice-counter region holds one counter array per entry, at least kCntRegion
// bytes; segments after the first reuse the counter and partial regions from their start (the
// launches before them have finished and left their counters at zero).
// ------------------------------------------------------------------------------------------
struct LaunchGroup {
    int mask = 0;
    int64_t cs = 0;            // K-slice target of the group (chunks)
    int first = 0, count = 0;  // range in StackPlan::descs (or StackPlan::aqdescs)
    int total_wgu = 0;
    bool aq = false;           // an AQ2X8 launch
    bool epi = false;          // some descriptor applies an epilogue
    bool bi = false;           // batch-invariant instance
    bool lut = false;          // AQ2X8: the lookup-table kernel (else the matrix-core one)
    int64_t nwg = 0;           // AQ2X8: workgroups
    int am = 0;                // AQ2X8: activation rows of the launch when not all (rows 8.. at M > 8)
    int xq = -1;               // >= 0: one int8 quantizer launch for StackPlan::xq_order[xq, xq + nxq)
    int nxq = 0;
};

// An activation quantized to int8 for the TQ2 entries of a list (WQD_INT8_ACTIVATIONS): q, the
// block scales a and the block sums of q, in the workspace at base + off_*.
struct XQ {
    const void *x = nullptr;
    int64_t ldx = 0, K = 0;
    int64_t off_q = 0, off_a = 0, off_s = 0;
    bool issued = false;       // (planning) its quantizer launch is placed
};

struct StackPlan {
    std::vector<Desc> descs;
    std::vector<AqDesc> aqdescs;
    std::vector<LaunchGroup> groups;
    std::vector<XQ> xqs;
    std::vector<int> xq_order;  // indices into xqs, in the order their quantizer launches take them
    int64_t off_stamp = 0;     // the table's stamp: fingerprint of the list setup wrote it for
    int64_t off_descs = 0, off_aqdescs = 0, off_ctr = 0, off_cnt = 0, cnt_bytes = 0, off_xq = 0, off_part = 0;
    int64_t part_bytes = 0;    // partial bytes this mode uses
    bool needs_ws = false;     // some launch counts slices (split K or a gate/up pair)
    int64_t total() const { return off_part + part_bytes; }
};

// A list entry with its weight view's format and shape copied out (views validated first).
struct Proj {
    int32_t fmt, epi;
    int64_t N, K;
    const wqd_weight *w;
    const void *x;
    int64_t ldx;
    float *y;
    int64_t ldy;
};

static int to_projs(const wqd_proj *p, int32_t count, std::vector<Proj> &out) {
    if (!p || count < 1) return WQD_EINVAL;
    out.resize(size_t(count));
    for (int i = 0; i < count; i++) {
        const int rc = check_weight(p[i].w);
        if (rc != WQD_OK) return rc;
        Proj &q = out[size_t(i)];
        q.fmt = p[i].w->fmt;
        q.epi = p[i].epi;
        q.N = p[i].w->N;
        q.K = p[i].w->K;
        q.w = p[i].w;
        q.x = p[i].x;
        q.ldx = p[i].ldx;
        q.y = p[i].y;
        q.ldy = p[i].ldy;
    }
    return WQD_OK;
}

// Entries, with the epilogue rules: a WQD_EPI_SILU_GATE entry is followed by its
// WQD_EPI_SILU_UP entry (same format and N; the pair writes the gate entry's y), and AQ2X8
// entries take no epilogue.
static int check_list(const Proj *p, int32_t count, int64_t M, int64_t mmax) {
    if (!p || count < 1) return WQD_EINVAL;
    if (M < 1 || M > mmax) return WQD_ESHAPE;
    for (int i = 0; i < count; i++) {
        const Proj &q = p[i];
        if (q.epi < WQD_EPI_NONE || q.epi > WQD_EPI_SILU_UP) return WQD_EINVAL;
        if (q.epi != WQD_EPI_NONE && q.fmt == AQ2X8) return WQD_EINVAL;
        const Proj *out = &q;
        if (q.epi == WQD_EPI_SILU_GATE) {
            if (i + 1 >= count || p[i + 1].epi != WQD_EPI_SILU_UP || p[i + 1].fmt != q.fmt || p[i + 1].N != q.N)
                return WQD_EINVAL;
        } else if (q.epi == WQD_EPI_SILU_UP) {
            if (i == 0 || p[i - 1].epi != WQD_EPI_SILU_GATE) return WQD_EINVAL;
            out = &p[i - 1];
        }
        const int rc = check_proj(q.w, q.x, M, q.ldx, out->y, out->ldy, mmax);
        if (rc != WQD_OK) return rc;
    }
    return WQD_OK;
}

static bool fuse_with(const Proj &a, const Proj &b) {
    return a.fmt == b.fmt && a.fmt != AQ2X8 && a.x == b.x && a.ldx == b.ldx;
}

static void list_segments(const Proj *p, int count, int mode, std::vector<std::pair<int, int>> &seg) {
    seg.clear();
    if (mode == WQD_PERSISTENT) {
        seg.push_back({0, count});
        return;
    }
    int i = 0;
    while (i < count) {
        int j = (p[i].epi == WQD_EPI_SILU_GATE) ? i + 2 : i + 1;
        if (mode == WQD_FUSED) {
            while (j < count && fuse_with(p[i], p[j])) {
                const int take = (p[j].epi == WQD_EPI_SILU_GATE) ? 2 : 1;
                if (j + take - i > kInlineDescs) break;
                j += take;
            }
        }
        seg.push_back({i, j});
        i = j;
    }
}

// Plans the launches of entries [b, e) onto counters from cnt_off and partials from part_off
// (offsets into the workspace at `base`, which may be null when only sizes are wanted).
// The index in SP.xqs of entry q's quantized activation (int8 lists, TQ2 entries), or -1.
static int xq_of(const StackPlan &SP, const Proj &q) {
    for (size_t k = 0; k < SP.xqs.size(); k++)
        if (SP.xqs[k].x == q.x && SP.xqs[k].ldx == q.ldx && SP.xqs[k].K == q.K) return int(k);
    return -1;
}

static void plan_segment(const Proj *p, int b, int e, int64_t M, int mode, bool bi, bool i8, uint8_t *base,
                         int64_t &cnt_off, int64_t &part_off, StackPlan &SP, int cus) {
    // kernel format of entry i: TQ2 entries of an int8 list run the int8 product
    auto kfmt = [&](int i) { return (i8 && p[i].fmt == TQ2) ? TQ2I8 : p[i].fmt; };
    // quantize the activations this segment is the first to use (after the launches before it,
    // which may have produced them), all in one launch (up to kMaxQuantJobs per launch)
    for (int i = b; i < e; i++) {
        if (kfmt(i) != TQ2I8) continue;
        const int k = xq_of(SP, p[i]);
        XQ &xq = SP.xqs[k];
        if (xq.issued) continue;
        xq.issued = true;
        if (SP.groups.empty() || SP.groups.back().xq < 0 || SP.groups.back().nxq == kMaxQuantJobs ||
            SP.groups.back().xq + SP.groups.back().nxq != int(SP.xq_order.size())) {
            LaunchGroup Q;
            Q.xq = int(SP.xq_order.size());
            SP.groups.push_back(Q);
        }
        SP.xq_order.push_back(k);
        SP.groups.back().nxq++;
    }
    int present = 0;
    for (int i = b; i < e; i++) present |= fmt_bit(kfmt(i));
    const bool has_aq = (present & fmt_bit(AQ2X8)) != 0;
    present &= ~fmt_bit(AQ2X8);
    std::vector<int> masks;
    if ((present & kMaskCB48) == kMaskCB48 && mode == WQD_PERSISTENT && M < WQD_MFMA_MIN_M && !bi) {
        masks.push_back(kMaskCB48);
        present &= ~kMaskCB48;
    }
    for (int fmt = 1; fmt <= TQ2I8; fmt++)
        if (present & fmt_bit(fmt)) masks.push_back(fmt_bit(fmt));

    for (const int mask : masks) {
        // the K-slice size of a launch group follows its total work
        int64_t total_cc = 0;
        for (int i = b; i < e; i++) {
            if (!(mask & fmt_bit(kfmt(i)))) continue;
            Layout L = make_layout(p[i].fmt, p[i].N, p[i].K);
            total_cc += L.RG * L.C;
        }
        LaunchGroup G;
        G.mask = mask;
        const SliceTarget tgt = slice_target(mask, total_cc, resident_waves(mask, M, cus), M);
        G.cs = tgt.ws ? 0 : tgt.cs;  // (the dynamic tail serves long slices only)
        // The shortest M = 1 launches run the matrix-core instance (the batch-invariant one):
        // its activation windows arrive with the code loads, where the vector-ALU instance waits
        // for scalar loads of x at the start of each of its few units.
        G.bi = bi || (WQD_M1_MF_SHORT && M == 1 && tgt.tiny && mask != kMaskCB48);
        G.first = int(SP.descs.size());
        // Batch-invariant lists cut every projection the same way whatever M and whatever else
        // is in the list (workgroup-split slices of about WQD_BI_CW chunks per wave, or wave
        // slices of WQD_BI_CS chunks when WQD_BI_CW is 0), so its sums are added in one order.
        auto plan_of = [&](int f, int64_t N, int64_t K) {
            if (f == TQ2I8) f = TQ2;  // (TQ2 weights)
            if (!bi) return plan_target(f, N, K, M, tgt);
            return WQD_BI_CW > 0 ? plan_ws(f, N, K, M, WQD_BI_CW) : plan_cs(f, N, K, M, WQD_BI_CS);
        };
        // int8 activations of a TQ2 entry: the descriptor reads q, a and the sums of q
        auto to_i8 = [&](Desc &D, const Proj &q) {
            if (D.fmt != TQ2 || !i8) return;
            const XQ &xq = SP.xqs[xq_of(SP, q)];
            D.fmt = TQ2I8;
            D.x = base ? reinterpret_cast<const uint16_t *>(base + xq.off_q) : nullptr;
            D.ldx = xq.K;
            D.cbk = base ? reinterpret_cast<const uint16_t *>(base + xq.off_a) : nullptr;
        };
        int wgu = 0;
        auto push = [&](Desc D) {
            D.wgu_begin = wgu;
            wgu += (D.wu_count + kWaves - 1) / kWaves;
            SP.descs.push_back(D);
        };
        for (int fmt = 1; fmt <= TQ2I8; fmt++) {
            if (!(mask & fmt_bit(fmt))) continue;
            for (int i = b; i < e; i++) {
                const Proj &q = p[i];
                if (kfmt(i) != fmt || q.epi == WQD_EPI_SILU_UP) continue;
                const Plan P = plan_of(fmt, q.N, q.K);
                if (q.epi == WQD_EPI_SILU_GATE) {
                    // gate and up share one slice counter per row group and one partial array
                    const Proj &r = p[i + 1];
                    const Plan U = plan_of(fmt, r.N, r.K);
                    const int64_t S_all = P.S + U.S;
                    int *cnt = base ? reinterpret_cast<int *>(base + cnt_off) : nullptr;
                    float *part = base ? reinterpret_cast<float *>(base + part_off) : nullptr;
                    cnt_off += align_up(P.L.RG * 4, 256);
                    part_off += align_up(M * S_all * P.L.Npad * 4, 256);
                    Desc Dg = make_desc(P, q.w, q.x, q.ldx, q.y, q.ldy, part, cnt);
                    Desc Du = make_desc(U, r.w, r.x, r.ldx, q.y, q.ldy, part, cnt);
                    Dg.part = Du.part = part;
                    Dg.cnt = Du.cnt = cnt;
                    Dg.epi = Du.epi = kEpiSiluPair;
                    Dg.S_all = Du.S_all = int32_t(S_all);
                    Dg.S_first = Du.S_first = int32_t(P.S);
                    Dg.slot0 = 0;
                    Du.slot0 = int32_t(P.S);
                    to_i8(Dg, q);
                    to_i8(Du, r);
                    push(Dg);
                    push(Du);
                    SP.needs_ws = true;
                } else {
                    int *cnt = base ? reinterpret_cast<int *>(base + cnt_off) : nullptr;
                    float *part = base ? reinterpret_cast<float *>(base + part_off) : nullptr;
                    cnt_off += P.cnt_bytes;
                    part_off += P.part_bytes;
                    Desc D = make_desc(P, q.w, q.x, q.ldx, q.y, q.ldy, part, cnt);
                    D.epi = (q.epi == WQD_EPI_ADD) ? kEpiAdd : kEpiNone;
                    to_i8(D, q);
                    push(D);
                    SP.needs_ws |= P.S > 1;
                }
            }
        }
        G.count = int(SP.descs.size()) - G.first;
        G.total_wgu = wgu;
        for (int k = G.first; k < G.first + G.count; k++) G.epi |= SP.descs[k].epi != kEpiNone;
        SP.groups.push_back(G);
    }
    if (has_aq) {
        // AQ2X8 projections: one launch over all of them (batch-invariant lists plan every
        // projection as if it had every CU, so the pieces do not depend on M or on the list)
        const bool lut = aq_lut(M, bi);
        LaunchGroup G;
        G.mask = fmt_bit(AQ2X8);
        G.aq = true;
        G.bi = bi;
        G.lut = lut;
        G.first = int(SP.aqdescs.size());
        std::vector<AqPlan> plans;
        std::vector<int> idx;
        for (int i = b; i < e; i++) {
            if (p[i].fmt != AQ2X8) continue;
            plans.push_back(plan_aq(p[i].N, p[i].K, M, cus, lut));
            idx.push_back(i);
        }
        std::vector<AqShare> share;
        G.nwg = aq_assign(plans, cus, lut, share);
        if (!lut && !bi) {
            // the matrix-core kernel: each projection re-planned for the workgroups it gets
            for (size_t k = 0; k < plans.size(); k++) plans[k] = plan_aq(p[idx[k]].N, p[idx[k]].K, M, share[k].nw, lut);
            G.nwg = aq_assign(plans, cus, lut, share);
        }
        for (size_t k = 0; k < plans.size(); k++) {
            const AqPlan &A = plans[k];
            const Proj &q = p[idx[k]];
            void *part = base ? static_cast<void *>(base + part_off) : nullptr;
            void *cnt = base ? static_cast<void *>(base + cnt_off) : nullptr;
            part_off += A.part_bytes;
            cnt_off += A.cnt_bytes;
            SP.needs_ws |= A.b > 1;
            SP.aqdescs.push_back(make_aq_desc(A, q.w, q.x, q.ldx, q.y, q.ldy, part, cnt, share[k].off, share[k].nw));
        }
        G.count = int(plans.size());
        if (M > kAqMaxMmaM) {
            // (a batch-invariant verify of 9..16 rows) the matrix-core kernel takes 8 rows: a
            // second launch runs rows 8.. of the same entries, with the same pieces, on the same
            // partials and counters (left at zero by the first)
            G.am = kAqMaxMmaM;
            SP.groups.push_back(G);
            LaunchGroup G2 = G;
            G2.first = int(SP.aqdescs.size());
            G2.am = int(M) - kAqMaxMmaM;
            for (int k = 0; k < G.count; k++) {
                AqDesc D = SP.aqdescs[size_t(G.first + k)];
                D.x = D.x ? D.x + kAqMaxMmaM * D.ldx : nullptr;
                D.y = D.y ? D.y + kAqMaxMmaM * D.ldy : nullptr;
                SP.aqdescs.push_back(D);
            }
            SP.groups.push_back(G2);
        } else {
            SP.groups.push_back(G);
        }
    }
}

static int build_stack_plan(const wqd_proj *pub, int32_t count, int64_t M, int mode_flags, void *ws, StackPlan &SP,
                            int cus) {
    std::vector<Proj> list;
    int rc = to_projs(pub, count, list);
    if (rc != WQD_OK) return rc;
    const Proj *p = list.data();
    const bool bi = (mode_flags & WQD_BATCH_INVARIANT) != 0;
    const bool i8 = (mode_flags & WQD_INT8_ACTIVATIONS) != 0;
    const int mode = mode_flags & ~(WQD_BATCH_INVARIANT | WQD_INT8_ACTIVATIONS);
    if (mode != WQD_ORDERED && mode != WQD_PERSISTENT && mode != WQD_FUSED) return WQD_EINVAL;
    // a batch-invariant list verifies up to WQD_MAX_M_VERIFY rows in one pass (fp16 activations)
    rc = check_list(p, count, M, bi && !i8 ? WQD_MAX_M_VERIFY : WQD_MAX_M);
    if (rc != WQD_OK) return rc;

    SP.off_stamp = 0;
    SP.off_descs = 256;
    SP.off_aqdescs = align_up(SP.off_descs + int64_t(sizeof(Desc)) * count, 256);
    // (an AQ2X8 entry of a verify of more than 8 rows has two descriptors, one per launch)
    SP.off_ctr = align_up(SP.off_aqdescs + int64_t(sizeof(AqDesc)) * count * (M > kAqMaxMmaM ? 2 : 1), 256);
    SP.off_cnt = SP.off_ctr + 256;
    int64_t cnt_all = 0;
    for (int i = 0; i < count; i++) {
        if (p[i].epi == WQD_EPI_SILU_UP) continue;
        // (an AQ2X8 plan keeps its counters within kCntRegion bytes)
        cnt_all += p[i].fmt == AQ2X8 ? kCntRegion : align_up(make_layout(p[i].fmt, p[i].N, p[i].K).RG * 4, 256);
    }
    SP.cnt_bytes = cnt_all > kCntRegion ? cnt_all : kCntRegion;
    // int8 activations: one region per distinct TQ2 activation (the same layout in every mode,
    // with or without the flag, so the workspace is one size for all)
    SP.off_xq = SP.off_cnt + SP.cnt_bytes;
    int64_t xq_off = SP.off_xq;
    for (int i = 0; i < count; i++) {
        if (p[i].fmt != TQ2 || xq_of(SP, p[i]) >= 0) continue;
        XQ xq;
        xq.x = p[i].x;
        xq.ldx = p[i].ldx;
        xq.K = p[i].K;
        xq.off_q = xq_off;
        xq.off_a = align_up(xq.off_q + M * xq.K, 256);
        xq.off_s = xq.off_a + M * (xq.K / 128) * 4;
        xq_off = align_up(xq.off_s + M * (xq.K / 128) * 4, 256);
        SP.xqs.push_back(xq);
    }
    SP.off_part = xq_off;
    std::vector<std::pair<int, int>> seg;
    list_segments(p, count, mode, seg);
    uint8_t *base = static_cast<uint8_t *>(ws);
    int64_t part_used = 0;
    for (const auto &sg : seg) {
        int64_t cnt_off = SP.off_cnt, part_off = SP.off_part;
        plan_segment(p, sg.first, sg.second, M, mode, bi, i8, base, cnt_off, part_off, SP, cus);
        if (part_off - SP.off_part > part_used) part_used = part_off - SP.off_part;
    }
    SP.part_bytes = part_used;
    if (i8 && !SP.xqs.empty()) SP.needs_ws = true;
    return WQD_OK;
}

}  // namespace wqd

using namespace wqd;

extern "C" {

static int64_t workspace_bytes(int fmt, int64_t N, int64_t K, int64_t M) {
    if (fmt == AQ2X8) {
        AqPlan A = plan_aq(N, K, M, device_cus(), aq_lut(M, false));
        if (!A.L.ok) return WQD_ESHAPE;
        return A.ws_bytes();
    }
    Plan P = plan_single(fmt, N, K, M, device_cus());
    if (!P.L.ok) return WQD_ESHAPE;
    return P.ws_bytes();
}

WQD_API int64_t wqd_workspace_bytes(const wqd_weight *w, int64_t M) {
    const int rc = check_weight(w);
    if (rc != WQD_OK) return rc;
    if (M < 1 || M > WQD_MAX_M) return WQD_ESHAPE;
    return workspace_bytes(w->fmt, w->N, w->K, M);
}

}  // extern "C"

// One projection on a caller-provided (or the file-scope scratch) workspace: the body of wqd_gemm
// and wqd_gemm_noalloc.  The arguments are checked by the caller.
static int gemm_impl(const wqd_weight *w, const void *x, int64_t M, int64_t ldx, float *y, int64_t ldy,
                     void *workspace, int64_t workspace_bytes, void *stream) {
    const int cus = device_cus();
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    if (w->fmt == AQ2X8)
        return aq_gemm_launch(w->N, w->K, w, x, M, ldx, y, ldy, ws, workspace_bytes, static_cast<hipStream_t>(stream),
                              cus);
    Plan P = plan_single(w->fmt, w->N, w->K, M, cus);
    if (P.ws_bytes() > 0 && (!workspace || workspace_bytes < P.ws_bytes())) return WQD_ESPACE;
    int *cnt = reinterpret_cast<int *>(ws);
    float *part = ws ? reinterpret_cast<float *>(ws + kCntRegion) : nullptr;
    return gemm_launch(P, w, x, M, ldx, y, ldy, cnt, part, static_cast<hipStream_t>(stream), cus);
}

// ------------------------------------------------------------------------------------------
// Scratch of wqd_gemm_noalloc: the split-K counters and partial sums of one call, in a file-scope
// device array (one copy per GPU, held until the process ends) instead of a caller workspace.
// Host code never passes the array's name to a kernel: on the host it is a stand-in symbol, not a
// device address.  The device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that pointer is used afterwards.
// ------------------------------------------------------------------------------------------
constexpr int64_t kScratchBytes = WQD_NOALLOC_MAX_BYTES;
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4 *p, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
        p[i] = make_uint4(0, 0, 0, 0);
}

static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxScratchDevices];

// Device address of the scratch array on the current device.  The first call on a device looks
// the address up and clears the array with a fill kernel on `st` (the counters must start at
// zero; every later call leaves them at zero again).
static int scratch_on_device(hipStream_t st, uint8_t **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxScratchDevices) return WQD_EINVAL;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (!p) return hip_fail(hipErrorInvalidSymbol);
        hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, st, static_cast<uint4 *>(p), kScratchBytes / 16);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<uint8_t *>(g_scratch_ptr[dev]);
    return WQD_OK;
}

// ------------------------------------------------------------------------------------------
// Descriptor tables of WQD_PERSISTENT lists.  Setup writes them with kernels whose arguments
// carry the bytes (so nothing on the host has to outlive the call and the call can be captured),
// then zeroes the counters, then writes the stamp: a fingerprint of the plan.  Every launch from
// the tables carries the fingerprint of the plan it was called with and checks the stamp first.
// ------------------------------------------------------------------------------------------
constexpr int kWriteWords = 960;  // payload dwords per writer launch (arguments stay under 4 KiB)
struct WriteChunk {
    uint32_t *dst;
    int32_t nwords;
    int32_t pad_;
    uint32_t w[kWriteWords];
};
__global__ __launch_bounds__(256) void write_words_kernel(WriteChunk c) {
    // the payload is read where it lies, in the kernel-argument segment (indexing the parameter
    // itself would copy it to scratch first)
    const cu32p src = (cu32p)((uintptr_t)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(WriteChunk, w));
    for (int i = int(threadIdx.x); i < c.nwords; i += 256) c.dst[i] = src[i];
}

static int write_bytes(uint8_t *dst, const void *src, int64_t bytes, hipStream_t st) {
    const uint8_t *s = static_cast<const uint8_t *>(src);
    for (int64_t off = 0; off < bytes; off += 4 * kWriteWords) {
        WriteChunk c;
        memset(&c, 0, sizeof(c));
        const int64_t n = bytes - off < 4 * kWriteWords ? bytes - off : 4 * kWriteWords;
        c.dst = reinterpret_cast<uint32_t *>(dst + off);
        c.nwords = int32_t((n + 3) / 4);
        memcpy(c.w, s + off, size_t(n));
        hipLaunchKernelGGL(write_words_kernel, dim3(1), dim3(256), 0, st, c);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    return WQD_OK;
}

// Fingerprint of a plan: its descriptors (every pointer, shape and piece assignment), the mode
// and M.  Never 0 (a zero-filled workspace holds no table).
static uint64_t plan_fingerprint(const StackPlan &SP, int64_t M, int32_t mode) {
    uint64_t h = 0x243F6A8885A308D3ull ^ uint64_t(M) ^ (uint64_t(uint32_t(mode)) << 32);
    auto mix = [&](const void *p, size_t n) {
        const uint8_t *b = static_cast<const uint8_t *>(p);
        for (size_t i = 0; i + 8 <= n; i += 8) {
            uint64_t w;
            memcpy(&w, b + i, 8);
            h = (h ^ w) * 0x9E3779B97F4A7C15ull;
            h ^= h >> 29;
        }
        for (size_t i = n & ~size_t(7); i < n; i++) h = (h ^ b[i]) * 0x100000001B3ull;
        h = (h ^ uint64_t(n)) * 0x9E3779B97F4A7C15ull;
    };
    mix(SP.descs.data(), sizeof(Desc) * SP.descs.size());
    mix(SP.aqdescs.data(), sizeof(AqDesc) * SP.aqdescs.size());
    return h | 1;
}

// The per-device flag a launch raises when it finds a stale table (a file-scope device variable;
// its device address comes from hipGetSymbolAddress, once per device with the device current).
static __device__ int stale_flag;
static std::mutex g_flag_mu;
static void *g_flag_ptr[kMaxScratchDevices];
static int flag_on_device(int **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxScratchDevices) return WQD_EINVAL;
    std::lock_guard<std::mutex> lock(g_flag_mu);
    if (!g_flag_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(stale_flag));
        if (e != hipSuccess) return hip_fail(e);
        if (!p) return hip_fail(hipErrorInvalidSymbol);
        g_flag_ptr[dev] = p;
    }
    *out = static_cast<int *>(g_flag_ptr[dev]);
    return WQD_OK;
}

extern "C" {

WQD_API int wqd_gemm(const wqd_weight *w, const void *x, int64_t M, int64_t ldx, float *y, int64_t ldy, void *workspace,
                     int64_t workspace_bytes, void *stream) {
    int rc = check_proj(w, x, M, ldx, y, ldy);
    if (rc != WQD_OK) return rc;
    return gemm_impl(w, x, M, ldx, y, ldy, workspace, workspace_bytes, stream);
}

WQD_API int wqd_gemm_noalloc(const wqd_weight *w, const void *x, int64_t M, int64_t ldx, float *y, int64_t ldy,
                             void *stream) {
    int rc = check_proj(w, x, M, ldx, y, ldy);
    if (rc != WQD_OK) return rc;
    const int64_t need = workspace_bytes(w->fmt, w->N, w->K, M);
    if (need < 0) return int(need);
    if (need > kScratchBytes) return WQD_ESPACE;
    uint8_t *ws = nullptr;
    if (need > 0) {
        rc = scratch_on_device(static_cast<hipStream_t>(stream), &ws);
        if (rc != WQD_OK) return rc;
    }
    return gemm_impl(w, x, M, ldx, y, ldy, ws, need > 0 ? kScratchBytes : 0, stream);
}

// Workspace of wqd_gemm_i8: [wqd_gemm's counters and partials][q: M x K bytes][a: M x K/128 fp32]
// [sums of q: M x K/128 int32], each region 256-byte aligned.
struct I8Ws {
    int64_t off_q = 0, off_a = 0, off_s = 0, total = 0;
};
static I8Ws i8_workspace(const Plan &P, int64_t M, int64_t K) {
    I8Ws w;
    w.off_q = align_up(P.ws_bytes(), 256);
    w.off_a = align_up(w.off_q + M * K, 256);
    w.off_s = w.off_a + M * (K / 128) * 4;
    w.total = align_up(w.off_s + M * (K / 128) * 4, 256);
    return w;
}

WQD_API int64_t wqd_gemm_i8_workspace_bytes(const wqd_weight *w, int64_t M) {
    const int rc = check_weight(w);
    if (rc != WQD_OK) return rc;
    if (w->fmt != TQ2) return WQD_EINVAL;
    if (M < 1 || M > WQD_MAX_M) return WQD_ESHAPE;
    Plan P = plan_single(TQ2, w->N, w->K, M, device_cus());
    return i8_workspace(P, M, w->K).total;
}

WQD_API int wqd_gemm_i8(const wqd_weight *w, const void *x, int64_t M, int64_t ldx, float *y, int64_t ldy,
                        void *workspace, int64_t workspace_bytes, void *stream) {
    int rc = check_proj(w, x, M, ldx, y, ldy);
    if (rc != WQD_OK) return rc;
    if (w->fmt != TQ2) return WQD_EINVAL;
    const int64_t N = w->N, K = w->K;
    const int cus = device_cus();
    Plan P = plan_single(TQ2, N, K, M, cus);
    const I8Ws iw = i8_workspace(P, M, K);
    if (!workspace) return WQD_EINVAL;
    if (workspace_bytes < iw.total) return WQD_ESPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return WQD_EALIGN;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int8_t *q = reinterpret_cast<int8_t *>(ws + iw.off_q);
    float *a = reinterpret_cast<float *>(ws + iw.off_a);
    int32_t *qs = reinterpret_cast<int32_t *>(ws + iw.off_s);
    const int nb = int(K / 128);
    const unsigned blocks = unsigned((M * nb + 3) / 4);
    hipLaunchKernelGGL(quantize_i8_kernel<true>, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t *>(x), ldx,
                       int(M), nb, q, K, a, qs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
    GemvParams GP;
    memset(&GP, 0, sizeof(GP));
    GP.d[0] = make_desc(P, w, q, K, y, ldy, P.S > 1 ? reinterpret_cast<float *>(ws + kCntRegion) : nullptr,
                        reinterpret_cast<int *>(ws));
    GP.d[0].fmt = TQ2I8;
    GP.d[0].cbk = reinterpret_cast<const uint16_t *>(a);  // activation scales, then the sums of q
    GP.descs = nullptr;
    GP.ndesc = 1;
    GP.total_wgu = int32_t((GP.d[0].wu_count + kWaves - 1) / kWaves);
    return launch_gemv(fmt_bit(TQ2I8), int(M), GP, st, cus);
}

WQD_API int wqd_quantize_i8(const void *x, int64_t M, int64_t K, int64_t ldx, int8_t *q, float *a, int32_t *qsum,
                            void *stream) {
    if (!x || !q || !a || !qsum) return WQD_EINVAL;
    if (M < 1 || M > WQD_MAX_M || K < 128 || K % 128 || ldx < K || K > kMaxK) return WQD_ESHAPE;
    if ((reinterpret_cast<uintptr_t>(x) & 3) || (ldx & 1) || (reinterpret_cast<uintptr_t>(a) & 3) ||
        (reinterpret_cast<uintptr_t>(qsum) & 3))
        return WQD_EALIGN;
    const int nb = int(K / 128);
    hipLaunchKernelGGL(quantize_i8_kernel<false>, dim3(unsigned((M * nb + 3) / 4)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t *>(x), ldx, int(M), nb, q, K, a,
                       qsum);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

WQD_API int wqd_dequant_f32(const wqd_weight *w, float *out, void *stream) {
    int rc = check_weight(w);
    if (rc != WQD_OK) return rc;
    if (!out) return WQD_EINVAL;
    const int fmt = w->fmt;
    Layout L = make_layout(fmt, w->N, w->K);
    const int64_t threads = (fmt == AQ2X8) ? L.N * L.G : (fmt == AQ1X16) ? L.N * (L.K / 8) : L.N * L.C;
    const unsigned blocks = unsigned((threads + 255) / 256);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint8_t *wc = static_cast<const uint8_t *>(w->codes);
    const uint8_t *sc = static_cast<const uint8_t *>(w->scales);
    const uint16_t *cb = static_cast<const uint16_t *>(w->codebooks);
    const uint16_t *rs = static_cast<const uint16_t *>(w->scales);
    switch (fmt) {
    case Q4_0: hipLaunchKernelGGL(dequant_kernel<Q4_0>, dim3(blocks), dim3(256), 0, st, wc, sc, cb, L, out); break;
    case CB4: hipLaunchKernelGGL(dequant_kernel<CB4>, dim3(blocks), dim3(256), 0, st, wc, sc, cb, L, out); break;
    case CB8: hipLaunchKernelGGL(dequant_kernel<CB8>, dim3(blocks), dim3(256), 0, st, wc, sc, cb, L, out); break;
    case TQ2: hipLaunchKernelGGL(dequant_kernel<TQ2>, dim3(blocks), dim3(256), 0, st, wc, sc, cb, L, out); break;
    case AQ2X8: hipLaunchKernelGGL(dequant_aq2x8_kernel, dim3(blocks), dim3(256), 0, st, wc, rs, cb, L, out); break;
    case AQ1X16: hipLaunchKernelGGL(dequant_aq1x16_kernel, dim3(blocks), dim3(256), 0, st, wc, rs, cb, L, out); break;
    }
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

WQD_API int64_t wqd_stack_workspace_bytes(const wqd_proj *projs, int32_t count, int64_t M) {
    // enough for every mode
    int64_t need = 0;
    if (M > WQD_MAX_M) {  // batch-invariant lists only
        for (int mode : {WQD_ORDERED, WQD_PERSISTENT, WQD_FUSED}) {
            StackPlan SB;
            const int rc = build_stack_plan(projs, count, M, mode | WQD_BATCH_INVARIANT, nullptr, SB, device_cus());
            if (rc != WQD_OK) return rc;
            if (SB.total() > need) need = SB.total();
        }
        return need;
    }
    for (int mode : {WQD_ORDERED, WQD_PERSISTENT, WQD_FUSED}) {
        StackPlan SP;
        int rc = build_stack_plan(projs, count, M, mode, nullptr, SP, device_cus());
        if (rc != WQD_OK) return rc;
        if (SP.total() > need) need = SP.total();
        // the batch-invariant plans too (the int8 flag changes no region's size)
        StackPlan SB;
        if (build_stack_plan(projs, count, M, mode | WQD_BATCH_INVARIANT, nullptr, SB, device_cus()) == WQD_OK &&
            SB.total() > need)
            need = SB.total();
    }
    return need;
}

WQD_API int wqd_stack_setup(const wqd_proj *projs, int32_t count, int64_t M, int32_t mode, void *workspace,
                            int64_t workspace_bytes, void *stream) {
    if (!workspace) return WQD_EINVAL;
    if ((mode & ~(WQD_BATCH_INVARIANT | WQD_INT8_ACTIVATIONS)) != WQD_PERSISTENT) return WQD_EINVAL;
    StackPlan SP;
    int rc = build_stack_plan(projs, count, M, mode, workspace, SP, device_cus());
    if (rc != WQD_OK) return rc;
    if (workspace_bytes < SP.total()) return WQD_ESPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t *base = static_cast<uint8_t *>(workspace);
    if (!SP.descs.empty() && (rc = write_bytes(base + SP.off_descs, SP.descs.data(), int64_t(sizeof(Desc) * SP.descs.size()), st)) != WQD_OK)
        return rc;
    if (!SP.aqdescs.empty() &&
        (rc = write_bytes(base + SP.off_aqdescs, SP.aqdescs.data(), int64_t(sizeof(AqDesc) * SP.aqdescs.size()), st)) != WQD_OK)
        return rc;
    // launch-group and slice counters start at 0; every launch leaves them at 0 again
    hipLaunchKernelGGL(zero_fill_kernel, dim3(256), dim3(256), 0, st, reinterpret_cast<uint4 *>(base + SP.off_ctr),
                       (SP.off_part - SP.off_ctr) / 16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
    const uint64_t fp = plan_fingerprint(SP, M, mode);  // last: the tables are complete before it
    return write_bytes(base + SP.off_stamp, &fp, 8, st);
}

static int run_projections_impl(const wqd_proj *projs, int32_t count, int64_t M, int32_t mode,
                                void *workspace, int64_t workspace_bytes, hipStream_t st,
                                void *const *events, int32_t n_events) {
    if (n_events < 0 || (n_events > 0 && !events)) return WQD_EINVAL;
    const int cus = device_cus();
    StackPlan SP;
    int rc = build_stack_plan(projs, count, M, mode, workspace, SP, cus);
    if (rc != WQD_OK) return rc;
    uint8_t *base = static_cast<uint8_t *>(workspace);
    // WQD_PERSISTENT reads the descriptor tables wqd_stack_setup wrote; the other modes pass
    // their descriptors in the kernel arguments and need the workspace only to count slices.
    const bool persistent = (mode & ~(WQD_BATCH_INVARIANT | WQD_INT8_ACTIVATIONS)) == WQD_PERSISTENT;
    if (persistent && !base) return WQD_EINVAL;
    if ((persistent || SP.needs_ws) && (!base || workspace_bytes < SP.total())) return WQD_ESPACE;
    const int launches = int(SP.groups.size());
    if (n_events != 0 && n_events != 2 * launches) return WQD_ESPACE;
    int li = 0;
    auto mark = [&](int which) -> int {
        if (n_events == 0) return WQD_OK;
        hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[2 * li + which]), st);
        return e == hipSuccess ? WQD_OK : hip_fail(e);
    };
    const bool table = persistent;
    const Desc *dtab = table ? reinterpret_cast<const Desc *>(base + SP.off_descs) : nullptr;
    const AqDesc *atab = table ? reinterpret_cast<const AqDesc *>(base + SP.off_aqdescs) : nullptr;
    // launches from the tables check them against this list
    const uint64_t *stamp = table ? reinterpret_cast<const uint64_t *>(base + SP.off_stamp) : nullptr;
    const uint64_t fp = table ? plan_fingerprint(SP, M, mode) : 0;
    int *stale = nullptr;
    if (table && (rc = flag_on_device(&stale)) != WQD_OK) return rc;
    for (size_t gi = 0; gi < SP.groups.size(); gi++) {
        const LaunchGroup &G = SP.groups[gi];
        if (G.xq >= 0) {
            QuantJobs J;
            memset(&J, 0, sizeof(J));
            for (int t = 0; t < G.nxq; t++) {
                const XQ &xq = SP.xqs[SP.xq_order[size_t(G.xq + t)]];
                QuantJob &jb = J.j[t];
                jb.x = static_cast<const uint16_t *>(xq.x);
                jb.ldx = xq.ldx;
                jb.q = reinterpret_cast<int8_t *>(base + xq.off_q);
                jb.ldq = xq.K;
                jb.a = reinterpret_cast<float *>(base + xq.off_a);
                jb.qs = reinterpret_cast<int32_t *>(base + xq.off_s);
                jb.M = int32_t(M);
                jb.nb = int32_t(xq.K / 128);
                jb.wave0 = J.waves;
                J.waves += jb.M * jb.nb;
            }
            J.n = G.nxq;
            if ((rc = mark(0)) != WQD_OK) return rc;
            hipLaunchKernelGGL(quantize_i8_jobs_kernel, dim3(unsigned((J.waves + 3) / 4)), dim3(256), 0, st, J);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return hip_fail(e);
            if ((rc = mark(1)) != WQD_OK) return rc;
            li++;
            continue;
        }
        if (G.aq) {
            AqParams AP;
            memset(&AP, 0, sizeof(AP));
            AP.d0 = SP.aqdescs[G.first];
            AP.descs = table ? atab + G.first : nullptr;
            AP.ndesc = G.count;
            AP.nwg = int32_t(G.nwg);
            AP.stamp = stamp;
            AP.fp = fp;
            AP.stale = stale;
            if (!table && G.count != 1) return WQD_EINVAL;  // (segments hold one AQ2X8 entry)
            if ((rc = mark(0)) != WQD_OK) return rc;
            rc = launch_aq(G.am ? G.am : M, G.lut, aq_rec(&SP.aqdescs[G.first], G.count, G.lut), AP, st);
            if (rc != WQD_OK) return rc;
            if ((rc = mark(1)) != WQD_OK) return rc;
            li++;
            continue;
        }
        GemvParams GP;
        memset(&GP, 0, sizeof(GP));
        if (table) {
            GP.descs = dtab + G.first;
        } else {
            if (G.count > kInlineDescs) return WQD_EINVAL;  // (segments are cut to fit)
            for (int k = 0; k < G.count; k++) {
                GP.d[k] = SP.descs[G.first + k];
                GP.wgu_begin[k] = GP.d[k].wgu_begin;
            }
            GP.descs = nullptr;
        }
        GP.ndesc = G.count;
        GP.total_wgu = G.total_wgu;
        GP.stamp = stamp;
        GP.fp = fp;
        GP.stale = stale;
        // The dynamic tail pays a barrier, an atomic and a cold load pipeline per unit it hands
        // out: only units of long slices amortize that.  (Launches run one after another, and
        // each leaves its two counters at zero, so they share them.)
        if (WQD_POOL_PERCENT > 0 && G.cs >= WQD_POOL_MIN_CS && base) {
            GP.ctr = reinterpret_cast<int *>(base + SP.off_ctr);
            GP.pool_begin = int32_t(int64_t(G.total_wgu) * (100 - WQD_POOL_PERCENT) / 100);
        }
        if ((rc = mark(0)) != WQD_OK) return rc;
        rc = launch_gemv(G.mask, int(M), GP, st, cus, G.epi, G.bi);
        if (rc != WQD_OK) return rc;
        if ((rc = mark(1)) != WQD_OK) return rc;
        li++;
    }
    return WQD_OK;
}

WQD_API int wqd_run_projections(const wqd_proj *projs, int32_t count, int64_t M, int32_t mode,
                                void *workspace, int64_t workspace_bytes, void *stream) {
    return run_projections_impl(projs, count, M, mode, workspace, workspace_bytes,
                                static_cast<hipStream_t>(stream), nullptr, 0);
}

WQD_API int wqd_stack_launches(const wqd_proj *projs, int32_t count, int64_t M, int32_t mode) {
    StackPlan SP;
    int rc = build_stack_plan(projs, count, M, mode, nullptr, SP, device_cus());
    if (rc != WQD_OK) return rc;
    return int(SP.groups.size());
}

WQD_API int wqd_run_projections_timed(const wqd_proj *projs, int32_t count, int64_t M, int32_t mode,
                                      void *workspace, int64_t workspace_bytes, void *stream,
                                      void *const *events, int32_t n_events) {
    return run_projections_impl(projs, count, M, mode, workspace, workspace_bytes,
                                static_cast<hipStream_t>(stream), events, n_events);
}

WQD_API int wqd_stream_check(void *stream) {
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
    int *flag = nullptr;
    int rc = flag_on_device(&flag);
    if (rc != WQD_OK) return rc;
    int v = 0;
    e = hipMemcpy(&v, flag, sizeof(v), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e);
    if (v == 0) return WQD_OK;
    const int zero = 0;
    e = hipMemcpy(flag, &zero, sizeof(zero), hipMemcpyHostToDevice);
    return e == hipSuccess ? WQD_ESTALE : hip_fail(e);
}

WQD_API int wqd_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
