// Host launch code and C entry points of libwqd, plus the split-K reduction and the debug
// dequantize kernels.  The dequantize-and-multiply kernels live in gemv_<format>.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/wqd.h"
#include "common.h"

namespace wqd {

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// y[m][n] = sum_s part[m][s][n], s ascending.  Every projection's (m, n) range starts at a
// multiple of 256 in the flattened index space, so one workgroup never straddles two
// projections and its descriptor is found with scalar loads.
__global__ __launch_bounds__(256) void reduce_kernel(RedParams P) {
    const int64_t base = (int64_t)blockIdx.x * 256;
    RedDesc D = P.d0;
    if (P.descs) {
        typedef const int64_t __attribute__((address_space(4))) *ci64p;
        int lo = 0, hi = P.ndesc - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            const int64_t b = ((ci64p)(uintptr_t)&P.descs[mid].begin)[0];
            if (b <= base) lo = mid; else hi = mid - 1;
        }
        typedef const uint32_t __attribute__((address_space(4))) *cu32;
        uint32_t w[sizeof(RedDesc) / 4];
        cu32 src = (cu32)(uintptr_t)(P.descs + lo);
#pragma unroll
        for (unsigned k = 0; k < sizeof(RedDesc) / 4; k++) w[k] = src[k];
        __builtin_memcpy(&D, w, sizeof(RedDesc));
    }
    const int64_t j = base + threadIdx.x - D.begin;
    if (j >= (int64_t)D.M * D.N) return;
    const int m = (int)(j / D.N);
    const int n = (int)(j - (int64_t)m * D.N);
    const float *p = D.part + (int64_t)m * D.S * D.Npad + n;
    float s = 0.f;
    for (int k = 0; k < D.S; k++) s += p[(int64_t)k * D.Npad];
    D.y[(int64_t)m * D.ldy + n] = s;
}

// Debug decode of the prepared layout to dense fp32, one thread per (row, chunk).
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *w, Layout L, float *out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= L.N * L.C) return;
    const int64_t n = i / L.C, c = i - n * L.C;
    const int64_t g = n / 64, r = n % 64;
    const uint4 v = *reinterpret_cast<const uint4 *>(w + ((g * L.C + c) * 64 + r) * 16);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    float *orow = out + n * L.K;
    const uint16_t *cbk = reinterpret_cast<const uint16_t *>(w + L.off_cbk);
    if constexpr (FMT == Q4_0 || FMT == TQ2) {
        const int64_t b = (FMT == Q4_0) ? c : c / 2;
        const uint16_t dh = reinterpret_cast<const uint16_t *>(w + L.off_scales)[((g * L.Q + b / 4) * 64 + r) * 4 + b % 4];
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
    } else if constexpr (FMT == AQ2X8) {
        const float s = half_bits_to_float(reinterpret_cast<const uint16_t *>(w + L.off_scales)[n]);
        for (int gi = 0; gi < 8; gi++) {
            const int64_t k0 = c * 64 + gi * 8;
            if (k0 >= L.K) break;
            const uint32_t c0 = (w4[gi / 2] >> (16 * (gi % 2))) & 0xFF;
            const uint32_t c1 = (w4[gi / 2] >> (16 * (gi % 2) + 8)) & 0xFF;
            for (int j = 0; j < 8; j++) {
                const float e0 = half_bits_to_float(cbk[(0 * 256 + c0) * 8 + j]);
                const float e1 = half_bits_to_float(cbk[(1 * 256 + c1) * 8 + j]);
                orow[k0 + j] = __fmul_rn(__fadd_rn(e0, e1), s);
            }
        }
    }
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

struct Plan {
    Layout L;
    int64_t CS = 0, S = 1;
    int64_t part_bytes = 0;  // M * S * Npad * 4 when S > 1
};

static Plan finish_plan(Plan P, int64_t M) {
    P.S = (P.L.C + P.CS - 1) / P.CS;
    P.part_bytes = (P.S > 1) ? M * P.S * P.L.Npad * 4 : 0;
    return P;
}

// One projection alone: split K until the wave units cover the GPU about 4 times.
static Plan plan_single(int fmt, int64_t N, int64_t K, int64_t M, int cus) {
    Plan P;
    P.L = make_layout(fmt, N, K);
    if (!P.L.ok) return P;
    P.CS = choose_cs(P.L, int64_t(cus) * 16 / P.L.RG, 8);
    return finish_plan(P, M);
}

// A projection inside a persistent stack launch: K-slices of about WQD_STACK_MIN_CS chunks.
static Plan plan_stack(int fmt, int64_t N, int64_t K, int64_t M) {
    Plan P;
    P.L = make_layout(fmt, N, K);
    if (!P.L.ok) return P;
    int64_t target = WQD_STACK_MIN_CS;
    int64_t splits = (P.L.C + target / 2) / target;
    P.CS = choose_cs(P.L, splits, 1);
    return finish_plan(P, M);
}

static Desc make_desc(const Plan &P, const void *w, const void *x, int64_t ldx, float *y, int64_t ldy,
                      float *part) {
    Desc D;
    memset(&D, 0, sizeof(D));
    const uint8_t *base = static_cast<const uint8_t *>(w);
    D.codes = base;
    D.scales = base + P.L.off_scales;
    D.cbk = reinterpret_cast<const uint16_t *>(base + P.L.off_cbk);
    D.x = static_cast<const uint16_t *>(x);
    D.y = y;
    D.part = part;
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
    D.wu_count = int32_t(P.L.RG * P.S);
    D.wgu_begin = 0;
    D.fmt = P.L.fmt;
    return D;
}

static GemvFn pick_gemv(int mask, int M) {
    switch (mask) {
    case 1 << Q4_0: return gemv_fn_q4_0(M);
    case 1 << CB4: return gemv_fn_cb4(M);
    case 1 << CB8: return gemv_fn_cb8(M);
    case 1 << TQ2: return gemv_fn_tq2(M);
    case 1 << AQ2X8: return gemv_fn_aq2x8(M);
    case kMaskCB48: return gemv_fn_cb48(M);
    }
    return nullptr;
}

// Resident workgroups per CU of a kernel (queried once per kernel and device).  The persistent
// grid never exceeds what is resident at once, so every workgroup starts immediately.
static int resident_per_cu(GemvFn fn) {
    struct Entry { GemvFn fn; int dev; int n; };
    static thread_local std::vector<Entry> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    for (const Entry &e : cache)
        if (e.fn == fn && e.dev == dev) return e.n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(fn), kThreads, 0) !=
            hipSuccess || n < 1)
        n = 1;
    cache.push_back({fn, dev, n});
    return n;
}

static int launch_gemv(int mask, int M, const GemvParams &GP, hipStream_t st, int cus) {
    GemvFn fn = pick_gemv(mask, M);
    if (!fn) return WQD_EINVAL;
    int64_t grid = int64_t(cus) * resident_per_cu(fn);
    if (grid > GP.total_wgu) grid = GP.total_wgu;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(fn, dim3(unsigned(grid)), dim3(kThreads), 0, st, GP);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

static int launch_reduce(const RedParams &RP, hipStream_t st) {
    if (RP.total <= 0) return WQD_OK;
    const int64_t blocks = (RP.total + 255) / 256;
    hipLaunchKernelGGL(reduce_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, RP);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

static int check_proj(int fmt, int64_t N, int64_t K, const void *w, const void *x, int64_t M,
                      int64_t ldx, const float *y, int64_t ldy) {
    if (k_multiple(fmt) == 0 || !w || !x || !y) return WQD_EINVAL;
    Layout L = make_layout(fmt, N, K);
    if (!L.ok || M < 1 || M > WQD_MAX_M || ldx < K || ldy < N) return WQD_ESHAPE;
    if ((reinterpret_cast<uintptr_t>(w) & 15) || (reinterpret_cast<uintptr_t>(x) & 3) ||
        (reinterpret_cast<uintptr_t>(y) & 3) || (ldx & 1))
        return WQD_EALIGN;
    return WQD_OK;
}

// One projection onto the stream (validated arguments).
static int gemm_one(int fmt, int64_t N, int64_t K, const void *w, const void *x, int64_t M, int64_t ldx,
                    float *y, int64_t ldy, void *ws, int64_t ws_bytes, hipStream_t st, int cus) {
    Plan P = plan_single(fmt, N, K, M, cus);
    if (P.part_bytes > 0 && (!ws || ws_bytes < P.part_bytes)) return WQD_ESPACE;
    float *part = P.part_bytes > 0 ? static_cast<float *>(ws) : nullptr;
    GemvParams GP;
    memset(&GP, 0, sizeof(GP));
    GP.d0 = make_desc(P, w, x, ldx, y, ldy, part);
    GP.descs = nullptr;
    GP.ndesc = 1;
    GP.total_wgu = int32_t((GP.d0.wu_count + kWaves - 1) / kWaves);
    int rc = launch_gemv(fmt_bit(fmt), int(M), GP, st, cus);
    if (rc != WQD_OK || P.S == 1) return rc;
    RedParams RP;
    memset(&RP, 0, sizeof(RP));
    RP.d0.part = part;
    RP.d0.y = y;
    RP.d0.ldy = ldy;
    RP.d0.N = int32_t(N);
    RP.d0.Npad = int32_t(P.L.Npad);
    RP.d0.S = int32_t(P.S);
    RP.d0.M = int32_t(M);
    RP.d0.begin = 0;
    RP.descs = nullptr;
    RP.ndesc = 1;
    RP.total = M * N;
    return launch_reduce(RP, st);
}

// Stack workspace: [Desc table][RedDesc table][partials...], each 256-byte aligned.  The
// projections are grouped into launches: all CB4/CB8 projections together when both appear,
// otherwise one launch per format; within a launch, descriptors are in format order.
struct LaunchGroup {
    int mask = 0;
    int first = 0, count = 0;  // range in StackPlan::descs
    int total_wgu = 0;
};

struct StackPlan {
    int64_t off_ctr = 0;           // 2 ints per launch group (dynamic-tail counters)
    std::vector<Desc> descs;
    std::vector<LaunchGroup> groups;
    std::vector<RedDesc> reds;
    int64_t red_total = 0;
    int64_t off_descs = 0, off_reds = 0, off_part = 0, total = 0;
    int64_t max_single_part = 0;   // for ORDERED mode
};

static int build_stack_plan(const wqd_proj *p, int32_t count, int64_t M, void *ws, StackPlan &SP, int cus) {
    if (!p || count < 1) return WQD_EINVAL;
    int present = 0;
    for (int i = 0; i < count; i++) {
        if (p[i].reserved != 0) return WQD_EINVAL;
        int rc = check_proj(p[i].fmt, p[i].N, p[i].K, p[i].w, p[i].x, M, p[i].ldx, p[i].y, p[i].ldy);
        if (rc != WQD_OK) return rc;
        present |= fmt_bit(p[i].fmt);
    }
    std::vector<int> masks;
    if ((present & kMaskCB48) == kMaskCB48) {
        masks.push_back(kMaskCB48);
        present &= ~kMaskCB48;
    }
    for (int fmt = 1; fmt <= 5; fmt++)
        if (present & fmt_bit(fmt)) masks.push_back(fmt_bit(fmt));
    SP.off_descs = 0;
    SP.off_ctr = align_up(int64_t(sizeof(Desc)) * count, 256);
    SP.off_reds = SP.off_ctr + 256;
    SP.off_part = SP.off_reds + align_up(int64_t(sizeof(RedDesc)) * count, 256);
    int64_t part_off = SP.off_part;
    uint8_t *base = static_cast<uint8_t *>(ws);
    for (int mask : masks) {
        LaunchGroup G;
        G.mask = mask;
        G.first = int(SP.descs.size());
        int wgu = 0;
        for (int fmt = 1; fmt <= 5; fmt++) {
            if (!(mask & fmt_bit(fmt))) continue;
            for (int i = 0; i < count; i++) {
                if (p[i].fmt != fmt) continue;
                Plan P = plan_stack(fmt, p[i].N, p[i].K, M);
                float *part = nullptr;
                if (P.part_bytes > 0) {
                    part = base ? reinterpret_cast<float *>(base + part_off) : nullptr;
                    RedDesc R;
                    memset(&R, 0, sizeof(R));
                    R.part = part;
                    R.y = p[i].y;
                    R.ldy = p[i].ldy;
                    R.N = int32_t(p[i].N);
                    R.Npad = int32_t(P.L.Npad);
                    R.S = int32_t(P.S);
                    R.M = int32_t(M);
                    R.begin = SP.red_total;
                    SP.red_total += align_up(M * p[i].N, 256);
                    SP.reds.push_back(R);
                    part_off += align_up(P.part_bytes, 256);
                }
                Desc D = make_desc(P, p[i].w, p[i].x, p[i].ldx, p[i].y, p[i].ldy, part);
                D.wgu_begin = wgu;
                wgu += (D.wu_count + kWaves - 1) / kWaves;
                SP.descs.push_back(D);
                Plan Q = plan_single(p[i].fmt, p[i].N, p[i].K, M, cus);
                if (Q.part_bytes > SP.max_single_part) SP.max_single_part = Q.part_bytes;
            }
        }
        G.count = int(SP.descs.size()) - G.first;
        G.total_wgu = wgu;
        SP.groups.push_back(G);
    }
    SP.total = part_off;
    if (SP.max_single_part > SP.total) SP.total = SP.max_single_part;
    return WQD_OK;
}

}  // namespace wqd

using namespace wqd;

extern "C" {

WQD_API int64_t wqd_gemm_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t M) {
    if (k_multiple(fmt) == 0) return WQD_EINVAL;
    if (M < 1 || M > WQD_MAX_M) return WQD_ESHAPE;
    Plan P = plan_single(fmt, N, K, M, device_cus());
    if (!P.L.ok) return WQD_ESHAPE;
    return P.part_bytes;
}

WQD_API int wqd_gemm(int fmt, int64_t N, int64_t K, const void *w, const void *x, int64_t M, int64_t ldx,
                     float *y, int64_t ldy, void *workspace, int64_t workspace_bytes, void *stream) {
    int rc = check_proj(fmt, N, K, w, x, M, ldx, y, ldy);
    if (rc != WQD_OK) return rc;
    return gemm_one(fmt, N, K, w, x, M, ldx, y, ldy, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream), device_cus());
}

WQD_API int wqd_dequant_f32(int fmt, int64_t N, int64_t K, const void *w, float *out, void *stream) {
    if (k_multiple(fmt) == 0 || !w || !out) return WQD_EINVAL;
    Layout L = make_layout(fmt, N, K);
    if (!L.ok) return WQD_ESHAPE;
    if (reinterpret_cast<uintptr_t>(w) & 15) return WQD_EALIGN;
    const int64_t threads = L.N * L.C;
    const unsigned blocks = unsigned((threads + 255) / 256);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    switch (fmt) {
    case Q4_0: hipLaunchKernelGGL(dequant_kernel<Q4_0>, dim3(blocks), dim3(256), 0, st, wb, L, out); break;
    case CB4: hipLaunchKernelGGL(dequant_kernel<CB4>, dim3(blocks), dim3(256), 0, st, wb, L, out); break;
    case CB8: hipLaunchKernelGGL(dequant_kernel<CB8>, dim3(blocks), dim3(256), 0, st, wb, L, out); break;
    case TQ2: hipLaunchKernelGGL(dequant_kernel<TQ2>, dim3(blocks), dim3(256), 0, st, wb, L, out); break;
    case AQ2X8: hipLaunchKernelGGL(dequant_kernel<AQ2X8>, dim3(blocks), dim3(256), 0, st, wb, L, out); break;
    }
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

WQD_API int64_t wqd_stack_workspace_bytes(const wqd_proj *projs, int32_t count, int64_t M) {
    if (M < 1 || M > WQD_MAX_M) return WQD_ESHAPE;
    StackPlan SP;
    int rc = build_stack_plan(projs, count, M, nullptr, SP, device_cus());
    if (rc != WQD_OK) return rc;
    return SP.total;
}

WQD_API int wqd_stack_setup(const wqd_proj *projs, int32_t count, int64_t M, void *workspace,
                            int64_t workspace_bytes, void *stream) {
    if (M < 1 || M > WQD_MAX_M) return WQD_ESHAPE;
    if (!workspace) return WQD_EINVAL;
    StackPlan SP;
    int rc = build_stack_plan(projs, count, M, workspace, SP, device_cus());
    if (rc != WQD_OK) return rc;
    if (workspace_bytes < SP.total) return WQD_ESPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t *base = static_cast<uint8_t *>(workspace);
    hipError_t e = hipMemcpyAsync(base + SP.off_descs, SP.descs.data(), sizeof(Desc) * SP.descs.size(),
                                  hipMemcpyHostToDevice, st);
    if (e == hipSuccess && !SP.reds.empty())
        e = hipMemcpyAsync(base + SP.off_reds, SP.reds.data(), sizeof(RedDesc) * SP.reds.size(),
                           hipMemcpyHostToDevice, st);
    static const int zeros[64] = {0};  // dynamic-tail counters start at 0 (each launch resets them)
    if (e == hipSuccess) e = hipMemcpyAsync(base + SP.off_ctr, zeros, sizeof(zeros), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

static int run_projections_impl(const wqd_proj *projs, int32_t count, int64_t M, int32_t mode,
                                void *workspace, int64_t workspace_bytes, hipStream_t st,
                                void *const *events, int32_t n_events) {
    if (M < 1 || M > WQD_MAX_M) return WQD_ESHAPE;
    if (mode != WQD_ORDERED && mode != WQD_PERSISTENT) return WQD_EINVAL;
    if (n_events < 0 || (n_events > 0 && !events)) return WQD_EINVAL;
    const int cus = device_cus();
    if (mode == WQD_ORDERED) {
        if (!projs || count < 1) return WQD_EINVAL;
        if (n_events != 0) return WQD_EINVAL;
        for (int i = 0; i < count; i++) {
            const wqd_proj &q = projs[i];
            if (q.reserved != 0) return WQD_EINVAL;
            int rc = check_proj(q.fmt, q.N, q.K, q.w, q.x, M, q.ldx, q.y, q.ldy);
            if (rc != WQD_OK) return rc;
            rc = gemm_one(q.fmt, q.N, q.K, q.w, q.x, M, q.ldx, q.y, q.ldy, workspace, workspace_bytes, st, cus);
            if (rc != WQD_OK) return rc;
        }
        return WQD_OK;
    }
    if (!workspace) return WQD_EINVAL;
    StackPlan SP;
    int rc = build_stack_plan(projs, count, M, workspace, SP, cus);
    if (rc != WQD_OK) return rc;
    if (workspace_bytes < SP.total) return WQD_ESPACE;
    const int launches = int(SP.groups.size()) + (SP.reds.empty() ? 0 : 1);
    if (n_events != 0 && n_events != 2 * launches) return WQD_ESPACE;
    int li = 0;
    auto mark = [&](int which) -> int {
        if (n_events == 0) return WQD_OK;
        hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[2 * li + which]), st);
        return e == hipSuccess ? WQD_OK : hip_fail(e);
    };
    const uint8_t *base = static_cast<const uint8_t *>(workspace);
    const Desc *dtab = reinterpret_cast<const Desc *>(base + SP.off_descs);
    for (const LaunchGroup &G : SP.groups) {
        GemvParams GP;
        memset(&GP, 0, sizeof(GP));
        GP.d0 = SP.descs[G.first];
        GP.descs = dtab + G.first;
        GP.ndesc = G.count;
        GP.total_wgu = G.total_wgu;
        if (WQD_POOL_PERCENT > 0) {
            GP.ctr = reinterpret_cast<int *>(const_cast<uint8_t *>(base) + SP.off_ctr) + 2 * (&G - SP.groups.data());
            GP.pool_begin = int32_t(int64_t(G.total_wgu) * (100 - WQD_POOL_PERCENT) / 100);
        }
        if ((rc = mark(0)) != WQD_OK) return rc;
        rc = launch_gemv(G.mask, int(M), GP, st, cus);
        if (rc != WQD_OK) return rc;
        if ((rc = mark(1)) != WQD_OK) return rc;
        li++;
    }
    if (!SP.reds.empty()) {
        RedParams RP;
        memset(&RP, 0, sizeof(RP));
        RP.d0 = SP.reds[0];
        RP.descs = reinterpret_cast<const RedDesc *>(base + SP.off_reds);
        RP.ndesc = int32_t(SP.reds.size());
        RP.total = SP.red_total;
        if ((rc = mark(0)) != WQD_OK) return rc;
        rc = launch_reduce(RP, st);
        if (rc != WQD_OK) return rc;
        if ((rc = mark(1)) != WQD_OK) return rc;
        li++;
    }
    return rc;
}

WQD_API int wqd_run_projections(const wqd_proj *projs, int32_t count, int64_t M, int32_t mode,
                                void *workspace, int64_t workspace_bytes, void *stream) {
    return run_projections_impl(projs, count, M, mode, workspace, workspace_bytes,
                                static_cast<hipStream_t>(stream), nullptr, 0);
}

WQD_API int wqd_stack_launches(const wqd_proj *projs, int32_t count, int64_t M) {
    if (M < 1 || M > WQD_MAX_M) return WQD_ESHAPE;
    StackPlan SP;
    int rc = build_stack_plan(projs, count, M, nullptr, SP, device_cus());
    if (rc != WQD_OK) return rc;
    return int(SP.groups.size()) + (SP.reds.empty() ? 0 : 1);
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
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

WQD_API int wqd_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
