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

// y[m][n] = sum_s part[m][s][n], s ascending.
__global__ __launch_bounds__(256) void reduce_kernel(RedParams P) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= P.total) return;
    RedDesc D = P.d0;
    if (P.descs) {
        int lo = 0, hi = P.ndesc - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (P.descs[mid].begin <= i) lo = mid; else hi = mid - 1;
        }
        D = P.descs[lo];
    }
    const int64_t j = i - D.begin;
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

static bool has_table(int fmt) { return fmt == CB4 || fmt == CB8 || fmt == AQ2X8; }

// Chunks per split for a single projection: enough wave units to cover the GPU.
static int64_t choose_cs(const Layout &L, int64_t target_units, int64_t min_cs) {
    int64_t splits = target_units / L.RG;
    if (splits < 1) splits = 1;
    int64_t cs = (L.C + splits - 1) / splits;
    if (cs < min_cs) cs = min_cs;
    int64_t mult = (L.fmt == TQ2) ? 8 : 4;
    cs = align_up(cs, mult);
    int64_t cap = (L.fmt == Q4_0) ? 64 : (L.fmt == TQ2) ? 128 : (int64_t(1) << 30);
    if (cs > cap) cs = cap;
    if (cs >= L.C) cs = L.C;  // one split: the whole row
    return cs;
}

struct Plan {
    Layout L;
    int64_t CS = 0, S = 1;
    int64_t part_bytes = 0;  // M * S * Npad * 4 when S > 1
};

static Plan plan_single(int fmt, int64_t N, int64_t K, int64_t M, int cus) {
    Plan P;
    P.L = make_layout(fmt, N, K);
    if (!P.L.ok) return P;
    P.CS = choose_cs(P.L, int64_t(cus) * 16, 8);
    P.S = (P.L.C + P.CS - 1) / P.CS;
    P.part_bytes = (P.S > 1) ? M * P.S * P.L.Npad * 4 : 0;
    return P;
}

static Plan plan_stack(int fmt, int64_t N, int64_t K, int64_t M) {
    Plan P;
    P.L = make_layout(fmt, N, K);
    if (!P.L.ok) return P;
    P.CS = choose_cs(P.L, 1, 32);  // about 32 KiB of codes per wave unit
    P.S = (P.L.C + P.CS - 1) / P.CS;
    P.part_bytes = (P.S > 1) ? M * P.S * P.L.Npad * 4 : 0;
    return P;
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
    return D;
}

static GemvFn pick_gemv(int fmt, int M) {
    switch (fmt) {
    case Q4_0: return gemv_fn_q4_0(M);
    case CB4: return gemv_fn_cb4(M);
    case CB8: return gemv_fn_cb8(M);
    case TQ2: return gemv_fn_tq2(M);
    case AQ2X8: return gemv_fn_aq2x8(M);
    }
    return nullptr;
}

static int grid_for(int fmt, int64_t total_wgu, int cus) {
    int64_t per_cu = has_table(fmt) ? (fmt == AQ2X8 ? 4 : 2) : 4;
    int64_t g = int64_t(cus) * per_cu;
    if (g > total_wgu) g = total_wgu;
    return int(g < 1 ? 1 : g);
}

static int launch_gemv(int fmt, int M, const GemvParams &GP, int grid, hipStream_t st) {
    GemvFn fn = pick_gemv(fmt, M);
    if (!fn) return WQD_EINVAL;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), 0, st, GP);
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
    int rc = launch_gemv(fmt, int(M), GP, grid_for(fmt, GP.total_wgu, cus), st);
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

// Stack workspace: [Desc table][RedDesc table][partials...], each 256-byte aligned.
struct StackPlan {
    std::vector<Desc> descs;       // grouped by format, in format order
    std::vector<int> fmt_begin;    // index into descs of each format group (size 6)
    std::vector<int> wgu_total;    // per format
    std::vector<RedDesc> reds;
    int64_t red_total = 0;
    int64_t off_descs = 0, off_reds = 0, off_part = 0, total = 0;
    int64_t max_single_part = 0;   // for ORDERED mode
};

static int build_stack_plan(const wqd_proj *p, int32_t count, int64_t M, void *ws, StackPlan &SP, int cus) {
    if (!p || count < 1) return WQD_EINVAL;
    for (int i = 0; i < count; i++) {
        if (p[i].reserved != 0) return WQD_EINVAL;
        int rc = check_proj(p[i].fmt, p[i].N, p[i].K, p[i].w, p[i].x, M, p[i].ldx, p[i].y, p[i].ldy);
        if (rc != WQD_OK) return rc;
    }
    SP.off_descs = 0;
    SP.off_reds = align_up(int64_t(sizeof(Desc)) * count, 256);
    SP.off_part = SP.off_reds + align_up(int64_t(sizeof(RedDesc)) * count, 256);
    int64_t part_off = SP.off_part;
    uint8_t *base = static_cast<uint8_t *>(ws);
    SP.fmt_begin.assign(7, 0);
    SP.wgu_total.assign(7, 0);
    for (int fmt = 1; fmt <= 5; fmt++) {
        SP.fmt_begin[fmt] = int(SP.descs.size());
        int wgu = 0;
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
                SP.red_total += M * p[i].N;
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
        SP.wgu_total[fmt] = wgu;
    }
    SP.fmt_begin[6] = int(SP.descs.size());
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
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

WQD_API int wqd_run_projections(const wqd_proj *projs, int32_t count, int64_t M, int32_t mode,
                                void *workspace, int64_t workspace_bytes, void *stream) {
    if (M < 1 || M > WQD_MAX_M) return WQD_ESHAPE;
    if (mode != WQD_ORDERED && mode != WQD_PERSISTENT) return WQD_EINVAL;
    const int cus = device_cus();
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mode == WQD_ORDERED) {
        if (!projs || count < 1) return WQD_EINVAL;
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
    const uint8_t *base = static_cast<const uint8_t *>(workspace);
    const Desc *dtab = reinterpret_cast<const Desc *>(base + SP.off_descs);
    for (int fmt = 1; fmt <= 5; fmt++) {
        const int nd = SP.fmt_begin[fmt + 1] - SP.fmt_begin[fmt];
        if (nd == 0) continue;
        GemvParams GP;
        memset(&GP, 0, sizeof(GP));
        GP.d0 = SP.descs[SP.fmt_begin[fmt]];
        GP.descs = dtab + SP.fmt_begin[fmt];
        GP.ndesc = nd;
        GP.total_wgu = SP.wgu_total[fmt];
        rc = launch_gemv(fmt, int(M), GP, grid_for(fmt, GP.total_wgu, cus), st);
        if (rc != WQD_OK) return rc;
    }
    if (!SP.reds.empty()) {
        RedParams RP;
        memset(&RP, 0, sizeof(RP));
        RP.d0 = SP.reds[0];
        RP.descs = reinterpret_cast<const RedDesc *>(base + SP.off_reds);
        RP.ndesc = int32_t(SP.reds.size());
        RP.total = SP.red_total;
        rc = launch_reduce(RP, st);
    }
    return rc;
}

WQD_API int wqd_stream_check(void *stream) {
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
    return e == hipSuccess ? WQD_OK : hip_fail(e);
}

WQD_API int wqd_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
