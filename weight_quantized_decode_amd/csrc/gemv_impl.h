// HIP kernels (gfx950) and the C entry points of libwqd that launch them.
//
// Design (one projection y = x W^T, M <= 8 activation rows per call, up to 16 in a batch-invariant
// verify):
//   * One wavefront lane per weight row: a wave covers a group of 64 rows, and every load
//     instruction reads chunk c of those 64 rows, 1 KiB of contiguous prepared code bytes
//     (layout.h).  Each row's dot product stays inside its lane, so no cross-lane reduction.
//   * The activations are the same for all 64 lanes, so they are read with scalar loads into
//     SGPRs and fed to v_dot2 (two fp16 products accumulated in fp32 per instruction).
//   * Work unit of a wave = (row group, K-slice).  K is split only as far as needed to give the
//     GPU enough waves; each slice writes fp32 partial sums and counts itself done on its row
//     group, and the wave that finishes the last slice adds them in slice order, so results are
//     the same bits from run to run (the only atomic is the per-row-group arrival counter).
//   * Codebook formats decode through tables in LDS replicated per lane slot (one copy per bank),
//     indexed with one v_perm per byte; the block formats decode with AND masks that leave the
//     codes as fp16 subnormals (code * 2^-24 * 4^j) and apply the -8 / -1 offset through the
//     per-block sum of the activations.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace wqd {

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}
__device__ __forceinline__ cu32p scalar_ptr(const void *p) {
    return (cu32p)(uintptr_t)p;
}
// Descriptor read with scalar loads, so its fields live in SGPRs and count as wave-uniform.
__device__ __forceinline__ Desc load_desc(const Desc *p) {
    static_assert(sizeof(Desc) % 4 == 0, "descriptor must be whole dwords");
    uint32_t w[sizeof(Desc) / 4];
    cu32p s = scalar_ptr(p);
#pragma unroll
    for (unsigned i = 0; i < sizeof(Desc) / 4; i++) w[i] = s[i];
    Desc D;
    __builtin_memcpy(&D, w, sizeof(Desc));
    return D;
}
__device__ __forceinline__ int load_wgu_begin(const Desc *p) {
    return (int)scalar_ptr(&p->wgu_begin)[0];
}
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// LDS dword at a byte offset (the offset is already a multiple of 4).
__device__ __forceinline__ uint32_t lds_word(const uint32_t *lds, uint32_t byte_off) {
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lds) + byte_off);
}

// Loads through the global address space (global_load_*, counted by vmcnt only; a generic
// pointer would compile to flat loads, which also hold up LDS waits).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ T gld(const void *p) {
    return *(const T __attribute__((address_space(1))) *)(uintptr_t)p;
}
__device__ __forceinline__ uint4 ld16(const uint8_t *p) {
    const u32x4 v = gld<u32x4>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// Streaming read of packed codes: each byte is used once, so the load is marked nontemporal
// (it then does not displace reused data such as activations and tables in the caches).
__device__ __forceinline__ uint4 ld16_stream(const uint8_t *p) {
#if WQD_NT_CODES
    const u32x4 v = __builtin_nontemporal_load((const u32x4 __attribute__((address_space(1))) *)(uintptr_t)p);
#else
    const u32x4 v = gld<u32x4>(p);
#endif
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8(const uint8_t *p) {
    const u32x2 v = gld<u32x2>(p);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld16(const uint4 *p) { return ld16(reinterpret_cast<const uint8_t *>(p)); }
// The same pointer in the global address space: atomics through it compile to global_* (a
// generic pointer gives flat_* instructions, which also count against the LDS/scalar wait
// counter and so hold up every later LDS wait until they complete).
template <typename T>
__device__ __forceinline__ T __attribute__((address_space(1))) *as_global(T *p) {
    return (T __attribute__((address_space(1))) *)(uintptr_t)p;
}
// A launch from a descriptor table first compares the table's stamp with the fingerprint of the
// list it was planned for (a table that setup wrote for another list).  On a mismatch every
// workgroup returns before touching any output, and workgroup 0 raises *stale.
__device__ __forceinline__ bool stale_table(const uint64_t *stamp, uint64_t fp, int *stale) {
    if (!stamp) return false;
    const cu32p s = (cu32p)(uintptr_t)stamp;
    const uint64_t v = uint64_t(s[0]) | (uint64_t(s[1]) << 32);
    if (v == fp) return false;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        __hip_atomic_store((int __attribute__((address_space(1))) *)(uintptr_t)stale, 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Workgroup barrier that orders LDS traffic only (global loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ void gst(float *p, float v) {
    *(float __attribute__((address_space(1))) *)(uintptr_t)p = v;
}

// Compile-time loop: f(Int<0>{}), ..., f(Int<N-1>{}), so the body can use the index where a
// constant expression is required (an MFMA operand-broadcast field).
template <int I>
struct Int {
    static constexpr int value = I;
};
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(Int<I>{});
        static_for<N, I + 1>(f);
    }
}

// Small-M matrix-core step.  v_mfma_f32_4x4x4_16b_f16 computes 16 independent 4x4x4 products,
// block b on lanes 4b..4b+3: D_b[i][j] += sum_k A_b[i][k] B_b[k][j], lane 4b+i holding row i of A_b
// and lane 4b+j column j of B_b (4 fp16 values each), and register v of lane 4b+j receiving
// D_b[v][j].  Here B is 4 consecutive decoded weights of the lane's own row and, with the A
// operand of block WIN broadcast to all 16 blocks, A[i][k] is activation row i at those 4 k: each
// lane gets the partial dot products of its row with 4 activation rows.  A window register pair
// holds 16 such 4-element k-blocks (64 consecutive k) of 4 activation rows: lane 4b+i holds row i,
// elements 4b..4b+3 of the window.
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int WIN>
__device__ __forceinline__ f32x4 mfma_xw(u32x2 xwin, u32x2 w, f32x4 d) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h16x4, xwin), __builtin_bit_cast(h16x4, w), d, 4,
                                              WIN, 0);
}

// Uniform read of NW consecutive x dwords (2*NW fp16 values starting at element k) of one row.
// FULL: the whole range lies inside K (scalar loads).  Otherwise elements at or beyond K read as
// zero (only a partial last chunk takes that path).
template <bool FULL, int NW>
__device__ __forceinline__ void load_x(uint32_t (&xs)[NW], const uint16_t *xrow, int k, int K) {
    if constexpr (FULL) {
        cu32p p = scalar_ptr(xrow + k);
#pragma unroll
        for (int i = 0; i < NW; i++) xs[i] = p[i];
    } else {
#pragma unroll
        for (int i = 0; i < NW; i++) {
            uint32_t lo = (k + 2 * i < K) ? gld<uint16_t>(xrow + k + 2 * i) : 0u;
            uint32_t hi = (k + 2 * i + 1 < K) ? gld<uint16_t>(xrow + k + 2 * i + 1) : 0u;
            xs[i] = lo | (hi << 16);
        }
    }
}

template <bool B>
struct FullTag {
    static constexpr bool value = B;
};

template <int FMT>
struct LdsSize {
    static constexpr int dwords = (FMT == CB4 || FMT == CB8) ? 256 * kTableCopies : 1;
};
constexpr int cmax(int a, int b) { return a > b ? a : b; }
template <int MASK>
struct LdsSizeMask {
    // tables of the codebook formats; per-wave block sums (WQD_MAX_M x 64 floats) of Q4_0 / TQ2
    static constexpr int dwords = cmax(cmax((MASK & (1 << CB4)) ? LdsSize<CB4>::dwords : 1,
                                            (MASK & (1 << CB8)) ? LdsSize<CB8>::dwords : 1),
                                       (MASK & ((1 << Q4_0) | (1 << TQ2))) ? kWaves * kMaxM * 64 : 1);
};

// Build the per-workgroup LDS table of a projection.
template <int FMT>
__device__ void build_table(uint32_t *lds, const Desc &D) {
    const int t = threadIdx.x;
    if constexpr (FMT == CB4 || FMT == CB8) {
        // entry e, copy j at dword e*64 + j: lane slot j reads bank j for any entry.
        for (int e = t; e < 256; e += kThreads) {
            uint32_t v;
            if constexpr (FMT == CB4) v = uint32_t(gld<uint16_t>(D.cbk + (e & 15))) | (uint32_t(gld<uint16_t>(D.cbk + (e >> 4))) << 16);
            else v = uint32_t(gld<uint16_t>(D.cbk + e));
            uint4 q = make_uint4(v, v, v, v);
            // not unrolled: unrolled, the 16 store addresses are hoisted out of the persistent
            // loop and held in registers for the whole kernel
#pragma unroll 1
            for (int j = 0; j < kTableCopies / 4; j++) {
                int jj = (j + e) % (kTableCopies / 4);
                reinterpret_cast<uint4 *>(lds)[e * (kTableCopies / 4) + jj] = q;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// AQ1X16 chunks [cb, ce) of row group g (lane = row): a chunk is 8 16-bit codes, 64 weights.  Each
// code selects a 16-byte entry (8 fp16) of the projection's 1 MiB codebook, gathered from the L2
// cache; the products are fp16 x fp16 summed in fp32 (v_dot2).  A ring of P code chunks stays in
// flight: the 8 gathers of a chunk are issued before the code load P chunks ahead, so the wait for
// the gathers leaves that prefetch outstanding.
// ------------------------------------------------------------------------------------------
template <int M, typename Hook>
__device__ __forceinline__ void aq16_chunks(const Desc &D, int g, int cb, int ce, int lane,
                                            const uint16_t *const (&xrow)[M], float (&acc)[M], Hook &&hook) {
    constexpr int P = 4;
    const uint8_t *cptr = D.codes + ((int64_t)g * D.C * 64 + lane) * 16;
    // The gathers are buffer loads on a resource over the 1 MiB codebook: each takes the entry's
    // 32-bit byte offset as it is (no 64-bit address arithmetic per gather).  Word 3 of the
    // resource (0x00020000) is the raw 32-bit buffer format of gfx950.
    const __amdgpu_buffer_rsrc_t cbr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(D.cbk), (short)0, 65536 * 16, 0x00020000);
    uint4 q[P];
    if (cb < ce) {
#pragma unroll
        for (int j = 0; j < P; j++) q[j] = ld16_stream(cptr + (int64_t)min(cb + j, ce - 1) * 1024);
    }
    hook();
    for (int c = cb; c < ce; c += P) {
        static_for<P>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int cc = c + j;
            if (cc < ce) {
                const uint32_t w[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
                u32x4 e[8];
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const uint32_t code = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                    e[i] = __builtin_amdgcn_raw_buffer_load_b128(cbr, code * 16, 0, 0);
                }
                q[j] = ld16_stream(cptr + (int64_t)min(cc + P, ce - 1) * 1024);
                const int ng = min(8, (D.K - cc * 64) >> 3);  // groups inside K (8 but in a tail)
                if (ng == 8) {
#pragma unroll
                    for (int m = 0; m < M; m++) {
                        cu32p xs = scalar_ptr(xrow[m] + cc * 64);
#pragma unroll
                        for (int i = 0; i < 8; i++)
#pragma unroll
                            for (int t = 0; t < 4; t++) acc[m] = dot2(e[i][t], xs[4 * i + t], acc[m]);
                    }
                } else {
#pragma unroll
                    for (int m = 0; m < M; m++) {
#pragma unroll
                        for (int i = 0; i < 8; i++) {
                            if (i < ng) {
                                cu32p xs = scalar_ptr(xrow[m] + cc * 64 + 8 * i);
#pragma unroll
                                for (int t = 0; t < 4; t++) acc[m] = dot2(e[i][t], xs[t], acc[m]);
                            }
                        }
                    }
                }
            }
        });
    }
    // the row scale, once per unit
    const float sc = half_bits_to_float(reinterpret_cast<const uint16_t *>(D.scales)[g * 64 + lane]);
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] *= sc;
}

// ------------------------------------------------------------------------------------------
// TQ2 times int8 activations, chunks [cb, ce) of row group g (lane = row; the slice is a whole
// number of 128-weight blocks).  Per block: the 2-bit codes of a word shifted by 2j and masked with
// 0x03030303 give 4 codes in 4 bytes; v_dot4_i32_i8 multiplies them with the matching 4 int8
// activations (the quantizer stores each block's q in this field order) into an int32 sum, 32 per
// block; the -1 code offset comes off as the block's sum of q, and floating point is applied once
// per block: acc += (d * a) * (sum code*q - sum q).  D.x holds q ([M][ldx] bytes), D.cbk the
// per-block activation scales a[M][K/128] (fp32) followed by the sums of q [M][K/128] (int32).
// ------------------------------------------------------------------------------------------
template <int M, typename Hook>
__device__ __forceinline__ void tq2i8_chunks(const Desc &D, int g, int cb, int ce, int lane, float (&acc)[M],
                                             Hook &&hook) {
    constexpr int P = 4;  // code chunks in flight (two blocks)
    const uint8_t *cptr = D.codes + ((int64_t)g * D.C * 64 + lane) * 16;
    const int nb = D.K / 128;
    const int8_t *qb = reinterpret_cast<const int8_t *>(D.x);
    const float *ab = reinterpret_cast<const float *>(D.cbk);
    const int32_t *sb = reinterpret_cast<const int32_t *>(ab + (int64_t)M * nb);
    uint4 q[P];
    if (cb < ce) {
#pragma unroll
        for (int j = 0; j < P; j++) q[j] = ld16_stream(cptr + (int64_t)min(cb + j, ce - 1) * 1024);
    }
    hook();
    for (int c = cb; c < ce; c += P) {
        static_for<P / 2>([&](auto bc) {
            constexpr int jb = decltype(bc)::value;  // block of this round: chunks 2jb, 2jb+1
            const int cc = c + 2 * jb;
            if (cc < ce) {
                const int b = cc >> 1;
                const uint32_t dbits = gld<uint16_t>(D.scales + (((int64_t)g * D.Q + (b >> 2)) * 64 + lane) * 8 + (b & 3) * 2);
                int32_t isum[M];
#pragma unroll
                for (int m = 0; m < M; m++) isum[m] = 0;
                static_for<2>([&](auto hc) {
                    constexpr int h = decltype(hc)::value;
                    const uint4 v = q[2 * jb + h];
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int m = 0; m < M; m++) {
                        cu32p xs = scalar_ptr(qb + (int64_t)m * D.ldx + (int64_t)b * 128 + 64 * h);
#pragma unroll
                        for (int t = 0; t < 4; t++)
#pragma unroll
                            for (int j = 0; j < 4; j++)
                                isum[m] = __builtin_amdgcn_sdot4((int)((w4[t] >> (2 * j)) & 0x03030303u),
                                                                 (int)xs[4 * t + j], isum[m], false);
                    }
                });
                q[2 * jb] = ld16_stream(cptr + (int64_t)min(cc + P, ce - 1) * 1024);
                q[2 * jb + 1] = ld16_stream(cptr + (int64_t)min(cc + P + 1, ce - 1) * 1024);
                const float d = half_bits_to_float(dbits);
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const float da = d * __builtin_bit_cast(float, scalar_ptr(ab + (int64_t)m * nb + b)[0]);
                    acc[m] = fmaf(da, (float)(isum[m] - (int32_t)scalar_ptr(sb + (int64_t)m * nb + b)[0]), acc[m]);
                }
            }
        });
    }
}

// ------------------------------------------------------------------------------------------
// One wave unit: rows 64g..64g+63 (one per lane) times chunks [cb, ce).
// ------------------------------------------------------------------------------------------
// `hook` runs once, right after the first loads of the unit are issued: the workgroup uses it
// to (re)build its LDS table while those loads are in flight.
template <int FMT, int M, bool EPI, bool BI, typename Hook>
__device__ __forceinline__ void run_unit(const Desc &D, int wu, int lane, uint32_t *lds, float *red, Hook &&hook) {
    // Wave unit -> (row group g, K-slice s, chunks [cb, ce)).  Workgroup-split descriptors give
    // the kWaves waves of a workgroup unit consecutive pieces of one slice of D.CS chunks (the
    // last pieces of a row may be empty); otherwise a wave unit is a whole slice.
    int g, s, cb, ce;
    if (D.wsplit) {
        const int q = wu / kWaves, w = wu - q * kWaves;
        g = q / D.S;
        s = q - g * D.S;
        const int cw = D.CS / kWaves;
        cb = min(D.C, s * D.CS + w * cw);
        ce = min(D.C, cb + cw);
    } else {
        g = wu / D.S;
        s = wu - g * D.S;
        cb = s * D.CS;
        ce = min(D.C, cb + D.CS);
    }
    // These are wave-uniform, which the compiler cannot prove by itself; marked as such, the
    // chunk loop's counters and the activation addresses stay in SGPRs instead of costing vector
    // instructions per chunk.
    cb = __builtin_amdgcn_readfirstlane(cb);
    ce = __builtin_amdgcn_readfirstlane(ce);
    g = __builtin_amdgcn_readfirstlane(g);
    // TQ2 slices start at a multiple of 8 chunks (the planners align them to scale quads, which
    // the scale loads rely on too), so a load group starts on an even chunk and the compiler knows
    // which chunk of a group opens a 128-weight block (no branches or register copies for it).
    // Only an empty range can start elsewhere (a workgroup-split piece past the end of a row whose
    // chunk count is not a multiple of 8): it is moved to a quad boundary, still empty.
    if constexpr (FMT == TQ2) {
        if (cb >= ce) cb = ce = cb & ~7;
        __builtin_assume((cb & 7) == 0);
    }
    const int row = g * 64 + lane;
    const uint8_t *cptr = D.codes + ((int64_t)g * D.C * 64 + lane) * 16;
    const uint16_t *xrow[M];
#pragma unroll
    for (int m = 0; m < M; m++) xrow[m] = D.x + (int64_t)m * D.ldx;

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;

    if constexpr (FMT == AQ1X16) {
        aq16_chunks<M>(D, g, cb, ce, lane, xrow, acc, hook);
    } else if constexpr (FMT == TQ2I8) {
        tq2i8_chunks<M>(D, g, cb, ce, lane, acc, hook);
    } else {
    // Chunks [cb, cfe) are whole chunks (x read with scalar loads); a partial last chunk of the
    // row, if this unit owns it, is handled after the pipelined loop.
    const int cfe = min(ce, D.C_full);

    // Matrix-core path (M >= WQD_MFMA_MIN_M): the whole chunks are multiplied by
    // v_mfma_f32_4x4x4_16b_f16 into MFA (activation rows 4h..4h+3 in MFA[.][h]).  With H = 1 there
    // are two accumulator chains, so consecutive MFMAs do not wait for each other; with H = 2 the
    // two activation-row quads already alternate.  A load group of U chunks spans NWIN
    // activation windows of 64 k, loaded with the group's codes (in-order completion then makes
    // one wait cover both).  The matrix-core path takes longer per chunk, so it loads larger
    // groups (more bytes in flight per wave while a group is processed).
    // The block formats decode to exact fp16 values (code - 8, code - 1) for it, and their
    // MFA holds one scale block at a time, added to acc times the block scale.
    // Batch-invariant instances (BI) take the matrix-core path at every M, with one accumulator
    // chain per activation quad, so a row's instruction sequence does not depend on M.
    constexpr bool MF = (M >= WQD_MFMA_MIN_M || BI) && (FMT == CB4 || FMT == CB8 || FMT == Q4_0 || FMT == TQ2);
    constexpr bool BLK = (FMT == Q4_0 || FMT == TQ2);
    constexpr int WPC = (FMT == CB8) ? 16 : (FMT == TQ2) ? 64 : 32;  // weights per chunk
    constexpr int CPW = 64 / WPC;                // chunks per window
    constexpr int H = MF ? (M + 3) / 4 : 1;
    // CB4 with two activation quads needs twice the window registers: a shorter group keeps it
    // within 128 VGPRs
    constexpr int U = MF ? ((FMT == CB4 && H > 1) ? WQD_MF_U_WIDE : WQD_MF_U) : kU;
    static_assert(!MF || U % CPW == 0, "a load group holds whole activation windows");
    static_assert(!MF || !BLK || U == 4, "a load group of a block format lies in one scale quad");
    constexpr int NWIN = MF ? U / CPW : 1;
    constexpr int NCH = (H == 1 && !BI) ? 2 : 1;
    const uint16_t *xw[H];  // lane 4b+i: activation row 4h+i (clamped to M-1), at element 4b
#pragma unroll
    for (int h = 0; h < H; h++) xw[h] = D.x + (int64_t)min(4 * h + (lane & 3), M - 1) * D.ldx + 4 * (lane >> 2);
    const int kwin_max = cfe * WPC - 4 - 4 * (lane >> 2);  // window loads stay below K
    auto load_win = [&](u32x2 (&X)[NWIN][H], int c) {
        if constexpr (MF) {
#pragma unroll
            for (int w = 0; w < NWIN; w++)
#pragma unroll
                for (int h = 0; h < H; h++) {
                    const uint16_t *p = xw[h] + min(c * WPC + 64 * w, kwin_max);
                    X[w][h] = u32x2{gld<uint32_t>(p), gld<uint32_t>(p + 2)};
                }
        }
    };
    u32x2 XA[NWIN][H], XB[NWIN][H];
    f32x4 MFA[NCH][H];
#pragma unroll
    for (int q = 0; q < NCH; q++)
#pragma unroll
        for (int h = 0; h < H; h++) MFA[q][h] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load_group = [&](uint4 (&buf)[U], u32x2 (&X)[NWIN][H], int c) {
#pragma unroll
        for (int j = 0; j < U; j++) {
            const int cc = min(c + j, cfe - 1);
            buf[j] = ld16_stream(cptr + (int64_t)cc * 1024);
        }
        load_win(X, c);
    };
    // Scale quad of the chunk group starting at c (block formats only).
    auto load_sq = [&](int c) -> uint2 {
        if constexpr (FMT == Q4_0 || FMT == TQ2) {
            const int q = (FMT == Q4_0) ? (c >> 2) : (c >> 3);
            return ld8(D.scales + (((int64_t)g * D.Q + q) * 64 + lane) * 8);
        } else {
            return make_uint2(0, 0);
        }
    };
    uint4 A[U], B[U];
    uint2 sqA = make_uint2(0, 0), sqB = make_uint2(0, 0);
    if (cb < cfe) {
        sqA = load_sq(cb);
        load_group(A, XA, cb);
    }
    hook();

    // Per-block activation sums for the block formats (the -8 / -1 code offsets are applied
    // through them).  All 64 lanes load the unit's slice of x together, SEG lanes per block, and
    // the sums are parked in this wave's LDS area; the main loop reads them back with a uniform
    // (broadcast) address.
    int b0 = 0;
    constexpr int WPB = (FMT == Q4_0) ? 32 : 128;   // weights per scale block
    float *bs = nullptr;
    if constexpr ((FMT == Q4_0 || FMT == TQ2) && !MF) {
        const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        bs = reinterpret_cast<float *>(lds) + wid * (kMaxM * 64);
        b0 = (FMT == Q4_0) ? cb : cb / 2;
        const int b1 = (FMT == Q4_0) ? ce : ce / 2;
        constexpr int SEG = WPB / 8;   // lanes per block, 8 activations per lane
        constexpr int BPR = 64 / SEG;  // blocks per round of the wave
        const int rounds = (b1 - b0 + BPR - 1) / BPR;
        constexpr uint32_t ones = 0x3C003C00u;  // (1.0, 1.0) in fp16
#pragma unroll
        for (int m = 0; m < M; m++) {
            for (int r = 0; r < rounds; r++) {
                const int blk = b0 + r * BPR + lane / SEG;
                float sacc = 0.f;
                if (blk < b1) {
                    const uint16_t *xp = xrow[m] + (int64_t)blk * WPB + (lane % SEG) * 8;
#pragma unroll
                    for (int i = 0; i < 4; i++) sacc = dot2(gld<uint32_t>(xp + 2 * i), ones, sacc);
                }
#pragma unroll
                for (int o = 1; o < SEG; o <<= 1) sacc += __shfl_xor(sacc, o);
                if ((lane % SEG) == 0 && blk < b1) bs[m * 64 + (blk - b0)] = sacc;
            }
        }
    }

    const uint32_t loff = uint32_t(lane) * 4u;  // lane slot byte offset inside a table entry
    // TQ2 per-block partial accumulators (weights scaled by 4^j * 2^-24)
    float ta[M][5];

    auto process = [&](auto full_tag, const uint4 &v, int c, uint2 sq) {
        constexpr bool FULL = decltype(full_tag)::value;
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        if constexpr (FMT == CB4) {
#pragma unroll
            for (int t = 0; t < 4; t++) {
                uint32_t e[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    uint32_t a = __builtin_amdgcn_perm(w4[t], loff, 0x0c0c0400u + (uint32_t(i) << 8));
                    e[i] = lds_word(lds, a);
                }
#pragma unroll
                for (int m = 0; m < M; m++) {
                    uint32_t xs[4];
                    load_x<FULL, 4>(xs, xrow[m], c * 32 + t * 8, D.K);
#pragma unroll
                    for (int i = 0; i < 4; i++) acc[m] = dot2(e[i], xs[i], acc[m]);
                }
            }
        } else if constexpr (FMT == CB8) {
#pragma unroll
            for (int t = 0; t < 4; t++) {
                uint32_t pr[2];
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    uint32_t a0 = __builtin_amdgcn_perm(w4[t], loff, 0x0c0c0400u + (uint32_t(2 * i) << 8));
                    uint32_t a1 = __builtin_amdgcn_perm(w4[t], loff, 0x0c0c0400u + (uint32_t(2 * i + 1) << 8));
                    uint32_t e0 = lds_word(lds, a0), e1 = lds_word(lds, a1);
                    pr[i] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);
                }
#pragma unroll
                for (int m = 0; m < M; m++) {
                    uint32_t xs[2];
                    load_x<FULL, 2>(xs, xrow[m], c * 16 + t * 4, D.K);
                    acc[m] = dot2(pr[0], xs[0], acc[m]);
                    acc[m] = dot2(pr[1], xs[1], acc[m]);
                }
            }
        } else if constexpr (FMT == Q4_0) {
            uint32_t q[4][4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                uint32_t w = w4[t], w8 = w4[t] >> 8;
                q[t][0] = w & 0x000F000Fu;
                q[t][1] = w & 0x00F000F0u;
                q[t][2] = w8 & 0x000F000Fu;
                q[t][3] = w8 & 0x00F000F0u;
            }
            const int bq = c & 3;
            const uint32_t dbits = (bq < 2 ? sq.x : sq.y) >> ((bq & 1) * 16);
            const float d = half_bits_to_float(dbits & 0xFFFFu);
#pragma unroll
            for (int m = 0; m < M; m++) {
                uint32_t xs[16];
                load_x<FULL, 16>(xs, xrow[m], c * 32, D.K);
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    a0 = dot2(q[t][0], xs[4 * t + 0], a0);
                    a1 = dot2(q[t][1], xs[4 * t + 1], a1);
                    a0 = dot2(q[t][2], xs[4 * t + 2], a0);
                    a1 = dot2(q[t][3], xs[4 * t + 3], a1);
                }
                const float sb = bs[m * 64 + (c - b0)];
                const float p = fmaf(a1, 0.0625f, a0);               // 2^-24 * sum code*x
                const float blk = fmaf(p, 16777216.0f, -8.0f * sb);  // sum (code-8)*x
                acc[m] = fmaf(d, blk, acc[m]);
            }
        } else if constexpr (FMT == TQ2) {
            const bool first = (c & 1) == 0;
#pragma unroll
            for (int m = 0; m < M; m++) {
                if (first) {
#pragma unroll
                    for (int j = 0; j < 5; j++) ta[m][j] = 0.f;
                }
            }
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t w = w4[t], w10 = w4[t] >> 10;
                uint32_t q[8];
                q[0] = w & 0x00030003u;
                q[1] = w & 0x000C000Cu;
                q[2] = w & 0x00300030u;
                q[3] = w & 0x00C000C0u;
                q[4] = w & 0x03000300u;
                q[5] = w10 & 0x00030003u;
                q[6] = w10 & 0x000C000Cu;
                q[7] = w10 & 0x00300030u;
#pragma unroll
                for (int m = 0; m < M; m++) {
                    uint32_t xs[8];
                    load_x<FULL, 8>(xs, xrow[m], c * 64 + t * 16, D.K);
                    ta[m][0] = dot2(q[0], xs[0], ta[m][0]);
                    ta[m][1] = dot2(q[1], xs[1], ta[m][1]);
                    ta[m][2] = dot2(q[2], xs[2], ta[m][2]);
                    ta[m][3] = dot2(q[3], xs[3], ta[m][3]);
                    ta[m][4] = dot2(q[4], xs[4], ta[m][4]);
                    ta[m][0] = dot2(q[5], xs[5], ta[m][0]);
                    ta[m][1] = dot2(q[6], xs[6], ta[m][1]);
                    ta[m][2] = dot2(q[7], xs[7], ta[m][2]);
                }
            }
            if (!first) {
                const int b = c >> 1;
                const int bq = b & 3;
                const uint32_t dbits = (bq < 2 ? sq.x : sq.y) >> ((bq & 1) * 16);
                const float d = half_bits_to_float(dbits & 0xFFFFu);
#pragma unroll
                for (int m = 0; m < M; m++) {
                    float p = fmaf(ta[m][4], 0.00390625f, ta[m][3] * 0.015625f);
                    p = fmaf(ta[m][2], 0.0625f, p);
                    p = fmaf(ta[m][1], 0.25f, p);
                    p += ta[m][0];                                   // 2^-24 * sum code*x
                    const float sb = bs[m * 64 + (b - b0)];
                    const float blk = fmaf(p, 16777216.0f, -sb);     // sum (code-1)*x
                    acc[m] = fmaf(d, blk, acc[m]);
                }
            }
        }
    };

    // Matrix-core form of one whole chunk, j-th of its group (static: it fixes the window and the
    // 4-k block of every MFMA).  Chunk j of a group at chunk c covers k = (c+j)*WPC ..; window w
    // starts at k = c*WPC + 64w, so chunk j lies in window j / CPW at block (j % CPW) * WPC / 4.
    auto process_mf = [&](auto jc, const uint4 &v, const u32x2 (&X)[NWIN][H], int c, uint2 sq) {
        constexpr int j = decltype(jc)::value;
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        static_for<4>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            if constexpr (BLK) {
                // Q4_0 word t: nibbles i and i+4 are weights 8t+2i, 8t+2i+1; TQ2 word t: fields i
                // and i+8 are weights 16t+2i, 16t+2i+1.  OR-ing a code into 0x6400 (fp16 1024)
                // gives 1024 + code exactly; one packed fp16 add of -1032 / -1025 leaves code - 8
                // / code - 1.  B operand q: weights 4q..4q+3 of the word.
                constexpr int NP = (FMT == Q4_0) ? 4 : 8, SH = (FMT == Q4_0) ? 4 : 2;
                constexpr uint32_t MSK = (FMT == Q4_0) ? 0x000F000Fu : 0x00030003u;
                constexpr uint32_t OFF = (FMT == Q4_0) ? 0xE408E408u : 0xE401E401u;
                uint32_t pr[NP];
#pragma unroll
                for (int i = 0; i < NP; i++)
                    pr[i] = __builtin_bit_cast(uint32_t, as_h2(((w4[t] >> (SH * i)) & MSK) | 0x64006400u) + as_h2(OFF));
                static_for<NP / 2>([&](auto qc) {
                    constexpr int q = decltype(qc)::value;
                    constexpr int win = j / CPW, blk = (FMT == Q4_0) ? 8 * (j % CPW) + 2 * t + q : 4 * t + q;
#pragma unroll
                    for (int h = 0; h < H; h++) MFA[q % NCH][h] = mfma_xw<blk>(X[win][h], u32x2{pr[2 * q], pr[2 * q + 1]}, MFA[q % NCH][h]);
                });
            } else if constexpr (FMT == CB4) {
                // word t: byte i -> weights 8t+2i, 8t+2i+1; pair p of bytes -> weights 8t+4p..+3
                uint32_t e[4];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    e[i] = lds_word(lds, __builtin_amdgcn_perm(w4[t], loff, 0x0c0c0400u + (uint32_t(i) << 8)));
                static_for<2>([&](auto pc) {
                    constexpr int p = decltype(pc)::value;
                    constexpr int win = j / CPW, blk = 8 * (j % CPW) + 2 * t + p;
#pragma unroll
                    for (int h = 0; h < H; h++) MFA[p % NCH][h] = mfma_xw<blk>(X[win][h], u32x2{e[2 * p], e[2 * p + 1]}, MFA[p % NCH][h]);
                });
            } else {
                // word t: weights 4t..4t+3 of the chunk
                uint32_t pr[2];
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    uint32_t a0 = __builtin_amdgcn_perm(w4[t], loff, 0x0c0c0400u + (uint32_t(2 * i) << 8));
                    uint32_t a1 = __builtin_amdgcn_perm(w4[t], loff, 0x0c0c0400u + (uint32_t(2 * i + 1) << 8));
                    pr[i] = __builtin_amdgcn_perm(lds_word(lds, a1), lds_word(lds, a0), 0x05040100u);
                }
                constexpr int win = j / CPW, blk = 4 * (j % CPW) + t;
#pragma unroll
                for (int h = 0; h < H; h++) MFA[t % NCH][h] = mfma_xw<blk>(X[win][h], u32x2{pr[0], pr[1]}, MFA[t % NCH][h]);
            }
        });
        if constexpr (BLK) {
            // end of a scale block (every Q4_0 chunk; every second TQ2 chunk, groups start even)
            if constexpr (FMT == Q4_0 || (j & 1) == 1) {
                const int bq = (FMT == Q4_0) ? ((c + j) & 3) : (((c + j) >> 1) & 3);
                const uint32_t dbits = (bq < 2 ? sq.x : sq.y) >> ((bq & 1) * 16);
                const float d = half_bits_to_float(dbits & 0xFFFFu);
#pragma unroll
                for (int h = 0; h < H; h++) {
#pragma unroll
                    for (int vv = 0; vv < 4; vv++) {
                        const float bsum = (NCH == 2) ? MFA[0][h][vv] + MFA[NCH - 1][h][vv] : MFA[0][h][vv];
                        if (4 * h + vv < M) acc[4 * h + vv] = fmaf(d, bsum, acc[4 * h + vv]);
                    }
#pragma unroll
                    for (int qq = 0; qq < NCH; qq++) MFA[qq][h] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    };

    // (full: every chunk of the group is below cfe, so no chunk needs its guard.  The batch-
    // invariant instances keep it: they also run the shortest M = 1 launches, where a second,
    // unguarded copy of the matrix-core body cost more than the guards: the fused decode step
    // took 1.2% longer)
    auto proc_group = [&](auto full, const uint4 (&buf)[U], const u32x2 (&X)[NWIN][H], int c, uint2 sq) {
        constexpr bool kFull = decltype(full)::value;
        if constexpr (MF) {
            static_for<U>([&](auto jc) {
                if ((kFull && !BI) || c + decltype(jc)::value < cfe) process_mf(jc, buf[decltype(jc)::value], X, c, sq);
            });
        } else {
#pragma unroll
            for (int j = 0; j < U; j++)
                if (kFull || c + j < cfe) process(FullTag<true>{}, buf[j], c + j, sq);
        }
    };

    // Double-buffered pipeline: the loads of group g+1 are in flight while group g is decoded.
    // Each branch below is straight-line code, so the compiler can wait for exactly the older
    // group (vmcnt = U) instead of draining every load.
    if (cb < cfe) {
        const int ng = (cfe - cb + U - 1) / U;
        int gi = 0;
        // (a group with a successor is full)
        while (true) {
            const int c = cb + gi * U;
            if (gi + 1 >= ng) {
                proc_group(FullTag<false>{}, A, XA, c, sqA);
                break;
            }
            sqB = load_sq(c + U);
            load_group(B, XB, c + U);
            proc_group(FullTag<true>{}, A, XA, c, sqA);
            gi++;
            if (gi + 1 >= ng) {
                proc_group(FullTag<false>{}, B, XB, c + U, sqB);
                break;
            }
            sqA = load_sq(c + 2 * U);
            load_group(A, XA, c + 2 * U);
            proc_group(FullTag<true>{}, B, XB, c + U, sqB);
            gi++;
        }
    }
    if constexpr (MF && !BLK) {
        // The partial last chunk (when this unit owns it): its window reads zero at k >= K, so
        // the zero padding of the codes (which decodes to a codebook entry) adds nothing.
        for (int c = max(cb, cfe); c < ce; c++) {
            const uint4 v = ld16(cptr + (int64_t)c * 1024);
            u32x2 X[NWIN][H];
            const int k0 = c * WPC + 4 * (lane >> 2);
#pragma unroll
            for (int h = 0; h < H; h++) {
                const uint16_t *p = D.x + (int64_t)min(4 * h + (lane & 3), M - 1) * D.ldx;
                uint32_t e[4];
#pragma unroll
                for (int i = 0; i < 4; i++) e[i] = (k0 + i < D.K) ? uint32_t(gld<uint16_t>(p + k0 + i)) : 0u;
#pragma unroll
                for (int w = 0; w < NWIN; w++) X[w][h] = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
            }
            process_mf(Int<0>{}, v, X, c, make_uint2(0, 0));
        }
    } else if constexpr (FMT != Q4_0 && FMT != TQ2) {
        for (int c = max(cb, cfe); c < ce; c++) {
            const uint4 v = ld16(cptr + (int64_t)c * 1024);
            process(FullTag<false>{}, v, c, make_uint2(0, 0));
        }
    }
    if constexpr (MF && !BLK) {
        // register v of MFA[.][h] is activation row 4h+v of this lane's row
#pragma unroll
        for (int h = 0; h < H; h++)
#pragma unroll
            for (int v = 0; v < 4; v++)
                if (4 * h + v < M) acc[4 * h + v] += (NCH == 2) ? MFA[0][h][v] + MFA[NCH - 1][h][v] : MFA[0][h][v];
    }

    }  // (generic formats)

    if (D.wsplit) {
        // Workgroup split: add the kWaves pieces in wave order through LDS (RM activation rows
        // per round); wave 0 goes on with the slice's sums.  The first barrier of a round keeps
        // the buffer until wave 0 has read the previous round (or the previous unit).
        const int w = wu % kWaves;
        constexpr int RM = M < 4 ? M : 4;
#pragma unroll
        for (int m0 = 0; m0 < M; m0 += RM) {
            lds_barrier();
#pragma unroll
            for (int r = 0; r < RM; r++)
                if (m0 + r < M) red[(r * kWaves + w) * 64 + lane] = acc[m0 + r];
            lds_barrier();
            if (w == 0) {
#pragma unroll
                for (int r = 0; r < RM; r++) {
                    if (m0 + r < M) {
                        float t = red[(r * kWaves) * 64 + lane];
#pragma unroll
                        for (int v = 1; v < kWaves; v++) t += red[(r * kWaves + v) * 64 + lane];
                        acc[m0 + r] = t;
                    }
                }
            }
        }
        if (w != 0) return;
    }

    if (D.S_all == 1) {
        // (two uniform branches: the residual is loaded only when it is added)
        if (row < D.N) {
            if (EPI && D.epi == kEpiAdd) {
                float old[M];
#pragma unroll
                for (int m = 0; m < M; m++) old[m] = gld<float>(D.y + (int64_t)m * D.ldy + row);
#pragma unroll
                for (int m = 0; m < M; m++) gst(D.y + (int64_t)m * D.ldy + row, old[m] + acc[m]);
            } else {
#pragma unroll
                for (int m = 0; m < M; m++) gst(D.y + (int64_t)m * D.ldy + row, acc[m]);
            }
        }
        return;
    }
    // Split K: publish this slice's partial sums, then count the finished slices of the row
    // group; the wave that finishes the last slice adds all slices in ascending order, applies
    // the epilogue and writes y.  A gate/up pair shares one counter and one partial array: the
    // gate's slices are slots [0, S_first), the up's [S_first, S_all), and the last of all its
    // slices writes SiLU(gate) * up.  The partials are written and read with device-coherent
    // (agent scope) accesses, which go through to memory instead of a single XCD's L2; the wait
    // below makes the stores complete before the counter is incremented, so whoever sees the
    // final count sees them.
#pragma unroll
    for (int m = 0; m < M; m++)
        __hip_atomic_store(as_global(D.part + ((int64_t)m * D.S_all + D.slot0 + s) * D.Npad + row), acc[m],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int done = 0;
    if (lane == 0) done = __hip_atomic_fetch_add(as_global(D.cnt + g), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    done = __builtin_amdgcn_readfirstlane(done);
    if (done == D.S_all - 1) {
        // slots [s0, s1) of one activation row, 8 loads in flight at a time, added in ascending order
        auto slot_sum = [&](const float *pm, int s0, int s1) {
            float sum = 0.f;
            for (int k0 = s0; k0 < s1; k0 += 8) {
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; j++)
                    v[j] = (k0 + j < s1) ? __hip_atomic_load(as_global(pm + (int64_t)(k0 + j) * D.Npad), __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT)
                                         : 0.f;
#pragma unroll
                for (int j = 0; j < 8; j++) sum += v[j];
            }
            return sum;
        };
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float *pm = D.part + (int64_t)m * D.S_all * D.Npad + row;
            float *py = D.y + (int64_t)m * D.ldy + row;
            float out;
            if (EPI && D.epi == kEpiSiluPair) {
                const float gsum = slot_sum(pm, 0, D.S_first);
                const float usum = slot_sum(pm, D.S_first, D.S_all);
                out = gsum / (1.f + expf(-gsum)) * usum;  // SiLU(g) = g * sigma(g); -0 for g -> -inf
            } else {
                out = slot_sum(pm, 0, D.S_all);
                if (EPI && D.epi == kEpiAdd && row < D.N) out = gld<float>(py) + out;
            }
            if (row < D.N) gst(py, out);
        }
        if (lane == 0) __hip_atomic_store(as_global(D.cnt + g), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Index of the projection owning workgroup unit u (uniform binary search over the descriptors).
__device__ __forceinline__ int find_proj(const Desc *tab, int ndesc, int u) {
    int lo = 0, hi = ndesc - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (load_wgu_begin(tab + mid) <= u) lo = mid; else hi = mid - 1;
    }
    return lo;
}
// The launch's descriptors: a table in device memory, or the array in the kernel arguments.  The
// latter is addressed in the kernel-argument segment, where the kernel's only argument (the
// GemvParams, descriptor array first) starts at offset 0; taking the address of the parameter
// itself would make the compiler copy all of it to scratch memory.
__device__ __forceinline__ const Desc *desc_table(const GemvParams &P) {
    static_assert(offsetof(GemvParams, d) == 0, "inline descriptors open the kernel arguments");
    return P.descs ? P.descs : (const Desc *)(uintptr_t)__builtin_amdgcn_kernarg_segment_ptr();
}

// One workgroup unit: kWaves wave units of one projection, one per wave.  The LDS table is
// rebuilt (between two barriers, so all waves of the workgroup take part) when the projection
// changes.
template <int MASK, int M, bool EPI, bool BI>
__device__ __forceinline__ void run_wgu(const GemvParams &P, int u, int &cur, Desc &D, uint32_t *lds, float *red, int wid,
                                        int lane) {
    // Units are visited in increasing order: search only for the first one, then step forward.
    // Inline descriptors: their first units are in the kernel arguments beside them.
    const Desc *tab = desc_table(P);
    int p;
    if (!P.descs) {
        p = 0;
#pragma unroll
        for (int i = 1; i < kInlineDescs; i++) p += (i < P.ndesc && P.wgu_begin[i] <= u) ? 1 : 0;
    } else if (cur < 0) {
        p = find_proj(tab, P.ndesc, u);
    } else {
        p = cur;
        while (p + 1 < P.ndesc && load_wgu_begin(tab + p + 1) <= u) p++;
    }
    bool rebuild = false;
    if (p != cur) {
        D = load_desc(tab + p);
        rebuild = true;
        cur = p;
    }
    // All waves take part in the table rebuild (two barriers), after issuing their first loads.
    auto hook = [&]() {
        if constexpr ((MASK & ((1 << CB4) | (1 << CB8))) != 0) {
            if (rebuild) {
                __syncthreads();
                if constexpr ((MASK & (1 << CB4)) != 0) if (D.fmt == CB4) build_table<CB4>(lds, D);
                if constexpr ((MASK & (1 << CB8)) != 0) if (D.fmt == CB8) build_table<CB8>(lds, D);
                __syncthreads();
            }
        }
    };
    const int wu = (u - D.wgu_begin) * kWaves + wid;
    if (wu < D.wu_count) {
        if constexpr (MASK == kMaskCB48) {
            // two formats: one branch or the other (not two independent ifs, which let
            // the compiler keep values of both bodies live at once)
            if (D.fmt == CB4) run_unit<CB4, M, EPI, BI>(D, wu, lane, lds, red, hook);
            else run_unit<CB8, M, EPI, BI>(D, wu, lane, lds, red, hook);
        } else {
            if constexpr ((MASK & (1 << Q4_0)) != 0) if (D.fmt == Q4_0) run_unit<Q4_0, M, EPI, BI>(D, wu, lane, lds, red, hook);
            if constexpr ((MASK & (1 << CB4)) != 0) if (D.fmt == CB4) run_unit<CB4, M, EPI, BI>(D, wu, lane, lds, red, hook);
            if constexpr ((MASK & (1 << CB8)) != 0) if (D.fmt == CB8) run_unit<CB8, M, EPI, BI>(D, wu, lane, lds, red, hook);
            if constexpr ((MASK & (1 << TQ2)) != 0) if (D.fmt == TQ2) run_unit<TQ2, M, EPI, BI>(D, wu, lane, lds, red, hook);
            if constexpr ((MASK & (1 << AQ1X16)) != 0) if (D.fmt == AQ1X16) run_unit<AQ1X16, M, EPI, BI>(D, wu, lane, lds, red, hook);
            if constexpr ((MASK & (1 << TQ2I8)) != 0) if (D.fmt == TQ2I8) run_unit<TQ2I8, M, EPI, BI>(D, wu, lane, lds, red, hook);
        }
    } else {
        hook();
    }
}

// Every instance is compiled for WQD_WG_PER_CU (2) resident 8-wave workgroups per CU, i.e. 4
// waves per SIMD and at most 128 VGPRs, except the 9..16-row batch-invariant ones (one workgroup
// per CU, 256 VGPRs); the launch sizes its persistent grid from the same constants (the runtime
// occupancy query under-reports kernels without AGPRs).
constexpr int kMinWavesPerEU = WQD_WG_PER_CU * kWaves / 4;

// Persistent kernel over a list of projections whose formats are in MASK.  Workgroup units
// [0, pool_begin) are split into equal contiguous ranges, one per workgroup; the rest are handed
// out one by one from a device-wide counter to whichever workgroup is free, which evens out the
// finish times (workgroups on different XCDs stream at different speeds).  EPI: the instance
// applies the descriptors' epilogues (lists without any use the instance without that code).
// BI: the batch-invariant instance (every M on the matrix cores, one chain per quad).
template <int MASK, int M, bool EPI, bool BI = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(M > kMaxM ? kThreads / 256 : kMinWavesPerEU))) void gemv_kernel(GemvParams P) {
    __shared__ uint32_t lds[LdsSizeMask<MASK>::dwords];
    __shared__ float red[kWaves * (M < 4 ? M : 4) * 64];  // workgroup-split sums
    __shared__ int next_u;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int total = P.total_wgu;
    // The dynamic tail is compiled in only when WQD_POOL_PERCENT > 0 (a second copy of the unit
    // loop costs registers in every instance).
    constexpr bool kPool = WQD_POOL_PERCENT > 0;
    const int nstatic = (kPool && P.ctr) ? P.pool_begin : total;
    const int per = nstatic / (int)gridDim.x, rem = nstatic % (int)gridDim.x;
    const int b = blockIdx.x;
    const int u0 = b * per + min(b, rem);
    const int u1 = u0 + per + (b < rem ? 1 : 0);
    // (after the arithmetic on the arguments, so that their loads go out with the stamp's
    // pointer in one round trip: a launch without a table has no stamp to wait for)
    if (stale_table(P.stamp, P.fp, P.stale)) return;
    int cur = -1;
    Desc D;
    for (int u = u0; u < u1; u++) run_wgu<MASK, M, EPI, BI>(P, u, cur, D, lds, red, wid, lane);
    if (kPool && P.ctr) {
        while (true) {
            __syncthreads();
            if (threadIdx.x == 0)
                next_u = nstatic + __hip_atomic_fetch_add(as_global(P.ctr), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const int u = __builtin_amdgcn_readfirstlane(next_u);
            if (u >= total) break;
            run_wgu<MASK, M, EPI, BI>(P, u, cur, D, lds, red, wid, lane);
        }
        // Every workgroup has taken its last index once it reaches here; the last one to arrive
        // resets the counters for the next launch on this workspace.
        if (threadIdx.x == 0) {
            if (__hip_atomic_fetch_add(as_global(P.ctr + 1), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (int)gridDim.x - 1) {
                __hip_atomic_store(as_global(P.ctr), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(as_global(P.ctr + 1), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

template <int MASK, bool EPI, bool BI>
GemvFn gemv_fn_var(int M) {
    switch (M) {
    case 1: return gemv_kernel<MASK, 1, EPI, BI>;
    case 2: return gemv_kernel<MASK, 2, EPI, BI>;
    case 3: return gemv_kernel<MASK, 3, EPI, BI>;
    case 4: return gemv_kernel<MASK, 4, EPI, BI>;
    case 5: return gemv_kernel<MASK, 5, EPI, BI>;
    case 6: return gemv_kernel<MASK, 6, EPI, BI>;
    case 7: return gemv_kernel<MASK, 7, EPI, BI>;
    case 8: return gemv_kernel<MASK, 8, EPI, BI>;
    }
    return nullptr;
}
// Batch-invariant instances for a verify of 9..16 rows in one pass (one workgroup per CU: the
// four activation quads need up to 256 registers).
template <int MASK>
GemvFn gemv_fn_bi_wide(int M) {
    switch (M) {
    case 9: return gemv_kernel<MASK, 9, true, true>;
    case 10: return gemv_kernel<MASK, 10, true, true>;
    case 11: return gemv_kernel<MASK, 11, true, true>;
    case 12: return gemv_kernel<MASK, 12, true, true>;
    case 13: return gemv_kernel<MASK, 13, true, true>;
    case 14: return gemv_kernel<MASK, 14, true, true>;
    case 15: return gemv_kernel<MASK, 15, true, true>;
    case 16: return gemv_kernel<MASK, 16, true, true>;
    }
    return nullptr;
}
// The batch-invariant instances always carry the epilogue code (one set of them per format).
// WIDE: with the 9..16-row batch-invariant instances.
template <int MASK, bool WIDE = true>
GemvFn gemv_fn(int M, bool epi, bool bi) {
    if (bi) {
        if (M <= kMaxM) return gemv_fn_var<MASK, true, true>(M);
        if constexpr (WIDE) return gemv_fn_bi_wide<MASK>(M);
        return nullptr;
    }
    return epi ? gemv_fn_var<MASK, true, false>(M) : gemv_fn_var<MASK, false, false>(M);
}

}  // namespace wqd
