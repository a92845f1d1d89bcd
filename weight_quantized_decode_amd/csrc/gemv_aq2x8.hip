// AQ2X8 dequantize-and-multiply kernels (gfx950), on the transposed tile layout of layout.h: one
// wavefront lane per group of 8 weights, and 8 rows per 16-byte lane load.
//
// The weights of row n, group g are s_n * (C_0[c0] + C_1[c1]) with two 8-bit codes into two
// codebooks of 256 fp16 8-vectors (trapetum "Benchmarks", the additive vector-quantization GEMV
// section), so
//     y_n = s_n * sum_g ( T_0,g[c0(n,g)] + T_1,g[c1(n,g)] ),   T_b,g[c] = sum_j C_b[c][j] x[8g+j]:
// a per-group lookup table built from the activations, after which only the codes are read.
//
// M = 1, lookup tables:
//   * For one K-slice of 64 groups the workgroup builds T in LDS as dword (c*64 + g) holding the
//     pair (T_0,g[c], T_1,g[c]) in fp16: 64 KiB.  T is the product C_b (256 x 8) . X (8 x 64),
//     X[j][g] = x[8g+j], on the 4x4x4 matrix core: with 4 codebook rows broadcast as the A
//     operand and each lane's own group activations as B, one pair of MFMAs (k = 0..3, 4..7)
//     leaves T[c][g = lane] for 4 codes in 4 registers of lane g (exact fp16 products, fp32
//     sums), already in table order.  Each wave builds 256/W codes of both codebooks.
//   * Two tables alternate: the table of the next slice is built while the current one is read,
//     with one workgroup barrier per slice.
//   * Lane g reads only bank g, so the lookups never conflict: two LDS reads per 8 weights (the
//     addresses made by one v_perm each from the code bytes) and one v_fma_mix that adds the low
//     fp16 half of one word to the high half of the other in fp32.
//   * The 64 lanes' terms of a row are summed by a transposed butterfly in a fixed order: per tile
//     the permlane32 and permlane16 swap stages fold 8 rows x 64 lanes into 2 values per lane,
//     which accumulate over the slices of a piece; the DPP stages finish the sum once per piece.
// M = 2, one table for both rows: dword (b*256 + c)*64 + g holds the fp16 pair (T_b,g[c] of row 0,
//   of row 1), 128 KiB, so it is single-buffered (a barrier, the build, a barrier per slice); the
//   same two lookups per 8 weights give both rows' terms.
// M = 3..8 (and batch-invariant calls), direct decode (at M = 3 and 4 the host runs row parts on
//   the table kernels instead): the codebooks sit in LDS, each lane decodes
//   its group's 8 rows (two 16-byte LDS reads and one packed fp16 add per row) and multiplies them
//   with each activation row; the 8 row sums are reduced across lanes per tile.
//
// Work: see AqDesc.  A workgroup walks its pieces in order, slice by slice; the loads of the next
// slice (of the same or the next piece) are in flight while a slice is processed.  With b > 1
// K-splits a piece stores one tagged 64-bit partial per row (no fence: a slot is either still zero or holds
// the tag and the value), and once all of its own pieces are done each of the b workgroups of a
// chunk adds the b partials, in split order, of its share of the chunk's rows.
#include <stddef.h>

#include "gemv_impl.h"

namespace wqd {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t u32(float f) { return __builtin_bit_cast(uint32_t, f); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return f32(uint32_t(__builtin_amdgcn_update_dpp(0, int(u32(v)), CTRL, 0xF, 0xF, false)));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRor8 = 0x128;         // row_ror:8 (lane i <-> i^8 within 16)
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i within 8

// Sum over the 64 lanes of v[r] for each of 8 rows r, in a fixed order, in two stages.
// fold_rows8: lanes l, l^32 and l^16 -> two values per lane, w[j] holding row j + 2*bit4 + 4*bit5
// of the lane (summed over its 4 lanes {l, l^16, l^32, l^48}).
__device__ __forceinline__ void fold_rows8(const float (&v)[8], float (&w)[2]) {
    float u[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {  // lanes l, l^32: row r in lanes 0-31, row r+4 in lanes 32-63
        const auto s = __builtin_amdgcn_permlane32_swap(u32(v[r]), u32(v[r + 4]), false, false);
        u[r] = f32(s[0]) + f32(s[1]);
    }
#pragma unroll
    for (int r = 0; r < 2; r++) {  // lanes l, l^16: row r + 2*bit4 + 4*bit5
        const auto s = __builtin_amdgcn_permlane16_swap(u32(u[r]), u32(u[r + 2]), false, false);
        w[r] = f32(s[0]) + f32(s[1]);
    }
}
// finish_rows8: the rest of the sum (lanes l^8, then the 8 lanes of an octet).  On return lanes
// 8r..8r+7 all hold the sum of row r.
__device__ __forceinline__ float finish_rows8(const float (&w)[2], int lane) {
    const float x0 = w[0] + dpp<kDppRor8>(w[0]);  // lanes l, l^8
    const float x1 = w[1] + dpp<kDppRor8>(w[1]);
    float z = (lane & 8) ? x1 : x0;               // row bit3 + 2*bit4 + 4*bit5
    z = z + dpp<kDppXor1>(z);
    z = z + dpp<kDppXor2>(z);
    z = z + dpp<kDppHalfMirror>(z);
    return z;
}

template <typename T>
__device__ __forceinline__ T load_uniform(const T *p) {
    static_assert(sizeof(T) % 4 == 0, "whole dwords");
    uint32_t w[sizeof(T) / 4];
    cu32p s = scalar_ptr(p);
#pragma unroll
    for (unsigned i = 0; i < sizeof(T) / 4; i++) w[i] = s[i];
    T D;
    __builtin_memcpy(&D, w, sizeof(T));
    return D;
}

// Descriptor p, read with scalar loads either from the table or, for a single projection, from
// the kernel argument itself (AqParams::d0 sits at the start of the kernarg segment).  Choosing
// between two pointers rather than two structs keeps the descriptor out of scratch memory.
__device__ __forceinline__ AqDesc get_desc(const AqParams &P, int p) {
    static_assert(offsetof(AqParams, d0) == 0, "d0 leads the kernel arguments");
    p = min(max(p, 0), P.ndesc - 1);  // never read outside the table
    const AqDesc *d = P.descs ? P.descs + p
                              : (const AqDesc *)(uintptr_t)__builtin_amdgcn_kernarg_segment_ptr();
    return load_uniform(d);
}

// A piece of this workgroup's work list (wave-uniform).
struct Piece {
    int p;          // projection; == ndesc past the end of the list
    int j;          // piece index within the projection
    int rb0, rb1;   // 8-row blocks [rb0, rb1)
    int s0, s1;     // K-slices [s0, s1)
    int split;
};

// The first piece of this workgroup at or after (projection p, piece j); j < 0: start of p.
__device__ __forceinline__ Piece find_piece(const AqParams &P, int wg, int p, int j) {
    while (p < P.ndesc) {
        const AqDesc D = get_desc(P, p);
        if (j < 0) {
            j = (wg - D.off) % P.nwg;
            if (j < 0) j += P.nwg;
        }
        if (j < D.npieces) {
            Piece q;
            q.p = p;
            q.j = j;
            q.split = j / D.a;
            const int chunk = j - q.split * D.a;
            q.rb0 = chunk * D.nrb;
            q.rb1 = min(D.RB, q.rb0 + D.nrb);
            q.s0 = q.split * D.ns;
            q.s1 = min(D.KS, q.s0 + D.ns);
            return q;
        }
        p++;
        j = -1;
    }
    Piece q;
    q.p = P.ndesc;
    q.j = 0;
    q.rb0 = q.rb1 = q.s0 = q.s1 = q.split = 0;
    return q;
}
__device__ __forceinline__ Piece next_piece(const AqParams &P, int wg, const Piece &q) {
    return find_piece(P, wg, q.p, q.j + P.nwg);
}

// Row block (from the piece's first) of tile i of wave wid in pass `pass` of a slice: a pass covers
// W * RW consecutive row blocks, RW consecutive ones per wave (each wave's tiles of a slice are
// one contiguous run of RW KiB; wave-interleaved tiles measured 2.5% slower on the 70B MLP).
template <int RW, int W>
__device__ __forceinline__ int tile_rb(int wid, int i, int pass) {
    return RW * (wid + W * pass) + i;
}

// Tile loader running ahead of the processing.  It walks units (piece, slice, pass): each slice
// of a piece is read in NP passes of RW tiles per wave (tile_rb), so one table serves
// NP * W * RW row blocks.
template <int RW, int W, int NP>
struct Loader {
    const uint8_t *base;   // code plane (wave-uniform; the lane's 16 bytes are added at the load)
    int64_t s_stride;      // bytes between slices (R8 = Npad/8 KiB)
    int s_max, rb_max;     // last slice and row block of the plane (tile addresses stay inside)
    int rb0, rb1;          // the piece's row blocks
    int wv;                // this wave
    const uint16_t *x, *cbk;  // operands of the slice's table / activation stage
    int64_t ldx;
    int G;
    Piece q;  // current piece
    int s, pass;
    bool done;

    // (the next piece is looked up only when this one ends: at the start of the kernel, one
    // descriptor read stands before the first loads instead of two)
    __device__ __forceinline__ void setup(const AqParams &P, const Piece n, int wg, int wid, int lane) {
        q = n;
        s = n.s0;
        pass = 0;
        const AqDesc D = get_desc(P, n.p);
        base = D.codes;
        s_stride = int64_t(D.Npad / 8) * 1024;
        x = D.x;
        cbk = D.cbk;
        ldx = D.ldx;
        G = D.G;
        s_max = D.KS - 1;
        rb_max = D.Npad / 8 - 1;
        rb0 = n.rb0;
        wv = wid;
        rb1 = n.rb1;
    }
    // A missing tile (past the piece, or past the end of the list) still takes its place in the
    // ring (every load stays unconditional): it reads 1 KiB of the codebooks, which the table
    // build keeps in L2, instead of HBM.
    __device__ __forceinline__ const uint8_t *addr(int i) const {
        const int r = rb0 + tile_rb<RW, W>(wv, i, pass);
        return (done || r >= rb1) ? reinterpret_cast<const uint8_t *>(cbk)
                                  : base + int64_t(min(s, s_max)) * s_stride + int64_t(min(r, rb_max)) * 1024;
    }
    // After the tiles of a unit: step to the next pass, slice or piece.
    __device__ __forceinline__ void step(const AqParams &P, int wg, int wid, int lane) {
        if (done) return;
        if (++pass < NP) return;
        pass = 0;
        if (++s < q.s1) return;
        const Piece qn = next_piece(P, wg, q);
        if (qn.p >= P.ndesc) {
            done = true;
            s = q.s1 - 1;
        } else {
            setup(P, qn, wg, wid, lane);
        }
    }
};

constexpr int kSpinMax = 1 << 22;   // polls of a missing partial before giving up (NaN result)
constexpr int kFinLoads = 8;        // partial loads in flight per row in the finalize (32 measured slower)

// Adds the b tagged partials of rows of the pieces this workgroup ran, then scales and writes y
// and clears the slots.  The rows of a row chunk are shared out over its b splits: the workgroup
// that ran split t finalizes rows [t*R/b, (t+1)*R/b) of the chunk's R rows.  A row takes L lanes
// (L = b/8 rounded up to a power of two): lane j of the row loads partials 8j..8j+7 in one round
// and adds them in split order, then the L lane sums are combined in a fixed tree.  The shares of
// all of the workgroup's pieces are finalized at once: each share takes whole waves (its rows x L
// lanes, rounded up to 64), numbered over the pieces in order, and wave w takes numbers w, w + W,
// ..., so the partial loads of the pieces are in flight together rather than one memory round
// trip per piece.  Runs after all of the workgroup's own pieces; a partial not yet written is
// polled again (bounded), and its writer never waits on another workgroup, so the wait ends.
template <int M, int W>
__device__ __forceinline__ void finalize(const AqParams &P, int wg, int wid, int lane) {
    int first = 0;  // first wave number of the piece's share
    for (Piece q = find_piece(P, wg, 0, -1); q.p < P.ndesc; q = next_piece(P, wg, q)) {
        const AqDesc D = get_desc(P, q.p);
        if (D.b == 1) continue;
        int L = 1;
        while (L * kFinLoads < D.b) L *= 2;  // (b <= 64 keeps L <= 8)
        const int r0 = q.rb0 * 8, R = min((q.rb1 - q.rb0) * 8, D.N - r0);
        const int lo = r0 + (R * q.split) / D.b, hi = r0 + (R * (q.split + 1)) / D.b;
        const int nw = ((hi - lo) * L + 63) / 64;  // waves of this share
        const int sub = lane & (L - 1);            // this lane's group of partials
        const int t0 = sub * kFinLoads;
        // wave numbers [first, first + nw) are this share's; wave wid takes those = wid mod W
        for (int v = first + ((wid - first) % W + W) % W; v < first + nw; v += W) {
            const int k = ((v - first) * 64 + lane) / L;  // row of the share (L lanes per row)
            const bool live = k < hi - lo;                // (every lane still takes the combine)
            const int row = lo + min(k, hi - lo - 1);
            const float sc = half_bits_to_float(gld<uint16_t>(D.rscale + row));
#pragma unroll
            for (int m = 0; m < M; m++) {
                uint64_t *slot = D.part + (int64_t(m) * D.b) * D.Npad + row;
                uint64_t v8[kFinLoads];
#pragma unroll
                for (int j = 0; j < kFinLoads; j++)
                    v8[j] = (live && t0 + j < D.b) ? __hip_atomic_load(as_global(slot + int64_t(t0 + j) * D.Npad), __ATOMIC_RELAXED,
                                                                      __HIP_MEMORY_SCOPE_AGENT)
                                                   : (uint64_t(kAqTag) << 32);
                float sum = 0.f;
                int ok = 1;
#pragma unroll
                for (int j = 0; j < kFinLoads; j++) {
                    int spins = 0;
                    while (uint32_t(v8[j] >> 32) != kAqTag && spins < kSpinMax) {
                        __builtin_amdgcn_s_sleep(2);
                        v8[j] = __hip_atomic_load(as_global(slot + int64_t(t0 + j) * D.Npad), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                        spins++;
                    }
                    ok &= uint32_t(v8[j] >> 32) == kAqTag;
                    if (t0 + j < D.b) sum += f32(uint32_t(v8[j]));  // split order
                }
                // combine the L lanes of the row: pairs, then pairs of pairs (a fixed order)
                for (int o = 1; o < L; o <<= 1) {
                    sum += __shfl_xor(sum, o);
                    ok &= __shfl_xor(ok, o);
                }
                if (live && sub == 0) gst(D.y + int64_t(m) * D.ldy + row, ok ? sum * sc : __builtin_nanf(""));
                if (live)
                    for (int j = 0; j < kFinLoads && t0 + j < D.b; j++)
                        __hip_atomic_store(as_global(slot + int64_t(t0 + j) * D.Npad), uint64_t(0), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        first += nw;
    }
}

template <int M, bool LUT>
struct LdsWords {
    static constexpr int value = LUT ? 2 * 256 * 64 : 2048 + 256 * M;
};

// ------------------------------------------------------------------------------------------
// The kernel.  RW: 8-row blocks per wave per slice (a piece has at most W * RW of them).
//
// Pipeline: the tiles (RW per wave) and operands of the next two slices are in flight while a
// slice is processed.  At the start of a slice the wave waits for that slice's loads (the oldest
// it has in flight), then issues the loads of the slice two ahead, then builds the table and
// processes.  With W * RW = 64 row blocks a workgroup keeps about 128 KiB in flight.
// ------------------------------------------------------------------------------------------

// Per-slice operands of the table build (M = 1: activation pairs of the two 32-group blocks and
// this wave's two codebook rows) or of the stage (M > 1: one activation row, a codebook part).
struct SliceOps {
    u32x2 B[2], A[2];
    u32x2 B1[2];  // M = 2 tables: the second activation row's halves
    u32x4 X, C;
    int gval;  // groups of the slice inside K (M = 1: the table masks the rest)
};

// fp32 T_0 (low half of d0) + T_1 (high half of d1), both fp16 table entries.
__device__ __forceinline__ float add_lo_hi(uint32_t d0, uint32_t d1) {
    float r;
    __asm__("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(d0), "v"(d1));
    return r;
}
// fp32 sums of the low halves and of the high halves of two fp16 pairs.
__device__ __forceinline__ float add_lo_lo(uint32_t d0, uint32_t d1) {
    float r;
    __asm__("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(d0), "v"(d1));
    return r;
}
__device__ __forceinline__ float add_hi_hi(uint32_t d0, uint32_t d1) {
    float r;
    __asm__("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(d0), "v"(d1));
    return r;
}
// fp16 pair (a, b), round to nearest even.
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
}

// M = 1: the 128 KiB table allows one workgroup per CU, i.e. 2 waves per SIMD, so each wave may
// use 256 VGPRs (the compiler would otherwise aim for more waves than can ever be resident).
// BI: the batch-invariant instance, which takes the direct decode at every M (M = 1 included), so
// that a row's arithmetic does not depend on M.
template <int M, int RW, int NP, bool BI = false>
__global__ __launch_bounds__(aq_waves(M) * 64) __attribute__((amdgpu_waves_per_eu(1, aq_waves_per_simd(M))))
void aq_kernel(AqParams P) {
    constexpr int W = aq_waves(M);  // waves per workgroup
    constexpr bool LUT = (M <= 2 && !BI);  // lookup tables (else the direct decode)
    constexpr bool LUT2 = LUT && M == 2;   // one table of both activation rows, single-buffered
    __shared__ uint32_t lds[LdsWords<M, LUT>::value];

    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wg = blockIdx.x;

    Piece pp = find_piece(P, wg, 0, -1);  // piece being processed
    if (pp.p >= P.ndesc) return;          // no work for this workgroup (same for all its waves)
    int ps = pp.s0;                       // slice being processed

    AqDesc pd = get_desc(P, pp.p);        // its descriptor

    Loader<RW, W, NP> ld;
    static_assert(LUT || NP == 1, "passes share a lookup table (M = 1)");
    ld.done = false;
    ld.setup(P, pp, wg, wid, lane);

    // M = 1 table share of this wave: NQ quads of codes (4NQ codes from 4NQ*wid) of both
    // codebooks.  Its MFMA A operands hold 4NQ blocks (codebook, quad, k-half) of 4 codebook
    // rows: block n = 16r + b sits in lanes 4b..4b+3 of A[r], as codebook n / 2NQ, quad
    // (n % 2NQ) / 2, k-half n % 2.
    constexpr int NQ = 64 / W;
    static_assert(!LUT || (4 * NQ <= 32 && W * NQ == 64), "the A operands hold the wave's blocks");

    // Issue the loads of the loader's slice: operands first, then the RW tiles; step the loader.
    // Every load is unconditional with a clamped address (a load under a lane condition makes
    // the compiler wait for it at once); groups past G are zeroed where the operands are used.
    auto load_slice = [&](u32x4 (&t)[RW], SliceOps &o) __attribute__((always_inline)) {
        if constexpr (LUT) {
            o.gval = ld.G - ld.s * 64;
            const int g = min(ld.s * 64 + lane, ld.G - 1);  // lane = group
#pragma unroll
            for (int h = 0; h < 2; h++) o.B[h] = gld<u32x2>(ld.x + int64_t(g) * 8 + 4 * h);
            if constexpr (LUT2) {
#pragma unroll
                for (int h = 0; h < 2; h++) o.B1[h] = gld<u32x2>(ld.x + ld.ldx + int64_t(g) * 8 + 4 * h);
            }
#pragma unroll
            for (int r = 0; r < (4 * NQ + 15) / 16; r++) {
                const int n = min(16 * r + (lane >> 2), 4 * NQ - 1);
                const int cb = n / (2 * NQ), quad = (n % (2 * NQ)) / 2, half = n % 2;
                const int code = wid * 4 * NQ + 4 * quad + (lane & 3);
                o.A[r] = gld<u32x2>(ld.cbk + (int64_t(cb) * 256 + code) * 8 + 4 * half);
            }
        } else {
            const int g = min(ld.s * 64 + lane, ld.G - 1);
            o.X = gld<u32x4>(ld.x + int64_t(min(wid, M - 1)) * ld.ldx + int64_t(g) * 8);
            o.C = gld<u32x4>(reinterpret_cast<const uint8_t *>(ld.cbk) + (threadIdx.x & 511) * 16);
        }
#pragma unroll
        for (int i = 0; i < RW; i++) {  // uniform tile base + the lane's 16 bytes
#if WQD_NT_CODES
            t[i] = __builtin_nontemporal_load((const u32x4 __attribute__((address_space(1))) *)(uintptr_t)(ld.addr(i) + lane * 16));
#else
            t[i] = gld<u32x4>(ld.addr(i) + lane * 16);
#endif
        }
        ld.step(P, wg, wid, lane);
    };
    // Wait for a slice's tiles and operands: an empty asm statement that reads them.
    auto settle_tiles = [&](u32x4 (&t)[RW]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RW; i++) __asm__ volatile("" ::"v"(t[i]));
    };
    auto settle_ops = [&](SliceOps &o) __attribute__((always_inline)) {
        if constexpr (LUT) {
            __asm__ volatile("" ::"v"(o.B[0]), "v"(o.B[1]), "v"(o.A[0]), "v"(o.A[1]));
            if constexpr (LUT2) __asm__ volatile("" ::"v"(o.B1[0]), "v"(o.B1[1]));
        } else {
            __asm__ volatile("" ::"v"(o.X), "v"(o.C));
        }
    };

    // per row block and activation row: two folded row sums (see fold_rows8), finished once per
    // piece
    constexpr int NACC = 2 * M;
    float acc[NP][RW][NACC];
#pragma unroll
    for (int p = 0; p < NP; p++)
#pragma unroll
        for (int i = 0; i < RW; i++)
#pragma unroll
            for (int r = 0; r < NACC; r++) acc[p][i][r] = 0.f;

    int tb = 0;   // M = 1: table buffer of the slice being processed

    // Piece epilogue: row sums -> y (b == 1) or this split's tagged partial slots.
    auto epilogue = [&](const Piece &q, const AqDesc &D) __attribute__((always_inline)) {
#pragma unroll
        for (int pi = 0; pi < NP * RW; pi++) {
            const int p = pi / RW, i = pi % RW;
            const int rb = q.rb0 + tile_rb<RW, W>(wid, i, p);
            const int row = rb * 8 + (lane >> 3);
            const bool ok = (lane & 7) == 0 && rb < q.rb1 && row < D.N && q.split < D.b;
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float w2[2] = {acc[p][i][2 * m], acc[p][i][2 * m + 1]};
                const float z = finish_rows8(w2, lane);
                if (ok) {
                    if (D.b == 1) {
                        // (the scale is loaded here, not ahead: an early load's result would be
                        // waited for behind every tile in flight)
                        const float sc = half_bits_to_float(gld<uint16_t>(D.rscale + row));
                        gst(D.y + int64_t(m) * D.ldy + row, z * sc);
                    } else {
                        const uint64_t v = (uint64_t(kAqTag) << 32) | u32(z);
                        __hip_atomic_store(as_global(D.part + (int64_t(m) * D.b + q.split) * D.Npad + row), v, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < NACC; r++) acc[p][i][r] = 0.f;
        }
    };

    // M = 1: build the table of a slice (its operands o) into table buffer tb.
    auto build_table = [&](const SliceOps &o, int tb) __attribute__((always_inline)) {
        const bool in = lane < o.gval;  // groups past K read as zero
        const u32x2 B0 = in ? o.B[0] : u32x2{0u, 0u}, B1 = in ? o.B[1] : u32x2{0u, 0u};
        uint32_t *tab = lds + tb * (256 * 64);
        if constexpr (LUT2) {
            // dword (cb*256 + c)*64 + g holds (T_cb[c] for row 0, for row 1) of group g
            const u32x2 R0 = in ? o.B1[0] : u32x2{0u, 0u}, R1 = in ? o.B1[1] : u32x2{0u, 0u};
            static_for<NQ>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                static_for<2>([&](auto cc) {
                    constexpr int cb = decltype(cc)::value;
                    constexpr int n0 = cb * 2 * NQ + 2 * q, n1 = n0 + 1;
                    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
                    const f32x4 D0 = mfma_xw<n1 % 16>(o.A[n1 / 16], B1, mfma_xw<n0 % 16>(o.A[n0 / 16], B0, z));
                    const f32x4 D1 = mfma_xw<n1 % 16>(o.A[n1 / 16], R1, mfma_xw<n0 % 16>(o.A[n0 / 16], R0, z));
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        tab[(cb * 256 + wid * 4 * NQ + 4 * q + i) * 64 + lane] = pack_h2(D0[i], D1[i]);
                });
            });
            return;
        }
        static_for<NQ>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            f32x4 D[2];
            static_for<2>([&](auto cc) {
                constexpr int cb = decltype(cc)::value;
                constexpr int n0 = cb * 2 * NQ + 2 * q, n1 = n0 + 1;  // k-halves 0 and 1
                const f32x4 d = mfma_xw<n0 % 16>(o.A[n0 / 16], B0, f32x4{0.f, 0.f, 0.f, 0.f});
                D[cb] = mfma_xw<n1 % 16>(o.A[n1 / 16], B1, d);
            });
            // register i of lane g: T_b[code 4NQ*wid + 4q + i][group g]
#pragma unroll
            for (int i = 0; i < 4; i++) tab[(wid * 4 * NQ + 4 * q + i) * 64 + lane] = pack_h2(D[0][i], D[1][i]);
        });
    };

    // M > 1: stage the activations of a slice.
    auto slice_start = [&](const SliceOps &o) __attribute__((always_inline)) {
        const int G = pd.G;
        if constexpr (LUT) {
        } else {
            const bool in = ps * 64 + lane < G;
            const u32x4 X = in ? o.X : u32x4{0u, 0u, 0u, 0u};
            lds_barrier();  // every wave is done with the previous stage
            u32x4 *cbl = reinterpret_cast<u32x4 *>(lds);
            u32x4 *xl = cbl + 512;
            if (threadIdx.x < 512) cbl[threadIdx.x] = o.C;
            if (wid < M) xl[wid * 64 + lane] = X;  // (waves >= M loaded a copy of row M-1)
            lds_barrier();
        }
    };

    // One tile: this lane's group for 8 rows of row block i (M = 1: lk selects the table).
    auto process = [&](const u32x4 &v, float (&a)[NACC], uint32_t lk) __attribute__((always_inline)) {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        if constexpr (LUT2) {
            // codebook 0 entries in table half 0, codebook 1 in half 1 (byte 2 of the address);
            // each dword gives the term of both activation rows
            const uint32_t lk1 = lk | 0x10000u;
            float v0[8], v1[8];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t d0 = lds_word(lds, __builtin_amdgcn_perm(w4[t], lk, 0x0c020400u));
                const uint32_t d1 = lds_word(lds, __builtin_amdgcn_perm(w4[t], lk1, 0x0c020500u));
                const uint32_t d2 = lds_word(lds, __builtin_amdgcn_perm(w4[t], lk, 0x0c020600u));
                const uint32_t d3 = lds_word(lds, __builtin_amdgcn_perm(w4[t], lk1, 0x0c020700u));
                v0[2 * t] = add_lo_lo(d0, d1);
                v1[2 * t] = add_hi_hi(d0, d1);
                v0[2 * t + 1] = add_lo_lo(d2, d3);
                v1[2 * t + 1] = add_hi_hi(d2, d3);
            }
            float w[2];
            fold_rows8(v0, w);
            a[0] += w[0];
            a[1] += w[1];
            fold_rows8(v1, w);
            a[2] += w[0];
            a[3] += w[1];
        } else if constexpr (LUT) {
            float v[8];
#pragma unroll
            for (int t = 0; t < 4; t++) {  // word t: (c0, c1) of rows 2t and 2t+1
                // address (tb*256 + c)*256 + 4*lane: byte 0 from lk, byte 1 the code, byte 2 tb
                const uint32_t a0 = __builtin_amdgcn_perm(w4[t], lk, 0x0c020400u);
                const uint32_t a1 = __builtin_amdgcn_perm(w4[t], lk, 0x0c020500u);
                const uint32_t a2 = __builtin_amdgcn_perm(w4[t], lk, 0x0c020600u);
                const uint32_t a3 = __builtin_amdgcn_perm(w4[t], lk, 0x0c020700u);
                v[2 * t] = add_lo_hi(lds_word(lds, a0), lds_word(lds, a1));
                v[2 * t + 1] = add_lo_hi(lds_word(lds, a2), lds_word(lds, a3));
            }
            float w[2];
            fold_rows8(v, w);
            a[0] += w[0];
            a[1] += w[1];
        } else {
            // decode the 8 rows of this lane's group once, then take the activation rows one at a
            // time (staged in LDS), folding each row's 64 lane terms to two per lane
            const u32x4 *cbl = reinterpret_cast<const u32x4 *>(lds);
            const u32x4 *xl = cbl + 512;
            uint32_t wv[8][4];
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const uint32_t c0 = (w4[r >> 1] >> (16 * (r & 1))) & 0xFFu;
                const uint32_t c1 = (w4[r >> 1] >> (16 * (r & 1) + 8)) & 0xFFu;
                const u32x4 E0 = cbl[c0], E1 = cbl[256 + c1];
                const uint32_t e0[4] = {E0.x, E0.y, E0.z, E0.w}, e1[4] = {E1.x, E1.y, E1.z, E1.w};
#pragma unroll
                for (int k = 0; k < 4; k++) wv[r][k] = __builtin_bit_cast(uint32_t, as_h2(e0[k]) + as_h2(e1[k]));
            }
#pragma unroll
            for (int m = 0; m < M; m++) {
                const u32x4 X = xl[m * 64 + lane];
                const uint32_t xw[4] = {X.x, X.y, X.z, X.w};
                float val[8];
#pragma unroll
                for (int r = 0; r < 8; r++) {
                    float sm = 0.f;
#pragma unroll
                    for (int k = 0; k < 4; k++) sm = dot2(wv[r][k], xw[k], sm);
                    val[r] = sm;
                }
                float w2[2];
                fold_rows8(val, w2);
                a[2 * m] += w2[0];
                a[2 * m + 1] += w2[1];
            }
        }
    };

    // One slice: wait for it, prefetch the one two ahead, build, process, advance.  Returns true
    // after the last slice of the last piece.
    // M = 1: the operands of the slice after it (oa) are waited for too, and its table is built
    // into the other buffer before this slice's lookups; the barrier at the end makes it
    // complete for every wave and frees this slice's table for the slice after next.
    // A unit is one pass over a slice; the table of the next slice is built (and the barrier
    // taken) in the last pass.
    auto step = [&](auto pc, u32x4 (&cur)[RW], SliceOps &oc, SliceOps &oa, u32x4 (&nxt)[RW], SliceOps &on) __attribute__((always_inline)) -> bool {
        constexpr int pass = decltype(pc)::value;
        constexpr bool last = pass == NP - 1;
        settle_tiles(cur);
        if constexpr (LUT2) {
            if constexpr (pass == 0) settle_ops(oc);
        } else if constexpr (LUT) {
            if constexpr (last) settle_ops(oa);
        } else {
            settle_ops(oc);
        }
        load_slice(nxt, on);
        auto lookups = [&](uint32_t lk) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < RW; i++) {
                // (the ring slots past the piece's end hold no tile)
                if (pp.rb0 + tile_rb<RW, W>(wid, i, pass) < pp.rb1) process(cur[i], acc[pass][i], lk);
                // one tile at a time: hoisting the address math of every tile blows the register budget
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if constexpr (LUT2) {
            if constexpr (pass == 0) {  // the slice's table replaces the previous slice's
                lds_barrier();          // every wave is done with the previous table
                build_table(oc, 0);
                lds_barrier();          // the table is complete
            }
            lookups(uint32_t(lane) << 2);
        } else if constexpr (LUT) {
            if constexpr (last) build_table(oa, tb ^ 1);
            lookups((uint32_t(lane) << 2) | (uint32_t(tb) << 16));
            if constexpr (last) {
                lds_barrier();
                tb ^= 1;
            }
        } else {
            slice_start(oc);
            lookups(0);
        }
        if constexpr (!last) return false;
        if (++ps < pp.s1) return false;
        epilogue(pp, pd);
        const Piece pn = next_piece(P, wg, pp);
        if (pn.p >= P.ndesc) return true;
        pp = pn;
        ps = pp.s0;
        pd = get_desc(P, pp.p);
        return false;
    };

    // Three slice buffers: while slice s is processed, slices s+1 and s+2 are in flight.
    u32x4 buf0[RW], buf1[RW], buf2[RW];
    SliceOps ops0, ops1, ops2;
    load_slice(buf0, ops0);
    load_slice(buf1, ops1);
    if constexpr (LUT && !LUT2) {  // the first table (M = 2: built by the first slice's step)
        settle_ops(ops0);
        build_table(ops0, 0);
        lds_barrier();
    }
    // (the ring has 3 buffers and a slice NP passes: 3 * NP steps per round)
    while (true) {
        if (step(Int<0>{}, buf0, ops0, ops1, buf2, ops2)) break;
        if (step(Int<1 % NP>{}, buf1, ops1, ops2, buf0, ops0)) break;
        if (step(Int<2 % NP>{}, buf2, ops2, ops0, buf1, ops1)) break;
        if constexpr (NP == 2) {
            if (step(Int<1>{}, buf0, ops0, ops1, buf2, ops2)) break;
            if (step(Int<0>{}, buf1, ops1, ops2, buf0, ops0)) break;
            if (step(Int<1>{}, buf2, ops2, ops0, buf1, ops1)) break;
        }
    }
    finalize<M, W>(P, wg, wid, lane);
}

}  // namespace

AqFn aq_fn(int M, int RW, bool bi) {
    if (bi) {  // one row block per wave per slice at every M
        switch (M) {
        case 1: return aq_kernel<1, 1, 1, true>;
        case 2: return aq_kernel<2, 1, 1, true>;
        case 3: return aq_kernel<3, 1, 1, true>;
        case 4: return aq_kernel<4, 1, 1, true>;
        case 5: return aq_kernel<5, 1, 1, true>;
        case 6: return aq_kernel<6, 1, 1, true>;
        case 7: return aq_kernel<7, 1, 1, true>;
        case 8: return aq_kernel<8, 1, 1, true>;
        }
        return nullptr;
    }
#define WQD_AQ_CASE(m)                                   \
    case m:                                              \
        return RW == 1 ? aq_kernel<m, 1, 1> : aq_kernel<m, 2, 1>;
    switch (M) {
    case 1:  // RW: row blocks per wave per slice; 8 = two passes of 4
        if (RW <= 1) return aq_kernel<1, 1, 1>;
        if (RW == 2) return aq_kernel<1, 2, 1>;
        if (RW == 4) return aq_kernel<1, 4, 1>;
        return aq_kernel<1, 4, 2>;
    case 2:  // lookup tables: RW 4 = two passes of 2
        if (RW <= 1) return aq_kernel<2, 1, 1>;
        if (RW == 2) return aq_kernel<2, 2, 1>;
        return aq_kernel<2, 2, 2>;
        WQD_AQ_CASE(3)
        WQD_AQ_CASE(4)
        WQD_AQ_CASE(5)
        WQD_AQ_CASE(6)
        WQD_AQ_CASE(7)
        WQD_AQ_CASE(8)
    }
#undef WQD_AQ_CASE
    return nullptr;
}

}  // namespace wqd
