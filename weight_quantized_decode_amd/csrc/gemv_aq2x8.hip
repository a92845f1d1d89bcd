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
//   * For one K-slice of 64 groups the workgroup builds T in LDS, fp32, as dword
//     ((b*256 + c)*64 + g): 128 KiB.  T is the product C_b (256 x 8) . X (8 x 64), X[j][g] =
//     x[8g+j]; each of the 16 waves computes one (codebook, 32 codes) block with two 32x32x8 f16
//     MFMAs (exact fp16 products, fp32 sums) and, after a permlane32 swap, writes whole 64-group
//     rows of the table.
//   * Lane g reads only bank g, so the lookups never conflict: two LDS reads and two fp32 adds per
//     8 weights, the address made by one v_perm from the code byte.
//   * The 64 lanes' terms of a row are summed by a transposed butterfly in a fixed order: per tile
//     the permlane32 and permlane16 swap stages fold 8 rows x 64 lanes into 2 values per lane,
//     which accumulate over the slices of a piece; the DPP stages finish the sum once per piece.
// M = 2..8, direct decode: the codebooks sit in LDS, each lane decodes its group's 8 rows (two
//   16-byte LDS reads and one packed fp16 add per row) and multiplies them with each activation
//   row; the 8 row sums are reduced across lanes per tile.
//
// Work: see AqDesc.  A workgroup walks its pieces in order, slice by slice; the loads of the next
// slice (of the same or the next piece) are in flight while a slice is processed.  With b > 1
// K-splits a piece stores one tagged 64-bit partial per row (no fence: a slot is either still zero or holds
// the tag and the value), and the workgroup that ran the last split of a chunk adds the b
// partials of its rows, in split order, once all of its own pieces are done.
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
__device__ __forceinline__ float reduce_rows8(const float (&v)[8], int lane) {
    float w[2];
    fold_rows8(v, w);
    return finish_rows8(w, lane);
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

// Tile loader running ahead of the processing: (piece, slice), RW tiles per slice.
template <int RW, int W>
struct Loader {
    const uint8_t *base;   // code plane (wave-uniform; the lane's 16 bytes are added at the load)
    int64_t s_stride;      // bytes between slices (R8 = Npad/8 KiB)
    int s_max, rb_max;     // last slice and row block of the plane (tile addresses stay inside)
    int rb[RW];            // this wave's row blocks, clamped into the piece
    const uint16_t *x, *cbk;  // operands of the slice's table / activation stage
    int64_t ldx;
    int G;
    Piece q, qn;  // current piece and the next one (looked up a piece ahead)
    int s;
    bool done;

    // (n by value: step() passes the member qn, which is overwritten below)
    __device__ __forceinline__ void setup(const AqParams &P, const Piece n, int wg, int wid, int lane) {
        q = n;
        s = n.s0;
        qn = next_piece(P, wg, n);
        const AqDesc D = get_desc(P, n.p);
        base = D.codes;
        s_stride = int64_t(D.Npad / 8) * 1024;
        x = D.x;
        cbk = D.cbk;
        ldx = D.ldx;
        G = D.G;
        s_max = D.KS - 1;
        rb_max = D.Npad / 8 - 1;
#pragma unroll
        for (int i = 0; i < RW; i++) rb[i] = min(min(n.rb0 + wid + W * i, n.rb1 - 1), rb_max);
    }
    __device__ __forceinline__ const uint8_t *addr(int i) const {
        return base + int64_t(min(s, s_max)) * s_stride + int64_t(rb[i]) * 1024;
    }
    // After the last tile of a slice: step to the next slice (or piece).  Past the end of the
    // list the loader keeps re-reading the last tile, so the ring never has a hole.
    __device__ __forceinline__ void step(const AqParams &P, int wg, int wid, int lane) {
        if (done) return;
        if (++s < q.s1) return;
        if (qn.p >= P.ndesc) {
            done = true;
            s = q.s1 - 1;
        } else {
            setup(P, qn, wg, wid, lane);
        }
    }
};

constexpr int kSpinMax = 1 << 22;   // polls of a missing partial before giving up (NaN result)

// Adds the b tagged partials of rows [8*rb, 8*rb + 8) of every row block of this wave in the
// pieces whose last split this workgroup ran, in split order, then scales and writes y and clears
// the slots.  Runs after all of the workgroup's own pieces.
template <int M, int RW, int W>
__device__ __forceinline__ void finalize(const AqParams &P, int wg, int wid, int lane) {
    for (Piece q = find_piece(P, wg, 0, -1); q.p < P.ndesc; q = next_piece(P, wg, q)) {
        const AqDesc D = get_desc(P, q.p);
        if (D.b == 1 || q.split != D.b - 1) continue;
        const int i = lane >> 3, r = lane & 7;
        const int rb = q.rb0 + wid + W * i;
        const int row = rb * 8 + r;
        if (i >= RW || rb >= q.rb1 || row >= D.N) continue;
        const float sc = half_bits_to_float(gld<uint16_t>(D.rscale + row));
#pragma unroll
        for (int m = 0; m < M; m++) {
            uint64_t *slot = D.part + (int64_t(m) * D.b) * D.Npad + row;
            float sum = 0.f;
            bool ok = true;
            // up to 8 slot loads in flight; a slot still untagged is polled again (bounded)
            for (int t0 = 0; t0 < D.b; t0 += 8) {
                uint64_t v[8];
#pragma unroll
                for (int j = 0; j < 8; j++)
                    v[j] = (t0 + j < D.b) ? __hip_atomic_load(as_global(slot + int64_t(t0 + j) * D.Npad), __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT)
                                          : (uint64_t(kAqTag) << 32);
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    int spins = 0;
                    while (uint32_t(v[j] >> 32) != kAqTag && spins < kSpinMax) {
                        __builtin_amdgcn_s_sleep(2);
                        v[j] = __hip_atomic_load(as_global(slot + int64_t(t0 + j) * D.Npad), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                        spins++;
                    }
                    ok = ok && uint32_t(v[j] >> 32) == kAqTag;
                    if (t0 + j < D.b) sum += f32(uint32_t(v[j]));  // split order
                }
            }
            gst(D.y + int64_t(m) * D.ldy + row, ok ? sum * sc : __builtin_nanf(""));
            for (int t = 0; t < D.b; t++)
                __hip_atomic_store(as_global(slot + int64_t(t) * D.Npad), uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int M>
struct LdsWords {
    static constexpr int value = (M == 1) ? 2 * 256 * 64 : 2048 + 256 * M;
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
    u32x4 X, C;
};

// M = 1: the 128 KiB table allows one workgroup per CU, i.e. 2 waves per SIMD, so each wave may
// use 256 VGPRs (the compiler would otherwise aim for more waves than can ever be resident).
template <int M, int RW>
__global__ __launch_bounds__(aq_waves(M) * 64) __attribute__((amdgpu_waves_per_eu(1, M == 1 ? 2 : 4)))
void aq_kernel(AqParams P) {
    constexpr int W = aq_waves(M);  // waves per workgroup
    __shared__ uint32_t lds[LdsWords<M>::value];

    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wg = blockIdx.x;

    Piece pp = find_piece(P, wg, 0, -1);  // piece being processed
    if (pp.p >= P.ndesc) return;          // no work for this workgroup (same for all its waves)
    int ps = pp.s0;                       // slice being processed

    AqDesc pd = get_desc(P, pp.p);        // its descriptor
    Piece pn = next_piece(P, wg, pp);     // the next piece, looked up a piece ahead

    Loader<RW, W> ld;
    ld.done = false;
    ld.setup(P, pp, wg, wid, lane);

    // M = 1 table blocks of this wave: codebook bsel, code blocks cblk0 .. cblk0 + 32/W - 1
    // (32 codes each; 16 blocks over W waves).
    constexpr int NBLK = 16 / W;  // blocks per wave: 2 (M = 1, W = 8)
    const int bsel = (wid * NBLK) >> 3, cblk0 = (wid * NBLK) & 7;

    // Issue the loads of the loader's slice: operands first, then the RW tiles; step the loader.
    // Every load is unconditional with a clamped address (a load under a lane condition makes
    // the compiler wait for it at once); groups past G are zeroed where the operands are used.
    auto load_slice = [&](u32x4 (&t)[RW], SliceOps &o) __attribute__((always_inline)) {
        if constexpr (M == 1) {
#pragma unroll
            for (int gb = 0; gb < 2; gb++) {
                const int g = min(ld.s * 64 + gb * 32 + (lane & 31), ld.G - 1);
                o.B[gb] = gld<u32x2>(ld.x + int64_t(g) * 8 + 4 * (lane >> 5));
            }
#pragma unroll
            for (int h = 0; h < NBLK; h++)
                o.A[h] = gld<u32x2>(ld.cbk + (int64_t(bsel) * 256 + (cblk0 + h) * 32 + (lane & 31)) * 8 + 4 * (lane >> 5));
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
    auto settle = [&](u32x4 (&t)[RW], SliceOps &o) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RW; i++) __asm__ volatile("" ::"v"(t[i]));
        if constexpr (M == 1) {
            __asm__ volatile("" ::"v"(o.B[0]), "v"(o.B[1]), "v"(o.A[0]), "v"(o.A[1]));
        } else {
            __asm__ volatile("" ::"v"(o.X), "v"(o.C));
        }
    };

    // per row block: two folded row sums (M = 1, see fold_rows8) or M finished row sums
    constexpr int NACC = (M == 1) ? 2 : M;
    float acc[RW][NACC];
#pragma unroll
    for (int i = 0; i < RW; i++)
#pragma unroll
        for (int r = 0; r < NACC; r++) acc[i][r] = 0.f;

    u32x4 Xc[M];  // M > 1: this lane's group activations for the current slice
    const uint32_t lk = (uint32_t(lane) << 2) | (1u << 16);

    // Piece epilogue: row sums -> y (b == 1) or this split's tagged partial slots.
    auto epilogue = [&](const Piece &q, const AqDesc &D) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RW; i++) {
            const int rb = q.rb0 + wid + W * i;
            const int row = rb * 8 + (lane >> 3);
            const bool ok = (lane & 7) == 0 && rb < q.rb1 && row < D.N && q.split < D.b;
#pragma unroll
            for (int m = 0; m < M; m++) {
                float z;
                if constexpr (M == 1) z = finish_rows8(acc[i], lane);
                else z = acc[i][m];
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
            for (int r = 0; r < NACC; r++) acc[i][r] = 0.f;
        }
    };

    // Start of a slice: build its table (M = 1) or stage its activations (M > 1).
    auto slice_start = [&](const SliceOps &o) __attribute__((always_inline)) {
        const int G = pd.G;
        if constexpr (M == 1) {
            u32x2 B[2];
#pragma unroll
            for (int gb = 0; gb < 2; gb++) {
                const bool in = ps * 64 + gb * 32 + (lane & 31) < G;
                B[gb] = in ? o.B[gb] : u32x2{0u, 0u};
            }
            lds_barrier();  // every wave is done with the previous table
            const f32x16 zero = {};
#pragma unroll
            for (int h = 0; h < NBLK; h++) {
                const h4 A = __builtin_bit_cast(h4, o.A[h]);
                const f32x16 d0 = __builtin_amdgcn_mfma_f32_32x32x8f16(A, __builtin_bit_cast(h4, B[0]), zero, 0, 0, 0);
                const f32x16 d1 = __builtin_amdgcn_mfma_f32_32x32x8f16(A, __builtin_bit_cast(h4, B[1]), zero, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    // d0: groups 0-31, d1: groups 32-63; after the swap sw[0] holds code row
                    // 8(v/4) + v%4 of the block for all 64 groups, sw[1] the row 4 further on.
                    const auto sw = __builtin_amdgcn_permlane32_swap(u32(d0[v]), u32(d1[v]), false, false);
                    const int c = (cblk0 + h) * 32 + 8 * (v >> 2) + (v & 3);
                    lds[(bsel * 256 + c) * 64 + lane] = sw[0];
                    lds[(bsel * 256 + c + 4) * 64 + lane] = sw[1];
                }
            }
            lds_barrier();
        } else {
            const bool in = ps * 64 + lane < G;
            const u32x4 X = in ? o.X : u32x4{0u, 0u, 0u, 0u};
            lds_barrier();  // every wave is done with the previous stage
            u32x4 *cbl = reinterpret_cast<u32x4 *>(lds);
            u32x4 *xl = cbl + 512;
            if (threadIdx.x < 512) cbl[threadIdx.x] = o.C;
            if (wid < M) xl[wid * 64 + lane] = X;  // (waves >= M loaded a copy of row M-1)
            lds_barrier();
#pragma unroll
            for (int m = 0; m < M; m++) Xc[m] = xl[m * 64 + lane];
        }
    };

    // One tile: this lane's group for 8 rows of row block i.
    auto process = [&](const u32x4 &v, float (&a)[NACC]) __attribute__((always_inline)) {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        if constexpr (M == 1) {
            float v[8];
#pragma unroll
            for (int t = 0; t < 4; t++) {  // word t: (c0, c1) of rows 2t and 2t+1
                const uint32_t a0 = __builtin_amdgcn_perm(w4[t], lk, 0x0c0c0400u);
                const uint32_t a1 = __builtin_amdgcn_perm(w4[t], lk, 0x0c020500u);
                const uint32_t a2 = __builtin_amdgcn_perm(w4[t], lk, 0x0c0c0600u);
                const uint32_t a3 = __builtin_amdgcn_perm(w4[t], lk, 0x0c020700u);
                v[2 * t] = f32(lds_word(lds, a0)) + f32(lds_word(lds, a1));
                v[2 * t + 1] = f32(lds_word(lds, a2)) + f32(lds_word(lds, a3));
            }
            float w[2];
            fold_rows8(v, w);
            a[0] += w[0];
            a[1] += w[1];
        } else {
            const u32x4 *cbl = reinterpret_cast<const u32x4 *>(lds);
            float val[M][8];
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const uint32_t c0 = (w4[r >> 1] >> (16 * (r & 1))) & 0xFFu;
                const uint32_t c1 = (w4[r >> 1] >> (16 * (r & 1) + 8)) & 0xFFu;
                const u32x4 E0 = cbl[c0], E1 = cbl[256 + c1];
                const uint32_t e0[4] = {E0.x, E0.y, E0.z, E0.w}, e1[4] = {E1.x, E1.y, E1.z, E1.w};
                uint32_t wv[4];
#pragma unroll
                for (int k = 0; k < 4; k++) wv[k] = __builtin_bit_cast(uint32_t, as_h2(e0[k]) + as_h2(e1[k]));
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const uint32_t xw[4] = {Xc[m].x, Xc[m].y, Xc[m].z, Xc[m].w};
                    float sm = 0.f;
#pragma unroll
                    for (int k = 0; k < 4; k++) sm = dot2(wv[k], xw[k], sm);
                    val[m][r] = sm;
                }
            }
#pragma unroll
            for (int m = 0; m < M; m++) a[m] += reduce_rows8(val[m], lane);
        }
    };

    // One slice: wait for it, prefetch the one two ahead, build, process, advance.  Returns true
    // after the last slice of the last piece.
    auto step = [&](u32x4 (&cur)[RW], SliceOps &oc, u32x4 (&nxt)[RW], SliceOps &on) __attribute__((always_inline)) -> bool {
        settle(cur, oc);
        load_slice(nxt, on);
        slice_start(oc);
#pragma unroll
        for (int i = 0; i < RW; i++) {
            process(cur[i], acc[i]);
            // one tile at a time: hoisting the address math of every tile blows the register budget
            __builtin_amdgcn_sched_barrier(0);
        }
        if (++ps < pp.s1) return false;
        epilogue(pp, pd);
        if (pn.p >= P.ndesc) return true;
        pp = pn;
        ps = pp.s0;
        pd = get_desc(P, pp.p);
        pn = next_piece(P, wg, pp);
        return false;
    };

    // Three slice buffers: while slice s is processed, slices s+1 and s+2 are in flight.
    u32x4 buf0[RW], buf1[RW], buf2[RW];
    SliceOps ops0, ops1, ops2;
    load_slice(buf0, ops0);
    load_slice(buf1, ops1);
    while (true) {
        if (step(buf0, ops0, buf2, ops2)) break;
        if (step(buf1, ops1, buf0, ops0)) break;
        if (step(buf2, ops2, buf1, ops1)) break;
    }
    finalize<M, RW, W>(P, wg, wid, lane);
}

}  // namespace

AqFn aq_fn(int M, int RW) {
#define WQD_AQ_CASE(m)                                   \
    case m:                                              \
        return RW == 1 ? aq_kernel<m, 1> : aq_kernel<m, 2>;
    switch (M) {
    case 1:
        return RW <= 2 ? aq_kernel<1, 2> : RW == 4 ? aq_kernel<1, 4> : aq_kernel<1, 8>;
        WQD_AQ_CASE(2)
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
