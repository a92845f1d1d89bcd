// AQ2X8 dequantize-and-multiply kernels (gfx950) on the tile layout of layout.h: a tile is 16 rows
// x 32 groups of 8 weights, and lane 32h + g holds the code pairs (c0, c1) of rows 8h..8h+7 of
// group g.
//
// The weights of row n, group g are s_n * (C_0[c0] + C_1[c1]) with two 8-bit codes into two
// codebooks of 256 fp16 8-vectors (trapetum "Benchmarks", "Additive vector-quantization GEMV
// (AQLM-style, 2-bit)"), so
//     y_n = s_n * sum_g ( T_0,g[c0(n,g)] + T_1,g[c1(n,g)] ),   T_b,g[c] = sum_j C_b[c][j] x[8g+j]:
// a per-group lookup table built from the activations, after which only the codes are read.  The
// same page keeps such group sums in f32 (its 1x16 kernel moved to f32 after fp16 group sums
// drifted from the dequantized weights), and so do both kernels here: no intermediate value is
// rounded to fp16.
//
// Lookup-table kernel (M = 1):
//   * For one slice of 32 groups the workgroup builds T in LDS, fp32, at dword c*64 + b*32 + g:
//     64 KiB.  Two tables alternate: the table of the next slice is built while the current one
//     is read, with one workgroup barrier per slice.
//   * The build is T_b = C_b (256 x 8) . X (8 x 32), X[j][g] = x[8g+j]: one 32x32x8 matrix-core
//     product per wave (16 waves: codebook w/8, codes 32(w%8)..+31), whose 16 result registers
//     per lane are written as 16 dwords (exact fp16 products, fp32 sums).
//   * Per row of a tile, lane 32h + g reads T_h[c_h] and T_(1-h)[c_(1-h)] of its group: in one LDS
//     instruction the lanes of half 0 read codebook-0 entries (columns 0..31) and the lanes of
//     half 1 codebook-1 entries (columns 32..63), so no two lanes meet in a bank.  Each address is
//     one v_perm of the code word with a per-lane byte selector.  The two fp32 entries of each of
//     the lane's 8 rows are added, folded with the lane 16 apart (4 sums per lane) and accumulated;
//     the rest of the sum over the 32 lanes of a half is taken once per piece.
// Matrix-core kernel (M = 1..8; every batch-invariant call takes it):
//   * y = x W^T on the 16x16x32 fp16 matrix core: A = 16 activation rows (rows past M repeat row
//     M-1 and are never stored) x 32 k (4 groups), B = 32 k x 16 weight rows, whose operand in
//     lane 16q + n is the 8 fp16 values of codebook entry C_b[c_b(n, 4t + q)].  The two codebooks
//     are two products into the same fp32 accumulators: every product is exact, every sum fp32.
//   * The codebooks sit in LDS in 16 copies, entry e of copy j at ((b*256 + e)*16 + j)*16 bytes:
//     lane 16q + n gathers from copy n, so the 16 lanes of one LDS pass hit 16 different 16-byte
//     bank groups.
//   * A tile goes through the wave's LDS staging area, from which each lane reads the 8 code pairs
//     it needs (row n, groups 4t + q), 2 bytes each.  The activations of a slice are staged in
//     LDS (double-buffered, one barrier per slice).
//   * A wave's one or two tiles of a slice share each step: the lookups of step t + 1 (both
//     tiles, both codebooks) are issued before the products of step t.  A slice lasts as long as
//     its busiest wave, so the planner charges a piece whole passes of the 16 waves over its row
//     blocks (api.hip, plan_aq).
//
// Work (AqDesc): a workgroup walks its pieces in order, slice by slice; the tile loads of the next
// two slices are in flight while a slice is processed.  When a workgroup serves few pieces (the
// usual case: one piece of each projection), wave 0 writes all of them as LDS records at the start,
// so moving to the next piece is an LDS read; otherwise every wave walks the descriptors.  Pieces with b > 1 store fp32 partials.
// Once all of its pieces are done, the workgroup counts each split piece done on its row chunk,
// and the workgroup that arrives last adds the chunk's partials in split order: no workgroup ever
// waits for another, and results are the same bits from run to run.
#include <stddef.h>

#include "gemv_impl.h"

namespace wqd {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int W = kAqWaves;
#ifndef WQD_AQ_LUT_RING
#define WQD_AQ_LUT_RING 3  // unit buffers of the lookup-table kernel's load ring
#endif

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

// Sums over the 32 lanes of each half (lanes 32h .. 32h+31) of v[r], r < 8, in a fixed order (a
// transposed butterfly), in two parts.  fold16: lanes l and l^16, leaving row r + 4*bit4 in u[r],
// r < 4.  finish_half4: the rest; on return lane l holds the sum of row (l >> 2) & 7 of its half.
__device__ __forceinline__ void fold16(const float (&v)[8], float (&u)[4]) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const auto s = __builtin_amdgcn_permlane16_swap(u32(v[r]), u32(v[r + 4]), false, false);
        u[r] = f32(s[0]) + f32(s[1]);
    }
}
__device__ __forceinline__ float finish_half4(const float (&u)[4], int lane) {
    const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
    float w[2];
#pragma unroll
    for (int r = 0; r < 2; r++) {  // lanes l, l^8: row r + 2*bit3 + 4*bit4
        const float keep = b3 ? u[r + 2] : u[r], give = b3 ? u[r] : u[r + 2];
        w[r] = keep + dpp<kDppRor8>(give);
    }
    // lanes i, 7-i within 8 (bit 2 differs): row bit2 + 2*bit3 + 4*bit4
    const float keep = b2 ? w[1] : w[0], give = b2 ? w[0] : w[1];
    float z = keep + dpp<kDppHalfMirror>(give);
    z = z + dpp<kDppXor1>(z);  // the 4 lanes of a quad hold the same row
    z = z + dpp<kDppXor2>(z);
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
// the kernel argument itself (AqParams::d0 sits at the start of the kernarg segment).
__device__ __forceinline__ AqDesc get_desc(const AqParams &P, int p) {
    static_assert(offsetof(AqParams, d0) == 0, "d0 leads the kernel arguments");
    p = min(max(p, 0), P.ndesc - 1);  // never read outside the table
    const AqDesc *d = P.descs ? P.descs + p
                              : (const AqDesc *)(uintptr_t)__builtin_amdgcn_kernarg_segment_ptr();
    return load_uniform(d);
}

// A piece of this workgroup's work list (wave-uniform), as the descriptor defines it.
struct Piece {
    int p;          // projection; == ndesc past the end of the list
    int j;          // piece index within the projection
    int nw;         // workgroups serving the projection (piece stride)
    int chunk, split;
    int rb0, rb1;   // 16-row blocks [rb0, rb1)
    int s0, s1;     // 32-group slices [s0, s1)
};

__device__ __forceinline__ Piece piece_of(const AqDesc &D, int p, int j) {
    Piece q;
    q.p = p;
    q.j = j;
    q.nw = D.nw;
    q.split = j / D.a;
    q.chunk = j - q.split * D.a;
    q.rb0 = q.chunk * D.nrb;
    q.rb1 = min(D.RB, q.rb0 + D.nrb);
    q.s0 = q.split * D.ns;
    q.s1 = min(D.KS, q.s0 + D.ns);
    return q;
}

// The first piece of this workgroup at or after (projection p, piece j); j < 0: start of p.
// Workgroup wg serves pieces j = (wg - off) mod nwg, then every nw-th, of each projection whose
// workgroups it is among (0 <= off < nwg).
__device__ __forceinline__ Piece find_piece(const AqParams &P, int wg, int p, int j) {
    while (p < P.ndesc) {
        const AqDesc D = get_desc(P, p);
        if (j < 0) {
            j = wg - D.off;
            if (j < 0) j += P.nwg;
            if (j >= D.nw) j = D.npieces;  // not one of the projection's workgroups
        }
        if (j < D.npieces) return piece_of(D, p, j);
        p++;
        j = -1;
    }
    Piece q;
    q.p = P.ndesc;
    q.j = 0;
    q.nw = 1;
    q.chunk = q.split = q.rb0 = q.rb1 = q.s0 = q.s1 = 0;
    return q;
}

// Everything the kernels use of one piece: its row blocks and slices, and the fields of its
// projection that the loads, the epilogue and the split sum read.
struct PieceRec {
    const uint8_t *codes;    // tile plane
    const uint8_t *x;        // activations (row 0)
    const uint8_t *cbk;      // codebooks
    float *y;                // output (row 0)
    float *part;             // partials [M][b][Npad] when b > 1
    const uint16_t *rscale;  // row scales
    int *cnt;                // the piece's row-chunk arrival counter when b > 1
    int64_t ldx;             // bytes between activation rows
    int64_t ldy;             // elements between output rows
    int32_t rb0, rb1, s0, s1;
    int32_t N, Npad, G, b;
    int32_t split, pad[5];
};
static_assert(sizeof(PieceRec) == 128, "record of 8 x 16 bytes");

__device__ __forceinline__ PieceRec make_rec(const Piece &q, const AqDesc &D) {
    PieceRec r;
    r.codes = D.codes;
    r.x = reinterpret_cast<const uint8_t *>(D.x);
    r.cbk = reinterpret_cast<const uint8_t *>(D.cbk);
    r.y = D.y;
    r.part = D.part;
    r.rscale = D.rscale;
    r.cnt = D.b > 1 ? D.cnt + q.chunk * kAqCntStride : nullptr;
    r.ldx = D.ldx * 2;
    r.ldy = D.ldy;
    r.rb0 = q.rb0;
    r.rb1 = q.rb1;
    r.s0 = q.s0;
    r.s1 = q.s1;
    r.N = D.N;
    r.Npad = D.Npad;
    r.G = D.G;
    r.b = D.b;
    r.split = q.split;
#pragma unroll
    for (int i = 0; i < 5; i++) r.pad[i] = 0;
    return r;
}

// A record in LDS, read by every lane of a wave at the same address (broadcast), made uniform.
__device__ __forceinline__ PieceRec read_rec(const PieceRec *p) {
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
    uint32_t w[32];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const u32x4 v = q[i];
        w[4 * i] = __builtin_amdgcn_readfirstlane(v.x);
        w[4 * i + 1] = __builtin_amdgcn_readfirstlane(v.y);
        w[4 * i + 2] = __builtin_amdgcn_readfirstlane(v.z);
        w[4 * i + 3] = __builtin_amdgcn_readfirstlane(v.w);
    }
    PieceRec r;
    __builtin_memcpy(&r, w, sizeof(r));
    return r;
}

// The workgroup's piece records, in walk order (projection, then piece index), built once by wave
// 0 at the start: lane l takes projection base + l, counts the pieces this workgroup serves of it,
// and writes their records after those of the lanes before it.  Returns the number of pieces (the
// host launches this form only when a bound on it, the sum over projections of
// ceil(npieces / nw), is at most CAP).
template <int CAP>
__device__ int build_recs(const AqParams &P, int wg, int lane, PieceRec *recs) {
    int total = 0;
    for (int base = 0; base < P.ndesc; base += 64) {
        const int p = min(base + lane, P.ndesc - 1);
        AqDesc D;
        if (P.descs) {  // lane p's descriptor from the table
            uint32_t w[sizeof(AqDesc) / 4];
#pragma unroll
            for (unsigned i = 0; i < sizeof(AqDesc) / 4; i++)
                w[i] = gld<uint32_t>(reinterpret_cast<const uint32_t *>(P.descs + p) + i);
            __builtin_memcpy(&D, w, sizeof(D));
        } else {  // the single projection of the kernel arguments
            D = get_desc(P, 0);
        }
        int j0 = wg - D.off;
        if (j0 < 0) j0 += P.nwg;
        const int cnt = (base + lane < P.ndesc && j0 < D.nw && j0 < D.npieces) ? (D.npieces - j0 + D.nw - 1) / D.nw : 0;
        int incl = cnt;  // inclusive prefix sum over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d, 64);
            if (lane >= d) incl += t;
        }
        const int first = total + incl - cnt;
        for (int r = 0; r < cnt && first + r < CAP; r++) recs[first + r] = make_rec(piece_of(D, p, j0 + r * D.nw), D);
        total += __shfl(incl, 63, 64);
    }
    return total;
}

// Where a walk over the workgroup's pieces stands: record k (records in LDS), or piece (p, j) of
// the list (walking the descriptors).
struct PiecePos {
    int k, p, j, nw;
};
template <bool REC>
struct Pieces {
    const AqParams &P;
    int wg;
    const PieceRec *recs;  // REC: the records
    int n;                 // REC: their number

    __device__ __forceinline__ bool first(PiecePos &pos, PieceRec &r) const {
        if constexpr (REC) {
            pos.k = 0;
            if (n < 1) return false;
            r = read_rec(recs);
            return true;
        } else {
            return walk_to(find_piece(P, wg, 0, -1), pos, r);
        }
    }
    __device__ __forceinline__ bool next(PiecePos &pos, PieceRec &r) const {
        if constexpr (REC) {
            if (++pos.k >= n) return false;
            r = read_rec(recs + pos.k);
            return true;
        } else {
            return walk_to(find_piece(P, wg, pos.p, pos.j + pos.nw), pos, r);
        }
    }
    // The record of the piece at pos (again).
    __device__ __forceinline__ PieceRec at(const PiecePos &pos) const {
        if constexpr (REC) {
            return read_rec(recs + pos.k);
        } else {
            const AqDesc D = get_desc(P, pos.p);
            return make_rec(piece_of(D, pos.p, pos.j), D);
        }
    }
    __device__ __forceinline__ bool walk_to(const Piece &q, PiecePos &pos, PieceRec &r) const {
        if (q.p >= P.ndesc) return false;
        pos.p = q.p;
        pos.j = q.j;
        pos.nw = q.nw;
        r = make_rec(q, get_desc(P, q.p));
        return true;
    }
};

// At the start: wave 0 builds the records (REC), every wave then sees them.  `nshared` is an int
// of LDS.
template <bool REC, int CAP>
__device__ __forceinline__ int start_pieces(const AqParams &P, int wg, int wid, int lane, PieceRec *recs, int *nshared) {
    if constexpr (!REC) return 0;
    if (wid == 0) {
        const int t = build_recs<CAP>(P, wg, lane, recs);
        if (lane == 0) *nshared = t;
    }
    lds_barrier();
    return min(__builtin_amdgcn_readfirstlane(*nshared), CAP);
}

// Row block (from the piece's first) of tile i of wave wid: the waves take turns, so a piece of
// fewer than W*RW row blocks leaves every wave with a nearly equal share.
__device__ __forceinline__ int tile_rb(int wid, int i) { return wid + W * i; }

// Load cursor, running ahead of the processing: where this wave's tiles of the next slice to load
// are, and that slice's activations and codebooks.  Going from one slice to the next only adds a
// stride to each address; the piece bookkeeping runs once per piece.  A missing tile (past the
// piece's row blocks, or past the end of the work) still takes its place in the load ring, so every
// load stays unconditional: it reads 1 KiB of the codebooks instead, with a stride of 0.
template <int RW, bool REC>
struct Cursor {
    const uint8_t *ta[RW];  // per lane: its 16 bytes of tile i of the next slice
    int64_t tstr[RW];       // bytes from one slice of tile i to the next (0 for a missing tile)
    const uint8_t *cbk;     // the projection's codebooks
    const uint8_t *xp;      // x of the next slice (bytes from row 0)
    int64_t ldx;            // bytes between activation rows
    int gl;                 // groups of the projection from the next slice on
    int left;               // slices of the piece after the next one
    PiecePos pos;
    bool done;

    __device__ __forceinline__ void setup(const PieceRec &r, int wid, int lane) {
        const int64_t stride = int64_t(r.Npad / 16) * 1024;
        cbk = r.cbk;
        xp = r.x + int64_t(r.s0) * 512;
        ldx = r.ldx;
        gl = r.G - 32 * r.s0;
        left = r.s1 - r.s0 - 1;
        done = false;
        const uint8_t *t0 = r.codes + int64_t(r.s0) * stride + int64_t(r.rb0 + wid) * 1024 + lane * 16;
#pragma unroll
        for (int i = 0; i < RW; i++) {
            const bool valid = r.rb0 + tile_rb(wid, i) < r.rb1;
            ta[i] = valid ? t0 + i * (W * 1024) : cbk + lane * 16;
            tstr[i] = valid ? stride : 0;
        }
    }
    // To the next slice: the piece's next, else the first of the workgroup's next piece.
    __device__ __forceinline__ void advance(const Pieces<REC> &pcs, int wid, int lane) {
        if (done) return;
        if (left > 0) {
            left--;
#pragma unroll
            for (int i = 0; i < RW; i++) ta[i] += tstr[i];
            xp += 512;
            gl -= 32;
            return;
        }
        PieceRec r;
        if (pcs.next(pos, r)) {
            setup(r, wid, lane);
            return;
        }
        done = true;  // the activation and codebook loads keep the last slice's (in bounds)
#pragma unroll
        for (int i = 0; i < RW; i++) {
            ta[i] = cbk + lane * 16;
            tstr[i] = 0;
        }
    }
};

template <int RW, bool REC>
__device__ __forceinline__ void load_tiles(const Cursor<RW, REC> &c, u32x4 (&t)[RW]) {
#pragma unroll
    for (int i = 0; i < RW; i++)
        t[i] = __builtin_nontemporal_load((const u32x4 __attribute__((address_space(1))) *)(uintptr_t)c.ta[i]);
}
template <int RW>
__device__ __forceinline__ void settle_tiles(u32x4 (&t)[RW]) {
#pragma unroll
    for (int i = 0; i < RW; i++) __asm__ volatile("" ::"v"(t[i]));
}

// ------------------------------------------------------------------------------------------
// Split pieces: arrival and the sum of the partials.
// ------------------------------------------------------------------------------------------

// Adds the b partials (in split order) of every row of piece r's row chunk, scales them and writes
// y, then clears the chunk's counter.  Items (activation row m, row of the chunk) are taken by the
// workgroup's threads in turn.  NL >= b loads per item, unconditional (indices past b - 1 repeat
// the last split and are not added), so every load of a thread is in flight at once.
template <int M, int RW, int NL>
__device__ __forceinline__ void add_splits_n(const PieceRec &r) {
    constexpr int ROWS = W * RW * 16;  // most rows of a chunk
    constexpr int NI = (M * ROWS + W * 64 - 1) / (W * 64);
    const int r0 = 16 * r.rb0, nrows = min(16 * r.rb1, r.N) - r0;
    float v[NI][NL];
    int rowv[NI], mv[NI];
    uint32_t scb[NI];  // the row scales, loaded with the partials (not after the sums)
    bool live[NI];
#pragma unroll
    for (int it = 0; it < NI; it++) {
        const int item = int(threadIdx.x) + W * 64 * it;
        const int m = item / ROWS, rr = item - m * ROWS;
        live[it] = m < M && rr < nrows;
        rowv[it] = live[it] ? r0 + rr : 0;
        mv[it] = live[it] ? m : 0;
        scb[it] = gld<uint16_t>(r.rscale + rowv[it]);
#pragma unroll
        for (int j = 0; j < NL; j++)
            v[it][j] = __hip_atomic_load(as_global(r.part + (int64_t(mv[it]) * r.b + min(j, r.b - 1)) * r.Npad + rowv[it]),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int it = 0; it < NI; it++) {
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < NL; j++)
            if (j < r.b) sum += v[it][j];
        if (live[it]) gst(r.y + int64_t(mv[it]) * r.ldy + rowv[it], sum * half_bits_to_float(scb[it]));
    }
    if (threadIdx.x == 0) __hip_atomic_store(as_global(r.cnt), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <int M, int RW, int BMAX>
__device__ __forceinline__ void add_splits(const PieceRec &r) {
    if (BMAX <= 8 || r.b <= 8) add_splits_n<M, RW, 8>(r);
    else if (BMAX <= 16 || r.b <= 16) add_splits_n<M, RW, (BMAX < 16 ? BMAX : 16)>(r);
    else if (BMAX <= 24 || r.b <= 24) add_splits_n<M, RW, (BMAX < 24 ? BMAX : 24)>(r);
    else add_splits_n<M, RW, BMAX>(r);
}

// The record form's split sums: the nc chunks whose records fl[0..nc) name (this workgroup
// arrived last on each; their split counts b <= NL), summed together.  An item is (chunk,
// activation row m, row of the chunk); each thread takes G items per round, NL loads each
// (unconditional, so that all are in flight at once), and issues every load of the round before
// the first sum, so a round costs one trip to memory however many chunks it covers.  Items past a
// chunk's rows load its first row instead and are not stored.
template <int M, int RW, int NL, int G>
__device__ __forceinline__ void add_splits_g(const PieceRec *recs, const int *fl, int nc) {
    constexpr int ROWS = W * RW * 16;              // most rows of a chunk
    const int per = M * ROWS, total = nc * per;
    for (int base = 0; base < total; base += G * W * 64) {
        float v[G][NL];
        float *yp[G];
        uint32_t scb[G];  // the row scales, loaded with the partials (not after the sums)
        int bb[G];
        bool live[G];
#pragma unroll
        for (int g = 0; g < G; g++) {
            const int item = base + g * W * 64 + int(threadIdx.x);
            const int c = min(item / per, nc - 1), rem = item - (item / per) * per;
            const int m = rem / ROWS, rr = rem - m * ROWS;
            const PieceRec *rp = recs + fl[c];
            const int b = rp->b, r0 = 16 * rp->rb0, nrows = min(16 * rp->rb1, rp->N) - r0;
            live[g] = item < total && rr < nrows;
            const int row = r0 + (live[g] ? rr : 0), mm = live[g] ? m : 0;
            const float *part = rp->part + int64_t(mm) * b * rp->Npad + row;
            scb[g] = gld<uint16_t>(rp->rscale + row);
#pragma unroll
            for (int j = 0; j < NL; j++)  // (unconditional: indices past b - 1 repeat the last split)
                v[g][j] = __hip_atomic_load(as_global(part + int64_t(min(j, b - 1)) * rp->Npad), __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
            yp[g] = rp->y + int64_t(mm) * rp->ldy + row;
            bb[g] = b;
        }
#pragma unroll
        for (int g = 0; g < G; g++) {
            if (!live[g]) continue;
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < NL; j++)
                if (j < bb[g]) sum += v[g][j];
            gst(yp[g], sum * half_bits_to_float(scb[g]));
        }
    }
    if (int(threadIdx.x) < nc) __hip_atomic_store(as_global(recs[fl[threadIdx.x]].cnt), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// G: as many items per thread as the chunks need (each thread then holds G x NL loads), at most
// what the registers allow.
template <int M, int RW, int NL>
__device__ __forceinline__ void add_splits_recs(const PieceRec *recs, const int *fl, int nc) {
    constexpr int GMAX = NL >= 24 ? 2 : (48 / NL > 4 ? 4 : 48 / NL);
    const int need = (nc * M * W * RW * 16 + W * 64 - 1) / (W * 64);  // items per thread for one round
    if (need <= 1 || GMAX == 1) add_splits_g<M, RW, NL, 1>(recs, fl, nc);
    else if (need <= 2 || GMAX == 2) add_splits_g<M, RW, NL, (GMAX < 2 ? GMAX : 2)>(recs, fl, nc);
    else if (need <= 3 || GMAX == 3) add_splits_g<M, RW, NL, (GMAX < 3 ? GMAX : 3)>(recs, fl, nc);
    else add_splits_g<M, RW, NL, GMAX>(recs, fl, nc);
}

// After all of the workgroup's pieces: once every wave's partial stores have completed, the
// workgroup counts each of its split pieces done on the piece's row chunk (lane k of wave 0 takes
// the k-th, so the atomics are one instruction per 64 pieces), and where it arrived last it adds
// the chunk's partials.  `flags`: 260 ints of LDS.
template <int M, int RW, int BMAX, bool REC>
__device__ __forceinline__ void finish(const Pieces<REC> &pcs, int wid, int lane, int *flags) {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // every wave's partials are stored
    if constexpr (REC) {  // at most 64 records
        if (wid == 0) {
            int last = 0, b = 0;
            if (lane < pcs.n) {
                const PieceRec *rp = pcs.recs + lane;
                b = rp->b;
                int *cnt = rp->cnt;
                if (b > 1) last = __hip_atomic_fetch_add(as_global(cnt), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == b - 1;
            }
            // the chunks this workgroup finishes, by split-count class (b <= 8, 16, 24, more), in
            // record order: the count of class c at flags[c], its list at flags[4 + 64 c ..]
            const int cls = b <= 8 ? 0 : b <= 16 ? 1 : b <= 24 ? 2 : 3;
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const uint64_t mask = __ballot(last && cls == c);
                const int pos = __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
                if (last && cls == c) flags[4 + 64 * c + pos] = lane;
                if (lane == 0) flags[c] = __popcll(mask);
            }
        }
        lds_barrier();
        int nc[4];
#pragma unroll
        for (int c = 0; c < 4; c++) nc[c] = __builtin_amdgcn_readfirstlane(flags[c]);
        if (nc[0]) add_splits_recs<M, RW, 8>(pcs.recs, flags + 4, nc[0]);
        if (BMAX > 8 && nc[1]) add_splits_recs<M, RW, (BMAX < 16 ? BMAX : 16)>(pcs.recs, flags + 4 + 64, nc[1]);
        if (BMAX > 16 && nc[2]) add_splits_recs<M, RW, (BMAX < 24 ? BMAX : 24)>(pcs.recs, flags + 4 + 128, nc[2]);
        if (BMAX > 24 && nc[3]) add_splits_recs<M, RW, BMAX>(pcs.recs, flags + 4 + 192, nc[3]);
        return;
    } else {
        PiecePos pos;
        PieceRec r;
        bool more = pcs.first(pos, r);
        while (more) {
            const PiecePos pos0 = pos;
            int *cnt = nullptr;  // lane k: the k-th split piece's counter and split count
            int bk = 0, n = 0;
            for (; more && n < 64; more = pcs.next(pos, r)) {
                if (r.b == 1) continue;
                if (lane == n) {
                    cnt = r.cnt;
                    bk = r.b;
                }
                n++;
            }
            if (wid == 0) {
                int last = 0;
                if (lane < n) last = __hip_atomic_fetch_add(as_global(cnt), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == bk - 1;
                flags[lane] = last;
            }
            lds_barrier();
            PiecePos q = pos0;
            PieceRec rq = pcs.at(q);
            for (int k = 0; k < n; ) {
                if (rq.b > 1) {
                    if (__builtin_amdgcn_readfirstlane(flags[k])) add_splits<M, RW, BMAX>(rq);
                    k++;
                }
                if (k < n) pcs.next(q, rq);
            }
            lds_barrier();  // flags are read before the next round overwrites them
        }
    }
}

// ------------------------------------------------------------------------------------------
// Lookup-table kernel, M = 1 or 2 activation rows.  RW: 16-row blocks per wave per slice (a piece
// has at most W*RW).  One workgroup per CU, 4 waves per SIMD; the tables take 128 KiB of LDS:
//   M = 1: two tables of one slice (fp32, dword c*64 + b*32 + g), the next slice's built while
//          the current one is read: one barrier per slice;
//   M = 2: one table whose entries hold both rows' sums (fp32 pairs, at byte (b << 16) | (c << 8) |
//          (g << 3)), built and then read: two barriers per slice.
// REC: the workgroup's pieces as LDS records (at most kAqLutRecs), else walked from the descriptors.
// ------------------------------------------------------------------------------------------
template <int M>
struct LutOps {
    u32x2 A;     // this wave's codebook rows (A operand of the table build)
    u32x2 B[M];  // the slice's activations of this lane's group, per row (B operands)
    int gval;    // groups of the slice inside K
};

template <int M, int RW, int R, bool REC>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(1, 4))) void aq_lut_kernel(AqParams P) {
    static_assert(M == 1 || M == 2, "one or two activation rows");
    constexpr bool DB = M == 1;  // double-buffered tables
    __shared__ uint32_t lds[2 * 256 * 64];
    __shared__ PieceRec recs[REC ? kAqLutRecs : 1];
    __shared__ int nshared;

    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wg = blockIdx.x;
    const int h = lane >> 5, g = lane & 31;

    if (stale_table(P.stamp, P.fp, P.stale)) return;
    const int nrecs = start_pieces<REC, kAqLutRecs>(P, wg, wid, lane, recs, &nshared);
    const Pieces<REC> pcs{P, wg, recs, nrecs};
    PiecePos pos;  // piece being processed
    PieceRec pr;
    if (!pcs.first(pos, pr)) return;  // no work for this workgroup (same for all its waves)
    int ps = pr.s0, ps_end = pr.s1;   // slice being processed, end of the piece's slices
    int rows_w = pr.rb1 - pr.rb0 - wid;  // tile i of this wave is in the piece when 16 i < rows_w

    Cursor<RW, REC> ld;
    ld.pos = pos;
    ld.setup(pr, wid, lane);

    // LDS byte address of a lookup: byte 0 and byte 2 come from lk, byte 1 is the code byte the
    // selector picks from the word (word t holds (c0, c1) of rows 2t and 2t+1).  M = 1: (tb << 16) |
    // (code << 8) | (b << 7) | (g << 2), tb the table buffer; M = 2: (b << 16) | (code << 8) |
    // (g << 3).  Lanes of half 0 look up codebook 0 (A) while those of half 1 look up codebook 1,
    // then the other way round (B), so no two lanes of a pass meet in a bank.
    const uint32_t lkA0 = DB ? (uint32_t(g) << 2) | (uint32_t(h) << 7) : (uint32_t(g) << 3) | (uint32_t(h) << 16);
    const uint32_t lkB0 = DB ? (uint32_t(g) << 2) | (uint32_t(1 - h) << 7) : (uint32_t(g) << 3) | (uint32_t(1 - h) << 16);
    const uint32_t selA[2] = {0x0c020000u | ((4u + h) << 8), 0x0c020000u | ((6u + h) << 8)};
    const uint32_t selB[2] = {0x0c020000u | ((5u - h) << 8), 0x0c020000u | ((7u - h) << 8)};

    // the build operands: this wave's codebook rows (codebook wid/8, codes 32(wid%8) + g), and
    // the 8 activations of group g per row (groups past K clamp to the last, then read as zero)
    const uint32_t aoff = ((wid >> 3) * 256 + 32 * (wid & 7) + g) * 16 + 8 * h;
    auto load_ops = [&](LutOps<M> &o) __attribute__((always_inline)) {
        o.A = gld<u32x2>(ld.cbk + aoff);
        o.gval = ld.gl;
#pragma unroll
        for (int m = 0; m < M; m++) o.B[m] = gld<u32x2>(ld.xp + m * ld.ldx + min(g, ld.gl - 1) * 16 + 8 * h);
    };
    auto load_slice = [&](u32x4 (&t)[RW], LutOps<M> &o) __attribute__((always_inline)) {
        load_ops(o);
        load_tiles(ld, t);
        ld.advance(pcs, wid, lane);
    };
    auto settle_ops = [&](LutOps<M> &o) __attribute__((always_inline)) {
        __asm__ volatile("" ::"v"(o.A));
#pragma unroll
        for (int m = 0; m < M; m++) __asm__ volatile("" ::"v"(o.B[m]));
    };

    // The table of a slice (into buffer tb when double-buffered): wave w computes
    // T_(w/8)[32(w%8) .. +31][g = 0..31], one 32x32x8 product per row.
    auto build = [&](const LutOps<M> &o, int tb) __attribute__((always_inline)) {
        f32x16 z;
#pragma unroll
        for (int v = 0; v < 16; v++) z[v] = 0.f;
        f32x16 D[M];
#pragma unroll
        for (int m = 0; m < M; m++) {
            const u32x2 B = g < o.gval ? o.B[m] : u32x2{0u, 0u};  // groups past K read as zero
            D[m] = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(h4, o.A), __builtin_bit_cast(h4, B), z, 0, 0, 0);
        }
        if constexpr (DB) {
            uint32_t *tab = lds + tb * (256 * 64) + (wid >> 3) * 32 + g;
#pragma unroll
            for (int v = 0; v < 16; v++) {  // register v of lane l: code row 8(v/4) + 4(l/32) + v%4
                const int code = 32 * (wid & 7) + 8 * (v >> 2) + 4 * h + (v & 3);
                tab[code * 64] = u32(D[0][v]);
            }
        } else {
            uint8_t *tab = reinterpret_cast<uint8_t *>(lds) + ((wid >> 3) << 16) + (g << 3);
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int code = 32 * (wid & 7) + 8 * (v >> 2) + 4 * h + (v & 3);
                *reinterpret_cast<u32x2 *>(tab + (code << 8)) = u32x2{u32(D[0][v]), u32(D[M - 1][v])};
            }
        }
    };

    // per row block and activation row: the lane's 8 row sums folded over lanes l, l^16 (fold16)
    float acc[RW][M][4];
#pragma unroll
    for (int i = 0; i < RW; i++)
#pragma unroll
        for (int m = 0; m < M; m++)
#pragma unroll
            for (int r = 0; r < 4; r++) acc[i][m][r] = 0.f;

    // One tile: the 8 rows of this lane's half, its group.  The 16 lookups go out as two groups of
    // 8 (rows 0, 1, 4, 5, then rows 2, 3, 6, 7); the second group's addresses are tied to the first
    // lookup's result, so at most 15 LDS reads are outstanding and every wait is counted exactly.
    auto process = [&](const u32x4 &v, float (&a)[M][4], uint32_t lkA, uint32_t lkB) __attribute__((always_inline)) {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        u32x2 e[2][8];  // M = 1: .x only
#pragma unroll
        for (int q = 0; q < 2; q++) {
            uint32_t ad[8];
#pragma unroll
            for (int k = 0; k < 4; k++) {  // row r = (k & 1) + 2q + 4(k >> 1) is word r/2, parity r%2
                const int r = (k & 1) + 2 * q + 4 * (k >> 1);
                ad[2 * k] = __builtin_amdgcn_perm(w4[r >> 1], lkA, selA[r & 1]);
                ad[2 * k + 1] = __builtin_amdgcn_perm(w4[r >> 1], lkB, selB[r & 1]);
            }
            if (q == 1)
                __asm__ volatile("" : "+v"(ad[0]), "+v"(ad[1]), "+v"(ad[2]), "+v"(ad[3]), "+v"(ad[4]), "+v"(ad[5]),
                                 "+v"(ad[6]), "+v"(ad[7]) : "v"(e[0][0].x));
#pragma unroll
            for (int k = 0; k < 8; k++) {
                if constexpr (M == 1)
                    e[q][k].x = lds_word(lds, ad[k]);
                else
                    e[q][k] = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint8_t *>(lds) + ad[k]);
            }
        }
#pragma unroll
        for (int m = 0; m < M; m++) {
            float r8[8], u[4];
#pragma unroll
            for (int q = 0; q < 2; q++)
#pragma unroll
                for (int k = 0; k < 4; k++)
                    r8[(k & 1) + 2 * q + 4 * (k >> 1)] = f32(e[q][2 * k][m]) + f32(e[q][2 * k + 1][m]);
            fold16(r8, u);
#pragma unroll
            for (int r = 0; r < 4; r++) a[m][r] += u[r];
        }
    };

    // Piece epilogue: row sums -> y (b == 1) or this split's partials.
    auto epilogue = [&](const PieceRec &r) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RW; i++) {
            const int rb = r.rb0 + tile_rb(wid, i);
            if (W * i < rows_w) {
                const int row = 16 * rb + 8 * h + ((lane >> 2) & 7);
                const bool st = (lane & 3) == 0 && row < r.N;
                const float sc = st && r.b == 1 ? half_bits_to_float(gld<uint16_t>(r.rscale + row)) : 0.f;
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const float z = finish_half4(acc[i][m], lane);
                    if (st) {
                        if (r.b == 1)
                            gst(r.y + int64_t(m) * r.ldy + row, z * sc);
                        else
                            __hip_atomic_store(as_global(r.part + (int64_t(m) * r.b + r.split) * r.Npad + row), z,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < M; m++)
#pragma unroll
                for (int q = 0; q < 4; q++) acc[i][m][q] = 0.f;
        }
    };

    int tb = 0;         // table of the slice being processed (double-buffered tables)
    bool fin = false;   // every piece is done (the remaining steps of the ring's round are empty)
    // One slice: issue the loads of the slice two ahead (into the buffers the previous slice
    // left), wait for this slice's tiles and the table operands, then (M = 1) build the next
    // slice's table into the other buffer and look up this slice, barrier, or (M = 2) build this
    // slice's table, barrier, look it up, barrier.  The loads and waits come first and on every
    // path, the same in every step, so that the waits of the ring are counted exactly.
    auto step = [&](u32x4 (&cur)[RW], LutOps<M> &ocur, LutOps<M> &on, u32x4 (&nxt)[RW], LutOps<M> &onew)
                    __attribute__((always_inline)) {
        load_slice(nxt, onew);
        settle_tiles(cur);
        if constexpr (DB)
            settle_ops(on);
        else
            settle_ops(ocur);
        if (fin) return;
        // (no scalar load may be pending during the build and lookups: the LDS waits are then
        // counted exactly instead of draining every lookup in flight)
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if constexpr (DB) {
            build(on, tb ^ 1);
        } else {
            build(ocur, 0);
            lds_barrier();
        }
        const uint32_t lkA = lkA0 | (uint32_t(DB ? tb : 0) << 16), lkB = lkB0 | (uint32_t(DB ? tb : 0) << 16);
#pragma unroll
        for (int i = 0; i < RW; i++) {
            if (W * i < rows_w) process(cur[i], acc[i], lkA, lkB);
            __builtin_amdgcn_sched_barrier(0);
        }
        lds_barrier();
        tb ^= 1;
        if (++ps < ps_end) return;
        epilogue(pcs.at(pos));
        PieceRec r;
        if (!pcs.next(pos, r)) {
            fin = true;
            return;
        }
        ps = r.s0;
        ps_end = r.s1;
        rows_w = r.rb1 - r.rb0 - wid;
    };

    // R unit buffers: while unit s is processed, units s+1 .. s+R-2 are in flight, and the loads of
    // unit s+R-1 go into the buffer unit s-1 freed.
    // At the start every wave issues the first table's operands before any tile load (the
    // barrier between), so the first build does not wait behind the workgroup's first tiles.
    static_assert(R == 3, "three unit buffers");
    u32x4 buf0[RW], buf1[RW], buf2[RW];
    LutOps<M> ops0, ops1, ops2;
    load_ops(ops0);
    __builtin_amdgcn_s_barrier();
    load_tiles(ld, buf0);
    ld.advance(pcs, wid, lane);
    load_slice(buf1, ops1);
    if constexpr (DB) {
        settle_ops(ops0);
        build(ops0, 0);
        lds_barrier();
    }
    do {
        step(buf0, ops0, ops1, buf2, ops2);
        step(buf1, ops1, ops2, buf0, ops0);
        step(buf2, ops2, ops0, buf1, ops1);
    } while (!fin);
    finish<M, RW, kAqLutMaxSplits, REC>(pcs, wid, lane, reinterpret_cast<int *>(lds));
}

// ------------------------------------------------------------------------------------------
// Matrix-core kernel, M activation rows.  RW: 16-row blocks per wave per slice.  REC as above
// (at most kAqMmaRecs records).
// ------------------------------------------------------------------------------------------
constexpr int kCbBytes = 2 * 256 * 16 * 16;  // 16 copies of the two codebooks
constexpr int kStageBytes = 2 * 544;         // per wave: a tile, half h at h*544 (padded)
constexpr int kXRow = 33 * 16;               // staged activations: one row of a slice (padded)

template <int M>
struct MmaLds {
    static constexpr int off_stage = kCbBytes;
    static constexpr int off_x = kCbBytes + W * kStageBytes;
    static constexpr int xbuf = M * kXRow;
    static constexpr int bytes = off_x + 2 * xbuf;
};

struct MmaOps {
    u32x4 X;   // this thread's 8 activations of the slice (row t/32, group t%32), t < 32M
    int gval;  // groups of the slice inside K
};

template <int M, int RW, bool REC>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(1, 4))) void aq_mma_kernel(AqParams P) {
    using L = MmaLds<M>;
    static_assert(L::bytes + (REC ? kAqMmaRecs : 1) * sizeof(PieceRec) + 16 <= 160 * 1024, "LDS of one workgroup");
    __shared__ __attribute__((aligned(16))) uint8_t lds[L::bytes];
    __shared__ PieceRec recs[REC ? kAqMmaRecs : 1];
    __shared__ int nshared;

    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wg = blockIdx.x;
    const int n = lane & 15, q4 = lane >> 4;     // MMA operand lane: row (weight or activation), k-block
    const int th = lane >> 5, tg = lane & 31;    // tile lane: half, group

    if (stale_table(P.stamp, P.fp, P.stale)) return;
    const int nrecs = start_pieces<REC, kAqMmaRecs>(P, wg, wid, lane, recs, &nshared);
    const Pieces<REC> pcs{P, wg, recs, nrecs};
    PiecePos pos;
    PieceRec pr;
    if (!pcs.first(pos, pr)) return;
    int ps = pr.s0, ps_end = pr.s1;
    int rows_w = pr.rb1 - pr.rb0 - wid;  // tile i of this wave is in the piece when 16 i < rows_w
    const uint8_t *pcbk = pr.cbk;        // codebooks in LDS

    Cursor<RW, REC> ld;
    ld.pos = pos;
    ld.setup(pr, wid, lane);

    // thread t < 32M stages the 8 activations of row t/32, group t%32 of a slice
    const int xt = min(int(threadIdx.x), 32 * M - 1);
    auto load_slice = [&](u32x4 (&t)[RW], MmaOps &o) __attribute__((always_inline)) {
        o.gval = ld.gl;
        o.X = gld<u32x4>(ld.xp + (xt >> 5) * ld.ldx + min(xt & 31, ld.gl - 1) * 16);
        load_tiles(ld, t);
        ld.advance(pcs, wid, lane);
    };
    auto settle_ops = [&](MmaOps &o) __attribute__((always_inline)) { __asm__ volatile("" ::"v"(o.X)); };
    auto stage_x = [&](const MmaOps &o, int xb) __attribute__((always_inline)) {
        if (threadIdx.x < 32 * M) {
            const bool in = int(threadIdx.x & 31) < o.gval;
            *reinterpret_cast<u32x4 *>(lds + L::off_x + xb * L::xbuf + (threadIdx.x >> 5) * kXRow + (threadIdx.x & 31) * 16) =
                in ? o.X : u32x4{0u, 0u, 0u, 0u};
        }
    };
    // The projection's codebooks into the 16 copies (all loads first, then the writes).
    auto codebooks = [&](const uint8_t *cbk) __attribute__((always_inline)) {
        u32x4 e[8];
#pragma unroll
        for (int k = 0; k < 8; k++) e[k] = gld<u32x4>(cbk + ((threadIdx.x + k * W * 64) >> 4) * 16);
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const int idx = threadIdx.x + k * W * 64;  // entry idx >> 4, copy idx & 15
            *reinterpret_cast<u32x4 *>(lds + (idx >> 4) * 256 + (idx & 15) * 16) = e[k];
        }
    };

    f32x4 Dacc[RW][2];
#pragma unroll
    for (int i = 0; i < RW; i++)
#pragma unroll
        for (int c = 0; c < 2; c++) Dacc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint8_t *stage = lds + L::off_stage + wid * kStageBytes;
    const uint8_t *code_src = stage + (n >> 3) * 544 + q4 * 16 + 2 * (n & 7);
    const uint32_t lkc = (1u << 16) | (uint32_t(n) << 4);
    // The wave's tiles of one slice into accumulators D[i]: each tile's codes transposed through
    // the staging area (lane 16q + n: the code pairs of row n, groups 4t + q), then 8 steps of 4
    // groups, each two products per tile (codebook 0, codebook 1).  The tiles' lookups and
    // products alternate within a step; every accumulator still takes its products in the order
    // t = 0..7, codebook 0 before 1.
    // (NT: the wave's first NT tiles of the slice, all in the piece; no branch inside)
    auto mma_tiles = [&](auto nt, const u32x4 (&v)[RW], const uint8_t *xs, f32x4 (&D)[RW][2])
                         __attribute__((always_inline)) {
        constexpr int NT = decltype(nt)::value;
        uint32_t cp[NT][8];
#pragma unroll
        for (int i = 0; i < NT; i++) {  // (the staging area is reused: the reads of tile i come first)
            *reinterpret_cast<u32x4 *>(stage + th * 544 + tg * 16) = v[i];
#pragma unroll
            for (int t = 0; t < 8; t++) cp[i][t] = *reinterpret_cast<const uint16_t *>(code_src + t * 64);
        }
        // step t's lookups are issued before step t-1's products (two register sets), so each
        // product waits for lookups issued one step earlier
        u32x4 Bg[2][NT][2], Ax[2];
        auto lookups = [&](int t, u32x4 (&B)[NT][2], u32x4 &A) __attribute__((always_inline)) {
            A = *reinterpret_cast<const u32x4 *>(xs + t * 64);
#pragma unroll
            for (int i = 0; i < NT; i++) {
                const uint32_t a0 = __builtin_amdgcn_perm(cp[i][t], lkc, 0x0c0c0400u);  // (c0 << 8) | (n << 4)
                const uint32_t a1 = __builtin_amdgcn_perm(cp[i][t], lkc, 0x0c020500u);  // 64 KiB + (c1 << 8) | (n << 4)
                B[i][0] = *reinterpret_cast<const u32x4 *>(lds + a0);
                B[i][1] = *reinterpret_cast<const u32x4 *>(lds + a1);
            }
        };
        lookups(0, Bg[0], Ax[0]);
#pragma unroll
        for (int t = 0; t < 8; t++) {
            if (t + 1 < 8) lookups(t + 1, Bg[(t + 1) & 1], Ax[(t + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            const h8 Ah = __builtin_bit_cast(h8, Ax[t & 1]);
#pragma unroll
            for (int i = 0; i < NT; i++) {
                D[i][t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, __builtin_bit_cast(h8, Bg[t & 1][i][0]), D[i][t & 1], 0, 0, 0);
                D[i][t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, __builtin_bit_cast(h8, Bg[t & 1][i][1]), D[i][t & 1], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Piece epilogue: register v of lane 16q + n is activation row 4q + v of weight row n.
    auto epilogue = [&](const PieceRec &r) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RW; i++) {
            const int rb = r.rb0 + tile_rb(wid, i);
            const int row = 16 * rb + n;
            if (W * i < rows_w && row < r.N) {
                const float sc = r.b == 1 ? half_bits_to_float(gld<uint16_t>(r.rscale + row)) : 0.f;
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const int m = 4 * q4 + v;
                    const float s = Dacc[i][0][v] + Dacc[i][1][v];
                    if (m < M) {
                        if (r.b == 1)
                            gst(r.y + int64_t(m) * r.ldy + row, s * sc);
                        else
                            __hip_atomic_store(as_global(r.part + (int64_t(m) * r.b + r.split) * r.Npad + row), s,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < 2; c++) Dacc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };

    int xb = 0;         // activation buffer of the slice being processed
    bool fin = false;   // every piece is done (the remaining steps of the ring's round are empty)
    // One slice: the loads of the slice two ahead, the waits for this slice's tiles and the next
    // slice's activations (first and on every path, as in the lookup-table kernel), the next
    // slice's activations into LDS, the products of this slice, barrier.
    auto step = [&](u32x4 (&cur)[RW], MmaOps &on, u32x4 (&nxt)[RW], MmaOps &onew) __attribute__((always_inline)) {
        load_slice(nxt, onew);
        settle_tiles(cur);
        settle_ops(on);
        if (fin) return;
        stage_x(on, xb ^ 1);
        // step t's A operand, lane 16q + m: activation row min(m, M-1), groups 4t + q of the slice
        const uint8_t *xs = lds + L::off_x + xb * L::xbuf + min(n, M - 1) * kXRow + q4 * 16;
        static_assert(RW == 2, "one or two tiles per wave and slice");
        if (W < rows_w)
            mma_tiles(std::integral_constant<int, 2>(), cur, xs, Dacc);
        else if (0 < rows_w)
            mma_tiles(std::integral_constant<int, 1>(), cur, xs, Dacc);
        lds_barrier();
        xb ^= 1;
        if (++ps < ps_end) return;
        epilogue(pcs.at(pos));
        PieceRec r;
        if (!pcs.next(pos, r)) {
            fin = true;
            return;
        }
        ps = r.s0;
        ps_end = r.s1;
        rows_w = r.rb1 - r.rb0 - wid;
        if (r.cbk != pcbk) {  // every wave is past its lookups of the old codebooks (the barrier above)
            pcbk = r.cbk;
            codebooks(pcbk);
            lds_barrier();
        }
    };

    u32x4 buf0[RW], buf1[RW], buf2[RW];
    MmaOps ops0, ops1, ops2;
    codebooks(pcbk);
    load_slice(buf0, ops0);
    load_slice(buf1, ops1);
    settle_ops(ops0);
    stage_x(ops0, 0);
    lds_barrier();
    do {
        step(buf0, ops1, buf2, ops2);
        step(buf1, ops2, buf0, ops0);
        step(buf2, ops0, buf1, ops1);
    } while (!fin);
    finish<M, RW, kAqMmaMaxSplits, REC>(pcs, wid, lane, reinterpret_cast<int *>(lds));
}

}  // namespace

AqFn aq_fn(int M, bool lut, bool rec) {
    if (lut) {
        if (M == 1)
            return rec ? aq_lut_kernel<1, kAqLutRW, WQD_AQ_LUT_RING, true> : aq_lut_kernel<1, kAqLutRW, WQD_AQ_LUT_RING, false>;
        if (M == 2)
            return rec ? aq_lut_kernel<2, kAqLut2RW, WQD_AQ_LUT_RING, true> : aq_lut_kernel<2, kAqLut2RW, WQD_AQ_LUT_RING, false>;
        return nullptr;
    }
    switch (M) {
    case 1: return rec ? aq_mma_kernel<1, kAqMmaRW, true> : aq_mma_kernel<1, kAqMmaRW, false>;
    case 2: return rec ? aq_mma_kernel<2, kAqMmaRW, true> : aq_mma_kernel<2, kAqMmaRW, false>;
    case 3: return rec ? aq_mma_kernel<3, kAqMmaRW, true> : aq_mma_kernel<3, kAqMmaRW, false>;
    case 4: return rec ? aq_mma_kernel<4, kAqMmaRW, true> : aq_mma_kernel<4, kAqMmaRW, false>;
    case 5: return rec ? aq_mma_kernel<5, kAqMmaRW, true> : aq_mma_kernel<5, kAqMmaRW, false>;
    case 6: return rec ? aq_mma_kernel<6, kAqMmaRW, true> : aq_mma_kernel<6, kAqMmaRW, false>;
    case 7: return rec ? aq_mma_kernel<7, kAqMmaRW, true> : aq_mma_kernel<7, kAqMmaRW, false>;
    case 8: return rec ? aq_mma_kernel<8, kAqMmaRW, true> : aq_mma_kernel<8, kAqMmaRW, false>;
    }
    return nullptr;
}

}  // namespace wqd
