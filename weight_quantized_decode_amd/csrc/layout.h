// Prepared (device) layout of the packed weights, shared by the host re-layout code and the
// kernels of libwqd.
//
// Rows are grouped in tiles of 64 (one wavefront lane per row).  Each row's code bytes are cut
// into 16-byte chunks; the code plane stores, for row group g, chunk c and lane r, the 16 bytes
// of row 64g+r at ((g*C + c)*64 + r)*16.  One wavefront load instruction therefore reads 1 KiB
// of contiguous memory: chunk c of 64 consecutive rows.  This is the "re-lay the misaligned
// blocks into planes at load time" step of the ternary vLLM page ("Anatomy of a PQ2_0 block",
// prepared weights: a code plane, then a scale plane, rows 16-byte aligned), applied to all six
// formats.  Within a chunk the codes are permuted so that the decoder can extract two weights
// with one AND (see the per-format notes below).  Byte counts per weight are unchanged; only
// the zero padding of the last row group (N up to a multiple of 64) and of a last partial chunk
// is added.
//
// Planes, each starting at a 256-byte aligned offset from the weight base pointer:
//   codes   : RG*C*64*16 bytes
//   scales  : Q4_0 / TQ2: per row group g, per quad q of blocks, per lane r: 4 fp16 scales of
//             blocks 4q..4q+3 (8 bytes), at ((g*Q + q)*64 + r)*8.  AQ2X8, AQ1X16: s[Npad] fp16.
//   codebook: CB4 16 fp16, CB8 256 fp16, AQ2X8 C[2][256][8] fp16, AQ1X16 C[65536][8] fp16.
//
// Intra-chunk code order (w = one 32-bit word of the chunk, t = its index 0..3):
//   Q4_0  chunk = one block of 32 weights.  Word t holds weights 8t..8t+7; weight 8t+i sits in
//         nibble p = i/2 + 4*(i%2), so masks 0x000F000F / 0x00F000F0 of w and of w>>8 each give a
//         pair of consecutive weights (the second mask scaled by 16).
//   TQ2   chunk = half a block, 64 weights.  Word t holds weights 16t..16t+15; weight 16t+i sits in
//         the 2-bit field p = i/2 + 8*(i%2), so masks (0x00030003 << 2j) of w (j < 5) and of
//         w>>10 (j < 3) each give a pair of consecutive weights scaled by 4^j.
//   CB4   chunk = 32 weights in canonical order: byte b holds weights 2b (low) and 2b+1 (high).
//   CB8   chunk = 16 weights, byte b = weight b.
//   AQ1X16 chunk = 8 groups of 8 weights, 64 weights: the 8 little-endian 16-bit codes in
//         canonical order.
//   AQ2X8 is tiled the other way round (one lane per group of 8 weights, not per row): tiles of
//         16 rows x 32 groups.  With G = K/8 groups, KS = ceil(G/32) slices of 32 groups,
//         R16 = Npad/16 row blocks and row block b16 = n/16, the tile (b16, s) sits at
//         ((s*R16 + b16)*64 + lane)*16 with lane = 32*h + g: g = group % 32 of slice s = group / 32,
//         h = (n % 16) / 8, and its 16 bytes are (c0, c1) of rows 16*b16 + 8*h + 0..7 of that
//         group, row by row.  One wavefront load reads one tile (1 KiB); the tiles of consecutive
//         row blocks of one slice are contiguous.  Groups past G and rows past N are zero.
//         C = 4*KS, so the plane still holds RG*C*1024 bytes.
#pragma once
#include <stdint.h>

namespace wqd {

constexpr int kRowsPerGroup = 64;
constexpr int kChunkBytes = 16;
constexpr int64_t kPlaneAlign = 256;

// Largest N and K (the kernels keep N, K, Npad and chunk counts in 32-bit fields).
constexpr int64_t kMaxN = int64_t(1) << 30;
constexpr int64_t kMaxK = int64_t(1) << 30;
enum Fmt : int { Q4_0 = 1, CB4 = 2, CB8 = 3, TQ2 = 4, AQ2X8 = 5, AQ1X16 = 6 };
// Kernel-side id of a TQ2 projection multiplied by int8-quantized activations (TQ2 weights).
constexpr int TQ2I8 = 7;

struct Layout {
    int fmt = 0;
    int64_t N = 0, K = 0;
    int64_t RG = 0;           // row groups (ceil(N / 64))
    int64_t Npad = 0;         // RG * 64
    int64_t row_code_bytes = 0;
    int64_t C = 0;            // 16-byte chunks per row
    int64_t C_full = 0;       // chunks entirely inside K (the rest is a partial tail chunk)
    int64_t weights_per_chunk = 0;
    int64_t blocks = 0;       // scale blocks per row (Q4_0, TQ2)
    int64_t Q = 0;            // quads of blocks per row (Q4_0, TQ2)
    int64_t G = 0, KS = 0;    // AQ2X8: groups of 8 weights per row, slices of 32 groups
    int64_t off_scales = 0, off_cbk = 0, total = 0;
    bool ok = false;
};

inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

inline int k_multiple(int fmt) {
    switch (fmt) {
    case Q4_0: return 32;
    case CB4: return 2;
    case CB8: return 1;
    case TQ2: return 128;
    case AQ2X8: return 8;
    case AQ1X16: return 8;
    default: return 0;
    }
}

inline Layout make_layout(int fmt, int64_t N, int64_t K) {
    Layout L;
    L.fmt = fmt;
    L.N = N;
    L.K = K;
    int km = k_multiple(fmt);
    if (km == 0 || N < 1 || K < 1 || K % km != 0 || N > kMaxN || K > kMaxK)
        return L;
    L.RG = (N + kRowsPerGroup - 1) / kRowsPerGroup;
    L.Npad = L.RG * kRowsPerGroup;
    switch (fmt) {
    case Q4_0: L.row_code_bytes = K / 2; L.weights_per_chunk = 32; L.blocks = K / 32; break;
    case CB4: L.row_code_bytes = K / 2; L.weights_per_chunk = 32; break;
    case CB8: L.row_code_bytes = K; L.weights_per_chunk = 16; break;
    case TQ2: L.row_code_bytes = K / 4; L.weights_per_chunk = 64; L.blocks = K / 128; break;
    case AQ2X8: L.row_code_bytes = K / 4; L.weights_per_chunk = 64; break;
    case AQ1X16: L.row_code_bytes = K / 4; L.weights_per_chunk = 64; break;
    }
    L.C = (L.row_code_bytes + kChunkBytes - 1) / kChunkBytes;
    L.C_full = K / L.weights_per_chunk;
    if (fmt == AQ2X8) {
        L.G = K / 8;
        L.KS = (L.G + 31) / 32;
        L.C = 4 * L.KS;
        L.C_full = L.C;
    }
    L.Q = (L.blocks + 3) / 4;
    int64_t codes = L.RG * L.C * kRowsPerGroup * kChunkBytes;
    int64_t scales = 0, cbk = 0;
    if (fmt == Q4_0 || fmt == TQ2) scales = L.RG * L.Q * kRowsPerGroup * 8;
    if (fmt == AQ2X8 || fmt == AQ1X16) scales = L.Npad * 2;
    if (fmt == CB4) cbk = 32;
    if (fmt == CB8) cbk = 512;
    if (fmt == AQ2X8) cbk = 8192;
    if (fmt == AQ1X16) cbk = 65536 * 8 * 2;
    L.off_scales = align_up(codes, kPlaneAlign);
    L.off_cbk = align_up(L.off_scales + scales, kPlaneAlign);
    L.total = align_up(L.off_cbk + cbk, kPlaneAlign);
    L.ok = true;
    return L;
}

inline int64_t canonical_bytes(int fmt, int64_t N, int64_t K) {
    switch (fmt) {
    case Q4_0: return N * (K / 32) * 18;
    case CB4: return 32 + N * (K / 2);
    case CB8: return 512 + N * K;
    case TQ2: return N * (K / 128) * 34;
    case AQ2X8: return 8192 + 2 * N + N * (K / 8) * 2;
    case AQ1X16: return 65536 * 8 * 2 + 2 * N + N * (K / 8) * 2;
    default: return -1;
    }
}

}  // namespace wqd
