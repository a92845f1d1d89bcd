// Host-side part of libwqd: byte counts and the one-time re-layout of canonical packed weights
// into the prepared device layout described in layout.h.  No HIP calls.
#include <string.h>

#include <vector>

#include "../../include/wqd.h"
#include "layout.h"

static_assert(WQD_MAX_N == wqd::kMaxN && WQD_MAX_K == wqd::kMaxK, "the header states the layout limits");

using namespace wqd;

namespace {

inline uint16_t rd16(const uint8_t *p) { return uint16_t(p[0] | (p[1] << 8)); }
inline void wr16(uint8_t *p, uint16_t v) {
    p[0] = uint8_t(v & 0xFF);
    p[1] = uint8_t(v >> 8);
}

// Destination of chunk c of row n in the code plane.
inline uint8_t *chunk_ptr(uint8_t *codes, const Layout &L, int64_t n, int64_t c) {
    int64_t g = n / kRowsPerGroup, r = n % kRowsPerGroup;
    return codes + ((g * L.C + c) * kRowsPerGroup + r) * kChunkBytes;
}

// Q4_0 row: canonical blocks (d, qs[16]) -> chunks with the nibble order of layout.h.
void prep_q4_0(const Layout &L, const uint8_t *src, uint8_t *dst) {
    uint8_t *codes = dst, *scales = dst + L.off_scales;
    for (int64_t n = 0; n < L.N; n++) {
        int64_t g = n / kRowsPerGroup, r = n % kRowsPerGroup;
        for (int64_t b = 0; b < L.blocks; b++) {
            const uint8_t *blk = src + (n * L.blocks + b) * 18;
            uint8_t code[32];
            for (int j = 0; j < 16; j++) {
                code[j] = blk[2 + j] & 0xF;
                code[j + 16] = blk[2 + j] >> 4;
            }
            uint8_t *out = chunk_ptr(codes, L, n, b);
            for (int t = 0; t < 4; t++) {
                uint32_t w = 0;
                for (int i = 0; i < 8; i++) {
                    int p = i / 2 + 4 * (i % 2);
                    w |= uint32_t(code[8 * t + i]) << (4 * p);
                }
                memcpy(out + 4 * t, &w, 4);
            }
            uint8_t *sd = scales + ((g * L.Q + b / 4) * kRowsPerGroup + r) * 8 + (b % 4) * 2;
            wr16(sd, rd16(blk));
        }
    }
}

// TQ2 row: canonical blocks (d, qs[32]) -> two chunks per block with the 2-bit order of layout.h.
void prep_tq2(const Layout &L, const uint8_t *src, uint8_t *dst) {
    uint8_t *codes = dst, *scales = dst + L.off_scales;
    for (int64_t n = 0; n < L.N; n++) {
        int64_t g = n / kRowsPerGroup, r = n % kRowsPerGroup;
        for (int64_t b = 0; b < L.blocks; b++) {
            const uint8_t *blk = src + (n * L.blocks + b) * 34;
            uint8_t code[128];
            for (int j = 0; j < 128; j++) code[j] = (blk[2 + j / 4] >> (2 * (j % 4))) & 3;
            for (int h = 0; h < 2; h++) {
                uint8_t *out = chunk_ptr(codes, L, n, 2 * b + h);
                for (int t = 0; t < 4; t++) {
                    uint32_t w = 0;
                    for (int i = 0; i < 16; i++) {
                        int p = i / 2 + 8 * (i % 2);
                        w |= uint32_t(code[64 * h + 16 * t + i]) << (2 * p);
                    }
                    memcpy(out + 4 * t, &w, 4);
                }
            }
            uint8_t *sd = scales + ((g * L.Q + b / 4) * kRowsPerGroup + r) * 8 + (b % 4) * 2;
            wr16(sd, rd16(blk));
        }
    }
}

// CB4 / CB8: row code bytes copied in canonical order into 16-byte chunks.
void prep_bytes(const Layout &L, const uint8_t *row_codes, uint8_t *dst) {
    for (int64_t n = 0; n < L.N; n++) {
        const uint8_t *row = row_codes + n * L.row_code_bytes;
        for (int64_t c = 0; c < L.C; c++) {
            int64_t nb = L.row_code_bytes - c * kChunkBytes;
            if (nb > kChunkBytes) nb = kChunkBytes;
            memcpy(chunk_ptr(dst, L, n, c), row + c * kChunkBytes, size_t(nb));
        }
    }
}

// AQ2X8: canonical rows of (c0, c1) pairs -> transposed 16-row x 32-group tiles (layout.h).
void prep_aq2x8(const Layout &L, const uint8_t *row_codes, uint8_t *dst) {
    const int64_t R16 = L.Npad / 16;
    for (int64_t n = 0; n < L.N; n++) {
        const uint8_t *row = row_codes + n * L.G * 2;
        const int64_t b16 = n / 16, h = (n % 16) / 8, r = n % 8;
        for (int64_t g = 0; g < L.G; g++) {
            uint8_t *t = dst + ((g / 32 * R16 + b16) * 64 + 32 * h + g % 32) * kChunkBytes + 2 * r;
            t[0] = row[2 * g];
            t[1] = row[2 * g + 1];
        }
    }
}

}  // namespace

extern "C" {

WQD_API int64_t wqd_canonical_bytes(int fmt, int64_t N, int64_t K) {
    if (k_multiple(fmt) == 0) return WQD_EINVAL;
    Layout L = make_layout(fmt, N, K);
    if (!L.ok) return WQD_ESHAPE;
    return canonical_bytes(fmt, N, K);
}

WQD_API int64_t wqd_prepared_bytes(int fmt, int64_t N, int64_t K) {
    if (k_multiple(fmt) == 0) return WQD_EINVAL;
    Layout L = make_layout(fmt, N, K);
    if (!L.ok) return WQD_ESHAPE;
    return L.total;
}

WQD_API int wqd_prepare_host(int fmt, int64_t N, int64_t K, const void *canonical_host,
                             int64_t canonical_cap, void *prepared_host, int64_t prepared_cap) {
    if (k_multiple(fmt) == 0 || !canonical_host || !prepared_host) return WQD_EINVAL;
    Layout L = make_layout(fmt, N, K);
    if (!L.ok) return WQD_ESHAPE;
    if (canonical_cap < canonical_bytes(fmt, N, K) || prepared_cap < L.total) return WQD_ESPACE;
    const uint8_t *src = static_cast<const uint8_t *>(canonical_host);
    uint8_t *dst = static_cast<uint8_t *>(prepared_host);
    memset(dst, 0, size_t(L.total));
    switch (fmt) {
    case Q4_0: prep_q4_0(L, src, dst); break;
    case TQ2: prep_tq2(L, src, dst); break;
    case CB4:
        prep_bytes(L, src + 32, dst);
        memcpy(dst + L.off_cbk, src, 32);
        break;
    case CB8:
        prep_bytes(L, src + 512, dst);
        memcpy(dst + L.off_cbk, src, 512);
        break;
    case AQ2X8:
        prep_aq2x8(L, src + 8192 + 2 * N, dst);
        memcpy(dst + L.off_scales, src + 8192, size_t(2 * N));
        memcpy(dst + L.off_cbk, src, 8192);
        break;
    case AQ1X16: {
        const int64_t cbk = 65536 * 8 * 2;
        prep_bytes(L, src + cbk + 2 * N, dst);
        memcpy(dst + L.off_scales, src + cbk, size_t(2 * N));
        memcpy(dst + L.off_cbk, src, size_t(cbk));
        break;
    }
    }
    return WQD_OK;
}

WQD_API int wqd_bind(int fmt, int64_t N, int64_t K, const void *prepared, wqd_weight *out) {
    if (k_multiple(fmt) == 0 || !prepared || !out) return WQD_EINVAL;
    Layout L = make_layout(fmt, N, K);
    if (!L.ok) return WQD_ESHAPE;
    if (reinterpret_cast<uintptr_t>(prepared) & 15) return WQD_EALIGN;
    const uint8_t *base = static_cast<const uint8_t *>(prepared);
    const bool has_scales = fmt == Q4_0 || fmt == TQ2 || fmt == AQ2X8 || fmt == AQ1X16;
    const bool has_cbk = fmt == CB4 || fmt == CB8 || fmt == AQ2X8 || fmt == AQ1X16;
    wqd_weight w;
    memset(&w, 0, sizeof(w));
    w.fmt = fmt;
    w.N = int32_t(N);
    w.K = int32_t(K);
    w.codes = base;
    w.scales = has_scales ? base + L.off_scales : nullptr;
    w.codebooks = has_cbk ? base + L.off_cbk : nullptr;
    w.code_row_bytes = L.row_code_bytes;
    w.scale_row_elems = fmt == Q4_0 ? K / 32 : fmt == TQ2 ? K / 128 : (fmt == AQ2X8 || fmt == AQ1X16) ? 1 : 0;
    *out = w;
    return WQD_OK;
}

WQD_API const char *wqd_status_str(int status) {
    switch (status) {
    case WQD_OK: return "ok";
    case WQD_EINVAL: return "invalid argument (null pointer, unknown format or mode)";
    case WQD_ESHAPE: return "bad shape (N, K multiple, M range or leading dimension)";
    case WQD_EALIGN: return "misaligned pointer or leading dimension";
    case WQD_ESPACE: return "buffer or workspace too small";
    case WQD_EHIP: return "HIP runtime error";
    case WQD_ESTALE: return "a persistent launch found a descriptor table set up for another list";
    default: return "unknown status";
    }
}

}  // extern "C"
