/* wqd.h -- C ABI of the MI355X (gfx950) weight-quantized decode library (libwqd.so).
 *
 * The library computes the projection of batch-1 and small-batch LLM decode,
 *
 *     y[m][n] = sum_k x[m][k] * dequant(Wq)[n][k]       (0 <= m < M, 0 <= n < N, 0 <= k < K)
 *
 * with M <= 8 activation rows per call (16 in a batch-invariant list, WQD_MAX_M_VERIFY), packed
 * low-bit weights streamed from HBM once, decoded in registers and multiplied by a short fp16
 * activation row, accumulating in fp32.  The operation and the formats are those of:
 *   - trapetum "Benchmarks" (trapetum.neuralboot.com), "Kernel microbenchmarks" (4-bit and 8-bit
 *     codebook GEMV), "Additive vector-quantization GEMV (AQLM-style, 2-bit)", and the November
 *     update's fused, graphed decode step;
 *   - "Making a ternary reasoning model fast in vLLM", "Anatomy of a PQ2_0 block" and "The ideal
 *     kernel, as a checklist" (the 2-bit ternary block and the batch-1 projection y = x W^T with
 *     M input rows, N outputs and K inputs);
 *   - "Model quantization, read carefully" (blog.localai.hex7.com), "The ladder" table (Q4_0).
 *
 * Conventions
 *   - Every pointer is a device pointer unless its name ends in _host.  The caller owns every
 *     buffer; the library allocates no device memory and never synchronizes the stream except in
 *     wqd_stream_check.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Kernels are enqueued
 *     on it asynchronously; calls are stream-ordered and reentrant.
 *   - Functions return a wqd_status.  Argument errors are detected before any HIP call.  A launch
 *     failure returns WQD_EHIP (see wqd_last_hip_error); a fault inside a kernel surfaces later,
 *     through wqd_stream_check.
 *   - x is fp16 (IEEE binary16 bit patterns), row-major with leading dimension ldx (elements).
 *     y is fp32, row-major with leading dimension ldy (elements).
 *
 * Formats (fmt) and their canonical (interchange) bytes, all little-endian:
 *   WQD_Q4_0  per row, K/32 blocks of 18 B: fp16 scale d, then 16 bytes of 4-bit codes; byte j
 *             holds weight j (low nibble) and weight j+16 (high nibble); weight = (code - 8) * d.
 *   WQD_CB4   16 fp16 centroids (32 B), then codes [N][K/2]: low nibble = even k; weight = cb[code].
 *   WQD_CB8   256 fp16 centroids (512 B), then codes [N][K]; weight = cb[code].
 *   WQD_TQ2   per row, K/128 blocks of 34 B: fp16 scale d, then 32 bytes of 2-bit codes, weight j
 *             of the block at bits 2*(j%4) of byte j/4; weight = (code - 1) * d (code 3 -> +2d).
 *   WQD_AQ2X8 codebooks C[2][256][8] fp16 (8192 B), row scales s[N] fp16, codes [N][K/8][2]
 *             (codebook 0 first); weight k of row n = s[n] * (C[0][c0][k%8] + C[1][c1][k%8]) with
 *             (c0, c1) the codes of group k/8.
 *   WQD_AQ1X16 one codebook C[65536][8] fp16 (1 MiB), row scales s[N] fp16, codes [N][K/8] as
 *             little-endian uint16; weight k of row n = s[n] * C[code][k%8] with code the code of
 *             group k/8 (trapetum "Benchmarks", November update: the 70B PV-tuned model in AQLM's
 *             1x16 layout, 2 bits per weight).
 *   K must be a multiple of 32 (Q4_0), 2 (CB4), 1 (CB8), 128 (TQ2) or 8 (AQ2X8, AQ1X16).
 *
 * Prepared (device) layout: the same bytes re-laid once at load time into planes ("prepared
 * weights": a code plane, then the scale plane, then codebooks), built by wqd_prepare_host and
 * uploaded by the caller.  Its size is wqd_prepared_bytes(); it must be 16-byte aligned on the
 * device.  wqd_bind turns a prepared buffer into a wqd_weight view (one pointer per plane), and
 * every compute entry point takes that view (the ternary page's prepared-weight planes, "Anatomy
 * of a PQ2_0 block"; trapetum "Benchmarks", "Per-layer PyTorch op speedup vs torch dense fp16": the
 * per-projection op that replaces torch.mv takes such a weight and a short activation row).
 */
#ifndef WQD_H
#define WQD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WQD_API __attribute__((visibility("default")))

typedef enum { WQD_Q4_0 = 1, WQD_CB4 = 2, WQD_CB8 = 3, WQD_TQ2 = 4, WQD_AQ2X8 = 5, WQD_AQ1X16 = 6 } wqd_format;

typedef enum {
    WQD_OK = 0,
    WQD_EINVAL = -1, /* null pointer, unknown format or mode */
    WQD_ESHAPE = -2, /* N or K outside 1..2^30, K not a whole number of blocks/groups, M outside
                        1..8, ld too small */
    WQD_EALIGN = -3, /* weight not 16-byte aligned, x or y not 4-byte aligned, odd ldx */
    WQD_ESPACE = -4, /* a capacity or workspace argument is smaller than required */
    WQD_EHIP = -5,   /* a HIP call failed; wqd_last_hip_error() gives its hipError_t */
    WQD_ESTALE = -6  /* (reported by wqd_stream_check) a WQD_PERSISTENT launch found the workspace's
                        descriptor table set up for another list, and wrote no output */
} wqd_status;

enum { WQD_MAX_M = 8 };
/* Rows of one batch-invariant list call (WQD_BATCH_INVARIANT without WQD_INT8_ACTIVATIONS): a
 * verify of up to 16 draft tokens in one pass over the weights. */
enum { WQD_MAX_M_VERIFY = 16 };
/* Largest N and K any call accepts (2^30 each): the kernels keep N, K and their chunk counts in
 * 32-bit fields. */
enum { WQD_MAX_N = 1 << 30, WQD_MAX_K = 1 << 30 };

/* ---------------------------------------------------------------- layout (host only, no HIP) */

/* Bytes of the canonical encoding of an N x K matrix, or a negative wqd_status. */
WQD_API int64_t wqd_canonical_bytes(int fmt, int64_t N, int64_t K);

/* Bytes of the prepared (device) layout, or a negative wqd_status. */
WQD_API int64_t wqd_prepared_bytes(int fmt, int64_t N, int64_t K);

/* Re-lay canonical bytes (host memory) into the prepared layout (host memory).  Pure host code:
 * canonical_bytes and prepared_bytes are the capacities of the two buffers; they must be at least
 * wqd_canonical_bytes() and wqd_prepared_bytes().  Padding bytes are written as zero. */
WQD_API int wqd_prepare_host(int fmt, int64_t N, int64_t K, const void *canonical_host,
                             int64_t canonical_bytes, void *prepared_host, int64_t prepared_bytes);

/* ---------------------------------------------------------------- bound weights */

/* A prepared weight matrix of one format, as plane pointers (device memory owned by the caller;
 * the planes need not be contiguous).  Fields:
 *   fmt, N, K          format and shape (N, K <= 2^30; K a whole number of blocks or groups);
 *   codes              the code plane (16-byte aligned);
 *   scales             Q4_0 / TQ2 block scales (8-byte aligned), AQ2X8 / AQ1X16 row scales
 *                      (2-byte aligned); NULL for CB4, CB8;
 *   codebooks          CB4 16 / CB8 256 entries (2-byte aligned), AQ2X8 C[2][256][8] / AQ1X16
 *                      C[65536][8] (16-byte aligned); NULL for Q4_0, TQ2;
 *   code_row_bytes     packed code bytes per row: K/2 (Q4_0, CB4), K (CB8), K/4 (TQ2, AQ2X8, AQ1X16);
 *   scale_row_elems    scales per row: K/32 (Q4_0), K/128 (TQ2), 1 (AQ2X8, AQ1X16), 0 (CB4, CB8).
 * Calls check every field and return WQD_EINVAL (missing plane, unknown format), WQD_ESHAPE
 * (shape, or row sizes that do not match it) or WQD_EALIGN before any HIP call. */
typedef struct {
    int32_t fmt, N, K, pad;
    const void *codes, *scales, *codebooks;
    int64_t code_row_bytes, scale_row_elems;
} wqd_weight;

/* Fill *out with the planes of a prepared buffer (wqd_prepared_bytes(fmt, N, K) bytes, 16-byte
 * aligned, laid out by wqd_prepare_host).  Pure host arithmetic: `prepared` is not read.  Errors:
 * WQD_EINVAL (NULL argument, unknown format), WQD_ESHAPE, WQD_EALIGN. */
WQD_API int wqd_bind(int fmt, int64_t N, int64_t K, const void *prepared, wqd_weight *out);

/* ---------------------------------------------------------------- one projection */

/* Device workspace wqd_gemm needs for this weight and M, in bytes (0 = none): split-K counters and
 * partial sums.  Or a negative wqd_status. */
WQD_API int64_t wqd_workspace_bytes(const wqd_weight *w, int64_t M);

/* y[m*ldy + n] = sum_k x[m*ldx + k] * W[n][k] for 1 <= M <= 8 (N, K and W from the view w),
 * enqueued on `stream`.
 * x: M rows of K fp16 values, ldx >= K and even, 4-byte aligned.  y: M rows of N fp32, ldy >= N.
 * workspace: at least wqd_workspace_bytes(w, M) bytes of device memory (may be NULL when that is
 * 0).  It must be zero-filled before its first use; every call leaves its counters
 * at zero again, so it can be reused by later calls on the same stream (calls that overlap in
 * time must not share a workspace).  When K is split, the wave that finishes the last K-slice of
 * a 64-row group adds the slices' partial sums in ascending order, so results are the same bits
 * from run to run.  Every call is one launch.  AQ2X8 forms its group sums in fp32 at every M:
 * fp32 lookup tables of the activations at M = 1 and 2, exact fp16 products of codebook entries
 * summed in fp32 on the matrix cores at M > 2; its K-splits are added in split order by the
 * workgroup that finishes last. */
WQD_API int wqd_gemm(const wqd_weight *w, const void *x, int64_t M, int64_t ldx, float *y, int64_t ldy,
                     void *workspace, int64_t workspace_bytes, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): wqd_gemm without a workspace argument.  The split-K counters and
 * partial sums live in a file-scope device array of WQD_NOALLOC_MAX_BYTES bytes, one copy per GPU,
 * held from the first call on that GPU until the process ends.  The first call on a device looks
 * the array's address up and clears it with a kernel on `stream`; every call leaves its counters
 * at zero again.  The call allocates nothing (no hipMalloc, no allocating library routine).  All
 * calls on one GPU share the array: calls that overlap in time on one GPU (other streams, other
 * threads) race and must not be made.  Arguments and results as wqd_gemm; WQD_ESPACE when the
 * shape needs more than WQD_NOALLOC_MAX_BYTES (wqd_workspace_bytes() gives the need). */
#define WQD_NOALLOC_MAX_BYTES (16ll << 20)
WQD_API int wqd_gemm_noalloc(const wqd_weight *w, const void *x, int64_t M, int64_t ldx, float *y,
                             int64_t ldy, void *stream);

/* ---------------------------------------------------------------- TQ2 with int8 activations */

/* Device workspace wqd_gemm_i8 needs (always > 0): the quantized activations and wqd_gemm's
 * counters and partial sums.  w must be a WQD_TQ2 weight (WQD_EINVAL otherwise). */
WQD_API int64_t wqd_gemm_i8_workspace_bytes(const wqd_weight *w, int64_t M);

/* The TQ2 projection with int8 activations ("Making a ternary reasoning model fast in vLLM", "Why
 * small integers are a good fit"): each 128-element block of each row of x is quantized to int8,
 * a = max|x| / 127 and q = x / a rounded to nearest even (both fp32; q = 0 for an all-zero
 * block), then y[m][n] = sum_b d_b * a[m][b] * sum_{k in b} (code_k - 1) * q[m][k] with exact
 * integer block sums (v_dot4_i32_i8) and fp32 accumulation over blocks.  Two launches: the
 * quantizer, then the product.  Lossy against wqd_gemm: each activation moves by at most a/2, so
 * |y_i8 - y| <= sum_k |w[n][k]| * a(k) / 2.  Arguments as wqd_gemm (w must be WQD_TQ2); the
 * workspace (256-byte aligned, at least wqd_gemm_i8_workspace_bytes) is required and must be
 * zero-filled before its first use, like wqd_gemm's. */
WQD_API int wqd_gemm_i8(const wqd_weight *w, const void *x, int64_t M, int64_t ldx, float *y, int64_t ldy,
                        void *workspace, int64_t workspace_bytes, void *stream);

/* Inspection of the quantizer wqd_gemm_i8 runs first: q[m*K + k] (int8, natural order), a[m*(K/128)
 * + b] (fp32) and qsum[m*(K/128) + b] (int32, the block's sum of q) for M <= 8 rows of x, K a
 * multiple of 128.  The values are those wqd_gemm_i8 uses (it stores q in another order). */
WQD_API int wqd_quantize_i8(const void *x, int64_t M, int64_t K, int64_t ldx, int8_t *q, float *a,
                            int32_t *qsum, void *stream);

/* Debug decode: out[n*K + k] = dequantized weight in fp32, bit-exact: the exact value for Q4_0,
 * CB4, CB8, TQ2 and AQ1X16 (all representable in fp32); for AQ2X8 fp32(fp32(C0 + C1) * s) with
 * round-to-nearest-even after the add and after the product. */
WQD_API int wqd_dequant_f32(const wqd_weight *w, float *out, void *stream);

/* ---------------------------------------------------------------- layer / stack */

/* Epilogue of a projection in a list (trapetum "Benchmarks", "Short-context decode, step by
 * step": the fused decode kernels apply SiLU(gate) times up in the reduce of the gate/up
 * projection and add the residual inside the reduces of the o and down projections).  The
 * epilogue runs where the projection's K-slices are summed, so it costs no extra launch and no
 * extra pass over y.  AQ2X8 entries take WQD_EPI_NONE only. */
typedef enum {
    WQD_EPI_NONE = 0,      /* y[m][n] = sum_k x[m][k] W[n][k] */
    WQD_EPI_ADD = 1,       /* y[m][n] += sum_k x[m][k] W[n][k]: y holds the residual on entry */
    WQD_EPI_SILU_GATE = 2, /* gate of a gate/up pair; the next entry must be its WQD_EPI_SILU_UP */
    WQD_EPI_SILU_UP = 3    /* up of the pair (same fmt and N as the gate; K, w and x its own):
                              the gate entry's y[m][n] = SiLU(g[m][n]) * u[m][n], with
                              g = x_gate W_gate^T, u = x_up W_up^T and SiLU(g) = g / (1 + e^-g),
                              evaluated in fp32 on the fp32 sums.  This entry's y and ldy are
                              not used (y may be NULL). */
} wqd_epilogue;

typedef struct {
    const wqd_weight *w; /* bound weights (format and shape come from the view); host memory, read
                            during the call only */
    int32_t epi;         /* wqd_epilogue */
    int32_t pad;
    const void *x;       /* fp16 activations, M rows of ldx */
    int64_t ldx;
    float *y;            /* fp32 outputs, M rows of ldy */
    int64_t ldy;
} wqd_proj;

enum {
    WQD_ORDERED = 0,    /* entries one after another, each its own launch (a gate/up pair is one
                           entry) */
    WQD_PERSISTENT = 1, /* one persistent launch per format set (CB4 and CB8 together at M = 1)
                           over the whole list; valid when no entry's x is another entry's y and
                           no two entries write the same y elements.  Needs wqd_stack_setup. */
    WQD_FUSED = 2       /* runs of consecutive entries of one format that read the same x (same
                           pointer and ldx) share one launch, at most 4 entries per launch and a
                           gate/up pair never split (q/k/v in one launch, gate/up in one); runs
                           follow one another in list order, so a later run may read what an
                           earlier one wrote.  AQ2X8 entries launch one at a time.  Entries
                           of one run must not write the same y elements. */
};

/* Flag OR-ed into a mode: batch-invariant results (trapetum "Benchmarks", November update: a
 * draft of M tokens verified in one pass whose rows carry, bit for bit, the logits of M decode
 * steps).  With it, row m of a call with M activation rows is bitwise equal to the same call
 * made with row m alone (M = 1), for every M <= WQD_MAX_M_VERIFY (16), in every mode and whatever
 * else the list holds: every projection is sliced the same way at every M, and every M runs the
 * same per-row instruction sequence (the matrix-core path with one accumulator chain per 4 rows).
 * A verify of 9..16 rows reads the weights once (one workgroup per CU); its AQ2X8 entries run as
 * two launches of rows 0..7 and 8.. (the matrix-core kernel takes 8 rows; those weights are read
 * twice).  WQD_INT8_ACTIVATIONS lists take at most 8 rows.  AQ2X8 entries take the matrix-core kernel at every M
 * (the M <= 2 lookup-table kernel rounds differently), with pieces planned for every CU whatever
 * the list.  Results differ in rounding (within the bound) from calls without the flag. */
enum { WQD_BATCH_INVARIANT = 0x10 };

/* Flag OR-ed into a mode: the TQ2 entries of the list multiply int8-quantized activations, as
 * wqd_gemm_i8 does ("Making a ternary reasoning model fast in vLLM": "Why small integers are a
 * good fit", and "prepare each input once" of its checklist).  Each distinct activation (x, ldx,
 * K) of the list's TQ2 entries is quantized once per call, before the first launch that reads it
 * (after the launches before it, which may have written x): the activations a segment of the list
 * is the first to read are quantized together by one launch placed before the segment's launches
 * (in WQD_PERSISTENT mode, one quantizer launch for the whole list; up to 8 activations per
 * launch).  Entries that share x share its int8 copy.  Other formats are unaffected. */
enum { WQD_INT8_ACTIVATIONS = 0x20 };

/* Device workspace bytes for wqd_run_projections over this list in any mode (descriptor
 * tables, counters and partial sums).  In WQD_ORDERED and WQD_FUSED modes the workspace is used
 * like wqd_gemm's: zero-filled before its first use (or initialised by wqd_stack_setup), and
 * left with its counters at zero by every call; it may be NULL when no launch of the list splits
 * K and the list holds no gate/up pair.  In WQD_PERSISTENT mode wqd_stack_setup initialises it. */
WQD_API int64_t wqd_stack_workspace_bytes(const wqd_proj *projs_host, int32_t count, int64_t M);

/* Write the descriptor tables of this projection list for `mode` (WQD_PERSISTENT, optionally
 * with WQD_BATCH_INVARIANT and WQD_INT8_ACTIVATIONS) into the workspace, zero its counters and
 * stamp the tables with a fingerprint of the list.  Everything is enqueued on `stream` as kernel
 * launches whose data travel in their arguments (no host synchronization, no memset or copy
 * node: the call may be captured in a graph).
 * Must be called before wqd_run_projections in that mode, and again whenever a pointer, shape,
 * epilogue or mode of the list changes.  A WQD_PERSISTENT call whose list does not match the
 * stamp (setup not repeated after a change) writes no output: its kernels return at once and
 * the next wqd_stream_check reports WQD_ESTALE.  Errors: WQD_EINVAL for another mode. */
WQD_API int wqd_stack_setup(const wqd_proj *projs_host, int32_t count, int64_t M, int32_t mode,
                            void *workspace, int64_t workspace_bytes, void *stream);

/* Run every projection of the list with its epilogue.  `mode` is WQD_ORDERED, WQD_PERSISTENT
 * or WQD_FUSED, optionally OR-ed with WQD_BATCH_INVARIANT and WQD_INT8_ACTIVATIONS.  Errors: WQD_EINVAL for a bad mode or epilogue, a gate entry not followed by
 * its up entry (or an up entry without its gate, or the two differing in fmt or N), an epilogue
 * on an AQ2X8 entry, or a NULL workspace in WQD_PERSISTENT mode; WQD_ESPACE for a workspace
 * smaller than wqd_stack_workspace_bytes when one is needed; the wqd_gemm checks per entry. */
WQD_API int wqd_run_projections(const wqd_proj *projs_host, int32_t count, int64_t M, int32_t mode,
                                void *workspace, int64_t workspace_bytes, void *stream);

/* Profiling variant: the same work as wqd_run_projections, with hipEvent_t events[2i] recorded
 * on the stream just before the i-th kernel launch of the call and events[2i+1] just after it.
 * Launch order in WQD_PERSISTENT mode: the int8 quantizer (WQD_INT8_ACTIVATIONS), the CB4+CB8
 * launch if both formats are present, then one launch per remaining format (ascending format
 * id); in the other modes, list order (a segment's quantizer first).
 * n_events must be 2 * wqd_stack_launches(); the events are created and owned by the caller. */
WQD_API int wqd_run_projections_timed(const wqd_proj *projs_host, int32_t count, int64_t M,
                                      int32_t mode, void *workspace, int64_t workspace_bytes,
                                      void *stream, void *const *events, int32_t n_events);

/* Number of kernel launches one call in `mode` issues for this list (or a negative status). */
WQD_API int wqd_stack_launches(const wqd_proj *projs_host, int32_t count, int64_t M, int32_t mode);

/* ---------------------------------------------------------------- errors */

/* Synchronize `stream` and map any pending asynchronous error to WQD_EHIP; then WQD_ESTALE if a
 * WQD_PERSISTENT launch on this device found a stale descriptor table since the last check
 * (the report is per device, and clears it). */
WQD_API int wqd_stream_check(void *stream);
/* hipError_t of the last WQD_EHIP returned on this thread (0 if none). */
WQD_API int wqd_last_hip_error(void);
WQD_API const char *wqd_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* WQD_H */
