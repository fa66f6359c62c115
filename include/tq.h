/*
 * tq.h -- C ABI of libtq: packed-ternary weights x q8_K activations on
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow the statement of the problem on the pages
 * "how i made a 27b ternary model 3.8x faster on a laptop cpu by reordering
 * its bits" (page 1) and the ciot README (page 2):
 *
 *   - weights w in {-1, 0, +1}, one fp16 scale per 128 weights of a row;
 *     pq2_0 stores u = w + 1 in 2 bits (page 1, "what's running"),
 *     ptq1_0 stores five trits per byte (page 1, "the detour that lost");
 *   - activations are quantized on the fly to q8_K: blocks of 256 int8, one
 *     float scale, 16 partial sums (page 2, intro; page 1, "the paperwork");
 *   - a load-time repack reorders the weight bits once (page 1, "the layout");
 *   - the product is exact integer arithmetic per 128-weight group, with the
 *     float scales applied afterwards (page 1, "the trick with 4 and 16");
 *   - a decode step is a matrix-vector product, a prompt step a product with
 *     a small batch of tokens (page 1, "prefill wants a different shape").
 *
 * Conventions (all entry points):
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise, owned
 *     by the caller.  The library never allocates, frees or synchronizes.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *     null stream) and runs asynchronously; buffers must stay alive until it
 *     completes.
 *   - Arguments are validated on the host before anything is launched.  On any
 *     error nothing is launched and no output is touched.
 *   - Return value: TQ_OK, or a negative TQ_ERR_* code.  TQ_ERR_HIP means a
 *     HIP call failed; tq_last_hip_error() then holds its hipError_t value.
 *   - Outputs are overwritten, never accumulated into.
 *   - Shapes: rows >= 1; cols >= 256 and a multiple of 256 (so every 128-weight
 *     group lies inside one 256-value q8_K block); tokens >= 1.  Otherwise
 *     TQ_ERR_SHAPE.  Limits: rows <= 2^26, cols <= 2^20 (ptq1_0: cols <=
 *     32768), rows * cols <= 2^36, tokens <= 2^20, tokens * cols <= 2^36.
 *   - Alignment: weight buffers and q 16 bytes; x, d, y, idots 4 bytes;
 *     bsums 2 bytes.  Otherwise TQ_ERR_ALIGN.
 *
 * Canonical (file) formats, row-major by (row, group):
 *   pq2_0  34-byte block per 128 weights: little-endian fp16 d, then qs[32];
 *          weight k of the group is the 2-bit code u = w + 1 at bits
 *          2*(k&3)..2*(k&3)+1 of qs[k>>2] (low bits first).  Code 3 is not a
 *          pq2_0 value (three values need only codes 0..2).
 *   ptq1_0 28-byte block per 128 weights: little-endian fp16 d, then qs[26];
 *          weight k is trit (k%5) of qs[k/5]: with v = (qs[k/5] * 3^(k%5))
 *          mod 256, trit = floor(3 v / 256) and w = trit - 1.  Trits 3 and 4
 *          of qs[25] are padding and never used.  Every byte value decodes.
 *   q8_K   for T tokens and K columns: q int8 [T][K], d fp32 [T][K/256],
 *          bsums int16 [T][K/16] (bsums[t][j] = sum of q[t][16j .. 16j+15]).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TQ_FMT_PQ2_0 = 1, TQ_FMT_PTQ1_0 = 2 } tq_format;

enum {
    TQ_OK = 0,
    TQ_ERR_NULL = -1,        /* a required pointer is NULL */
    TQ_ERR_SHAPE = -2,       /* rows/cols/tokens outside the supported shapes */
    TQ_ERR_ALIGN = -3,       /* a pointer is not aligned as required */
    TQ_ERR_FORMAT = -4,      /* unknown tq_format value */
    TQ_ERR_UNSUPPORTED = -5, /* valid arguments, operation not provided */
    TQ_ERR_HIP = -6          /* a HIP runtime call failed */
};

/* Shape check ("the selector"): the pages' repack is chosen only for shapes it
 * handles and rejects the others (page 1, "did i break the model?": shapes
 * the selector should reject).  Returns TQ_OK or TQ_ERR_SHAPE/TQ_ERR_FORMAT. */
int tq_check_shape(int fmt, int64_t rows, int64_t cols, int64_t tokens);

/* Bytes of the canonical matrix (ciot README, format notes: a pq2_0 block is
 * an fp16 scale and 32 bytes of 2-bit codes, a ptq1_0 block an fp16 scale and
 * 26 bytes of base-3 codes): 34 (pq2_0) or 28 (ptq1_0) per 128 weights.
 * Returns 0 for an invalid format or shape. */
int64_t tq_canonical_bytes(int fmt, int64_t rows, int64_t cols);

/* Bytes of the repacked device layout, including the internal padding of the
 * row count to a multiple of 64 (and, for ptq1_0, of the group count to a
 * multiple of 8).  Returns 0 for an invalid format or shape. */
int64_t tq_repacked_bytes(int fmt, int64_t rows, int64_t cols);

/* Load-time repack (page 1, "the layout": runs once when the model loads and
 * costs nothing per token afterwards).  Reads the canonical matrix `src`
 * (tq_canonical_bytes) and writes the device layout into `dst`
 * (tq_repacked_bytes; out of place, `src` may be freed afterwards).  The
 * layout is private to this library: pass it only to tq_gemv, tq_gemm,
 * tq_group_dots and tq_unrepack of the same library version.
 * `bad_flag` (nullable, device int32): for pq2_0, every thread that meets a
 * code 3 stores 1 into it (the caller clears it beforehand); products over a
 * matrix that holds code 3 are unspecified.  Ignored for ptq1_0. */
int tq_repack(int fmt, const void *src, void *dst, int64_t rows, int64_t cols, int32_t *bad_flag, void *stream);

/* Inverse of tq_repack, for tests and export: writes the canonical matrix
 * (tq_canonical_bytes).  Both formats round-trip byte for byte (pq2_0 for
 * codes 0..2; ptq1_0 including the padding trits, which are copied as is). */
int tq_unrepack(int fmt, const void *src_repacked, void *dst, int64_t rows, int64_t cols, void *stream);

/* q8_K quantization (page 2 intro; page 1 "the paperwork": activations are
 * squashed to int8 on the fly).  x fp32 [tokens][cols] -> q, d, bsums as in the
 * q8_K format above.  Per 256-block: d = max|x| / 127 (fp32, correctly
 * rounded); q = round-to-nearest-even(x / d) (fp32 division); a block with
 * d == 0 gives q = 0 and bsums = 0.  Inputs must be finite. */
int tq_quantize_q8k(const float *x, int64_t tokens, int64_t cols, int8_t *q, float *d, int16_t *bsums, void *stream);

/* Bytes of the optional workspace of tq_gemv / tq_gemv_f32 / tq_gemv_f32_batch
 * for this shape (tq_gemm uses it only for a single token).  The workspace lets a product
 * split its columns over several workgroups per 64-row tile (fp64 partial
 * sums plus per-tile arrival counters), which keeps all compute units busy
 * when the row count is small.  It holds one block of 16400 bytes per 64-row
 * tile, laid out alike for every shape, format and entry point: the tile's
 * 32-bit arrival counter, then fp64 partial sums that are always written
 * before they are read.
 *
 * Contract: device memory of at least this size, 16-byte aligned, whose
 * counters are zero when a call starts.  Zero it once before first use
 * (tq_workspace_clear, or any zero fill).  Every call that completes returns
 * the counters it used to zero, so the workspace can then be reused by later
 * calls of any shape, format and token count whose tile count it covers (also
 * inside a captured graph) without clearing.  Calls that run at the same time
 * must not share one.
 *
 * What breaks the contract: a counter that is not zero at entry (a workspace
 * never cleared, or two overlapping calls on one workspace) makes a tile's
 * reduction run early or never: its y entries are then wrong or left
 * unwritten, with no error reported.  A call cannot be interrupted part-way
 * except by a fault that ends the HIP context.  Recover by calling
 * tq_workspace_clear on the workspace (stream-ordered) before the next call.
 * Returns 0 for an invalid shape. */
int64_t tq_workspace_bytes(int fmt, int64_t rows, int64_t cols, int64_t tokens);

/* Zero `bytes` bytes of a workspace (device memory, 16-byte aligned) with a
 * kernel on `stream`.  It records no memset, so it may be captured in a
 * graph.  Returns TQ_OK (nothing launched for bytes == 0), TQ_ERR_NULL,
 * TQ_ERR_ALIGN, TQ_ERR_SHAPE (bytes < 0) or TQ_ERR_HIP. */
int tq_workspace_clear(void *workspace, int64_t bytes, void *stream);

/* Matrix-vector product, one token (page 1, "the trick with 4 and 16" and
 * "did it reach the wall?"):
 *   y[r] = sum_g d_w[r][g] * d[g/2] * I[r][g],
 *   I[r][g] = sum_{k<128} w[r][128g+k] * q[128g+k]   (exact integer),
 * the float part evaluated in fp64 and rounded to fp32 once.  `w` is the
 * repacked matrix.  `bsums` is read for ptq1_0 and may be NULL for pq2_0.
 * `workspace` (nullable, see tq_workspace_bytes): without it each 64-row tile
 * is one workgroup.  Results are deterministic either way; with and without a
 * workspace they agree to within the fp64 rounding of the partial sums. */
int tq_gemv(int fmt, const void *w, int64_t rows, int64_t cols, const int8_t *q, const float *d, const int16_t *bsums,
            float *y, void *workspace, void *stream);

/* Quantize and multiply in one call, one token (page 1, "the paperwork":
 * activations are squashed to int8 on the fly, right before the product):
 * x fp32 [cols] -> y fp32 [rows].  Every workgroup quantizes the slice of x
 * it needs to q8_K in on-chip memory, with the arithmetic of
 * tq_quantize_q8k, so y is bit-identical to tq_quantize_q8k followed by
 * tq_gemv (same workspace argument); no q8_K buffer is written.  pq2_0
 * only.  x: 16-byte aligned, finite.  The q8_K of one
 * workgroup's column slice must fit on chip (at most 126 blocks of 256, i.e.
 * 32256 columns): with n = cols / 256 and tiles = ceil(rows / 64), a slice is
 * ceil(n / s) blocks, s = 1 without a workspace or when tiles >= 384, else
 * s = the smallest value from 1 up to min(16, max(1, n / 4)) with
 * ceil(n / s) <= 12 and tiles * s >= 224 (that cap if none).  Shapes beyond
 * that, and
 * ptq1_0, return TQ_ERR_UNSUPPORTED (checked before the pointers) and touch
 * nothing. */
int tq_gemv_f32(int fmt, const void *w, int64_t rows, int64_t cols, const float *x, float *y, void *workspace,
                void *stream);

/* tq_gemv_f32 without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the column split's workspace is the library's own
 * static device scratch (6,297,600 bytes per GPU, held until the process
 * ends), so the call allocates nothing.  The result is bit-identical to
 * tq_gemv_f32 with a zeroed workspace of tq_workspace_bytes.  The scratch is
 * looked up and zero-filled (with a kernel, on `stream`) at the first call on
 * a device.  Every call on one GPU shares that GPU's scratch, which keeps the
 * last call's contents (the tile counters are back at zero after each
 * call): calls that overlap on one GPU (concurrent streams, or threads) race
 * and may return wrong or unwritten outputs.  Shapes and errors as for
 * tq_gemv_f32; a shape whose split would need more than the scratch returns
 * TQ_ERR_UNSUPPORTED (none does: the split is used only below 384 row tiles,
 * which the scratch covers). */
int tq_gemv_f32_scratch(int fmt, const void *w, int64_t rows, int64_t cols, const float *x, float *y, void *stream);

/* Several independent tq_gemv_f32 products with the same column count in one
 * launch (page 1, "what's running": a decode step runs one product after
 * another for every projection of every layer; products that do not depend
 * on one another, such as the gate and up projections of a layer, can share
 * a launch).  Problem m (m < n, 1 <= n <= 4): w[m] (repacked pq2_0, rows[m] x
 * cols), x[m] fp32 [cols] (16-byte aligned), y[m] fp32 [rows[m]].  The
 * host arrays w, rows, x and y are read during the call only.  Each y[m] is
 * the same as a tq_gemv_f32 call would give it with the same workspace
 * treatment for a matrix of all the problems' row tiles together: with no
 * workspace, or 384 or more row tiles in total, bit-identical to separate
 * tq_gemv_f32 calls without a workspace.  `workspace` (nullable): at least
 * tq_workspace_bytes(fmt, R, cols, 1) bytes, R = the sum of the rows[m] each
 * rounded up to a multiple of 64.  The on-chip rule of tq_gemv_f32 applies
 * to that R (TQ_ERR_UNSUPPORTED, checked before the per-problem pointers).
 * pq2_0 only. */
int tq_gemv_f32_batch(int fmt, int n, const void *const *w, const int64_t *rows, int64_t cols, const float *const *x,
                      float *const *y, void *workspace, void *stream);

/* Matrix product with a small batch of tokens (page 1, "prefill wants a
 * different shape" and "the leftovers"): y[t][r] for t < tokens, the same
 * arithmetic as tq_gemv per token.  Token counts that are not a multiple of
 * the kernel's tile are padded internally; padded outputs are never written.
 * A single token runs the matrix-vector kernel.  `workspace` as for tq_gemv;
 * with more than one token it is not used.  With tokens > 1, y[t] is
 * bit-identical to tq_gemv of token t without a workspace, for both formats,
 * so a batch of a few tokens gives exactly the outputs of one product per
 * token.  pq2_0 runs on int8 matrix cores.  ptq1_0 with up to 7 tokens
 * decodes each base-3 byte once per block of 2 tokens and takes the dot
 * products on the vector units; from 8 tokens on it decodes once per 16
 * tokens and runs on int8 matrix cores. */
int tq_gemm(int fmt, const void *w, int64_t rows, int64_t cols, int64_t tokens, const int8_t *q, const float *d,
            const int16_t *bsums, float *y, void *workspace, void *stream);

/* Test export: the exact integer group dots I[t][r][g] (page 1, "the trick
 * with 4 and 16": the integer dot of one 128-weight group with its int8
 * activations, before any scale) (int32, [tokens][rows][cols/128]), computed
 * by the same kernels as tq_gemv (tokens == 1) and tq_gemm (tokens > 1). */
int tq_group_dots(int fmt, const void *w, int64_t rows, int64_t cols, int64_t tokens, const int8_t *q,
                  const int16_t *bsums, int32_t *idots, void *stream);

/* Static description of a status code. */
const char *tq_status_str(int status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int tq_last_hip_error(void);

/* Library version (major * 10000 + minor * 100 + patch). */
int tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
