/*
 * bi.h -- C ABI of the deterministic, batch-invariant training GEMM library
 * for AMD Instinct MI355X (gfx950).
 *
 * Operations (each defined by the pages cited beside it):
 *   bi_forward              Y  = RNE_T(X W + b)
 *   bi_backward_dx          dX = RNE_T(dY W^T)
 *   bi_backward_dw          dW = RNE_T(X^T dY)           (fixed-order two-pass)
 *   bi_linear_backward      dX and dW together (same bits as the two calls)
 *   bi_linear_backward_static   the same without a caller workspace
 *   bi_bias_grad            db = RNE_T(sum over rows of dY) (fixed order)
 *   bi_fp8_mm               Y  = RNE_bf16((A B^T) dA dB) (fp8 e4m3fn inputs)
 *   bi_fp8_quantize         q  = FP8(bf16 * scale_inv), amax (e4m3fn / e5m2)
 *   bi_fp8_transpose_quantize   the same into the transposed layout
 *   bi_fp8_linear_forward   Y  = RNE_bf16((q(x) q(w)^T) sx sw + b)
 *   bi_fp8_linear_backward  dX = RNE_bf16((q(g) q(w)) sg sw),
 *                           dW = RNE_bf16((q(g)^T q(x)) sg sx)
 *   bi_grouped_nt           Y[m] = in[m] Wt[e(m)]^T, zero rows for padding ids
 *   bi_grouped_nt_backward  dIn and f32 dWt of the grouped GEMM
 *
 * Common conventions
 *   Layout     Every matrix is dense row-major with no padding between rows.
 *              The linear weight W is stored [in, out] = [K, N] (sgemm-bi
 *              PyPI page, "Use": weight stored [in, out]).  Pointers of 16-bit
 *              types must be 2-byte aligned, f32 pointers 4-byte aligned;
 *              16-byte alignment of every row lets the kernels use vector loads
 *              (other alignments take a slower load path with the same bits).
 *   Memory     Every tensor pointer is a device pointer on the current HIP
 *              device, owned by the caller.  The library allocates nothing,
 *              keeps no per-call state, and never writes an input.  Outputs
 *              must not overlap inputs or each other.
 *   Execution  Work is enqueued on `stream` (0 = the null stream) and runs
 *              asynchronously; BI_OK means "validated and enqueued".
 *   Errors     All arguments are validated before anything is enqueued; on a
 *              validation error nothing is enqueued and no output is touched.
 *              A launch failure returns BI_ERR_HIP and is never retried on
 *              another tier (rublas tensor_grouped/mod.rs, strategy
 *              documentation: launch errors are propagated, never treated as a
 *              fallback).  bi_status_string() names every code.
 *   Sizes      m, k, n, e are int64; each tensor may hold at most 2^40
 *              elements (BI_ERR_TOO_LARGE beyond).  m == 0 is a valid empty
 *              batch: nothing is enqueued (except bi_backward_dw and the
 *              grouped backward, which then write zero gradients).
 *   dtype      BI_F32, BI_BF16 or BI_F16 for operands and outputs of the
 *              linear and grouped ops; accumulation is always f32 and the
 *              output is rounded once, to nearest-even (sgemm-bi PyPI page,
 *              "Determinism contracts").
 *   tc         Tensor-core (MFMA) tier request.  tc = 0 always selects the
 *              scalar FMA tier.  tc = 1 ("auto") selects the MFMA tier for
 *              bf16/f16 (and fp8) unless a non-M output dimension is below 64,
 *              in which case the scalar tier runs (sgemm-bi PyPI page,
 *              "Determinism contracts": shape-only fallback below 64); f32
 *              operands always use the scalar tier.  tc = 2 requires the MFMA
 *              tier: where tc = 1 would fall back, the call returns
 *              BI_ERR_UNSUPPORTED before enqueuing anything (rublas
 *              tensor_grouped: an explicit tensor-core strategy errors instead
 *              of falling back silently).  The tier depends only on (op,
 *              dtype, tc, the non-M output dims, the reduction length) --
 *              never on m -- so the forward is batch-invariant: a row's
 *              output bits do not depend on how many other rows are in the
 *              batch.  The two tiers do not give the same bits (different
 *              summation); results of either tier are bit-identical run to
 *              run.
 *              tc = 3 applies to the fp8 GEMMs only (bi_fp8_mm and the
 *              scaled fp8 linear): the tier is chosen as for tc = 1, and on
 *              the MFMA tier the fp8 matrix instruction multiplies the codes
 *              (about twice the throughput; it aligns the products of each
 *              group of 8 reduction indices to the group's largest one before
 *              adding them, so results are less exact than with tc = 1, whose
 *              products are all added at f32 precision).  Every other tc value
 *              returns BI_ERR_UNSUPPORTED.
 *
 * Determinism contracts
 *   Every entry point is bit-identical from run to run for the same inputs.
 *   Scalar tier: each output is one fmaf chain over the reduction index in
 *   ascending order from +0, then (+bias in f32), then one RNE; bf16/f16
 *   results equal RNE of the f32 tier run on the upcast inputs.
 *   MFMA tier: one MFMA instruction kind per dtype and a fixed ascending
 *   sequence of 16-deep reduction steps per output element in every tile
 *   shape (fp8 e4m3 codes are widened exactly to bf16 and take the bf16
 *   instruction; with tc = 3, 64-deep steps of the fp8 instruction), so all
 *   tile shapes give identical bits.
 *   No atomic accumulation anywhere (the quantisers fold max-abs with one
 *   integer atomic max per workgroup, which gives the same value in any order).
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BI_F32 = 0,  /* IEEE binary32 */
    BI_BF16 = 1, /* bfloat16 */
    BI_F16 = 2   /* IEEE binary16 */
} bi_dtype;

/* fp8 storage formats of the quantisers (one byte per element) */
typedef enum {
    BI_FP8_E4M3 = 3, /* OCP e4m3fn: bias 7, no infinities, largest finite 448 */
    BI_FP8_E5M2 = 4  /* OCP e5m2: bias 15, infinities, largest finite 57344 */
} bi_fp8_format;

typedef enum {
    BI_OK = 0,
    BI_ERR_NULL = -1,        /* a required pointer is NULL */
    BI_ERR_DTYPE = -2,       /* dtype code not supported by this entry point */
    BI_ERR_SHAPE = -3,       /* negative or zero-where-forbidden dimension */
    BI_ERR_TOO_LARGE = -4,   /* a tensor exceeds 2^40 elements */
    BI_ERR_WORKSPACE = -5,   /* workspace missing or too small */
    BI_ERR_HIP = -6,         /* a HIP launch failed (hipGetLastError) */
    BI_ERR_UNSUPPORTED = -7  /* tc/dtype combination has no tier */
} bi_status;

/* Forward of the training linear (sgemm-bi PyPI page, "Use" and
 * "Determinism contracts"; ViperLLM ffma.py, _FFMAAddmm.forward):
 *   y[m,n] = RNE_dtype( sum_k x[m,k] * w[k,n] + bias[n] )
 * x: [m,k], w: [k,n] ([in,out]), bias: [n] or NULL, y: [m,n]; all of `dtype`.
 * The bias is added in f32 to the f32 accumulator before the single rounding.
 * k == 0 gives y = RNE(bias) (or +0).  Batch-invariant in m. */
int bi_forward(void *y, const void *x, const void *w, const void *bias, int64_t m, int64_t k,
               int64_t n, int dtype, hipStream_t stream, int tc);

/* Input gradient (ffma.py, _FFMAAddmm.backward: gx = gy W^T):
 *   dx[m,k] = RNE_dtype( sum_n dy[m,n] * w[k,n] )
 * dy: [m,n], w: [k,n], dx: [m,k].  The tier depends on (k, n) only; the tile
 * may also follow m (identical bits, see bi_plan). */
int bi_backward_dx(void *dx, const void *dy, const void *w, int64_t m, int64_t k, int64_t n,
                   int dtype, hipStream_t stream, int tc);

/* Workspace bytes bi_backward_dw needs for these sizes (0 when the reduction
 * over m fits in one chunk).  Returns 0 for invalid arguments as well. */
size_t bi_backward_dw_workspace_bytes(int64_t m, int64_t k, int64_t n, int dtype, int tc);

/* Weight gradient (ffma.py, _FFMAAddmm.backward: gW = x^T gy, returned in the
 * weight dtype; sgemm-bi PyPI page, "Use": f32-accumulated dW):
 *   dw[k,n] = RNE_dtype( sum_m x[m,k] * dy[m,n] )
 * x: [m,k], dy: [m,n], dw: [k,n].  No atomics.  The m rows are cut into chunks
 * of C rows, C fixed by (dtype, tc, k, n) and never by m; pass 1 writes one f32
 * partial per chunk into the workspace, pass 2 sums the partials in ascending
 * chunk order and rounds once.  With a single chunk pass 1 rounds and stores
 * directly (same bits).  workspace: device memory of at least
 * bi_backward_dw_workspace_bytes(...) bytes (may be NULL when that is 0).
 * m == 0 writes dw = +0. */
int bi_backward_dw(void *dw, const void *x, const void *dy, int64_t m, int64_t k, int64_t n,
                   int dtype, void *workspace, size_t workspace_bytes, hipStream_t stream,
                   int tc);

/* Both gradients of a linear layer from one dY (ffma.py, _FFMAAddmm.backward:
 * gx = gy W^T and gW = x^T gy from the same gy).  Each output has exactly the
 * bits of bi_backward_dx / bi_backward_dw with the same arguments; where both
 * run the direct-load MFMA kernel on the 128x96 dX and 96x96 dW tiles (bf16 /
 * f16, aligned rows, dW in one chunk, at least 192 dX tiles) their tiles share
 * one launch, so a CU that finishes a dX tile starts a dW
 * tile while others are still busy; otherwise the two calls run in sequence.
 * dx or dw may be NULL to skip that gradient (not both, unless both outputs
 * are empty: BI_ERR_NULL); the other arguments, shapes, workspace and errors
 * are those of the two calls, all checked before anything is enqueued
 * (workspace: see bi_backward_dw_workspace_bytes). */
int bi_linear_backward(void *dx, void *dw, const void *dy, const void *x, const void *w,
                       int64_t m, int64_t k, int64_t n, int dtype, void *workspace,
                       size_t workspace_bytes, hipStream_t stream, int tc);

/* Bytes of the static scratch array behind bi_linear_backward_static: one
 * copy per GPU the library runs on, held until the process ends. */
#define BI_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, arguments (without the workspace) and bits as
 * bi_linear_backward, with dW's f32 chunk partials in a library-owned static
 * device array of BI_STATIC_SCRATCH_BYTES on the current GPU instead of a
 * caller workspace.  Nothing here allocates (no hipMalloc, no allocating
 * library call).  Errors: BI_ERR_WORKSPACE when the partials would need more
 * than BI_STATIC_SCRATCH_BYTES (bi_backward_dw_workspace_bytes(m, k, n,
 * dtype, tc) above it), checked before anything is enqueued; otherwise those
 * of bi_linear_backward, plus BI_ERR_HIP if the array's device address cannot
 * be looked up (done once per GPU, on the first call there).  All calls on
 * one GPU share its array and every call overwrites the partials it reads:
 * calls that overlap on one GPU (on different streams, or from several host
 * threads without ordering) race. */
int bi_linear_backward_static(void *dx, void *dw, const void *dy, const void *x, const void *w,
                              int64_t m, int64_t k, int64_t n, int dtype, hipStream_t stream,
                              int tc);

/* Workspace bytes bi_bias_grad needs (0 when m <= 256).  Returns 0 for invalid
 * arguments as well. */
size_t bi_bias_grad_workspace_bytes(int64_t m, int64_t n, int dtype);

/* Bias gradient (ffma.py, _FFMAAddmm.backward: gb = gy.sum(0) accumulated in
 * f32 and cast back to the bias dtype; sgemm-bi PyPI page, "Determinism
 * contracts": the bias gradient is a plain f32 column sum, deterministic for a
 * fixed shape and outside the batch-invariance contract):
 *   db[n] = RNE_dtype( sum_m dy[m,n] )
 * dy: [m,n], db: [n], both of `dtype`.  The order is fixed by m alone: rows in
 * chunks of 256; inside a chunk 64 interleaved running sums (rows t, t+64,
 * ...) combined in a fixed tree; chunk partials (f32, in the workspace) added in
 * ascending chunk order; one rounding.  workspace: 4-byte aligned device memory
 * of at least bi_bias_grad_workspace_bytes(m, n, dtype) bytes (may be NULL when
 * that is 0), else BI_ERR_WORKSPACE.  m == 0 writes db = +0. */
int bi_bias_grad(void *db, const void *dy, int64_t m, int64_t n, int dtype, void *workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* Per-tensor-scaled fp8 GEMM (AstrAI fp8_mm.cu: fp8_mm takes e4m3fn a[M,K]
 * and b[N,K] and returns bf16 [M,N]; fp8_gemm_into applies the per-tensor f32
 * scales inside the GEMM, D = A_SCALE * B_SCALE * A * B):
 *   y[m,n] = RNE_bf16( ((sum_k a[m,k] * bt[n,k]) * a_dequant) * b_dequant )
 * a: [m,k] OCP e4m3fn codes, bt: [n,k] e4m3fn codes (both k-contiguous),
 * a_dequant / b_dequant: device pointers to one f32 each, y: [m,n] bf16.
 * Products are exact; the sum is f32 (f32 compute type, as fp8_gemm_into asks
 * of cuBLASLt): on the MFMA tier the codes are widened exactly to bf16 and
 * every product is added by the bf16 matrix instruction at f32 precision
 * (tc = 1, 2); tc = 3 uses the fp8 matrix instruction instead (faster, less
 * exact: see tc above).  The two scale multiplies are f32, left to right; one
 * RNE to bf16.  Batch-invariant in m. */
int bi_fp8_mm(void *y, const void *a, const void *bt, const float *a_dequant,
              const float *b_dequant, int64_t m, int64_t k, int64_t n, hipStream_t stream,
              int tc);

/* fp8 quantisation (AstrAI fp8_mm.cu: quantize_kernel and cast_fp8):
 *   dst[i] = FP8( f32(src[i]) * (*scale_inv) ),  0 <= i < n
 * src: n bf16 elements, dst: n bytes of `fmt` (BI_FP8_E4M3 or BI_FP8_E5M2).
 * The product is an f32 multiplication; the conversion rounds to nearest even
 * and saturates values beyond the largest finite one to it (NaN stays NaN).
 * amax (nullable, device f32): *amax = max(*amax, max_i |src[i]|) over the
 * unscaled source, NaN ignored -- the caller sets *amax (e.g. to 0) first, as
 * the page's kernel expects a zeroed amax.  The max is exact, so the result
 * does not depend on the order in which workgroups fold it in.
 * n == 0 does nothing.  Errors: BI_ERR_DTYPE (fmt), BI_ERR_SHAPE (n < 0),
 * BI_ERR_NULL (a pointer other than amax is NULL while n > 0). */
int bi_fp8_quantize(void *dst, const void *src, const float *scale_inv, float *amax, int64_t n,
                    int fmt, hipStream_t stream);

/* Transposing fp8 quantisation (fp8_mm.cu: transpose_quantize_kernel): src
 * [rows, cols] bf16 row-major, dst [cols, rows] codes, dst[c*rows + r] =
 * FP8(f32(src[r*cols + c]) * (*scale_inv)); amax as in bi_fp8_quantize.
 * rows must not exceed 65535 * 64 (BI_ERR_TOO_LARGE).  rows or cols == 0 does
 * nothing. */
int bi_fp8_transpose_quantize(void *dst, const void *src, const float *scale_inv, float *amax,
                              int64_t rows, int64_t cols, int fmt, hipStream_t stream);

/* Workspace bytes for bi_fp8_linear_forward and bi_fp8_linear_backward on
 * (m, k, n): the larger of the two needs (quantised copies of the operands),
 * so one buffer serves both.  0 for invalid arguments.  A 256-byte-aligned
 * workspace keeps the fp8 GEMMs on their fast path. */
size_t bi_fp8_linear_workspace_bytes(int64_t m, int64_t k, int64_t n);

/* Scaled fp8 linear forward (fp8_mm.cu: fp8_linear_forward_scaled):
 *   y[m,n] = RNE_bf16( ((sum_k qx[m,k] * qw[n,k]) * sx) * sw + bias[n] )
 *   qx = FP8_e4m3(x * sx_inv), qw = FP8_e4m3(w * sw_inv)
 * x: [m,k] bf16, w: [n,k] bf16 (weight stored [out,in] as on the page),
 * bias: [n] bf16 or NULL, y: [m,n] bf16; sx, sw, sx_inv, sw_inv: device f32
 * scalars (sx_inv = 1/sx is the caller's); amax_x / amax_w (nullable) are set
 * to max |x| and max |w|.  The bias joins in f32 before the single rounding
 * (the page adds it to the rounded bf16 output, which rounds twice).
 * workspace: at least bi_fp8_linear_workspace_bytes(m, k, n) bytes. */
int bi_fp8_linear_forward(void *y, const void *x, const void *w, const void *bias,
                          const float *sx, const float *sw, const float *sx_inv,
                          const float *sw_inv, float *amax_x, float *amax_w, int64_t m,
                          int64_t k, int64_t n, void *workspace, size_t workspace_bytes,
                          hipStream_t stream, int tc);

/* Scaled fp8 linear backward (fp8_mm.cu: fp8_linear_backward_scaled):
 *   dx[m,k] = RNE_bf16( ((sum_n qg[m,n] * qw[n,k]) * sg) * sw )
 *   dw[n,k] = RNE_bf16( ((sum_m qg[m,n] * qx[m,k]) * sg) * sx )
 *   qg = FP8_e4m3(g * sg_inv), qw, qx as in the forward
 * g: [m,n], x: [m,k], w: [n,k] bf16; dx (nullable: skipped) [m,k] and dw
 * (nullable: skipped) [n,k] bf16.  amax_g (nullable) is set to max |g|; the
 * transposed copies of w and x record no max-abs (the page keeps theirs in a
 * scratch value apart from amax_g that nothing reads).  g is read once when dw
 * is wanted (its row-major and transposed codes come from the same read).  The
 * bias gradient is not computed here (bi_bias_grad on g gives it).  workspace:
 * at least bi_fp8_linear_workspace_bytes(m, k, n) bytes. */
int bi_fp8_linear_backward(void *dx, void *dw, const void *g, const void *x, const void *w,
                           const float *sg, const float *sw, const float *sx,
                           const float *sg_inv, const float *sw_inv, const float *sx_inv,
                           float *amax_g, int64_t m, int64_t k, int64_t n, void *workspace,
                           size_t workspace_bytes, hipStream_t stream, int tc);

/* Row-routed grouped GEMM (rublas tensor_grouped/mod.rs, grouped_matmul_nt:
 * [M,K] @ [E,N,K]^T selecting one expert per row; ids outside [0,E) are padding
 * and produce zero rows; f32 accumulation, one output rounding):
 *   y[m,n] = row_experts[m] < e ? RNE_dtype( sum_k input[m,k] * weights[row_experts[m],n,k] )
 *                               : +0
 * input: [m,k], weights: [e,n,k], y: [m,n], all of `dtype`;
 * row_experts: [m] uint32; offsets: [e+1] uint32 or NULL.
 * offsets (required when tc selects the MFMA tier): offsets[0] = 0 and the rows
 * of expert j are [offsets[j], offsets[j+1]); rows [offsets[e], m) are padding.
 * That is, rows are sorted by expert with padding last, and offsets describes
 * the same grouping as row_experts -- a caller invariant that is not checked
 * on the device (rublas: GPU values are not copied to the CPU to validate
 * grouping).  The scalar tier reads row_experts only, in any row order.
 * k, n, e must be > 0 (BI_ERR_SHAPE). */
int bi_grouped_nt(void *y, const void *input, const void *weights, const uint32_t *row_experts,
                  const uint32_t *offsets, int64_t m, int64_t k, int64_t n, int64_t e, int dtype,
                  hipStream_t stream, int tc);

/* Backward of the grouped GEMM (rublas tensor_grouped/mod.rs,
 * grouped_matmul_nt_backward_segmented and GroupedBackward: dinput in the
 * input dtype, dweights always f32):
 *   dinput[m,k]     = row_experts[m] < e ? RNE_dtype( sum_n grad_out[m,n] * weights[e(m),n,k] ) : +0
 *   dweights[j,n,k] = sum over rows m of expert j, ascending, of grad_out[m,n] * input[m,k]  (f32)
 * dinput: [m,k] of dtype, dweights: [e,n,k] f32, grad_out: [m,n] of dtype.
 * offsets: [e+1] uint32, required (same invariants as bi_grouped_nt); experts
 * with no rows get dweights = +0.  k, n, e must be > 0. */
int bi_grouped_nt_backward(void *dinput, float *dweights, const void *input, const void *weights,
                           const void *grad_out, const uint32_t *row_experts,
                           const uint32_t *offsets, int64_t m, int64_t k, int64_t n, int64_t e,
                           int dtype, hipStream_t stream, int tc);

/* Static, NUL-terminated name of a status code (never NULL). */
const char *bi_status_string(int status);

/* Tier and tile the dispatcher picks, without launching anything:
 * op: 0 forward, 1 dX, 2 dW, 3 fp8, 4 grouped forward, 5 grouped dinput,
 * 6 grouped dweights.  Returns 0 for the scalar tier, a positive tile id for
 * the MFMA tier, or a negative bi_status.  Depends on (op, dtype, tc, k, n)
 * only: the tier and the dW chunk length C never depend on m.  The tile
 * reported is the default of (k, n); forward, dX and fp8 calls run the tile a
 * launch-time model finds fastest for (m, k, n) among a few candidates, small
 * batches narrow 64x32 or 32x32 tiles (every tile issues the same MFMA
 * sequence per element, so the bits are the same).  For dW,
 * *chunk_rows (if not NULL) receives the chunk length C. */
int bi_plan(int op, int dtype, int tc, int64_t k, int64_t n, int64_t *chunk_rows);

/* The tile a call of `op` (as in bi_plan) with batch m launches when its rows
 * are 16-byte aligned, their lengths multiples of 8 elements and each operand
 * below 2^30 bytes (otherwise the register-staged kernel runs 256x256, 128x128
 * or 64x64): the batch-dependent choice of forward, dX, fp8, grouped forward
 * and grouped dinput calls (e = the grouped call's number of experts; ignored
 * by the other ops), the bi_plan tile for dW, the grouped dweights and m == 0.
 * Returns 0 for the scalar tier or a negative bi_status (as bi_plan;
 * BI_ERR_SHAPE for m < 0 or e < 0).  The m rows of a batch is the rows of A: x
 * for the forward, dy for dX, a for fp8, input / dY for the grouped forward / dinput.
 * A grouped forward on tile 112 (256x256) whose grid holds more than one round
 * of 256 workgroups may run the work left after the whole rounds as 256x128
 * column halves of the same tiles (decided on the device from the offsets;
 * same bits).  Launches nothing. */
int bi_plan_batch(int op, int dtype, int tc, int64_t m, int64_t k, int64_t n, int64_t e);

#ifdef __cplusplus
}
#endif

#endif /* BI_H */
