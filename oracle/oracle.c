/*
 * oracle.c -- plain, slow CPU oracle for the deterministic training-linear GEMM,
 * the per-tensor-scaled fp8 GEMM and the row-routed grouped GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or constant with the
 * HIP path.
 *
 * What it computes (every function below follows these four rules):
 *   1. Every input element is decoded to its exact value as a C double
 *      (f32, bf16, f16 and OCP fp8 e4m3fn are all exactly representable).
 *   2. Products of two decoded elements are exact in double: significand widths
 *      are 24+24, 8+8, 11+11 or 4+4 bits, all <= 53.
 *   3. The reduction is accumulated in double, one running sum per output
 *      element, in ascending order of the reduced index, starting from +0.
 *   4. The result is rounded ONCE, directly from double to the output type,
 *      with round-to-nearest-even and IEEE subnormal / overflow rules.
 *      (Never via f32 for bf16/f16 targets: that would round twice.)
 *
 * Definitions, with citations of the pages they restate:
 *   forward  Y[m,n]  = RNE_T( sum_k X[m,k] W[k,n] + b[n] )
 *            sgemm-bi PyPI page, "Use" (weight stored [in,out]) and
 *            "Determinism contracts" (f32 accumulate, single RNE downcast);
 *            ViperLLM ffma.py, _FFMAAddmm.forward (bias added before the one
 *            downcast).
 *   dX       dX[m,k] = RNE_T( sum_n dY[m,n] W[k,n] )
 *   dW       dW[k,n] = RNE_T( sum_m X[m,k] dY[m,n] )
 *            ffma.py, _FFMAAddmm.backward (gx = gy W^T, gW = x^T gy, both cast
 *            back to the operand dtype).
 *   fp8      Y[m,n]  = RNE_bf16( (sum_k A[m,k] B[n,k]) * dA * dB )
 *            AstrAI fp8_mm.cu, fp8_gemm_into (per-tensor f32 scales applied
 *            inside the GEMM, D = A_SCALE * B_SCALE * A * B) and fp8_mm
 *            (e4m3fn operands a[M,K], b[N,K], bf16 output).
 *   grouped  Y[m,n]  = e(m) < E ? RNE_T( sum_k in[m,k] Wt[e(m),n,k] ) : +0
 *            dIn[m,k]= e(m) < E ? RNE_T( sum_n dY[m,n] Wt[e(m),n,k] ) : +0
 *            dWt[e,n,k] = RNE_f32( sum_{m : e(m)=e} dY[m,n] in[m,k] )
 *            rublas tensor_grouped/mod.rs, grouped_matmul_nt (ids outside
 *            [0,E) are padding and give zero rows; one output rounding),
 *            GroupedBackward (dweights always f32) and the backward of
 *            Y[m,n] = sum_k input[m,k] weights[expert(m),n,k].
 *   The grouped oracle routes rows by row_experts alone; it never reads an
 *   offsets array.
 *   quantize  q[i] = FP8( f32( f32(src[i]) * scale_inv ) ), amax = max |src[i]|
 *            AstrAI fp8_mm.cu, quantize_kernel and cast_fp8: the bf16 value
 *            times the inverse scale in f32, then converted to e4m3fn or e5m2
 *            with round-to-nearest-even, values beyond the largest finite one
 *            saturating to it (NaN stays NaN); amax is the max-abs of the
 *            unscaled source (NaN ignored).  transpose_quantize_kernel: the
 *            same per element, stored transposed ([rows,cols] -> [cols,rows]).
 *   bias gradient  db[n] = RNE_T( sum_m dY[m,n] )
 *            ffma.py, _FFMAAddmm.backward (gb = gy.sum(0) in f32, cast back
 *            to the bias dtype).
 *   fp8 linear forward (fp8_linear_forward_scaled)
 *            Y[m,n] = RNE_bf16( (sum_k qx[m,k] qw[n,k]) * sx * sw + b[n] )
 *            with qx = quantize(x, 1/sx), qw = quantize(w, 1/sw), w stored
 *            [N,K]; the bias joins before the single rounding.
 *   fp8 linear backward (fp8_linear_backward_scaled)
 *            dX[m,k] = RNE_bf16( (sum_n qg[m,n] qw[n,k]) * sg * sw )
 *            dW[n,k] = RNE_bf16( (sum_m qg[m,n] qx[m,k]) * sg * sx )
 *            with qg = quantize(g, 1/sg); quantising a transposed copy gives
 *            the transposed codes, so the sums are written on qg, qw, qx.
 *
 * Every function also reports, per output element, the exact-in-double
 * pre-rounding value S and the absolute scale A = sum |a*b| (+ |bias|), which
 * the parity tests use for their tolerance.  The fp8 functions also report
 * G = sum over groups of 8 consecutive reduction indices (counted from the
 * first) of the largest |a*b| in the group, times the scales: the fp8 matrix
 * instruction adds each group of 8 products aligned to the group's largest
 * one, which bounds its difference from the exact sum by 2^-10 G.
 *
 * Threads: output rows are split over POSIX threads.  Each output element is
 * computed by exactly one thread with the order above, so the thread count does
 * not change any result.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F16 2
#define ORC_E4M3 3
#define ORC_E5M2 4

/* ------------------------------------------------------------------------- */
/* Decoding: bit pattern -> exact double                                      */
/* ------------------------------------------------------------------------- */

/* IEEE binary32: decoded by reinterpreting the bits; widening float->double
 * is exact. */
double orc_decode_f32_bits(uint32_t bits) {
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* bfloat16 is the upper half of a binary32: sign, 8 exponent bits (bias 127),
 * 7 fraction bits. */
double orc_decode_bf16(uint16_t bits) {
    return orc_decode_f32_bits((uint32_t)bits << 16);
}

/* IEEE binary16: sign, 5 exponent bits (bias 15), 10 fraction bits;
 * subnormals are frac * 2^-24; exponent 31 is inf/NaN. */
double orc_decode_f16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int ex = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)frac, -24);
    else if (ex == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), ex - 25);
    return sign ? -v : v;
}

/* OCP fp8 e4m3fn ("float8_e4m3fn" in the fp8 GEMM page): sign, 4 exponent bits
 * (bias 7), 3 fraction bits; subnormals are frac * 2^-9; no infinities; the
 * single pattern S.1111.111 is NaN, so the largest finite value is 448. */
double orc_decode_e4m3(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int ex = (bits >> 3) & 0xf;
    int frac = bits & 0x7;
    double v;
    if (ex == 15 && frac == 7)
        v = NAN;
    else if (ex == 0)
        v = ldexp((double)frac, -9);
    else
        v = ldexp((double)(8 + frac), ex - 10);
    return sign ? -v : v;
}

double orc_decode(int dt, const void *base, int64_t i) {
    switch (dt) {
    case ORC_F32: return orc_decode_f32_bits(((const uint32_t *)base)[i]);
    case ORC_BF16: return orc_decode_bf16(((const uint16_t *)base)[i]);
    case ORC_F16: return orc_decode_f16(((const uint16_t *)base)[i]);
    case ORC_E4M3: return orc_decode_e4m3(((const uint8_t *)base)[i]);
    }
    return NAN;
}

/* ------------------------------------------------------------------------- */
/* Rounding: exact double -> nearest representable value, ties to even         */
/* ------------------------------------------------------------------------- */

/* Round |x| to a binary format with p significand bits (incl. the hidden bit),
 * minimum normal exponent emin and largest finite value max_finite.  The value
 * is returned as a double (exactly representable in that format), or +inf on
 * overflow.  rint() rounds to nearest, ties to even, in the default mode;
 * dividing and multiplying by a power of two is exact here. */
static double round_mag(double ax, int p, int emin, double max_finite) {
    if (ax == 0.0 || isnan(ax)) return ax;
    if (isinf(ax)) return INFINITY;
    int e2;
    frexp(ax, &e2);          /* ax = f * 2^e2 with f in [0.5, 1) */
    int lead = e2 - 1;       /* exponent of the leading bit */
    if (lead < emin) lead = emin; /* subnormal range: fixed quantum */
    double q = ldexp(1.0, lead - (p - 1));
    double r = rint(ax / q) * q;
    /* Rounding with an unbounded exponent gives either a finite value of the
     * format or the next power of two above max_finite (when ax is at least
     * halfway past max_finite); the latter is an overflow. */
    if (r > max_finite) return INFINITY;
    return r;
}

/* double -> bfloat16 bits, RNE. */
uint16_t orc_rne_bf16(double x) {
    if (isnan(x)) return 0x7fc0;
    int neg = signbit(x) ? 1 : 0;
    double r = round_mag(fabs(x), 8, -126, 0x1.fep127);
    uint16_t mag;
    if (isinf(r)) {
        mag = 0x7f80;
    } else {
        float f = (float)r; /* exact: r has <= 8 significant bits */
        uint32_t b;
        memcpy(&b, &f, sizeof b);
        mag = (uint16_t)(b >> 16);
    }
    return (uint16_t)(mag | (neg << 15));
}

/* double -> binary16 bits, RNE. */
uint16_t orc_rne_f16(double x) {
    if (isnan(x)) return 0x7e00;
    int neg = signbit(x) ? 1 : 0;
    double r = round_mag(fabs(x), 11, -14, 65504.0);
    uint16_t mag;
    if (isinf(r)) {
        mag = 0x7c00;
    } else if (r == 0.0) {
        mag = 0;
    } else {
        int e2;
        frexp(r, &e2);
        int lead = e2 - 1;
        if (lead < -14) {
            mag = (uint16_t)ldexp(r, 24); /* subnormal: frac = r / 2^-24 */
        } else {
            int frac = (int)(ldexp(r, 10 - lead) - 1024.0);
            mag = (uint16_t)(((lead + 15) << 10) | frac);
        }
    }
    return (uint16_t)(mag | (neg << 15));
}

/* double -> binary32 bits, RNE.  C's double->float conversion rounds in the
 * current rounding mode, which is round-to-nearest-even by default, with IEEE
 * subnormals and overflow to inf. */
uint32_t orc_rne_f32(double x) {
    float f = (float)x;
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    return b;
}

/* double -> e4m3fn bits, RNE, saturating to +-448 (used only to describe the
 * format in tests; inputs are quantized by the input generator). */
uint8_t orc_rne_e4m3_sat(double x) {
    if (isnan(x)) return 0x7f;
    int neg = signbit(x) ? 1 : 0;
    double r = round_mag(fabs(x), 4, -6, 448.0);
    if (isinf(r)) r = 448.0;
    uint8_t mag;
    if (r == 0.0) {
        mag = 0;
    } else {
        int e2;
        frexp(r, &e2);
        int lead = e2 - 1;
        if (lead < -6)
            mag = (uint8_t)ldexp(r, 9);
        else
            mag = (uint8_t)(((lead + 7) << 3) | (int)(ldexp(r, 3 - lead) - 8.0));
    }
    return (uint8_t)(mag | (neg << 7));
}

static void store_rounded(int dt, void *base, int64_t i, double v) {
    switch (dt) {
    case ORC_F32: ((uint32_t *)base)[i] = orc_rne_f32(v); break;
    case ORC_BF16: ((uint16_t *)base)[i] = orc_rne_bf16(v); break;
    case ORC_F16: ((uint16_t *)base)[i] = orc_rne_f16(v); break;
    }
}

/* Decode a whole buffer of cnt elements to doubles (caller frees). */
static double *decode_all(int dt, const void *src, int64_t cnt) {
    double *d = (double *)malloc((size_t)(cnt > 0 ? cnt : 1) * sizeof(double));
    if (!d) return NULL;
    for (int64_t i = 0; i < cnt; ++i) d[i] = orc_decode(dt, src, i);
    return d;
}

/* ------------------------------------------------------------------------- */
/* Row-parallel driver                                                        */
/* ------------------------------------------------------------------------- */

typedef void (*row_fn)(void *ctx, int64_t sel_index);

struct worker {
    row_fn fn;
    void *ctx;
    int64_t begin, end;
};

static void *worker_main(void *p) {
    struct worker *w = (struct worker *)p;
    for (int64_t i = w->begin; i < w->end; ++i) w->fn(w->ctx, i);
    return NULL;
}

static void run_rows(row_fn fn, void *ctx, int64_t nsel, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nsel < nthreads) nthreads = (int)(nsel > 0 ? nsel : 1);
    pthread_t th[256];
    struct worker ws[256];
    int64_t per = (nsel + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        ws[t].fn = fn;
        ws[t].ctx = ctx;
        ws[t].begin = t * per;
        ws[t].end = (t + 1) * per < nsel ? (t + 1) * per : nsel;
        if (ws[t].begin >= ws[t].end) continue;
        if (t == 0) continue; /* run on the calling thread below */
        if (pthread_create(&th[t], NULL, worker_main, &ws[t]) != 0) {
            worker_main(&ws[t]); /* no thread available: run inline */
            ws[t].begin = ws[t].end;
        }
    }
    if (ws[0].begin < ws[0].end) worker_main(&ws[0]);
    for (int t = 1; t < nthreads; ++t)
        if (ws[t].begin < ws[t].end) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------- */
/* Generic "one output row" kernel: out[j] = sum_r a_row[r] * B(r, j)          */
/* ------------------------------------------------------------------------- */

/* Shared by all ops: given one decoded operand row a_row[0..red) and a decoded
 * operand matrix read as B(r, j) = b[r * b_rs + j * b_cs], accumulate
 * s[j] = sum over r ascending of a_row[r] * B(r, j) and abs[j] = sum |...|. */
static void row_dot(const double *a_row, int64_t red, const double *b, int64_t b_rs,
                    int64_t b_cs, int64_t ncols, double *s, double *ab) {
    for (int64_t j = 0; j < ncols; ++j) s[j] = 0.0, ab[j] = 0.0;
    for (int64_t r = 0; r < red; ++r) {
        double av = a_row[r];
        const double *br = b + r * b_rs;
        for (int64_t j = 0; j < ncols; ++j) {
            double p = av * br[j * b_cs]; /* exact */
            s[j] += p;
            ab[j] += fabs(p);
        }
    }
}

/* As row_dot, plus g[j] = sum over groups of 8 consecutive r (from r = 0) of
 * max |a_row[r] * B(r, j)| within the group. */
static void row_dot_g8(const double *a_row, int64_t red, const double *b, int64_t b_rs,
                       int64_t b_cs, int64_t ncols, double *s, double *ab, double *g) {
    double *gm = (double *)calloc((size_t)(ncols > 0 ? ncols : 1), sizeof(double));
    for (int64_t j = 0; j < ncols; ++j) s[j] = 0.0, ab[j] = 0.0, g[j] = 0.0;
    for (int64_t r = 0; r < red; ++r) {
        double av = a_row[r];
        const double *br = b + r * b_rs;
        for (int64_t j = 0; j < ncols; ++j) {
            double p = av * br[j * b_cs]; /* exact */
            s[j] += p;
            ab[j] += fabs(p);
            if (fabs(p) > gm[j]) gm[j] = fabs(p);
        }
        if (r % 8 == 7 || r == red - 1)
            for (int64_t j = 0; j < ncols; ++j) g[j] += gm[j], gm[j] = 0.0;
    }
    free(gm);
}

/* ------------------------------------------------------------------------- */
/* Linear forward / dX / dW                                                   */
/* ------------------------------------------------------------------------- */

struct lin_ctx {
    int dt;
    int64_t m, k, n;
    const double *X, *W, *B, *DY; /* decoded */
    const int64_t *rows;
    void *out;
    double *s_out, *a_out;
    int op; /* 0 fwd, 1 dx, 2 dw */
};

static void lin_row(void *p, int64_t i) {
    struct lin_ctx *c = (struct lin_ctx *)p;
    int64_t r = c->rows ? c->rows[i] : i;
    int64_t ncols = c->op == 1 ? c->k : c->n;
    double *s = (double *)malloc((size_t)ncols * sizeof(double));
    double *ab = (double *)malloc((size_t)ncols * sizeof(double));
    double *arow = NULL;
    if (c->op == 0) {
        /* Y[r, n] = sum_k X[r,k] W[k,n] + b[n] : W(k, n) = W[k*N + n] */
        row_dot(c->X + r * c->k, c->k, c->W, c->n, 1, c->n, s, ab);
        if (c->B)
            for (int64_t j = 0; j < c->n; ++j) s[j] += c->B[j], ab[j] += fabs(c->B[j]);
    } else if (c->op == 1) {
        /* dX[r, k] = sum_n dY[r,n] W[k,n] : B(n, k) = W[k*N + n] */
        row_dot(c->DY + r * c->n, c->n, c->W, 1, c->n, c->k, s, ab);
    } else {
        /* dW[r, n] = sum_m X[m,r] dY[m,n] : a_row[m] = X[m*K + r] */
        arow = (double *)malloc((size_t)(c->m > 0 ? c->m : 1) * sizeof(double));
        for (int64_t mm = 0; mm < c->m; ++mm) arow[mm] = c->X[mm * c->k + r];
        row_dot(arow, c->m, c->DY, c->n, 1, c->n, s, ab);
    }
    for (int64_t j = 0; j < ncols; ++j) {
        if (c->out) store_rounded(c->dt, c->out, i * ncols + j, s[j]);
        if (c->s_out) c->s_out[i * ncols + j] = s[j];
        if (c->a_out) c->a_out[i * ncols + j] = ab[j];
    }
    free(arow);
    free(s);
    free(ab);
}

static int lin_common(int op, int dt, const void *x, const void *w, const void *bias,
                      const void *dy, int64_t m, int64_t k, int64_t n, const int64_t *rows,
                      int64_t nrows, void *out, double *s_out, double *a_out, int nthreads) {
    if (dt < ORC_F32 || dt > ORC_F16) return -2;
    struct lin_ctx c;
    memset(&c, 0, sizeof c);
    c.dt = dt, c.m = m, c.k = k, c.n = n, c.rows = rows, c.out = out;
    c.s_out = s_out, c.a_out = a_out, c.op = op;
    double *X = NULL, *W = NULL, *B = NULL, *DY = NULL;
    if (op == 0 || op == 2) X = decode_all(dt, x, m * k);
    if (op == 0 || op == 1) W = decode_all(dt, w, k * n);
    if (op == 0 && bias) B = decode_all(dt, bias, n);
    if (op == 1 || op == 2) DY = decode_all(dt, dy, m * n);
    c.X = X, c.W = W, c.B = B, c.DY = DY;
    run_rows(lin_row, &c, nrows, nthreads);
    free(X), free(W), free(B), free(DY);
    return 0;
}

/* Y rows: rows[i] (or i when rows is NULL) for i < nrows; out is [nrows, n]. */
int orc_linear_forward(int dt, const void *x, const void *w, const void *bias, int64_t m,
                       int64_t k, int64_t n, const int64_t *rows, int64_t nrows, void *out,
                       double *s_out, double *a_out, int nthreads) {
    return lin_common(0, dt, x, w, bias, NULL, m, k, n, rows, nrows, out, s_out, a_out,
                      nthreads);
}

/* dX rows (indices into M); out is [nrows, k]. */
int orc_linear_dx(int dt, const void *dy, const void *w, int64_t m, int64_t k, int64_t n,
                  const int64_t *rows, int64_t nrows, void *out, double *s_out, double *a_out,
                  int nthreads) {
    return lin_common(1, dt, NULL, w, NULL, dy, m, k, n, rows, nrows, out, s_out, a_out,
                      nthreads);
}

/* dW rows (indices into K); out is [nrows, n]. */
int orc_linear_dw(int dt, const void *x, const void *dy, int64_t m, int64_t k, int64_t n,
                  const int64_t *rows, int64_t nrows, void *out, double *s_out, double *a_out,
                  int nthreads) {
    return lin_common(2, dt, x, NULL, NULL, dy, m, k, n, rows, nrows, out, s_out, a_out,
                      nthreads);
}

/* ------------------------------------------------------------------------- */
/* fp8 e4m3 GEMM with per-tensor dequantisation scales, bf16 output           */
/* ------------------------------------------------------------------------- */

struct fp8_ctx {
    int64_t k, n;
    const double *A, *BT;
    double da, db;
    const int64_t *rows;
    uint16_t *out;
    double *s_out, *a_out, *g_out;
};

static void fp8_row(void *p, int64_t i) {
    struct fp8_ctx *c = (struct fp8_ctx *)p;
    int64_t r = c->rows ? c->rows[i] : i;
    double *s = (double *)malloc((size_t)c->n * sizeof(double));
    double *ab = (double *)malloc((size_t)c->n * sizeof(double));
    double *g = (double *)malloc((size_t)c->n * sizeof(double));
    /* sum_k A[r,k] B[n,k] : B(k, n) = BT[n*K + k] */
    row_dot_g8(c->A + r * c->k, c->k, c->BT, 1, c->k, c->n, s, ab, g);
    for (int64_t j = 0; j < c->n; ++j) {
        double v = s[j] * c->da * c->db;
        double a = ab[j] * fabs(c->da) * fabs(c->db);
        if (c->out) c->out[i * c->n + j] = orc_rne_bf16(v);
        if (c->s_out) c->s_out[i * c->n + j] = v;
        if (c->a_out) c->a_out[i * c->n + j] = a;
        if (c->g_out) c->g_out[i * c->n + j] = g[j] * fabs(c->da) * fabs(c->db);
    }
    free(s);
    free(ab);
    free(g);
}

/* a8: [m,k] e4m3fn codes, bt8: [n,k] e4m3fn codes, da/db: the f32 dequant
 * scales (as passed to the GPU, widened exactly); out: bf16 bits [nrows, n]. */
int orc_fp8_mm(const uint8_t *a8, const uint8_t *bt8, float da, float db, int64_t m,
               int64_t k, int64_t n, const int64_t *rows, int64_t nrows, uint16_t *out,
               double *s_out, double *a_out, double *g_out, int nthreads) {
    struct fp8_ctx c;
    memset(&c, 0, sizeof c);
    double *A = decode_all(ORC_E4M3, a8, m * k);
    double *BT = decode_all(ORC_E4M3, bt8, n * k);
    c.k = k, c.n = n, c.A = A, c.BT = BT, c.da = (double)da, c.db = (double)db;
    c.rows = rows, c.out = out, c.s_out = s_out, c.a_out = a_out, c.g_out = g_out;
    run_rows(fp8_row, &c, nrows, nthreads);
    free(A), free(BT);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Row-routed grouped GEMM  [M,K] . [E,N,K]^T                                  */
/* ------------------------------------------------------------------------- */

struct grp_ctx {
    int dt, op; /* 0 fwd, 1 dinput, 2 dweights */
    int64_t m, k, n, e;
    const double *IN, *WT, *DY;
    const uint32_t *row_experts;
    const int64_t *rows;
    void *out;
    double *s_out, *a_out;
};

static void grp_row(void *p, int64_t i) {
    struct grp_ctx *c = (struct grp_ctx *)p;
    int64_t r = c->rows ? c->rows[i] : i;
    int64_t ncols = c->op == 1 ? c->k : (c->op == 0 ? c->n : c->k);
    double *s = (double *)malloc((size_t)ncols * sizeof(double));
    double *ab = (double *)malloc((size_t)ncols * sizeof(double));
    int out_dt = c->op == 2 ? ORC_F32 : c->dt;
    if (c->op == 0 || c->op == 1) {
        uint32_t ex = c->row_experts[r];
        if ((int64_t)ex >= c->e) {
            /* padding row: exact +0 */
            for (int64_t j = 0; j < ncols; ++j) s[j] = 0.0, ab[j] = 0.0;
        } else if (c->op == 0) {
            /* Y[r,n] = sum_k in[r,k] Wt[e,n,k] : B(k, n) = Wt[e*N*K + n*K + k] */
            row_dot(c->IN + r * c->k, c->k, c->WT + (int64_t)ex * c->n * c->k, 1, c->k, c->n,
                    s, ab);
        } else {
            /* dIn[r,k] = sum_n dY[r,n] Wt[e,n,k] : B(n, k) = Wt[e*N*K + n*K + k] */
            row_dot(c->DY + r * c->n, c->n, c->WT + (int64_t)ex * c->n * c->k, c->k, 1, c->k,
                    s, ab);
        }
    } else {
        /* selected dweights row r = e*N + n:
         * dWt[e,n,k] = sum over m ascending with row_experts[m] == e of
         *              dY[m,n] * in[m,k] */
        int64_t ee = r / c->n, nn = r % c->n;
        for (int64_t j = 0; j < ncols; ++j) s[j] = 0.0, ab[j] = 0.0;
        for (int64_t mm = 0; mm < c->m; ++mm) {
            if ((int64_t)c->row_experts[mm] != ee) continue;
            double g = c->DY[mm * c->n + nn];
            const double *inr = c->IN + mm * c->k;
            for (int64_t j = 0; j < c->k; ++j) {
                double pr = g * inr[j];
                s[j] += pr;
                ab[j] += fabs(pr);
            }
        }
    }
    for (int64_t j = 0; j < ncols; ++j) {
        if (c->out) store_rounded(out_dt, c->out, i * ncols + j, s[j]);
        if (c->s_out) c->s_out[i * ncols + j] = s[j];
        if (c->a_out) c->a_out[i * ncols + j] = ab[j];
    }
    free(s);
    free(ab);
}

static int grp_common(int op, int dt, const void *in, const void *wt, const void *dy,
                      const uint32_t *row_experts, int64_t m, int64_t k, int64_t n, int64_t e,
                      const int64_t *rows, int64_t nrows, void *out, double *s_out,
                      double *a_out, int nthreads) {
    if (dt < ORC_F32 || dt > ORC_F16) return -2;
    struct grp_ctx c;
    memset(&c, 0, sizeof c);
    c.dt = dt, c.op = op, c.m = m, c.k = k, c.n = n, c.e = e;
    c.row_experts = row_experts, c.rows = rows, c.out = out, c.s_out = s_out, c.a_out = a_out;
    double *IN = NULL, *WT = NULL, *DY = NULL;
    if (op == 0 || op == 2) IN = decode_all(dt, in, m * k);
    if (op == 0 || op == 1) {
        /* decoded weights plus one guard expert slot filled with NaN: a read
         * of expert slot E (a padding id mistaken for a real one) then shows
         * up as NaN instead of reading unrelated memory */
        WT = (double *)malloc((size_t)((e + 1) * n * k) * sizeof(double));
        if (WT) {
            for (int64_t i = 0; i < e * n * k; ++i) WT[i] = orc_decode(dt, wt, i);
            for (int64_t i = e * n * k; i < (e + 1) * n * k; ++i) WT[i] = NAN;
        }
    }
    if (op == 1 || op == 2) DY = decode_all(dt, dy, m * n);
    c.IN = IN, c.WT = WT, c.DY = DY;
    run_rows(grp_row, &c, nrows, nthreads);
    free(IN), free(WT), free(DY);
    return 0;
}

/* grouped forward rows (indices into M); out [nrows, n] in dt. */
int orc_grouped_fwd(int dt, const void *input, const void *weights,
                    const uint32_t *row_experts, int64_t m, int64_t k, int64_t n, int64_t e,
                    const int64_t *rows, int64_t nrows, void *out, double *s_out,
                    double *a_out, int nthreads) {
    return grp_common(0, dt, input, weights, NULL, row_experts, m, k, n, e, rows, nrows, out,
                      s_out, a_out, nthreads);
}

/* grouped dinput rows (indices into M); out [nrows, k] in dt. */
int orc_grouped_dinput(int dt, const void *grad_out, const void *weights,
                       const uint32_t *row_experts, int64_t m, int64_t k, int64_t n, int64_t e,
                       const int64_t *rows, int64_t nrows, void *out, double *s_out,
                       double *a_out, int nthreads) {
    return grp_common(1, dt, NULL, weights, grad_out, row_experts, m, k, n, e, rows, nrows,
                      out, s_out, a_out, nthreads);
}

/* grouped dweights rows (flattened indices e*N + n into [E*N]); out f32
 * [nrows, k]. */
int orc_grouped_dweights(int dt, const void *input, const void *grad_out,
                         const uint32_t *row_experts, int64_t m, int64_t k, int64_t n,
                         int64_t e, const int64_t *rows, int64_t nrows, float *out,
                         double *s_out, double *a_out, int nthreads) {
    return grp_common(2, dt, input, NULL, grad_out, row_experts, m, k, n, e, rows, nrows, out,
                      s_out, a_out, nthreads);
}

/* ------------------------------------------------------------------------- */
/* fp8 producer side: e5m2, quantisation, scaled fp8 linear                   */
/* ------------------------------------------------------------------------- */

/* OCP fp8 e5m2: sign, 5 exponent bits (bias 15), 2 fraction bits; subnormals
 * are frac * 2^-16; exponent 31 holds +-inf (frac 0) and NaN.  The largest
 * finite value is 1.75 * 2^15 = 57344. */
double orc_decode_e5m2(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int ex = (bits >> 2) & 0x1f;
    int frac = bits & 0x3;
    double v;
    if (ex == 31)
        v = frac ? NAN : INFINITY;
    else if (ex == 0)
        v = ldexp((double)frac, -16);
    else
        v = ldexp((double)(4 + frac), ex - 17);
    return sign ? -v : v;
}

/* double -> e5m2 bits, RNE, saturating to +-57344 (inf included). */
uint8_t orc_rne_e5m2_sat(double x) {
    if (isnan(x)) return 0x7f;
    int neg = signbit(x) ? 1 : 0;
    double r = round_mag(fabs(x), 3, -14, 57344.0);
    if (isinf(r)) r = 57344.0;
    uint8_t mag;
    if (r == 0.0) {
        mag = 0;
    } else {
        int e2;
        frexp(r, &e2);
        int lead = e2 - 1;
        if (lead < -14)
            mag = (uint8_t)ldexp(r, 16);
        else
            mag = (uint8_t)(((lead + 15) << 2) | (int)(ldexp(r, 2 - lead) - 4.0));
    }
    return (uint8_t)(mag | (neg << 7));
}

/* One quantised code: the bf16 source times the inverse scale, multiplied in
 * f32 (an IEEE single multiplication, round to nearest even: the compiler is
 * told not to contract or widen), then RNE to the fp8 format. */
static uint8_t quant_code(int fmt, uint16_t src_bits, float scale_inv) {
    const float raw = (float)orc_decode_bf16(src_bits); /* exact */
    volatile float v = raw * scale_inv;
    return fmt == ORC_E5M2 ? orc_rne_e5m2_sat((double)v) : orc_rne_e4m3_sat((double)v);
}

static float amax_of(const uint16_t *src, int64_t n) {
    float mx = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        const float a = fabsf((float)orc_decode_bf16(src[i]));
        if (a > mx) mx = a; /* NaN compares false: ignored */
    }
    return mx;
}

/* src: n bf16 bit patterns; dst: n codes; *amax = max |src|.  fmt: 3 e4m3fn,
 * 4 e5m2. */
int orc_fp8_quantize(int fmt, const uint16_t *src, float scale_inv, int64_t n, uint8_t *dst,
                     float *amax) {
    if (fmt != ORC_E4M3 && fmt != ORC_E5M2) return -2;
    for (int64_t i = 0; i < n; ++i) dst[i] = quant_code(fmt, src[i], scale_inv);
    if (amax) *amax = amax_of(src, n);
    return 0;
}

/* src: [rows, cols] bf16, row-major; dst: [cols, rows] codes. */
int orc_fp8_transpose_quantize(int fmt, const uint16_t *src, float scale_inv, int64_t rows,
                               int64_t cols, uint8_t *dst, float *amax) {
    if (fmt != ORC_E4M3 && fmt != ORC_E5M2) return -2;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            dst[c * rows + r] = quant_code(fmt, src[r * cols + c], scale_inv);
    if (amax) *amax = amax_of(src, rows * cols);
    return 0;
}

/* Decoded e4m3 codes of quantize(src, scale_inv) (caller frees). */
static double *quant_decoded(const uint16_t *src, float scale_inv, int64_t cnt) {
    double *d = (double *)malloc((size_t)(cnt > 0 ? cnt : 1) * sizeof(double));
    if (!d) return NULL;
    for (int64_t i = 0; i < cnt; ++i)
        d[i] = orc_decode_e4m3(quant_code(ORC_E4M3, src[i], scale_inv));
    return d;
}

struct fp8lin_ctx {
    int op; /* 0 forward, 1 dX, 2 dW */
    int64_t m, k, n;
    const double *QX, *QW, *QG, *B;
    double sa, sb;
    const int64_t *rows;
    uint16_t *out;
    double *s_out, *a_out, *g_out;
};

static void fp8lin_row(void *p, int64_t i) {
    struct fp8lin_ctx *c = (struct fp8lin_ctx *)p;
    int64_t r = c->rows ? c->rows[i] : i;
    int64_t ncols = c->op == 0 ? c->n : c->k;
    double *s = (double *)malloc((size_t)ncols * sizeof(double));
    double *ab = (double *)malloc((size_t)ncols * sizeof(double));
    double *g = (double *)malloc((size_t)ncols * sizeof(double));
    double *arow = NULL;
    if (c->op == 0) {
        /* Y[r, j] = sum_k QX[r,k] QW[j,k] : B(k, j) = QW[j*K + k] */
        row_dot_g8(c->QX + r * c->k, c->k, c->QW, 1, c->k, c->n, s, ab, g);
    } else if (c->op == 1) {
        /* dX[r, j] = sum_n QG[r,n] QW[n,j] : B(n, j) = QW[n*K + j] */
        row_dot_g8(c->QG + r * c->n, c->n, c->QW, c->k, 1, c->k, s, ab, g);
    } else {
        /* dW[r, j] = sum_m QG[m,r] QX[m,j] : a_row[m] = QG[m*N + r] */
        arow = (double *)malloc((size_t)(c->m > 0 ? c->m : 1) * sizeof(double));
        for (int64_t mm = 0; mm < c->m; ++mm) arow[mm] = c->QG[mm * c->n + r];
        row_dot_g8(arow, c->m, c->QX, c->k, 1, c->k, s, ab, g);
    }
    for (int64_t j = 0; j < ncols; ++j) {
        double v = s[j] * c->sa * c->sb;
        double a = ab[j] * fabs(c->sa) * fabs(c->sb);
        if (c->B) v += c->B[j], a += fabs(c->B[j]);
        if (c->out) c->out[i * ncols + j] = orc_rne_bf16(v);
        if (c->s_out) c->s_out[i * ncols + j] = v;
        if (c->a_out) c->a_out[i * ncols + j] = a;
        if (c->g_out) c->g_out[i * ncols + j] = g[j] * fabs(c->sa) * fabs(c->sb);
    }
    free(arow);
    free(s);
    free(ab);
    free(g);
}

/* x: [m,k] bf16, w: [n,k] bf16, bias: [n] bf16 or NULL; out: [nrows, n] bf16. */
int orc_fp8_linear_forward(const uint16_t *x, const uint16_t *w, const uint16_t *bias, float sx,
                           float sw, float sx_inv, float sw_inv, int64_t m, int64_t k,
                           int64_t n, const int64_t *rows, int64_t nrows, uint16_t *out,
                           double *s_out, double *a_out, double *g_out, float *amax_x,
                           float *amax_w, int nthreads) {
    struct fp8lin_ctx c;
    memset(&c, 0, sizeof c);
    double *QX = quant_decoded(x, sx_inv, m * k);
    double *QW = quant_decoded(w, sw_inv, n * k);
    double *B = bias ? decode_all(ORC_BF16, bias, n) : NULL;
    c.op = 0, c.m = m, c.k = k, c.n = n, c.QX = QX, c.QW = QW, c.B = B;
    c.sa = (double)sx, c.sb = (double)sw, c.rows = rows;
    c.out = out, c.s_out = s_out, c.a_out = a_out, c.g_out = g_out;
    run_rows(fp8lin_row, &c, nrows, nthreads);
    if (amax_x) *amax_x = amax_of(x, m * k);
    if (amax_w) *amax_w = amax_of(w, n * k);
    free(QX), free(QW), free(B);
    return 0;
}

/* g: [m,n], x: [m,k], w: [n,k] (bf16).  which = 1: dX rows (indices into M),
 * out [nrows, k]; which = 2: dW rows (indices into N), out [nrows, k]. */
int orc_fp8_linear_backward(int which, const uint16_t *g, const uint16_t *x, const uint16_t *w,
                            float sg, float sw, float sx, float sg_inv, float sw_inv,
                            float sx_inv, int64_t m, int64_t k, int64_t n, const int64_t *rows,
                            int64_t nrows, uint16_t *out, double *s_out, double *a_out,
                            double *g_out, float *amax_g, int nthreads) {
    if (which != 1 && which != 2) return -2;
    struct fp8lin_ctx c;
    memset(&c, 0, sizeof c);
    double *QG = quant_decoded(g, sg_inv, m * n);
    double *QW = which == 1 ? quant_decoded(w, sw_inv, n * k) : NULL;
    double *QX = which == 2 ? quant_decoded(x, sx_inv, m * k) : NULL;
    c.op = which, c.m = m, c.k = k, c.n = n, c.QX = QX, c.QW = QW, c.QG = QG;
    c.sa = (double)sg, c.sb = which == 1 ? (double)sw : (double)sx, c.rows = rows;
    c.out = out, c.s_out = s_out, c.a_out = a_out, c.g_out = g_out;
    run_rows(fp8lin_row, &c, nrows, nthreads);
    if (amax_g) *amax_g = amax_of(g, m * n);
    free(QG), free(QW), free(QX);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Bias gradient: column sums of dY                                           */
/* ------------------------------------------------------------------------- */

/* dy: [m, n] of dtype dt; out: [n] of dt; s_out / a_out: exact sum and sum of
 * absolute values per column (nullable). */
int orc_bias_grad(int dt, const void *dy, int64_t m, int64_t n, void *out, double *s_out,
                  double *a_out) {
    if (dt < ORC_F32 || dt > ORC_F16) return -2;
    for (int64_t j = 0; j < n; ++j) {
        double sum = 0.0, ab = 0.0;
        for (int64_t i = 0; i < m; ++i) {
            const double v = orc_decode(dt, dy, i * n + j);
            sum += v;
            ab += fabs(v);
        }
        if (out) store_rounded(dt, out, j, sum);
        if (s_out) s_out[j] = sum;
        if (a_out) a_out[j] = ab;
    }
    return 0;
}
