/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the bf16 grouped (ragged,
 * per-expert) GEMM and its fp8 block-scaled forward (stated with the fp8
 * functions below).  TEST INFRASTRUCTURE ONLY: the HIP library never links,
 * loads or calls this file, and this file shares no code with it.
 *
 * What it computes (restated from the pages, not copied):
 *
 *  - Ragged layout (PyTorch issue #152668, "Easy repro scenario": a 2-D
 *    activation [M,K], a 3-D weight [E,K,N] and int32 cumulative *end*
 *    offsets of length E): expert g owns the rows [end(g-1), end(g)) of the
 *    activation, with end(-1) = 0, and its output rows are that slice times
 *    W[g].  The backward of that call gives dgrad (dX = dY W[g]^T on the
 *    same rows) and wgrad (dW[g] = X[g]^T dY[g]).
 *  - Rows at or past end(E-1) belong to no expert.  They are reported as
 *    unused and never read (TransformerEngine PR #3542, "Changes": unused
 *    capacity of caller-owned outputs is preserved).
 *  - An expert with no rows contributes no output rows in fwd/dgrad and an
 *    all-zero dW[g] in wgrad (the empty sum).  The pages only report that
 *    this case hung the backward (PyTorch issue #152668, "Describe the
 *    bug"); the value +0.0 is the mathematical definition.
 *  - Masked layout (sglang PR #32385, "Evidence", reproduction and operand
 *    table): A[E, max_m, K], W[E, K, N], D[E, max_m, N] and a per-expert
 *    count masked_m[e]; rows r < masked_m[e] of expert e are active, the rest
 *    are inactive and neither read nor written.  Its backward on the same
 *    layout: dX[e, r] = dY[e, r] W[e]^T on active rows and dW[e] = X[e]^T
 *    dY[e] over active rows (+0.0 for an expert with none).
 *
 * Readings taken where the pages are silent:
 *  - Offsets are clamped into a monotone sequence, end(g) = min(max(offs[g],
 *    end(g-1)), M), so decreasing or oversize offsets give empty or
 *    truncated experts rather than out-of-range accesses.  masked_m is
 *    clamped into [0, max_m] the same way.
 *  - Sums run in fp64 over bf16 inputs decoded exactly; each product of two
 *    bf16 values is exact in fp64.  Alongside each output the oracle returns
 *    S = sum |a*b| over the same terms, the scale of the rounding error any
 *    fp32-accumulating implementation may make.
 *  - Results are rounded to the output type only by the caller, with
 *    oracle_round_bf16 (round to nearest, ties to even, straight from fp64)
 *    or an fp64 -> fp32 C cast (round to nearest even).
 *
 * Every entry point takes an explicit list of output rows (fwd, dgrad,
 * masked) or (expert, k) pairs (wgrad) so large problems can be checked on a
 * sample; a NULL list means "all".  Outputs are dense [count, width] fp64
 * arrays plus a per-entry status: 1 = computed, 0 = row belongs to no expert
 * (or is inactive) and its y/s entries are left untouched.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- bf16 codec (own implementation) ---------------------------------- */

/* bf16 is the top 16 bits of an IEEE binary32; decoding is exact. */
static double bf16_decode(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* fp64 -> bf16, round to nearest, ties to even, without an fp32 detour
 * (which would round twice).  bf16 keeps 8 significant bits: a finite value
 * of binary exponent E (2^E <= |v| < 2^(E+1)) is a multiple of 2^(E-7);
 * below the normal range the spacing stays 2^(-126-7).  rint() rounds to
 * even under the default rounding mode. */
uint16_t oracle_round_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                /* 2^e <= a < 2^(e+1) */
    if (e < -126) e = -126;
    double q = ldexp(1.0, e - 7);  /* spacing of bf16 values near a */
    double r = rint(a / q) * q;    /* a/q and the product are exact */
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;  /* overflow to inf */
    float rf = (float)r;           /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

double oracle_decode_bf16(uint16_t bits) { return bf16_decode(bits); }

/* Element-wise oracle_round_bf16 over an array. */
void oracle_round_bf16_array(const double* v, int64_t count, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_round_bf16(v[i]);
}

/* ---- group decode ------------------------------------------------------- */

/* end(g) = min(max(offs[g], end(g-1)), m), end(-1) = 0. */
static void group_ends(const int32_t* offs, int32_t num_groups, int64_t m,
                       int64_t* ends) {
    int64_t prev = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
        int64_t e = offs[g];
        if (e < prev) e = prev;
        if (e > m) e = m;
        ends[g] = e;
        prev = e;
    }
}

/* Expert owning row i, or -1 when i is at or past the last end. */
static int32_t group_of_row(const int64_t* ends, int32_t num_groups, int64_t i) {
    for (int32_t g = 0; g < num_groups; ++g)
        if (i < ends[g]) return g;
    return -1;
}

#define ORACLE_MAX_GROUPS (1 << 20)

/* ---- forward: Y[i, :] = X[i, :] . W[g] for each row i of expert g -------- */
int oracle_forward(const uint16_t* x, const uint16_t* w, const int32_t* offs,
                   int64_t m, int64_t k, int64_t n, int32_t num_groups,
                   const int64_t* rows, int64_t nrows,
                   double* y, double* s, int32_t* status) {
    if (num_groups < 1 || num_groups > ORACLE_MAX_GROUPS) return -1;
    int64_t* ends = (int64_t*)malloc(sizeof(int64_t) * (size_t)num_groups);
    if (!ends) return -2;
    group_ends(offs, num_groups, m, ends);
    int64_t count = rows ? nrows : m;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < count; ++r) {
        int64_t i = rows ? rows[r] : r;
        int32_t g = (i >= 0 && i < m) ? group_of_row(ends, num_groups, i) : -1;
        status[r] = g >= 0;
        if (g < 0) continue;
        double* yr = y + r * n;
        double* sr = s + r * n;
        for (int64_t j = 0; j < n; ++j) { yr[j] = 0.0; sr[j] = 0.0; }
        const uint16_t* wg = w + (int64_t)g * k * n;
        for (int64_t kk = 0; kk < k; ++kk) {
            double a = bf16_decode(x[i * k + kk]);
            const uint16_t* wrow = wg + kk * n;
            for (int64_t j = 0; j < n; ++j) {
                double p = a * bf16_decode(wrow[j]);
                yr[j] += p;
                sr[j] += fabs(p);
            }
        }
    }
    free(ends);
    return 0;
}

/* ---- dgrad: dX[i, kk] = sum_j dY[i, j] * W[g, kk, j] ---------------------- */
int oracle_dgrad(const uint16_t* dy, const uint16_t* w, const int32_t* offs,
                 int64_t m, int64_t k, int64_t n, int32_t num_groups,
                 const int64_t* rows, int64_t nrows,
                 double* dx, double* s, int32_t* status) {
    if (num_groups < 1 || num_groups > ORACLE_MAX_GROUPS) return -1;
    int64_t* ends = (int64_t*)malloc(sizeof(int64_t) * (size_t)num_groups);
    if (!ends) return -2;
    group_ends(offs, num_groups, m, ends);
    int64_t count = rows ? nrows : m;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < count; ++r) {
        int64_t i = rows ? rows[r] : r;
        int32_t g = (i >= 0 && i < m) ? group_of_row(ends, num_groups, i) : -1;
        status[r] = g >= 0;
        if (g < 0) continue;
        const uint16_t* wg = w + (int64_t)g * k * n;
        for (int64_t kk = 0; kk < k; ++kk) {
            double acc = 0.0, sabs = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                double p = bf16_decode(dy[i * n + j]) * bf16_decode(wg[kk * n + j]);
                acc += p;
                sabs += fabs(p);
            }
            dx[r * k + kk] = acc;
            s[r * k + kk] = sabs;
        }
    }
    free(ends);
    return 0;
}

/* ---- wgrad: dW[g, kk, :] = sum over rows i of g of X[i, kk] * dY[i, :] ---- */
/* pairs: nsel (expert, kk) pairs as int64 [nsel, 2]; NULL = all E*k rows of
 * dW in order.  An expert with no rows gives +0.0 everywhere. */
int oracle_wgrad(const uint16_t* x, const uint16_t* dy, const int32_t* offs,
                 int64_t m, int64_t k, int64_t n, int32_t num_groups,
                 const int64_t* pairs, int64_t nsel,
                 double* dw, double* s, int32_t* status) {
    if (num_groups < 1 || num_groups > ORACLE_MAX_GROUPS) return -1;
    int64_t* ends = (int64_t*)malloc(sizeof(int64_t) * (size_t)num_groups);
    if (!ends) return -2;
    group_ends(offs, num_groups, m, ends);
    int64_t count = pairs ? nsel : (int64_t)num_groups * k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < count; ++r) {
        int64_t g = pairs ? pairs[2 * r] : r / k;
        int64_t kk = pairs ? pairs[2 * r + 1] : r % k;
        int ok = g >= 0 && g < num_groups && kk >= 0 && kk < k;
        status[r] = ok;
        if (!ok) continue;
        double* out = dw + r * n;
        double* sr = s + r * n;
        for (int64_t j = 0; j < n; ++j) { out[j] = 0.0; sr[j] = 0.0; }
        int64_t start = g == 0 ? 0 : ends[g - 1];
        for (int64_t i = start; i < ends[g]; ++i) {
            double a = bf16_decode(x[i * k + kk]);
            const uint16_t* dyr = dy + i * n;
            for (int64_t j = 0; j < n; ++j) {
                double p = a * bf16_decode(dyr[j]);
                out[j] += p;
                sr[j] += fabs(p);
            }
        }
    }
    free(ends);
    return 0;
}

/* ---- masked forward: D[e, r, :] = A[e, r, :] . W[e], r < masked_m[e] ------ */
/* rows: flat indices e*max_m + r; NULL = all E*max_m. */
int oracle_masked_forward(const uint16_t* x, const uint16_t* w,
                          const int32_t* masked_m, int64_t max_m, int64_t k,
                          int64_t n, int32_t num_groups,
                          const int64_t* rows, int64_t nrows,
                          double* y, double* s, int32_t* status) {
    if (num_groups < 1) return -1;
    int64_t total = (int64_t)num_groups * max_m;
    int64_t count = rows ? nrows : total;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < count; ++r) {
        int64_t flat = rows ? rows[r] : r;
        int ok = flat >= 0 && flat < total;
        int64_t e = ok ? flat / max_m : 0, row = ok ? flat % max_m : 0;
        if (ok) {
            int64_t active = masked_m[e];
            if (active < 0) active = 0;
            if (active > max_m) active = max_m;
            ok = row < active;
        }
        status[r] = ok;
        if (!ok) continue;
        double* yr = y + r * n;
        double* sr = s + r * n;
        for (int64_t j = 0; j < n; ++j) { yr[j] = 0.0; sr[j] = 0.0; }
        const uint16_t* we = w + e * k * n;
        const uint16_t* xr = x + flat * k;
        for (int64_t kk = 0; kk < k; ++kk) {
            double a = bf16_decode(xr[kk]);
            for (int64_t j = 0; j < n; ++j) {
                double p = a * bf16_decode(we[kk * n + j]);
                yr[j] += p;
                sr[j] += fabs(p);
            }
        }
    }
    return 0;
}

/* Active rows of expert e in the masked layout: masked_m[e] clamped into
 * [0, max_m]. */
static int64_t masked_active(const int32_t* masked_m, int64_t e, int64_t max_m) {
    int64_t a = masked_m[e];
    if (a < 0) a = 0;
    if (a > max_m) a = max_m;
    return a;
}

/* ---- masked dgrad: dX[e, r, :] = dY[e, r, :] . W[e]^T, r < masked_m[e] ---- */
/* The backward of the masked forward through its activation: inactive rows
 * of dY are never read and of dX never written (sglang PR #32385, "Cause":
 * consumers of the masked layout must not depend on inactive rows).
 * rows: flat indices e*max_m + r; NULL = all E*max_m. */
int oracle_masked_dgrad(const uint16_t* dy, const uint16_t* w,
                        const int32_t* masked_m, int64_t max_m, int64_t k,
                        int64_t n, int32_t num_groups,
                        const int64_t* rows, int64_t nrows,
                        double* dx, double* s, int32_t* status) {
    if (num_groups < 1) return -1;
    int64_t total = (int64_t)num_groups * max_m;
    int64_t count = rows ? nrows : total;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < count; ++r) {
        int64_t flat = rows ? rows[r] : r;
        int ok = flat >= 0 && flat < total;
        int64_t e = ok ? flat / max_m : 0, row = ok ? flat % max_m : 0;
        if (ok) ok = row < masked_active(masked_m, e, max_m);
        status[r] = ok;
        if (!ok) continue;
        const uint16_t* we = w + e * k * n;
        const uint16_t* dyr = dy + flat * n;
        for (int64_t kk = 0; kk < k; ++kk) {
            double acc = 0.0, sabs = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                double p = bf16_decode(dyr[j]) * bf16_decode(we[kk * n + j]);
                acc += p;
                sabs += fabs(p);
            }
            dx[r * k + kk] = acc;
            s[r * k + kk] = sabs;
        }
    }
    return 0;
}

/* ---- masked wgrad: dW[e, kk, :] = sum over active rows r of X[e, r, kk] *
 * dY[e, r, :] ------------------------------------------------------------- */
/* pairs: nsel (expert, kk) pairs as int64 [nsel, 2]; NULL = all E*k rows of
 * dW in order.  An expert with no active rows gives +0.0 everywhere. */
int oracle_masked_wgrad(const uint16_t* x, const uint16_t* dy,
                        const int32_t* masked_m, int64_t max_m, int64_t k,
                        int64_t n, int32_t num_groups,
                        const int64_t* pairs, int64_t nsel,
                        double* dw, double* s, int32_t* status) {
    if (num_groups < 1) return -1;
    int64_t count = pairs ? nsel : (int64_t)num_groups * k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < count; ++r) {
        int64_t e = pairs ? pairs[2 * r] : r / k;
        int64_t kk = pairs ? pairs[2 * r + 1] : r % k;
        int ok = e >= 0 && e < num_groups && kk >= 0 && kk < k;
        status[r] = ok;
        if (!ok) continue;
        double* out = dw + r * n;
        double* sr = s + r * n;
        for (int64_t j = 0; j < n; ++j) { out[j] = 0.0; sr[j] = 0.0; }
        int64_t active = masked_active(masked_m, e, max_m);
        for (int64_t row = 0; row < active; ++row) {
            double a = bf16_decode(x[(e * max_m + row) * k + kk]);
            const uint16_t* dyr = dy + (e * max_m + row) * n;
            for (int64_t j = 0; j < n; ++j) {
                double p = a * bf16_decode(dyr[j]);
                out[j] += p;
                sr[j] += fabs(p);
            }
        }
    }
    return 0;
}

/* ---- FP8 (e4m3) block-scaled forward ------------------------------------- */
/*
 * sglang PR #32385 runs the masked MoE GEMMs of its fp8 rollout on fp8
 * operands with one scale per 128 reduction values ("Cause": G = D / 128 in
 * the table of models; "Evidence": activation scales of shape (E, max_m, G)
 * and weight scales per (expert, output column, k-block) in the operand
 * table), every scale a positive power of two -- UE8M0 -- checked by
 * masking an fp32's sign and mantissa bits ("Problem").  The weight is the
 * "nt" operand of that call: W[E, N, K], K contiguous.  So
 *
 *   Y[i, n] = sum_kk  x(i, kk) sx[i, kk / 128]  *  w(g, n, kk) sw[g, n, kk / 128]
 *
 * over the rows i of expert g, with x, w the e4m3 values and sx, sw the
 * scales (fp32 values).  The sums run in fp64; a product of two e4m3 values
 * and two powers of two is exact there.
 *
 * e4m3 here is the OCP 8-bit float with 4 exponent bits (bias 7) and 3
 * mantissa bits, no infinities, and NaN only at S.1111.111: a normal value
 * is (1 + m/8) 2^(e-7), a subnormal (e = 0) is m 2^-9, the largest 448. */
static double e4m3_decode(uint8_t b) {
    int sgn = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);   /* (1 + m/8) 2^(e-7) */
    return sgn ? -v : v;
}

double oracle_decode_e4m3(uint8_t b) { return e4m3_decode(b); }

/* The 256 e4m3 values, e4m3_decode of each code (a lookup for the row
 * loops below; the same values). */
static double e4m3_table[256];
static void e4m3_table_init(void) {
    for (int c = 0; c < 256; ++c) e4m3_table[c] = e4m3_decode((uint8_t)c);
}

/* One output row of the fp8 forward: xr, sxr the row's values and scales,
 * wg, swg the expert's weight [n, k] and scales [n, kb]; xs is room for k
 * doubles.  The row's scaled values x(i, kk) sx[i, kk / 128] are formed
 * once, then each output column sums its k products in order. */
static void fp8_row(const uint8_t* xr, const float* sxr, const uint8_t* wg,
                    const float* swg, int64_t k, int64_t n, double* yr, double* sr, double* xs) {
    int64_t kb = (k + 127) / 128;
    for (int64_t kk = 0; kk < k; ++kk) xs[kk] = e4m3_table[xr[kk]] * (double)sxr[kk / 128];
    for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0, sabs = 0.0;
        const uint8_t* wr = wg + j * k;
        const float* swr = swg + j * kb;
        for (int64_t kk = 0; kk < k; ++kk) {
            double p = xs[kk] * (e4m3_table[wr[kk]] * (double)swr[kk / 128]);
            acc += p;
            sabs += fabs(p);
        }
        yr[j] = acc;
        sr[j] = sabs;
    }
}

/* Ragged layout: x [m, k], sx [m, kb], w [E, n, k], sw [E, n, kb] with
 * kb = ceil(k / 128); the offsets as in oracle_forward. */
int oracle_fp8_forward(const uint8_t* x, const float* sx, const uint8_t* w,
                       const float* sw, const int32_t* offs, int64_t m, int64_t k,
                       int64_t n, int32_t num_groups, const int64_t* rows,
                       int64_t nrows, double* y, double* s, int32_t* status) {
    if (num_groups < 1 || num_groups > ORACLE_MAX_GROUPS) return -1;
    int64_t* ends = (int64_t*)malloc(sizeof(int64_t) * (size_t)num_groups);
    if (!ends) return -2;
    group_ends(offs, num_groups, m, ends);
    e4m3_table_init();
    int64_t kb = (k + 127) / 128;
    int64_t count = rows ? nrows : m;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < count; ++r) {
        int64_t i = rows ? rows[r] : r;
        int32_t g = (i >= 0 && i < m) ? group_of_row(ends, num_groups, i) : -1;
        status[r] = g >= 0;
        if (g < 0) continue;
        double* xs = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        if (!xs) {
            status[r] = 0;
#pragma omp atomic write
            failed = 1;
            continue;
        }
        fp8_row(x + i * k, sx + i * kb, w + (int64_t)g * n * k, sw + (int64_t)g * n * kb,
                k, n, y + r * n, s + r * n, xs);
        free(xs);
    }
    free(ends);
    return failed ? -2 : 0;
}

/* Masked layout: x [E, max_m, k], sx [E, max_m, kb], w [E, n, k],
 * sw [E, n, kb]; rows r < masked_m[e] are active, the others (values and
 * scales alike) are never read.  rows: flat indices e*max_m + r. */
int oracle_fp8_masked_forward(const uint8_t* x, const float* sx, const uint8_t* w,
                              const float* sw, const int32_t* masked_m, int64_t max_m,
                              int64_t k, int64_t n, int32_t num_groups,
                              const int64_t* rows, int64_t nrows, double* y, double* s,
                              int32_t* status) {
    if (num_groups < 1) return -1;
    e4m3_table_init();
    int64_t kb = (k + 127) / 128;
    int64_t total = (int64_t)num_groups * max_m;
    int64_t count = rows ? nrows : total;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < count; ++r) {
        int64_t flat = rows ? rows[r] : r;
        int ok = flat >= 0 && flat < total;
        int64_t e = ok ? flat / max_m : 0, row = ok ? flat % max_m : 0;
        if (ok) ok = row < masked_active(masked_m, e, max_m);
        status[r] = ok;
        if (!ok) continue;
        double* xs = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        if (!xs) {
            status[r] = 0;
#pragma omp atomic write
            failed = 1;
            continue;
        }
        fp8_row(x + flat * k, sx + flat * kb, w + e * n * k, sw + e * n * kb, k, n,
                y + r * n, s + r * n, xs);
        free(xs);
    }
    return failed ? -2 : 0;
}

/* Threads OpenMP will use for the calls above. */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 1; }
#endif
