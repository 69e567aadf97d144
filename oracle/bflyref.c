/*
 * bflyref.c -- fp64 CPU oracle for the learnable butterfly rotation and its
 * fused round-to-nearest quantizer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines what the GPU library must
 * compute; it is called by the test-suite, by the smoke check and by the CPU
 * baseline leg of the benchmark, and by nothing else.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * Sources (page titles as given on the pages):
 *  - "ButterflyQuant: Ultra-low-bit LLM Quantization through Learnable
 *    Orthogonal Butterfly Transforms" (arXiv 2509.09679 abstract, Fugu-MT
 *    page): the rotation Q is orthogonal by construction, parameterised by
 *    continuous Givens angles, costs O(n log n) with n log n / 2 parameters,
 *    and is applied before quantization using computational invariance
 *    y = Wx = (W Q^T)(Q x).
 *  - duidaima.com write-up of ButterflyQuant, section "butterfly" (蝴蝶展翅):
 *    Hadamard is a special case of the butterfly for n = 2^k; non-power-of-
 *    two widths such as 5120 use a Kronecker-product composite.
 *  - duidaima.com write-up, section "training and results": angles are
 *    learned by gradient descent (backward below).
 *  - WUSH page (gist.science, technical summary, section 2 "method"): the
 *    quantizer is round-to-nearest with absmax block scaling; the INT error
 *    model is proportional to the block's infinity norm.
 *
 * Readings where the pages are silent (each is a documented convention):
 *  - stage s (s = 0 .. L-1, applied in that order) pairs i with j = i + 2^s
 *    for every i whose bit s is clear;
 *  - the pair's angle is theta[s][p], p = the pair's rank among stage-s
 *    pairs ordered by increasing i;
 *  - the pair update is the textbook Givens rotation
 *    (u_i, u_j) <- (c u_i - s u_j, s u_i + c u_j), c = cos theta, s = sin theta;
 *  - quantization groups are contiguous runs of `group` output elements;
 *    symmetric mode: scale = fp16_rne(absmax / qmax), q = clamp(rne(y/scale));
 *    asymmetric mode: scale = fp16_rne((max-min)/levels),
 *    zero = clamp(rne(-min/scale), 0, levels), q = clamp(rne(y/scale)+zero);
 *    codes are packed little-endian, element 0 in the lowest bits.
 *
 * Everything is fp64; cos/sin are evaluated in fp64 from the fp32 angle.
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_F32 0
#define REF_BF16 1

/* ---------------------------------------------------------------------- */
/* Rounding helpers, written from the IEEE-754 definitions.               */
/* ---------------------------------------------------------------------- */

/* Round to nearest integer, ties to even.  Exact for |x| < 2^52. */
static double rne(double x)
{
    double f = floor(x);
    double d = x - f; /* exact */
    if (d > 0.5) return f + 1.0;
    if (d < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* Round x to a binary format with `prec` significand bits (implicit bit
 * included), smallest normal exponent emin (value 2^emin) and subnormal
 * spacing 2^(emin - prec + 1).  Returns the rounded value (may be +-inf). */
static double round_to_format(double x, int prec, int emin, double maxfinite)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    (void)frexp(x, &e); /* |x| = m 2^e, m in [0.5, 1) => 2^(e-1) <= |x| */
    int expo = e - 1;   /* unbiased exponent of x */
    if (expo < emin) expo = emin;
    double ulp = ldexp(1.0, expo - (prec - 1));
    double r = rne(x / ulp) * ulp; /* x / ulp and the product are exact */
    if (r == 0.0) return copysign(0.0, x); /* rounding keeps the sign of zero */
    /* overflow: the rounding boundary above maxfinite is maxfinite + ulp/2 */
    if (fabs(r) > maxfinite) return copysign(INFINITY, x);
    return r;
}

/* bf16: 8 significand bits, emin = -126. */
uint16_t bflyref_bf16_rne(double x)
{
    if (isnan(x)) return 0x7FC0;
    double maxf = ldexp(255.0, 120); /* (2 - 2^-7) 2^127 */
    double r = round_to_format(x, 8, -126, maxf);
    float f = (float)r; /* exact: r is representable in fp32 */
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)(b >> 16);
}

/* fp16: 11 significand bits, emin = -14, max 65504. */
uint16_t bflyref_fp16_rne(double x)
{
    if (isnan(x)) return 0x7E00;
    double r = round_to_format(x, 11, -14, 65504.0);
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (isinf(a)) return sign | 0x7C00;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) /* subnormal: a = k 2^-24 */
        return sign | (uint16_t)(a / ldexp(1.0, -24));
    int e;
    double m = frexp(a, &e); /* a = m 2^e, m in [0.5,1) */
    uint16_t biased = (uint16_t)(e - 1 + 15);
    uint16_t mant = (uint16_t)((m * 2.0 - 1.0) * 1024.0); /* exact */
    return sign | (uint16_t)(biased << 10) | mant;
}

double bflyref_fp16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int mant = h & 0x3FF;
    double v;
    if (ex == 0) v = ldexp((double)mant, -24);
    else if (ex == 31) v = mant ? NAN : INFINITY;
    else v = ldexp(1024.0 + mant, ex - 25);
    return sign ? -v : v;
}

void bflyref_round_bf16(const double* in, uint16_t* out, int64_t count)
{
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < count; ++k) out[k] = bflyref_bf16_rne(in[k]);
}

void bflyref_round_fp16(const double* in, uint16_t* out, int64_t count)
{
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < count; ++k) out[k] = bflyref_fp16_rne(in[k]);
}

static double widen(const void* x, int dtype, int64_t k)
{
    if (dtype == REF_BF16) {
        uint32_t b = (uint32_t)((const uint16_t*)x)[k] << 16;
        float f;
        memcpy(&f, &b, 4);
        return (double)f;
    }
    return (double)((const float*)x)[k];
}

static int log2_exact(int64_t n)
{
    if (n < 2) return -1;
    int L = 0;
    while ((1LL << L) < n) ++L;
    return ((1LL << L) == n) ? L : -1;
}

/* ---------------------------------------------------------------------- */
/* Butterfly                                                               */
/* ---------------------------------------------------------------------- */

/* cos/sin of every angle, evaluated once per call in fp64. */
static void angle_tables(const float* theta, int L, int n, double** cs, double** sn)
{
    int64_t count = (int64_t)L * (n / 2);
    *cs = (double*)malloc(sizeof(double) * count);
    *sn = (double*)malloc(sizeof(double) * count);
    for (int64_t k = 0; k < count; ++k) {
        (*cs)[k] = cos((double)theta[k]);
        (*sn)[k] = sin((double)theta[k]);
    }
}

/* One Givens stage: pair i (bit s clear) with j = i + 2^s; the pair's rank
 * within the stage is p = (i >> (s+1)) * 2^s + (i mod 2^s). */
static void stage_forward(double* u, int n, int s, const double* c_s, const double* s_s)
{
    int half = 1 << s;
    for (int i = 0; i < n; ++i) {
        if ((i >> s) & 1) continue;
        int j = i + half;
        int p = ((i >> (s + 1)) << s) + (i & (half - 1));
        double c = c_s[p], sn = s_s[p];
        double ui = u[i], uj = u[j];
        u[i] = c * ui - sn * uj;
        u[j] = sn * ui + c * uj;
    }
}

/* Transposed stage: (g_i, g_j) <- (c g_i + s g_j, -s g_i + c g_j). */
static void stage_transpose(double* g, int n, int s, const double* c_s, const double* s_s)
{
    int half = 1 << s;
    for (int i = 0; i < n; ++i) {
        if ((i >> s) & 1) continue;
        int j = i + half;
        int p = ((i >> (s + 1)) << s) + (i & (half - 1));
        double c = c_s[p], sn = s_s[p];
        double gi = g[i], gj = g[j];
        g[i] = c * gi + sn * gj;
        g[j] = -sn * gi + c * gj;
    }
}

static void butterfly_apply(double* u, int n, int L, const double* cs, const double* sn)
{
    for (int s = 0; s < L; ++s)
        stage_forward(u, n, s, cs + (int64_t)s * (n / 2), sn + (int64_t)s * (n / 2));
}

/* y[r] = Q(theta) x[r]; x is fp32 or bf16 bits, y is fp64; theta fp32 [L][n/2].
 * Returns 0 on success, -1 on bad arguments. */
int bflyref_forward(const void* x, int x_dtype, double* y, int64_t rows, int32_t n,
                    const float* theta)
{
    int L = log2_exact(n);
    if (L < 1 || rows < 0 || (rows > 0 && (!x || !y || !theta))) return -1;
    if (rows == 0) return 0;
    double *cs, *sn;
    angle_tables(theta, L, n, &cs, &sn);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double* u = y + r * n;
        for (int i = 0; i < n; ++i) u[i] = widen(x, x_dtype, r * n + i);
        butterfly_apply(u, n, L, cs, sn);
    }
    free(cs);
    free(sn);
    return 0;
}

/* Kronecker composite (O (x) B(theta_b)) x with n = m * nb and index
 * i = a * nb + b: the butterfly B acts on each segment a, then O mixes the m
 * segments column by column: y[a nb + b] = sum_a' O[a][a'] z[a' nb + b].
 * mix is fp32 [m][m] row-major. */
int bflyref_kron_forward(const void* x, int x_dtype, double* y, int64_t rows, int32_t m,
                         int32_t nb, const float* theta_b, const float* mix)
{
    int L = log2_exact(nb);
    if (L < 1 || m < 1 || rows < 0 || (rows > 0 && (!x || !y || !theta_b || !mix))) return -1;
    if (rows == 0) return 0;
    int64_t n = (int64_t)m * nb;
    double *cs, *sn;
    angle_tables(theta_b, L, nb, &cs, &sn);
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * m);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            double* u = y + r * n;
            for (int64_t i = 0; i < n; ++i) u[i] = widen(x, x_dtype, r * n + i);
            for (int a = 0; a < m; ++a) butterfly_apply(u + (int64_t)a * nb, nb, L, cs, sn);
            for (int b = 0; b < nb; ++b) {
                for (int a = 0; a < m; ++a) {
                    double acc = 0.0;
                    for (int a2 = 0; a2 < m; ++a2)
                        acc += (double)mix[a * m + a2] * u[(int64_t)a2 * nb + b];
                    w[a] = acc;
                }
                for (int a = 0; a < m; ++a) u[(int64_t)a * nb + b] = w[a];
            }
        }
        free(w);
    }
    free(cs);
    free(sn);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Quantizer                                                               */
/* ---------------------------------------------------------------------- */

#define REF_SYM 0
#define REF_ASYM 1

/* Per-group RTN quantization of fp64 rows y [rows][n].
 *   codes  u8  [rows][n*bits/8]   packed, element 0 of a byte in its low bits
 *   scales u16 [rows][n/group]    fp16 bits
 *   zeros  u16 [rows][n/group]    fp16 bits of the integer zero point (asym)
 *   s_pre  f64 [rows][n/group]    optional: the scale before fp16 rounding
 *   z_pre  f64 [rows][n/group]    optional (asym): -min/scale before rounding
 *   v      f64 [rows][n]          optional: y / scale, the value that is rounded
 * If use_given is 1, scales (and zeros) are INPUTS: the codes are computed
 * at those scales (used to re-quantize at another implementation's scale
 * when a scale rounding tie made both neighbours acceptable).  If use_given
 * is 2, the scales are inputs and the asymmetric zero points are derived at
 * them (clamp(rne(-min / scale))), as the quantizer would with that scale.
 * Returns 0, or -1 on bad arguments. */
int bflyref_quantize(const double* y, int64_t rows, int32_t n, int32_t group, int32_t bits,
                     int32_t mode, int32_t use_given, uint8_t* codes, uint16_t* scales,
                     uint16_t* zeros, double* s_pre, double* z_pre, double* v)
{
    if (rows < 0 || n < 1 || group < 1 || n % group != 0) return -1;
    if (use_given < 0 || use_given > 2) return -1;
    if (bits != 2 && bits != 4) return -1;
    if (mode != REF_SYM && mode != REF_ASYM) return -1;
    if (((int64_t)n * bits) % 8 != 0) return -1;
    if (rows == 0) return 0;
    if (!y || !codes || !scales || (mode == REF_ASYM && !zeros)) return -1;
    const int per_byte = 8 / bits;
    const int64_t row_bytes = (int64_t)n * bits / 8;
    const int ngroups = n / group;
    const int qmax = (1 << (bits - 1)) - 1; /* symmetric: 7 (INT4), 1 (INT2) */
    const int levels = (1 << bits) - 1;     /* asymmetric: 15 (INT4), 3 (INT2) */
    const uint8_t mask = (uint8_t)((1 << bits) - 1);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double* yr = y + r * n;
        uint8_t* cr = codes + r * row_bytes;
        memset(cr, 0, (size_t)row_bytes);
        for (int g = 0; g < ngroups; ++g) {
            const double* yg = yr + (int64_t)g * group;
            int64_t gi = r * ngroups + g;
            double spre, zp = 0.0;
            if (mode == REF_SYM) {
                double a = 0.0;
                for (int k = 0; k < group; ++k) a = fmax(a, fabs(yg[k]));
                spre = a / qmax;
            } else {
                double lo = yg[0], hi = yg[0];
                for (int k = 1; k < group; ++k) {
                    lo = fmin(lo, yg[k]);
                    hi = fmax(hi, yg[k]);
                }
                spre = (hi - lo) / levels;
                zp = -lo; /* divided by the scale below */
            }
            if (s_pre) s_pre[gi] = spre;
            uint16_t s16;
            if (use_given) {
                s16 = scales[gi];
            } else {
                /* a scale beyond the fp16 range saturates to the largest finite */
                s16 = bflyref_fp16_rne(spre > 65504.0 ? 65504.0 : spre);
                scales[gi] = s16;
            }
            double sc = bflyref_fp16_value(s16);
            double z = 0.0;
            if (mode == REF_ASYM) {
                if (sc != 0.0) {
                    double zq = zp / sc;
                    if (z_pre) z_pre[gi] = zq;
                    if (use_given == 1) {
                        z = bflyref_fp16_value(zeros[gi]);
                    } else {
                        z = rne(zq);
                        if (z < 0.0) z = 0.0;
                        if (z > levels) z = levels;
                        zeros[gi] = bflyref_fp16_rne(z);
                    }
                } else {
                    if (z_pre) z_pre[gi] = 0.0;
                    if (use_given != 1) zeros[gi] = 0;
                    z = use_given == 1 ? bflyref_fp16_value(zeros[gi]) : 0.0;
                }
            }
            for (int k = 0; k < group; ++k) {
                int64_t e = (int64_t)g * group + k;
                int q;
                if (sc == 0.0) {
                    q = 0;
                    if (v) v[r * n + e] = 0.0;
                } else {
                    double t = yg[k] / sc;
                    if (v) v[r * n + e] = t;
                    double qd = rne(t);
                    if (mode == REF_SYM) {
                        if (qd > qmax) qd = qmax;
                        if (qd < -qmax) qd = -qmax;
                    } else {
                        qd += z;
                        if (qd < 0.0) qd = 0.0;
                        if (qd > levels) qd = levels;
                    }
                    q = (int)qd;
                }
                cr[e / per_byte] |= (uint8_t)(((uint8_t)q & mask) << (bits * (e % per_byte)));
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Backward                                                                */
/* ---------------------------------------------------------------------- */

/* Given X and G = dL/dY (fp32 [rows][n]), with Y = Q(theta) X row by row:
 *   y      = Q x                       (fp64 [rows][n], optional)
 *   dx     = Q^T g                     (fp64 [rows][n], optional)
 *   dtheta = sum over rows of dL/dtheta (fp64 [L][n/2], OVERWRITTEN)
 *   dabs   = sum over rows of |g_j v_i| + |g_i v_j| (same shape, optional):
 *            the magnitude of the terms that cancel in dtheta.
 * For the pair (i, j) of stage s with stage output v and gradient g w.r.t.
 * that output, d(loss)/d(theta) = g_j v_i - g_i v_j.  Per-thread partial sums
 * are added in thread order. */
int bflyref_backward(const float* x, const float* g, int64_t rows, int32_t n,
                     const float* theta, double* y, double* dx, double* dtheta, double* dabs)
{
    int L = log2_exact(n);
    if (L < 1 || rows < 0 || !theta || !dtheta) return -1;
    if (rows > 0 && (!x || !g)) return -1;
    int64_t np = (int64_t)L * (n / 2);
    memset(dtheta, 0, sizeof(double) * np);
    if (dabs) memset(dabs, 0, sizeof(double) * np);
    if (rows == 0) return 0;
    double *cs, *sn;
    angle_tables(theta, L, n, &cs, &sn);
    int nthreads = 1;
#ifdef _OPENMP
    nthreads = omp_get_max_threads();
#endif
    double* part = (double*)calloc((size_t)nthreads * np * 2, sizeof(double));
#pragma omp parallel num_threads(nthreads)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double* pd = part + (int64_t)tid * np * 2;
        double* pa = pd + np;
        double* V = (double*)malloc(sizeof(double) * (size_t)(L + 1) * n);
        double* gv = (double*)malloc(sizeof(double) * n);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            for (int i = 0; i < n; ++i) V[i] = (double)x[r * n + i];
            for (int s = 0; s < L; ++s) {
                memcpy(V + (int64_t)(s + 1) * n, V + (int64_t)s * n, sizeof(double) * n);
                stage_forward(V + (int64_t)(s + 1) * n, n, s, cs + (int64_t)s * (n / 2),
                              sn + (int64_t)s * (n / 2));
            }
            if (y) memcpy(y + r * n, V + (int64_t)L * n, sizeof(double) * n);
            for (int i = 0; i < n; ++i) gv[i] = (double)g[r * n + i];
            for (int s = L - 1; s >= 0; --s) {
                const double* v = V + (int64_t)(s + 1) * n; /* stage-s output */
                int half = 1 << s;
                for (int i = 0; i < n; ++i) {
                    if ((i >> s) & 1) continue;
                    int j = i + half;
                    int p = ((i >> (s + 1)) << s) + (i & (half - 1));
                    double t1 = gv[j] * v[i], t2 = gv[i] * v[j];
                    pd[(int64_t)s * (n / 2) + p] += t1 - t2;
                    pa[(int64_t)s * (n / 2) + p] += fabs(t1) + fabs(t2);
                }
                stage_transpose(gv, n, s, cs + (int64_t)s * (n / 2), sn + (int64_t)s * (n / 2));
            }
            if (dx) memcpy(dx + r * n, gv, sizeof(double) * n);
        }
        free(V);
        free(gv);
    }
    for (int t = 0; t < nthreads; ++t) {
        const double* pd = part + (int64_t)t * np * 2;
        for (int64_t k = 0; k < np; ++k) {
            dtheta[k] += pd[k];
            if (dabs) dabs[k] += pd[np + k];
        }
    }
    free(part);
    free(cs);
    free(sn);
    return 0;
}

int bflyref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the parallel loops above use from now on (k >= 1). */
void bflyref_set_num_threads(int k)
{
#ifdef _OPENMP
    if (k >= 1) omp_set_num_threads(k);
#else
    (void)k;
#endif
}
