/* The oracle's C core under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built by tests/test_sanitize_cpu.py together with oracle/bflyref.c).  It
 * drives every exported function over small sizes, empty inputs and invalid
 * arguments, and checks a few exact properties on the way (norm
 * preservation, the adjoint identity <Q x, g> = <x, Q^T g>, code ranges), so
 * that a run that only avoids crashing does not pass. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t bflyref_bf16_rne(double x);
uint16_t bflyref_fp16_rne(double x);
double bflyref_fp16_value(uint16_t h);
void bflyref_round_bf16(const double* in, uint16_t* out, int64_t count);
void bflyref_round_fp16(const double* in, uint16_t* out, int64_t count);
int bflyref_forward(const void* x, int x_dtype, double* y, int64_t rows, int32_t n,
                    const float* theta);
int bflyref_kron_forward(const void* x, int x_dtype, double* y, int64_t rows, int32_t m,
                         int32_t nb, const float* theta_b, const float* mix);
int bflyref_quantize(const double* y, int64_t rows, int32_t n, int32_t group, int32_t bits,
                     int32_t mode, int32_t use_given, uint8_t* codes, uint16_t* scales,
                     uint16_t* zeros, double* s_pre, double* z_pre, double* v);
int bflyref_backward(const float* x, const float* g, int64_t rows, int32_t n,
                     const float* theta, double* y, double* dx, double* dtheta, double* dabs);
int bflyref_num_threads(void);
void bflyref_set_num_threads(int k);

static int failures = 0;
#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uniform(void) /* splitmix64, in [-1, 1) */
{
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1p-52 - 1.0;
}

static void rounding(void)
{
    const double special[] = {0.0, -0.0, 1.0, -1.0, 65504.0, 65520.0, 1e300, -1e300, 5.96e-8,
                              1e-300, 3.4e38, 3.5e38, INFINITY, -INFINITY, NAN};
    const int k = (int)(sizeof(special) / sizeof(special[0]));
    uint16_t b[16], h[16];
    bflyref_round_bf16(special, b, k);
    bflyref_round_fp16(special, h, k);
    for (int i = 0; i < k; ++i) {
        EXPECT(b[i] == bflyref_bf16_rne(special[i]));
        EXPECT(h[i] == bflyref_fp16_rne(special[i]));
        const double back = bflyref_fp16_value(h[i]);
        if (isfinite(special[i]) && fabs(special[i]) <= 65504.0)
            EXPECT(fabs(back - special[i]) <= fabs(special[i]) * 0x1p-11 + 0x1p-25);
    }
    for (uint32_t v = 0; v < 65536; ++v) (void)bflyref_fp16_value((uint16_t)v);
    bflyref_round_bf16(special, b, 0);
}

static void forward_backward(int n, int64_t rows)
{
    int L = 0;
    while ((1 << L) < n) ++L;
    float* theta = malloc(sizeof(float) * (size_t)L * (size_t)(n / 2));
    float* x = malloc(sizeof(float) * (size_t)(rows * n) + 1);
    float* g = malloc(sizeof(float) * (size_t)(rows * n) + 1);
    double* y = malloc(sizeof(double) * (size_t)(rows * n) + 1);
    double* y2 = malloc(sizeof(double) * (size_t)(rows * n) + 1);
    double* dx = malloc(sizeof(double) * (size_t)(rows * n) + 1);
    double* dth = malloc(sizeof(double) * (size_t)L * (size_t)(n / 2));
    double* dabs = malloc(sizeof(double) * (size_t)L * (size_t)(n / 2));
    for (int i = 0; i < L * (n / 2); ++i) theta[i] = (float)(3.14159 * uniform());
    for (int64_t i = 0; i < rows * n; ++i) {
        x[i] = (float)uniform();
        g[i] = (float)uniform();
    }
    EXPECT(bflyref_forward(x, 0, y, rows, n, theta) == 0);
    EXPECT(bflyref_backward(x, g, rows, n, theta, y2, dx, dth, dabs) == 0);
    for (int64_t r = 0; r < rows; ++r) {
        double nx = 0, ny = 0, qg = 0, xq = 0;
        for (int i = 0; i < n; ++i) {
            nx += (double)x[r * n + i] * x[r * n + i];
            ny += y[r * n + i] * y[r * n + i];
            qg += y[r * n + i] * g[r * n + i];
            xq += (double)x[r * n + i] * dx[r * n + i];
            EXPECT(y[r * n + i] == y2[r * n + i]);
        }
        EXPECT(fabs(nx - ny) <= 1e-12 * nx);
        EXPECT(fabs(qg - xq) <= 1e-12 * (sqrt(nx) * n));
    }
    for (int i = 0; i < L * (n / 2); ++i) EXPECT(fabs(dth[i]) <= dabs[i] * (1 + 1e-12));
    /* the same rows through a bf16 input and through the quantizer */
    uint16_t* xb = malloc(sizeof(uint16_t) * (size_t)(rows * n) + 1);
    for (int64_t i = 0; i < rows * n; ++i) xb[i] = bflyref_bf16_rne(x[i]);
    EXPECT(bflyref_forward(xb, 1, y2, rows, n, theta) == 0);
    for (int bits = 2; bits <= 4; bits += 2)
        for (int mode = 0; mode <= 1; ++mode)
            for (int group = 8; group <= n && group <= 512; group *= 4) {
                const int64_t ng = rows * (n / group);
                uint8_t* codes = malloc((size_t)(rows * n * bits / 8) + 1);
                uint16_t* sc = malloc(sizeof(uint16_t) * (size_t)ng + 1);
                uint16_t* zr = malloc(sizeof(uint16_t) * (size_t)ng + 1);
                double* sp = malloc(sizeof(double) * (size_t)ng + 1);
                double* zp = malloc(sizeof(double) * (size_t)ng + 1);
                double* v = malloc(sizeof(double) * (size_t)(rows * n) + 1);
                EXPECT(bflyref_quantize(y, rows, n, group, bits, mode, 0, codes, sc,
                                        mode ? zr : NULL, sp, zp, v) == 0);
                for (int use = 1; use <= 2; ++use)
                    EXPECT(bflyref_quantize(y, rows, n, group, bits, mode, use, codes, sc,
                                            mode ? zr : NULL, NULL, NULL, NULL) == 0);
                for (int64_t i = 0; i < ng; ++i) {
                    EXPECT(sp[i] >= 0 && isfinite(bflyref_fp16_value(sc[i])));
                    if (mode) EXPECT(bflyref_fp16_value(zr[i]) >= 0 &&
                                     bflyref_fp16_value(zr[i]) <= (1 << bits) - 1);
                }
                free(codes); free(sc); free(zr); free(sp); free(zp); free(v);
            }
    free(xb);
    /* the Kronecker composite with three segments of this butterfly */
    float mix[9];
    for (int i = 0; i < 9; ++i) mix[i] = (float)uniform();
    double* yk = malloc(sizeof(double) * (size_t)(rows * 3 * n) + 1);
    float* xk = malloc(sizeof(float) * (size_t)(rows * 3 * n) + 1);
    for (int64_t i = 0; i < rows * 3 * n; ++i) xk[i] = (float)uniform();
    EXPECT(bflyref_kron_forward(xk, 0, yk, rows, 3, n, theta, mix) == 0);
    free(yk); free(xk);
    free(theta); free(x); free(g); free(y); free(y2); free(dx); free(dth); free(dabs);
}

static void invalid(void)
{
    float t[4] = {0};
    double d[64] = {0};
    uint8_t c[64];
    uint16_t s[8];
    EXPECT(bflyref_forward(NULL, 0, d, 1, 8, t) == -1);
    EXPECT(bflyref_forward(d, 0, d, -1, 8, t) == -1);
    EXPECT(bflyref_forward(d, 0, d, 1, 6, t) == -1);
    EXPECT(bflyref_forward(NULL, 0, NULL, 0, 8, NULL) == 0);
    EXPECT(bflyref_kron_forward(d, 0, d, 1, 0, 4, t, t) == -1);
    EXPECT(bflyref_quantize(d, 1, 8, 3, 4, 0, 0, c, s, NULL, NULL, NULL, NULL) == -1);
    EXPECT(bflyref_quantize(d, 1, 8, 8, 3, 0, 0, c, s, NULL, NULL, NULL, NULL) == -1);
    EXPECT(bflyref_quantize(d, 1, 8, 8, 4, 2, 0, c, s, NULL, NULL, NULL, NULL) == -1);
    EXPECT(bflyref_quantize(d, 1, 8, 8, 4, 1, 0, c, s, NULL, NULL, NULL, NULL) == -1);
    EXPECT(bflyref_quantize(d, 1, 8, 8, 4, 0, 3, c, s, NULL, NULL, NULL, NULL) == -1);
    EXPECT(bflyref_quantize(d, 0, 8, 8, 4, 0, 0, NULL, NULL, NULL, NULL, NULL, NULL) == 0);
    EXPECT(bflyref_backward((const float*)t, NULL, 1, 8, t, NULL, NULL, d, NULL) == -1);
    EXPECT(bflyref_backward(NULL, NULL, 0, 8, t, NULL, NULL, d, NULL) == 0);
}

int main(void)
{
    EXPECT(bflyref_num_threads() >= 1);
    bflyref_set_num_threads(1);
    rounding();
    invalid();
    const int sizes[] = {2, 4, 8, 64, 256};
    for (int i = 0; i < 5; ++i) {
        forward_backward(sizes[i], 1);
        forward_backward(sizes[i], 5);
    }
    if (failures) {
        fprintf(stderr, "%d failed checks\n", failures);
        return 1;
    }
    printf("oracle_san: all checks passed\n");
    return 0;
}
