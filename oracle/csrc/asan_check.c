/*
 * asan_check.c -- host memory-safety check of the oracle's C core.
 *
 * TEST INFRASTRUCTURE ONLY. tests/test_oracle_asan.py compiles this file
 * together with bakron_oracle.c under gcc's AddressSanitizer and
 * UndefinedBehaviorSanitizer and runs it: every entry point of the core is
 * called on small shapes, including the edges (one row, one column, an empty
 * matrix, no L_O, a factorisation that fails), so an out-of-bounds access or
 * undefined operation in the loops stops the run. It also checks that the
 * naive and the accumulator sweeps agree code for code, which holds because
 * both evaluate the same rounding rule in the same order (YAQA article on
 * news.43b.com.cn, section 4, rounding rule).
 *
 * The inputs come from a small linear congruential generator of its own and
 * carry none of the method's arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint64_t orc_splitmix64(uint64_t seed, uint64_t idx);
double orc_uniform(uint64_t seed, uint64_t idx);
int orc_sweep_naive(int64_t m, int64_t n, const float* W, const double* LO, const double* LI,
                    const float* scales, int bits, int stochastic, uint64_t seed,
                    const double* u, uint8_t* codes, double* delta, double* tpre, double* eta,
                    double* margin, int64_t* clamped);
int orc_sweep_accum(int64_t m, int64_t n, const float* W, const double* LO, const double* LI,
                    const float* scales, int bits, int stochastic, uint64_t seed,
                    const double* u, uint8_t* codes, double* delta, double* tpre, double* eta,
                    double* margin, int64_t* clamped);
int orc_udu(int64_t d, const double* H, double* L, double* D, int64_t* bad);

static uint64_t lcg_state = 12345u;
static double lcg(void) { /* uniform on [-1, 1) */
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg_state >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

/* exact-size heap buffers, so that any overrun lands in a redzone */
static void* xalloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(3); }
    return p;
}

/* An SPD matrix B B^T / d + I of order d, then its factor's strict upper part. */
static int factor(int64_t d, double** L_out) {
    double* B = xalloc(sizeof(double) * (size_t)(d * d));
    double* H = xalloc(sizeof(double) * (size_t)(d * d));
    double* L = xalloc(sizeof(double) * (size_t)(d * d));
    double* D = xalloc(sizeof(double) * (size_t)d);
    for (int64_t i = 0; i < d * d; ++i) B[i] = lcg();
    for (int64_t i = 0; i < d; ++i)
        for (int64_t j = 0; j < d; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < d; ++k) s += B[i * d + k] * B[j * d + k];
            H[i * d + j] = s / (double)d + (i == j ? 1.0 : 0.0);
        }
    int64_t bad = 0;
    int rc = orc_udu(d, H, L, D, &bad);
    free(B);
    free(H);
    free(D);
    if (rc != 0) { free(L); return 1; }
    *L_out = L;
    return 0;
}

static int sweep_case(int64_t m, int64_t n, int bits, int stochastic, int one_sided) {
    double* LO = NULL;
    double* LI = NULL;
    if (!one_sided && m > 0 && factor(m, &LO)) return 1;
    if (n > 0 && factor(n, &LI)) return 1;
    const size_t mn = (size_t)(m * n);
    float* W = xalloc(sizeof(float) * mn);
    float* s = xalloc(sizeof(float) * (size_t)m);
    for (size_t i = 0; i < mn; ++i) W[i] = (float)(0.02 * lcg());
    for (int64_t i = 0; i < m; ++i) {
        float a = 0.0f;
        for (int64_t j = 0; j < n; ++j) a = fmaxf(a, fabsf(W[i * n + j]));
        s[i] = a > 0.0f ? 2.0f * a / (float)((1 << bits) - 1) : 1.0f;
    }
    uint8_t* c[2];
    double* buf[2][4];
    int64_t clamped[2];
    for (int v = 0; v < 2; ++v) {
        c[v] = xalloc(mn);
        for (int b = 0; b < 4; ++b) {
            buf[v][b] = xalloc(sizeof(double) * mn);
            memset(buf[v][b], 0, sizeof(double) * mn);
        }
    }
    int rc = orc_sweep_naive(m, n, W, LO, LI, s, bits, stochastic, 7u, NULL, c[0], buf[0][0], buf[0][1],
                             buf[0][2], buf[0][3], &clamped[0]);
    rc |= orc_sweep_accum(m, n, W, LO, LI, s, bits, stochastic, 7u, NULL, c[1], buf[1][0], buf[1][1],
                          buf[1][2], buf[1][3], &clamped[1]);
    int diff = 0;
    for (size_t i = 0; i < mn; ++i) diff += c[0][i] != c[1][i];
    if (rc || diff || clamped[0] != clamped[1]) {
        fprintf(stderr, "sweep %lldx%lld bits=%d stoch=%d one_sided=%d: rc=%d, %d code differences\n",
                (long long)m, (long long)n, bits, stochastic, one_sided, rc, diff);
        rc = 1;
    }
    for (int v = 0; v < 2; ++v) {
        free(c[v]);
        for (int b = 0; b < 4; ++b) free(buf[v][b]);
    }
    free(W);
    free(s);
    free(LO);
    free(LI);
    return rc;
}

int main(void) {
    int fails = 0;
    /* shapes: square, tall, wide, one row, one column, a single entry, empty */
    const int64_t shapes[][2] = {{9, 9}, {13, 6}, {5, 17}, {1, 12}, {11, 1}, {1, 1}, {0, 4}, {4, 0}};
    for (size_t k = 0; k < sizeof(shapes) / sizeof(shapes[0]); ++k)
        for (int bits = 2; bits <= 4; bits += 2)
            for (int st = 0; st < 2; ++st)
                for (int os = 0; os < 2; ++os) fails += sweep_case(shapes[k][0], shapes[k][1], bits, st, os);
    /* a factorisation that must fail: the negative of an SPD matrix */
    {
        const int64_t d = 6;
        double* H = xalloc(sizeof(double) * (size_t)(d * d));
        double* L = xalloc(sizeof(double) * (size_t)(d * d));
        double* D = xalloc(sizeof(double) * (size_t)d);
        for (int64_t i = 0; i < d * d; ++i) H[i] = (i % (d + 1) == 0) ? -1.0 : 0.0;
        int64_t bad = 0;
        if (orc_udu(d, H, L, D, &bad) != 2 || bad != d - 1) {
            fprintf(stderr, "failing factorisation not reported (bad=%lld)\n", (long long)bad);
            ++fails;
        }
        free(H);
        free(L);
        free(D);
    }
    /* the counter-based draws at the ends of the index range */
    double u = orc_uniform(~0ull, ~0ull - 1u) + orc_uniform(0u, 0u) + (double)(orc_splitmix64(1u, 2u) & 1u);
    if (!(u >= 0.0 && u < 3.0)) ++fails;
    if (fails) {
        fprintf(stderr, "%d failing cases\n", fails);
        return 1;
    }
    printf("asan_check ok\n");
    return 0;
}
