/*
 * bakron_oracle.c -- plain, slow, fp64 CPU reference for BaKron rounding.
 *
 * TEST INFRASTRUCTURE ONLY. This file is compiled into a separate shared
 * library that only the tests, the smoke check and the benchmark's CPU
 * baseline load. It shares no code, header or constant table with the HIP
 * library, and the HIP library never links or calls it.
 *
 * What it computes (sources are the web pages this project follows):
 *
 *  - The two-sided adaptive rounding rule of YAQA/BoA that the BaKron solver
 *    schedules (YAQA article on news.43b.com.cn, section 4 "adaptive rounding
 *    with Kronecker-factored Hessians", rounding rule; "BaKron: Efficient
 *    Quantization with Kronecker-Factored Hessians", Abstract):
 *        W_ij = Q( W*_ij + a_i^T D[:i,:j] b_j + a_i^T D[:i,j] + D[i,:j] b_j ),
 *    with D = W* - W the error already committed, a_i column i of the
 *    strictly upper triangular m x m factor L_O and b_j column j of the
 *    strictly upper n x n factor L_I. ":i" means indices 0..i-1.
 *  - The LDL form H = (L + I) diag(D) (L + I)^T with L strictly upper
 *    (same article and section, the factorisation paragraph).
 *
 * Everything is fp64 except the per-row scales, which are defined in fp32.
 * Matrices are dense row-major; L_O is m x m, L_I is n x n and only their
 * strict upper triangles are read.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Counter-based uniform draws for stochastic rounding.                      */
/*                                                                           */
/* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number   */
/* generators", OOPSLA 2014): the k-th output (k = 1, 2, ...) of a stream    */
/* whose state starts at `seed` is mix(seed + k * gamma) with gamma the      */
/* 64-bit golden-ratio increment and mix the variant-13 finaliser. Entry     */
/* (i, j) of an m x n matrix takes the output with k = i*n + j + 1, so the   */
/* draw does not depend on the order in which entries are visited.          */
/* ------------------------------------------------------------------------ */
uint64_t orc_splitmix64(uint64_t seed, uint64_t idx) {
    uint64_t z = seed + (idx + 1u) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Top 24 bits as a uniform on [0, 1): exactly representable in fp32 too. */
double orc_uniform(uint64_t seed, uint64_t idx) {
    return (double)(orc_splitmix64(seed, idx) >> 40) * (1.0 / 16777216.0);
}

/* ------------------------------------------------------------------------ */
/* Base quantiser Q on the per-row symmetric grid s_i * (c - Lq/2),          */
/* c in {0..Lq}, Lq = 2^bits - 1. Nearest: c = floor(y + 1/2); stochastic:   */
/* c = floor(y + u); both clamped to [0, Lq]; y = t / s_i + Lq/2 is t in     */
/* grid steps. The margin is the distance (in steps) from y, or y + u, to   */
/* the nearest boundary between two representable codes.                   */
/* ------------------------------------------------------------------------ */
static int quant_code(double y, int Lq, int stochastic, double u, double* margin) {
    double c, b;
    if (stochastic) {
        /* boundaries between codes k-1 and k sit at y + u = k, k = 1..Lq */
        double v = y + u;
        c = floor(v);
        b = floor(v + 0.5);
        if (b < 1.0) b = 1.0;
        if (b > (double)Lq) b = (double)Lq;
        *margin = fabs(v - b);
    } else {
        /* boundaries between codes k and k+1 sit at y = k + 1/2, k = 0..Lq-1 */
        c = floor(y + 0.5);
        b = floor(y);                 /* nearest k + 1/2 is at k = round(y - 1/2) */
        if (b < 0.0) b = 0.0;
        if (b > (double)(Lq - 1)) b = (double)(Lq - 1);
        *margin = fabs(y - (b + 0.5));
    }
    if (c < 0.0) c = 0.0;
    if (c > (double)Lq) c = (double)Lq;
    return (int)c;
}

typedef struct {
    int bits;
    int stochastic;
    uint64_t seed;
    const double* u;   /* optional m x n override of the uniform draws */
} orc_quant;

/* Round one entry given its pre-rounding value t; returns 1 if clamped. */
static int round_entry(const orc_quant* qd, int64_t i, int64_t j, int64_t n, double t,
                       double s, float wstar, uint8_t* code, double* delta, double* eta,
                       double* margin) {
    int Lq = (1 << qd->bits) - 1;
    double y = t / s + 0.5 * Lq;
    double u = 0.0;
    if (qd->stochastic)
        u = qd->u ? qd->u[i * n + j] : orc_uniform(qd->seed, (uint64_t)(i * n + j));
    double mg;
    int c = quant_code(y, Lq, qd->stochastic, u, &mg);
    double q = s * ((double)c - 0.5 * Lq);
    *code = (uint8_t)c;
    *delta = (double)wstar - q;
    *eta = t - q;
    *margin = mg;
    double raw = qd->stochastic ? floor(y + u) : floor(y + 0.5);
    return (raw < 0.0 || raw > (double)Lq) ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Naive sweep: every entry's feedback is the rule's three sums written out, */
/* O(m^2 n^2) in total. Row-major visiting order.                            */
/* ------------------------------------------------------------------------ */
int orc_sweep_naive(int64_t m, int64_t n, const float* W, const double* LO, const double* LI,
                    const float* scales, int bits, int stochastic, uint64_t seed,
                    const double* u, uint8_t* codes, double* delta, double* tpre, double* eta,
                    double* margin, int64_t* clamped) {
    orc_quant qd = {bits, stochastic, seed, u};
    int64_t nclamp = 0;
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            /* a_i^T D[:i,:j] b_j */
            double t1 = 0.0;
            for (int64_t k = 0; k < i; ++k) {
                double aki = LO ? LO[k * m + i] : 0.0;
                if (aki == 0.0) continue;
                for (int64_t l = 0; l < j; ++l) t1 += aki * delta[k * n + l] * LI[l * n + j];
            }
            /* a_i^T D[:i,j] */
            double t2 = 0.0;
            for (int64_t k = 0; k < i; ++k) t2 += (LO ? LO[k * m + i] : 0.0) * delta[k * n + j];
            /* D[i,:j] b_j */
            double t3 = 0.0;
            for (int64_t l = 0; l < j; ++l) t3 += delta[i * n + l] * LI[l * n + j];
            double t = (double)W[i * n + j] + t1 + t2 + t3;
            tpre[i * n + j] = t;
            nclamp += round_entry(&qd, i, j, n, t, (double)scales[i], W[i * n + j],
                                  &codes[i * n + j], &delta[i * n + j], &eta[i * n + j],
                                  &margin[i * n + j]);
        }
    }
    *clamped = nclamp;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Accumulator sweep: the same rule and the same row-major order, with the   */
/* sums re-associated so that the work is O(mn(m+n)):                        */
/*   P_ij = sum_{k<i} L_O[k,i] D_kj   (column feedback, a GEMV per row)      */
/*   G_ij = P_ij + D_ij                                                      */
/*   t_ij = W*_ij + P_ij + sum_{l<j} G_il L_I[l,j]                           */
/* since sum_{l<j} (P_il + D_il) L_I[l,j] is the rule's first and third term. */
/* ------------------------------------------------------------------------ */
int orc_sweep_accum(int64_t m, int64_t n, const float* W, const double* LO, const double* LI,
                    const float* scales, int bits, int stochastic, uint64_t seed,
                    const double* u, uint8_t* codes, double* delta, double* tpre, double* eta,
                    double* margin, int64_t* clamped) {
    orc_quant qd = {bits, stochastic, seed, u};
    double* P = (double*)calloc((size_t)n, sizeof(double));
    double* acc = (double*)calloc((size_t)n, sizeof(double));
    if (!P || !acc) { free(P); free(acc); return 1; }
    int64_t nclamp = 0;
    for (int64_t i = 0; i < m; ++i) {
        /* P_i = sum_{k<i} L_O[k,i] D_k,: */
#pragma omp parallel for schedule(static)
        for (int64_t j0 = 0; j0 < n; j0 += 256) {
            int64_t j1 = j0 + 256 < n ? j0 + 256 : n;
            for (int64_t j = j0; j < j1; ++j) P[j] = 0.0;
            if (LO) {
                for (int64_t k = 0; k < i; ++k) {
                    double aki = LO[k * m + i];
                    if (aki == 0.0) continue;
                    const double* dk = delta + k * n;
                    for (int64_t j = j0; j < j1; ++j) P[j] += aki * dk[j];
                }
            }
        }
        memset(acc, 0, (size_t)n * sizeof(double));
        for (int64_t j = 0; j < n; ++j) {
            double t = (double)W[i * n + j] + P[j] + acc[j];
            tpre[i * n + j] = t;
            nclamp += round_entry(&qd, i, j, n, t, (double)scales[i], W[i * n + j],
                                  &codes[i * n + j], &delta[i * n + j], &eta[i * n + j],
                                  &margin[i * n + j]);
            double g = P[j] + delta[i * n + j];
            const double* lrow = LI + j * n;
            for (int64_t jj = j + 1; jj < n; ++jj) acc[jj] += g * lrow[jj];
        }
    }
    free(P);
    free(acc);
    *clamped = nclamp;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* H = (L + I) diag(D) (L + I)^T with L strictly upper, by the column        */
/* recurrence taken from the last index to the first:                        */
/*   D_j  = H_jj - sum_{k>j} L_jk^2 D_k                                      */
/*   L_ij = (H_ij - sum_{k>j} L_ik L_jk D_k) / D_j      (i < j)              */
/* Reads the upper triangle of H. Returns 2 and the index in *bad if a       */
/* pivot is not positive.                                                    */
/* ------------------------------------------------------------------------ */
int orc_udu(int64_t d, const double* H, double* L, double* D, int64_t* bad) {
    memset(L, 0, (size_t)(d * d) * sizeof(double));
    *bad = -1;
    for (int64_t j = d - 1; j >= 0; --j) {
        double dj = H[j * d + j];
        const double* lj = L + j * d;
        for (int64_t k = j + 1; k < d; ++k) dj -= lj[k] * lj[k] * D[k];
        if (!(dj > 0.0)) { *bad = j; return 2; }
        D[j] = dj;
#pragma omp parallel for schedule(static) if (j > 256)
        for (int64_t i = 0; i < j; ++i) {
            const double* li = L + i * d;
            double v = H[i * d + j];
            for (int64_t k = j + 1; k < d; ++k) v -= li[k] * lj[k] * D[k];
            L[i * d + j] = v / dj;
        }
    }
    return 0;
}
