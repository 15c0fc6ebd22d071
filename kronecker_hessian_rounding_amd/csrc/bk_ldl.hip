// bk_ldl.hip -- damped LDL factorisation H + lambda I = (L + I) diag(D) (L + I)^T,
// L strictly upper (YAQA article, section 4, the factorisation paragraph;
// damping lambda = damp_rel * mean(diag H) as the factor estimates carry it,
// K-FAC tutorial on mlqm.cn, section 5).
//
// With J the index reversal, J H J = C' C'^T (lower Cholesky) gives H = C C^T
// with C = J C' J upper triangular; then L + I = C diag(C)^-1 and D = diag(C)^2.
// C is computed in fp64 by a right-looking blocked Cholesky that runs from the
// LAST 64-wide index block to the first. The working copy A holds the lower
// triangle (A[r][c] = H[r][c], r >= c), so a factored block column of C is
// stored as a block ROW of A (C^T), contiguous along the long index. Every
// contraction then has the "TN" form of bk_common.hpp (both operands K-major):
//   diag  : C22 = reverse Cholesky of the 64x64 diagonal block, and C22^-1
//   panel : C12^T = C22^-1 A[k0:k1, 0:k0]           (MFMA, in place)
//   inner : A[s0:k0, 0:k0] -= C12 C12^T restricted to the current 512-wide
//           super-panel's rows                        (MFMA, lower part)
//   outer : after each super-panel, A[0:s0, 0:s0] -= C_S C_S^T with
//           K = the super-panel width                 (MFMA, lower part)
// Orders up to 8192 take the same steps in one persistent launch (k_ldl_sched,
// one factor or a layer's two), scheduled per 64x64 tile; larger orders run them
// as a chain of launches, one per step.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>

#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

constexpr int kSuper = 512;  // super-panel width (K of the big trailing updates)
constexpr int kLdlKT = 32;   // k-slice depth of the fp64 panel / inner-update GEMMs (K = 64) and
                             // of the scheduled path's tile tasks; the wide outer updates use 16

struct LdlWs {
    double* A;     // d x d working copy, lower triangle used, ld = d
    double* Wt;    // one 64 x 64 slot per block: Wt[q][p] = (C22^-1)[p][q] of that diagonal block
    double* lam;   // damping lambda
    int64_t* info; // -1, the first failing pivot index, or -2 (a wait of the scheduled path timed out)
    int* cnt;      // scheduled path: one progress counter per 64x64 tile of A (nb x nb)
    int* ticket;   // scheduled path: next task ticket
    int* abort;    // scheduled path: nonzero once any workgroup gives up
};

static int64_t ldl_blocks(int64_t d) { return (d + kTile - 1) / kTile; }

static LdlWs carve(void* ws, int64_t d) {
    const size_t nb = (size_t)ldl_blocks(d);
    char* p = (char*)ws;
    LdlWs w;
    w.A = (double*)p;
    p += align256(sizeof(double) * (size_t)d * (size_t)d);
    w.Wt = (double*)p;
    p += align256(sizeof(double) * 4096 * nb);
    w.lam = (double*)p;
    p += 256;
    w.info = (int64_t*)p;
    p += 256;
    w.ticket = (int*)p;
    w.abort = w.ticket + 1;
    p += 256;
    w.cnt = (int*)p;
    return w;
}

size_t ldl_workspace_bytes(int64_t d) {
    const size_t nb = (size_t)ldl_blocks(d);
    return align256(sizeof(double) * (size_t)d * (size_t)d) + align256(sizeof(double) * 4096 * nb) +
           3 * 256 + align256(sizeof(int) * nb * nb);
}

// lambda = damp_rel * mean(diag H) in fp64; info = -1; the scheduler's ticket and abort flag 0.
__global__ __launch_bounds__(kThreads) void k_ldl_init(const float* __restrict__ H, int64_t d,
                                                       int64_t ldh, double damp_rel, LdlWs w) {
    __shared__ double red[kThreads];
    // thread t sums the diagonal entries t, t + 256, ... in that order, loading a batch
    // of them at once (each lies on a line of its own)
    constexpr int kIn = 16;
    double s = 0.0;
    for (int64_t i0 = threadIdx.x; i0 < d; i0 += (int64_t)kIn * kThreads) {
        float v[kIn];
#pragma unroll
        for (int u = 0; u < kIn; ++u) {
            const int64_t i = i0 + (int64_t)u * kThreads;
            v[u] = i < d ? H[i * ldh + i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kIn; ++u)
            if (i0 + (int64_t)u * kThreads < d) s += (double)v[u];
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        *w.lam = damp_rel * (red[0] / (double)d);
        *w.info = -1;
        *w.ticket = 0;
        *w.abort = 0;
    }
}

// A[r][c] = H[c][r] (upper triangle of H read, lower triangle of A written),
// plus lambda on the diagonal; 64x64 tiles transposed through LDS. Each tile's
// progress counter starts at 0. Whole tiles of an H with 16-byte aligned rows (and
// an even order, for A's rows) move in 16-byte pieces, every load in flight; the
// strict upper part of a diagonal tile of A is then written as zeros (A's upper
// triangle is never read). Other tiles go element by element.
__global__ __launch_bounds__(kThreads) void k_ldl_load(const float* __restrict__ H, int64_t d,
                                                       int64_t ldh, LdlWs w) {
    const int64_t rt = blockIdx.y, ct = blockIdx.x;  // tile of A: rows rt, cols ct, rt >= ct
    if (ct > rt) return;
    const int t = threadIdx.x;
    if (t == 0) w.cnt[rt * gridDim.x + ct] = 0;
    __shared__ float tile[kTile][kTile + 1];
    const int64_t r0 = rt * kTile, c0 = ct * kTile;
    const bool vec = r0 + kTile <= d && (ldh & 3) == 0 && (d & 1) == 0 &&
                     (reinterpret_cast<uintptr_t>(H) & 15) == 0;
    constexpr int kV4 = kTile * kTile / 4 / kThreads, kV2 = kTile * kTile / 2 / kThreads;
    if (vec) {
        // H rows c0 + a, columns r0 + b4 .. r0 + b4 + 3 (c0 <= r0: the columns exist too)
        f32x4 v[kV4];
#pragma unroll
        for (int u = 0; u < kV4; ++u) {
            const int q = t + u * kThreads;
            v[u] = *reinterpret_cast<const f32x4*>(H + (c0 + (q >> 4)) * ldh + r0 + ((q & 15) << 2));
        }
#pragma unroll
        for (int u = 0; u < kV4; ++u) {
            const int q = t + u * kThreads;
            const int a = q >> 4, b4 = (q & 15) << 2;
#pragma unroll
            for (int e = 0; e < 4; ++e) tile[a][b4 + e] = (rt > ct || a <= b4 + e) ? v[u][e] : 0.0f;
        }
    } else {
        for (int e = t; e < kTile * kTile; e += kThreads) {
            const int a = e / kTile, b = e % kTile;  // H row c0 + a, col r0 + b
            const int64_t hr = c0 + a, hc = r0 + b;
            tile[a][b] = (hr < d && hc < d && hr <= hc) ? H[hr * ldh + hc] : 0.0f;
        }
    }
    __syncthreads();
    const double lam = *w.lam;
    if (vec) {
#pragma unroll
        for (int u = 0; u < kV2; ++u) {
            const int q = t + u * kThreads;
            const int a = q >> 5, b2 = (q & 31) << 1;  // A row r0 + a, cols c0 + b2, +1
            f64x2 x = {(double)tile[b2][a], (double)tile[b2 + 1][a]};
            if (rt == ct) {
                if (a == b2) x[0] += lam;
                if (a == b2 + 1) x[1] += lam;
            }
            *reinterpret_cast<f64x2*>(w.A + (r0 + a) * d + c0 + b2) = x;
        }
    } else {
        for (int e = t; e < kTile * kTile; e += kThreads) {
            const int a = e / kTile, b = e % kTile;  // A row r0 + a, col c0 + b
            const int64_t r = r0 + a, c = c0 + b;
            if (r >= d || c > r) continue;
            double v = (double)tile[b][a];
            if (r == c) v += lam;
            w.A[r * d + c] = v;
        }
    }
}

// Reverse Cholesky of the diagonal block and the inverse of its factor.
// The block is held in LDS as the upper matrix u[i][j] = A[k0 + j][k0 + i]
// (i <= j), padded with the identity beyond nb, and factored in 16-wide block
// columns from the last. Wave 0 factors a block column with one lane per row:
// the pivot and the scaled column entries move between lanes by readlane, so
// the 16 columns of a block need no barrier. Each column first updates the
// next column and starts that pivot's reciprocal square root, then applies the
// rest of its rank-1 update, so the pivot chain overlaps the bulk of the work.
// All four waves then apply the rank-16 update to the block columns on its
// left with f64 MFMA. The inverse X = C^-1 is formed blockwise by waves 1-3
// while wave 0 factors the next block column, each block as soon as what it
// reads is final:
//   X[B][B]: back substitution on the 16x16 diagonal block (one wave),
//   X[I][J] = -X[I][I] sum_{I<Q<=J} C[I][Q] X[Q][J], J > I (MFMA, one wave).
// A pivot that is not positive and finite gives a reciprocal square root that
// is not positive and finite, and turns every later pivot into NaN, so the
// first failing pivot in factorisation order is the highest index whose
// 1 / C[j][j] is bad.
__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const long long b = __builtin_bit_cast(long long, v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), lane);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

// 1 / sqrt(x): the hardware estimate y, then y (1 + e/2 + 3 e^2 / 8) with e = 1 - x y^2,
// which leaves a relative error of order e^3 (below double rounding)
__device__ __forceinline__ double rsqrt_f64(double x) {
    const double y = __builtin_amdgcn_rsq(x);
    const double e = fma(-x * y, y, 1.0);
    return fma(y * e, fma(e, 0.375, 0.5), y);
}

constexpr int kUs = 65;  // LDS row stride (doubles) of the diagonal-block tiles

struct DiagSmem {
    double u[64][kUs];   // C, upper part
    double xs[64][kUs];  // X = C^-1, upper part
    double rcd[64];      // 1 / C[j][j]
    int badj;
};

// wave 0: factor block column b (columns 16b .. 16b+15), lane = row
template <int b>
__device__ __forceinline__ void ldl_factor_bcol(DiagSmem& s, int lane) {
    double r[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) r[q] = s.u[lane][16 * b + q];
    double rcs[16];
    double rc = rsqrt_f64(readlane_f64(r[15], 16 * b + 15));
#pragma unroll
    for (int jl = 15; jl >= 0; --jl) {
        const int jj = 16 * b + jl;
        rcs[jl] = rc;
        const double v = lane <= jj ? r[jl] * rc : 0.0;  // C[lane][jj]
        r[jl] = v;
        if (jl > 0) {  // the next column first: its pivot starts the next step's chain
            r[jl - 1] = fma(-v, readlane_f64(v, jj - 1), r[jl - 1]);
            rc = rsqrt_f64(readlane_f64(r[jl - 1], jj - 1));
        }
#pragma unroll
        for (int q = jl - 2; q >= 0; --q) r[q] = fma(-v, readlane_f64(v, 16 * b + q), r[q]);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) s.u[lane][16 * b + q] = r[q];
    if (lane == 0) {
#pragma unroll
        for (int q = 0; q < 16; ++q) s.rcd[16 * b + q] = rcs[q];
    }
}

// u[0:16b, 0:16b] -= P P^T with P = u[0:16b, 16b:16b+16], 16x16 tiles (I, K), I <= K
__device__ __forceinline__ void ldl_trailing(DiagSmem& s, int b, int wv, int lane) {
    for (int tile = wv; tile < b * (b + 1) / 2; tile += 4) {
        int I = 0, K = tile;
        while (K >= b - I) {
            K -= b - I;
            ++I;
        }
        K += I;
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int kq = 16 * b + 4 * kk + (lane >> 4);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(s.u[16 * I + (lane & 15)][kq],
                                                       s.u[16 * K + (lane & 15)][kq], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) s.u[16 * I + (lane >> 4) + 4 * r][16 * K + (lane & 15)] -= acc[r];
    }
}

// X[B][B]: lane k (mod 16) solves column k of the inverse of the 16x16 diagonal block by
// column-oriented back substitution: once x[m] is known it is removed from every
// equation above it, so the dependent chain is two operations per row
__device__ __forceinline__ void ldl_inv_diag(DiagSmem& s, int B, int lane) {
    const int B0 = 16 * B;
    const int k = lane & 15;
    double cu[16][16];  // C[B0 + q][B0 + m], q < m (upper part of the block)
#pragma unroll
    for (int m = 1; m < 16; ++m)
#pragma unroll
        for (int q = 0; q < m; ++q) cu[q][m] = s.u[B0 + q][B0 + m];
    double rc[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) rc[m] = s.rcd[B0 + m];
    double rhs[16], xl[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) rhs[m] = (m == k) ? 1.0 : 0.0;
#pragma unroll
    for (int m = 15; m >= 0; --m) {
        xl[m] = rhs[m] * rc[m];
#pragma unroll
        for (int q = m - 1; q >= 0; --q) rhs[q] = fma(-cu[q][m], xl[m], rhs[q]);
    }
    if (lane < 16) {
#pragma unroll
        for (int m = 0; m < 16; ++m) s.xs[B0 + m][B0 + k] = xl[m];
    }
}

// X[I][J] = -X[I][I] T, T = sum_{I<Q<=J} C[I][Q] X[Q][J]
__device__ __forceinline__ void ldl_inv_off(DiagSmem& s, int I, int J, int lane) {
    f64x4 tacc = {0.0, 0.0, 0.0, 0.0};
    for (int Q = I + 1; Q <= J; ++Q) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int kq = 4 * kk + (lane >> 4);
            tacc = __builtin_amdgcn_mfma_f64_16x16x4f64(s.u[16 * I + (lane & 15)][16 * Q + kq],
                                                        s.xs[16 * Q + kq][16 * J + (lane & 15)], tacc,
                                                        0, 0, 0);
        }
    }
    // tacc[kk] holds T[4 kk + lane / 16][lane % 16]: the B operand of k-step kk
    f64x4 xacc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        xacc = __builtin_amdgcn_mfma_f64_16x16x4f64(s.xs[16 * I + (lane & 15)][16 * I + 4 * kk + (lane >> 4)],
                                                    tacc[kk], xacc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) s.xs[16 * I + (lane >> 4) + 4 * r][16 * J + (lane & 15)] = -xacc[r];
}

// u[i][j] -= sum_p xs[p][i] xs[p][j] on and above the diagonal: the update of the
// block by the 64 rows held in xs (rows of the panel block just formed below it,
// zero past its last row). 32x32 quadrants, one wave each, K = 64.
__device__ __forceinline__ void diag_syrk(DiagSmem& s, int wv, int lane) {
    const int qi = wv >> 1, qj = wv & 1;
    if (qi > qj) return;
    const int ra = 32 * qi + (lane & 15), rb = 32 * qj + (lane & 15);
    const int kq = lane >> 4;
    f64x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int kk = 0; kk < 16; ++kk) {
        const int p = 4 * kk + kq;
        const double fa0 = s.xs[p][ra], fa1 = s.xs[p][ra + 16];
        const double fb0 = s.xs[p][rb], fb1 = s.xs[p][rb + 16];
        acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa0, fb0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa0, fb1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa1, fb0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa1, fb1, acc[1][1], 0, 0, 0);
    }
    // output layout: row = 16 bi + lane / 16 + 4 r, column = 16 bj + lane % 16
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 32 * qi + 16 * bi + (lane >> 4) + 4 * r;
                const int j = 32 * qj + 16 * bj + (lane & 15);
                if (i <= j) s.u[i][j] -= acc[bi][bj][r];
            }
}

// Factors the block held in s.u (identity past its nb rows) into C22 (left in
// s.u, upper part) and X = C22^-1 (s.xs, upper part). Returns -1, or the local
// index of the first failing pivot (uniform across the workgroup; the inverse
// is then incomplete). Starts and ends with every wave at a barrier.
__device__ __forceinline__ int diag_factor(DiagSmem& s, int nb, int wv, int lane) {
    // block column 3
    if (wv == 0) ldl_factor_bcol<3>(s, lane);
    __syncthreads();
    ldl_trailing(s, 3, wv, lane);
    __syncthreads();
    // block column 2; X[3][3] alongside
    if (wv == 0) ldl_factor_bcol<2>(s, lane);
    else if (wv == 1) ldl_inv_diag(s, 3, lane);
    __syncthreads();
    ldl_trailing(s, 2, wv, lane);
    __syncthreads();
    // block column 1; X[2][2] alongside
    if (wv == 0) ldl_factor_bcol<1>(s, lane);
    else if (wv == 1) ldl_inv_diag(s, 2, lane);
    __syncthreads();
    ldl_trailing(s, 1, wv, lane);
    __syncthreads();
    // block column 0; X[1][1] and X[2][3] alongside
    if (wv == 0) ldl_factor_bcol<0>(s, lane);
    else if (wv == 1) ldl_inv_diag(s, 1, lane);
    else if (wv == 2) ldl_inv_off(s, 2, 3, lane);
    __syncthreads();
    // X[0][0], X[1][2], X[1][3]; wave 0 looks for a failed pivot
    if (wv == 0) {
        const bool bad = lane < nb && !(s.rcd[lane] > 0.0 && s.rcd[lane] < INFINITY);
        const unsigned long long m = __ballot(bad);
        if (lane == 0) s.badj = m ? 63 - __clzll((long long)m) : -1;
    } else if (wv == 1) {
        ldl_inv_diag(s, 0, lane);
    } else if (wv == 2) {
        ldl_inv_off(s, 1, 2, lane);
    } else {
        ldl_inv_off(s, 1, 3, lane);
    }
    __syncthreads();
    const int badj = s.badj;
    if (badj >= 0) return badj;
    // X[0][1], X[0][2], X[0][3]
    if (wv > 0) ldl_inv_off(s, 0, wv, lane);
    __syncthreads();
    return -1;
}

// With pn, the block first takes the update of the panel block just formed below it:
// u[i][j] -= sum_{p < np} pn[p d + i] pn[p d + j] (np rows of C12^T, the block's 64 columns).
__device__ __forceinline__ void diag_body(int64_t d, int64_t k0, int nb, const LdlWs& w, DiagSmem& s,
                                          const double* pn = nullptr, int np = 0) {
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wv = t >> 6;
    {
        // the block, the panel rows and the status word in flight together
        constexpr int kPer = 64 * 64 / kThreads;
        double v[kPer], pv[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int e = t + r * kThreads;
            const int i = e & 63, j = e >> 6;
            v[r] = (i <= j && j < nb) ? w.A[(k0 + j) * d + k0 + i] : (i == j ? 1.0 : 0.0);
            pv[r] = (pn && j < np) ? pn[j * d + i] : 0.0;  // row j of the panel, column i
        }
        if (*w.info >= 0) return;  // an earlier block failed
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int e = t + r * kThreads;
            s.u[e & 63][e >> 6] = v[r];
            s.xs[e >> 6][e & 63] = pv[r];  // xs is free until the inverse
        }
    }
    __syncthreads();
    if (pn) {
        diag_syrk(s, wv, lane);
        __syncthreads();
    }
    const int badj = diag_factor(s, nb, wv, lane);
    if (badj >= 0) {
        if (t == 0) *w.info = k0 + badj;
        return;
    }

    // C22 back into A (lower storage: A[k0 + j][k0 + i] = C[i][j]); Wt[j][i] = X[i][j].
    // Every LDS read of the thread first, then the stores.
    constexpr int kPer = 64 * 64 / kThreads;
    double cv[kPer], xv[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int e = t + r * kThreads;
        const int i = e & 63, j = e >> 6;
        cv[r] = s.u[i][j];
        xv[r] = (i <= j) ? s.xs[i][j] : 0.0;
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int e = t + r * kThreads;
        const int i = e & 63, j = e >> 6;
        if (i <= j && j < nb) w.A[(k0 + j) * d + k0 + i] = cv[r];
        w.Wt[e] = xv[r];
    }
}

__global__ __launch_bounds__(kThreads) void k_ldl_diag(int64_t d, int64_t k0, int nb, LdlWs w) {
    __shared__ DiagSmem s;
    diag_body(d, k0, nb, w, s);
}

// C12^T[p][r] = sum_q (C22^-1)[p][q] A[k0 + q][r] for r in this workgroup's 64
// columns (r < k0), written back in place into A[k0 + p][r].
__global__ __launch_bounds__(kThreads) void k_ldl_panel(int64_t d, int64_t k0, int nb, LdlWs w) {
    if (*w.info >= 0) return;
    __shared__ GemmSmemF64<kLdlKT> sm;
    const int64_t r0 = (int64_t)blockIdx.x * kTile;
    const int Cn = (int)min<int64_t>(kTile, k0 - r0);
    f64x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    tile_gemm_f64<kLdlKT>(w.Wt, 64, nb, w.A + k0 * d + r0, d, Cn, nb, acc, sm);
    // every read of this workgroup's columns is complete (the tile loop ends in a barrier)
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pr = acc64_row(bi, r), rc = acc64_col(bj);
                if (pr < nb && rc < Cn) w.A[(k0 + pr) * d + r0 + rc] = acc[bi][bj][r];
            }
}

// One 64x64 tile (rows r0.., columns c0..) of A[r][c] -= sum_{q < K} A[q0 + q][r] A[q0 + q][c],
// rows below r_hi, columns below c_hi, lower triangle only (c <= r).
template <int KT>
__device__ __forceinline__ void update_tile(int64_t d, int64_t r0, int64_t r_hi, int64_t c0,
                                            int64_t c_hi, int64_t q0, int64_t K, const LdlWs& w,
                                            GemmSmemF64<KT>& sm) {
    const int R = (int)min<int64_t>(kTile, r_hi - r0);
    const int Cn = (int)min<int64_t>(kTile, c_hi - c0);
    f64x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    const double* P = w.A + q0 * d;
    tile_gemm_f64<KT>(P + r0, d, R, P + c0, d, Cn, K, acc, sm);
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lr = acc64_row(bi, r), lc = acc64_col(bj);
                const int64_t gi = r0 + lr, gj = c0 + lc;
                if (lr < R && lc < Cn && gj <= gi) w.A[gi * d + gj] -= acc[bi][bj][r];
            }
}

// The outer update A[r][c] -= sum_{q < K} A[q0 + q][r] A[q0 + q][c] over the lower
// triangle of [0, n) x [0, n), in 128 x 64 tiles of eight waves (4 x 2, each a 32 x 32
// quadrant of 2 x 2 MFMA blocks), grouped in squares of 4 x 8 tiles (512 x 512).
// Workgroups are dealt to the XCDs in turn (workgroup u to XCD u % 8), so square q
// goes to the workgroups of one XCD (those with u % 8 == q % 8): the panel columns
// that a square's tiles share are fetched into that XCD's L2 and reused there.
constexpr int kOutM = 128, kOutN = 64, kOutKT = 16, kOutThreads = 512;
constexpr int kSqR = 4, kSqC = 8;  // tiles per square: rows, columns (512 x 512 elements)
constexpr int kXcds = 8;

struct OuterSmem {
    double a[2][kOutKT][kOutM];
    double b[2][kOutKT][kOutN];
};

// rows k0 .. k0 + kOutKT - 1 of a W-wide panel: thread t loads 16-byte pairs (rows
// t / (W/2) + (512 / (W/2)) u, columns 2 (t % (W/2)), +1); zeros outside [0, K) x [0, R).
// kFast: a full width and 16-byte aligned rows (rows past K clamped here, zeroed by the store).
template <int W, bool kFast>
__device__ __forceinline__ void outer_load(const double* __restrict__ A, int64_t lda, int R, int64_t K,
                                           int64_t k0, f64x2 (&v)[kOutKT * W / 2 / kOutThreads], int t) {
    constexpr int PR = W / 2, RPP = kOutThreads / PR;
#pragma unroll
    for (int u = 0; u < kOutKT * W / 2 / kOutThreads; ++u) {
        const int64_t k = k0 + t / PR + RPP * u;
        const int c2 = (t % PR) * 2;
        if (kFast) {
            v[u] = *reinterpret_cast<const f64x2*>(A + min(k, K - 1) * lda + c2);
        } else {
            const double* p = A + k * lda + c2;
#pragma unroll
            for (int e = 0; e < 2; ++e) v[u][e] = (k < K && c2 + e < R) ? p[e] : 0.0;
        }
    }
}
template <int W>
__device__ __forceinline__ void outer_store(double (&dst)[kOutKT][W], const f64x2 (&v)[kOutKT * W / 2 / kOutThreads],
                                            int64_t K, int64_t k0, int t) {
    constexpr int PR = W / 2, RPP = kOutThreads / PR;
#pragma unroll
    for (int u = 0; u < kOutKT * W / 2 / kOutThreads; ++u) {
        const int r = t / PR + RPP * u;
        *reinterpret_cast<f64x2*>(&dst[r][(t % PR) * 2]) = k0 + r < K ? v[u] : f64x2{0.0, 0.0};
    }
}

template <bool kFast>
__device__ __forceinline__ void outer_gemm(const double* __restrict__ A, int R, const double* __restrict__ B, int Cn,
                                           int64_t lda, int64_t K, f64x4 (&acc)[2][2], OuterSmem& sm, int t) {
    const int lane = t & 63, wv = t >> 6;
    const int ra = (wv >> 1) * 32 + (lane & 15), rb = (wv & 1) * 32 + (lane & 15), kq = lane >> 4;
    f64x2 va[kOutKT * kOutM / 2 / kOutThreads], vb[kOutKT * kOutN / 2 / kOutThreads];
    outer_load<kOutM, kFast>(A, lda, R, K, 0, va, t);
    outer_load<kOutN, kFast>(B, lda, Cn, K, 0, vb, t);
    outer_store<kOutM>(sm.a[0], va, K, 0, t);
    outer_store<kOutN>(sm.b[0], vb, K, 0, t);
    __syncthreads();
    const int64_t nk = (K + kOutKT - 1) / kOutKT;
    for (int64_t it = 0; it < nk; ++it) {
        const int cur = (int)(it & 1);
        const bool more = it + 1 < nk;
        if (more) {
            outer_load<kOutM, kFast>(A, lda, R, K, (it + 1) * kOutKT, va, t);
            outer_load<kOutN, kFast>(B, lda, Cn, K, (it + 1) * kOutKT, vb, t);
        }
#pragma unroll
        for (int s = 0; s < kOutKT / 4; ++s) {
            const int kr = 4 * s + kq;
            const double fa0 = sm.a[cur][kr][ra], fa1 = sm.a[cur][kr][ra + 16];
            const double fb0 = sm.b[cur][kr][rb], fb1 = sm.b[cur][kr][rb + 16];
            acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa0, fb0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa0, fb1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa1, fb0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa1, fb1, acc[1][1], 0, 0, 0);
        }
        if (more) {
            outer_store<kOutM>(sm.a[cur ^ 1], va, K, (it + 1) * kOutKT, t);
            outer_store<kOutN>(sm.b[cur ^ 1], vb, K, (it + 1) * kOutKT, t);
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kOutThreads) void k_ldl_outer(int64_t d, int64_t n, int64_t q0, int64_t K, int nsq,
                                                           LdlWs w) {
    if (*w.info >= 0) return;
    const int u = blockIdx.x;
    constexpr int kPerSq = kSqR * kSqC;
    const int q = (u / kXcds / kPerSq) * kXcds + u % kXcds;
    if (q >= nsq) return;
    const int loc = (u / kXcds) % kPerSq;
    // square q = (I, J), J <= I, in row order of the lower triangle of squares
    int I = (int)((sqrt(8.0 * (double)q + 1.0) - 1.0) * 0.5);
    while (I * (I + 1) / 2 > q) --I;
    while ((I + 1) * (I + 2) / 2 <= q) ++I;
    const int J = q - I * (I + 1) / 2;
    const int64_t r0 = (int64_t)I * (kSqR * kOutM) + (loc / kSqC) * kOutM;
    const int64_t c0 = (int64_t)J * (kSqC * kOutN) + (loc % kSqC) * kOutN;
    if (r0 >= n || c0 >= n || c0 > r0 + kOutM - 1) return;  // past the edge, or above the diagonal
    const int R = (int)min<int64_t>(kOutM, n - r0), Cn = (int)min<int64_t>(kOutN, n - c0);
    __shared__ OuterSmem sm;
    const int t = tid_opaque();
    f64x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    const double* P = w.A + q0 * d;
    const bool fast = R == kOutM && Cn == kOutN && (d & 1) == 0 && (reinterpret_cast<uintptr_t>(w.A) & 15) == 0;
    if (fast) outer_gemm<true>(P + r0, R, P + c0, Cn, d, K, acc, sm, t);
    else outer_gemm<false>(P + r0, R, P + c0, Cn, d, K, acc, sm, t);
    const int lane = t & 63, wv = t >> 6;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lr = (wv >> 1) * 32 + 16 * bi + (lane >> 4) + 4 * r;
                const int lc = (wv & 1) * 32 + 16 * bj + (lane & 15);
                const int64_t gi = r0 + lr, gj = c0 + lc;
                if (lr < R && lc < Cn && gj <= gi) w.A[gi * d + gj] -= acc[bi][bj][r];
            }
}

// Workgroup 0 applies the update of the block just panelled (K rows at q0) to the
// diagonal block at kn (64 wide) and factors it; the others apply the same block's
// inner update to rows [r_lo, r_hi) x columns [0, c_hi), in a ct-wide grid of
// tiles, all but the tile (kn, kn). The two parts touch disjoint parts of A.
__global__ __launch_bounds__(kThreads) void k_ldl_diag_update(int64_t d, int64_t kn, int64_t r_lo,
                                                              int64_t r_hi, int64_t c_hi, int64_t q0,
                                                              int64_t K, int ct, LdlWs w) {
    __shared__ union {
        DiagSmem diag;
        GemmSmemF64<kLdlKT> g;
    } sm;
    if (blockIdx.x == 0) {
        // the block was last updated by the super-panel's earlier blocks; the panel
        // block at q0 (K rows) is applied here
        diag_body(d, kn, kTile, w, sm.diag, w.A + q0 * d + kn, (int)K);
        return;
    }
    if (*w.info >= 0) return;
    const int tile = (int)blockIdx.x - 1;
    const int64_t r0 = r_lo + (int64_t)(tile / ct) * kTile;
    const int64_t c0 = (int64_t)(tile % ct) * kTile;
    if (c0 > r0 + kTile - 1) return;     // entirely above the diagonal
    if (r0 == kn && c0 == kn) return;    // the next diagonal block
    update_tile<kLdlKT>(d, r0, r_hi, c0, c_hi, q0, K, w, sm.g);
}

// ---------------------------------------------------------------------------
// Scheduled factorisation: the same blocked algorithm in one persistent launch
// per factor, for orders up to kSchedMaxBlocks blocks, where the launch chain
// above leaves the GPU mostly idle.
//
// Block b (last to first) needs its diagonal tile (b, b) and its panel row
// (b, C), C < b, updated by every later block: tile (R, C) -= P_b,R^T P_b,C with
// P_b = C12^T, the panel row of block b. The first workgroup to start runs the
// chain alone: it factors each diagonal block and forms the panel tile
// (b, b - 1) in LDS, which is all that the next diagonal block waits for (its
// update by block b is applied straight from LDS). The other workgroups take
// tasks in ticket order from a table ordered by "phase" b = nb-1 .. 0:
//   panel  (b, C), C <= b - 2     C12^T tile = C22^-1 A(b, C)             (K = 64)
//   near   (R, C) by block b, for the kNear rows R just below b           (K = 64)
//   far    (R, C) by blocks b .. b + kSeg - 1, for the rows R = b - kNear - 1 - kSeg s
// so that a row's updates from blocks more than kNear above it come in segments
// of kSeg blocks, each as soon as its blocks are done and none longer than kSeg
// blocks (no workgroup is tied up for long while the chain waits on short tasks).
// Each tile's updates are applied in one fixed order (far segments from the
// highest, then the near blocks from the highest down) and counted in its
// progress counter; an update task computes its product first and waits for its
// turn only to read, subtract and store. The panel of tile (b, C) is marked by
// raising its counter one past the number of its updates. Every wait is on work
// earlier in ticket order (the chain counts as running ahead of phase b when it
// reaches block b), so the tasks cannot deadlock, and every wait is bounded in time.
// ---------------------------------------------------------------------------
constexpr int kSchedMaxBlocks = 128;  // orders up to 8192
constexpr int kNear = 3;              // rows that take a block's update on their own
constexpr int kSeg = 12;              // blocks per far update

struct SchedArgs {
    int64_t d;
    int nb;
    int ntask;            // tasks in the table; ticket 0 is the chain
    uint64_t spin_limit;  // wall-clock ticks a single wait may take
};

// last block whose update row R takes on its own
__host__ __device__ inline int sched_near_hi(int R, int nb) { return R + kNear < nb - 1 ? R + kNear : nb - 1; }
// far segments of row R: blocks R + kNear + 1 .. nb - 1 in groups of kSeg
__host__ __device__ inline int sched_nfar(int R, int nb) {
    const int lo = R + kNear + 1;
    return lo < nb ? (nb - lo + kSeg - 1) / kSeg : 0;
}
// updates tile (R, C) receives from tasks (the diagonal tile takes block R + 1's in the chain)
__host__ __device__ inline int sched_expect(int R, int C, int nb) {
    return sched_nfar(R, nb) + sched_near_hi(R, nb) - R - ((C == R && R + 1 < nb) ? 1 : 0);
}
// tasks of phase p, in table order: panels, near rows p-1 .. p-kNear, far rows p-kNear-1-kSeg s
__host__ __device__ inline int sched_phase_tasks(int p, int nb) {
    int n = p > 1 ? p - 1 : 0;
    for (int R = p - 1; R >= 0 && R >= p - kNear; --R) n += (R == p - 1) ? R : R + 1;
    for (int R = p - kNear - 1; R >= 0; R -= kSeg) n += R + 1;
    return n;
}

struct SchedTask {
    bool panel;
    int R, C;    // panel: tile (lo, C); update: tile (R, C)
    int lo, hi;  // blocks [lo, hi) whose panel rows update the tile
    int ord;     // the update's turn on the tile
};

// task i of phase p
__device__ __forceinline__ SchedTask sched_decode(int p, int i, int nb) {
    SchedTask k;
    const int npan = p > 1 ? p - 1 : 0;
    if (i < npan) {
        k.panel = true;
        k.lo = p;
        k.C = p - 2 - i;
        return k;
    }
    i -= npan;
    k.panel = false;
    for (int R = p - 1; R >= 0 && R >= p - kNear; --R) {
        const int top = (R == p - 1) ? R - 1 : R;  // row p - 1 leaves its diagonal tile to the chain
        if (i <= top) {
            k.R = R;
            k.C = top - i;
            k.lo = p;
            k.hi = p + 1;
            k.ord = sched_nfar(R, nb) + sched_near_hi(R, nb) - p;
            return k;
        }
        i -= top + 1;
    }
    // far: segment sg of row R = p - kNear - 1 - kSeg sg, blocks p .. p + kSeg - 1
    k.lo = p;
    k.hi = min(p + kSeg, nb);
    int R = p - kNear - 1, sg = 0;
    while (i > R) {
        i -= R + 1;
        R -= kSeg;
        ++sg;
    }
    k.R = R;
    k.C = R - i;
    k.ord = sched_nfar(R, nb) - 1 - sg;
    return k;
}

// thread 0: waits until *f >= v; false if the factorisation was abandoned or this
// wait ran past its limit (which abandons it: info = -2 unless already set)
__device__ __forceinline__ bool sched_wait(const SchedArgs& a, const LdlWs& w, const int* f, int v) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        if (ld_flag(f) >= v) return true;
        if (ld_flag(w.abort)) return false;
        if (__builtin_amdgcn_s_memrealtime() - t0 > a.spin_limit) {
            atomicCAS((unsigned long long*)w.info, ~0ull, (unsigned long long)-2ll);
            st_flag(w.abort, 1);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// thread 0's verdict to the whole workgroup, with the caches invalidated on success
__device__ __forceinline__ bool sched_share(bool ok, int& s_ok) {
    if (threadIdx.x == 0) {
        if (ok) acquire_agent();
        vm_wait_all();
        s_ok = ok;
    }
    __syncthreads();
    const bool r = s_ok != 0;
    __syncthreads();
    return r;
}

// thread 0 looks, without waiting, whether *f >= v; the answer goes to the whole
// workgroup, with the caches invalidated if so
__device__ __forceinline__ bool sched_ready(const int* f, int v, int& s_ok) {
    if (threadIdx.x == 0) {
        const bool r = ld_flag(f) >= v;
        if (r) acquire_agent();
        s_ok = r;
    }
    __syncthreads();
    const bool r = s_ok != 0;
    __syncthreads();
    return r;
}

// The chain: every diagonal block in turn, and the panel tile just below-left of it.
// Tiles whose updates are already all in are loaded ahead: the panel tile's loads go
// out with the diagonal block's stores, and the next diagonal tile's before the
// panel product.
__device__ __forceinline__ void sched_chain(const LdlWs& w, const SchedArgs& a, DiagSmem& s, int& s_ok) {
    const int64_t d = a.d;
    const int nb = a.nb;
    constexpr int kPer = 64 * 64 / kThreads;
    bool have_diag = false;  // s.u already holds block b's diagonal tile
    for (int b = nb - 1; b >= 0; --b) {
        const int t = tid_opaque(), lane = t & 63, wv = t >> 6;
        const int64_t k0 = (int64_t)b * kTile;
        const int nr = (int)min<int64_t>(kTile, d - k0);
        // 32-bit offsets from per-block bases keep the addresses to one register each;
        // thread t holds column i = t % 64 of rows j = t / 64 + 4 r
        const int i = t & 63, j0 = t >> 6;
        const int di4 = 4 * (int)d;
        double* const Ab = w.A + k0 * d + k0;
        double* const Pb = Ab - kTile;  // the panel tile (b, b - 1): rows k0.., columns k0 - 64..
        // (1) the diagonal block, once every update but block b + 1's is in
        if (!have_diag) {
            bool ok = true;
            if (t == 0) ok = sched_wait(a, w, &w.cnt[b * nb + b], sched_expect(b, b, nb));
            if (!sched_share(ok, s_ok)) return;
            double v[kPer];
#pragma unroll
            for (int r = 0; r < kPer; ++r) {
                const int j = j0 + 4 * r;
                v[r] = (i <= j && j < nr) ? Ab[j0 * (int)d + i + r * di4] : (i == j ? 1.0 : 0.0);
            }
#pragma unroll
            for (int r = 0; r < kPer; ++r) s.u[i][j0 + 4 * r] = v[r];
            __syncthreads();
        }
        if (b + 1 < nb) {  // s.xs holds the panel tile (b + 1, b) from the step before
            diag_syrk(s, wv, lane);
            __syncthreads();
        }
        const int badj = diag_factor(s, nr, wv, lane);
        if (badj >= 0) {
            if (t == 0) {
                atomicCAS((unsigned long long*)w.info, ~0ull, (unsigned long long)(k0 + badj));
                st_flag(w.abort, 1);
            }
            return;
        }
        const bool pre = b > 0 && sched_ready(&w.cnt[b * nb + b - 1], sched_expect(b, b - 1, nb), s_ok);
        double v[kPer];
        if (pre) {
#pragma unroll
            for (int r = 0; r < kPer; ++r) v[r] = j0 + 4 * r < nr ? Pb[j0 * (int)d + i + r * di4] : 0.0;
        }
        // C22 into A (lower storage: A[k0 + j][k0 + i] = C[i][j]), X^T into the block's Wt slot
        double* const wb = w.Wt + (size_t)b * 4096;
#pragma unroll 4
        for (int r = 0; r < kPer; ++r) {
            const int j = j0 + 4 * r;
            const double cv = s.u[i][j];
            const double xv = (i <= j) ? s.xs[i][j] : 0.0;
            if (i <= j && j < nr) st_coherent(&Ab[j0 * (int)d + i + r * di4], cv);
            st_coherent(&wb[t + r * kThreads], xv);
        }
        vm_wait_all();
        __syncthreads();
        if (t == 0) st_flag(&w.cnt[b * nb + b], sched_expect(b, b, nb) + 1);
        if (b == 0) return;

        // (2) the panel tile (b, b - 1): P = X A(b, b - 1), into A and into s.xs
        if (!pre) {
            bool ok = true;
            if (t == 0) ok = sched_wait(a, w, &w.cnt[b * nb + b - 1], sched_expect(b, b - 1, nb));
            if (!sched_share(ok, s_ok)) return;
#pragma unroll
            for (int r = 0; r < kPer; ++r) v[r] = j0 + 4 * r < nr ? Pb[j0 * (int)d + i + r * di4] : 0.0;
        }
#pragma unroll
        for (int r = 0; r < kPer; ++r) s.u[j0 + 4 * r][i] = v[r];
        __syncthreads();
        // the next diagonal tile (block b - 1, never the ragged last block)
        have_diag = sched_ready(&w.cnt[(b - 1) * nb + b - 1], sched_expect(b - 1, b - 1, nb), s_ok);
        double vn[kPer];
        if (have_diag) {
            const double* An = Ab - kTile * d - kTile;
#pragma unroll
            for (int r = 0; r < kPer; ++r) {
                const int j = j0 + 4 * r;
                vn[r] = i <= j ? An[j0 * (int)d + i + r * di4] : 0.0;
            }
        }
        // 32x32 quadrant per wave; X is upper triangular, so k starts at the quadrant's first row
        const int qi = wv >> 1, qj = wv & 1;
        f64x4 acc[2][2];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
        const int pa = 32 * qi + (lane & 15), pb = pa + 16, rc = 32 * qj + (lane & 15);
        for (int kk = 8 * qi; kk < 16; ++kk) {
            const int q = 4 * kk + (lane >> 4);
            const double fa0 = q >= pa ? s.xs[pa][q] : 0.0;
            const double fa1 = q >= pb ? s.xs[pb][q] : 0.0;
            const double fb0 = s.u[q][rc], fb1 = s.u[q][rc + 16];
            acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa0, fb0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa0, fb1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa1, fb0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa1, fb1, acc[1][1], 0, 0, 0);
        }
        __syncthreads();  // every read of X and of the tile is done
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int pr = 32 * qi + 16 * bi + (lane >> 4) + 4 * r;
                    const int c = 32 * qj + 16 * bj + (lane & 15);
                    s.xs[pr][c] = acc[bi][bj][r];
                    if (pr < nr) st_coherent(&Pb[pr * (int)d + c], acc[bi][bj][r]);
                }
        if (have_diag) {
#pragma unroll
            for (int r = 0; r < kPer; ++r) {
                const int j = j0 + 4 * r;
                s.u[i][j] = i <= j ? vn[r] : (i == j ? 1.0 : 0.0);
            }
        }
        vm_wait_all();
        __syncthreads();
        if (t == 0) st_flag(&w.cnt[b * nb + b - 1], sched_expect(b, b - 1, nb) + 1);
    }
}

// panel tile (b, C): C12^T = C22^-1 A(b, C), in place
__device__ __forceinline__ void sched_panel(const LdlWs& w, const SchedArgs& a, int b, int C,
                                            GemmSmemF64<kLdlKT>& sm, int& s_ok) {
    const int64_t d = a.d;
    const int nb = a.nb;
    const int64_t k0 = (int64_t)b * kTile, c0 = (int64_t)C * kTile;
    const int nr = (int)min<int64_t>(kTile, d - k0);
    bool ok = true;
    if (threadIdx.x == 0)
        ok = sched_wait(a, w, &w.cnt[b * nb + b], sched_expect(b, b, nb) + 1) &&
             sched_wait(a, w, &w.cnt[b * nb + C], sched_expect(b, C, nb));
    if (!sched_share(ok, s_ok)) return;
    f64x4 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
    tile_gemm_f64<kLdlKT>(w.Wt + (size_t)b * 4096, 64, nr, w.A + k0 * d + c0, d, kTile, nr, acc, sm);
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pr = acc64_row(bi, r), rc = acc64_col(bj);
                if (pr < nr) st_coherent(&w.A[(k0 + pr) * d + c0 + rc], acc[bi][bj][r]);
            }
    vm_wait_all();
    __syncthreads();
    if (threadIdx.x == 0) st_flag(&w.cnt[b * nb + C], sched_expect(b, C, nb) + 1);
}

// tile (R, C) -= sum over blocks [lo, hi) of P_b,R^T P_b,C, as update number `ord` of the tile
__device__ __forceinline__ void sched_update(const LdlWs& w, const SchedArgs& a, const SchedTask& k,
                                             GemmSmemF64<kLdlKT>& sm, int& s_ok) {
    const int64_t d = a.d;
    const int nb = a.nb;
    const int R = k.R, C = k.C;
    // the panel tiles (b, R) and (b, C) of every block b in [lo, hi): one thread per block
    bool ok = true;
    const int t = tid_opaque();
    if (t < k.hi - k.lo) {
        const int b = k.lo + t;
        ok = sched_wait(a, w, &w.cnt[b * nb + R], sched_expect(b, R, nb) + 1);
        if (ok && C != R) ok = sched_wait(a, w, &w.cnt[b * nb + C], sched_expect(b, C, nb) + 1);
    }
    if (t == 0) s_ok = 1;
    __syncthreads();
    if (!ok) s_ok = 0;
    __syncthreads();
    if (!s_ok) return;
    if (t == 0) {
        acquire_agent();
        vm_wait_all();
    }
    __syncthreads();
    const int64_t q0 = (int64_t)k.lo * kTile;
    const int64_t K = min<int64_t>((int64_t)k.hi * kTile, d) - q0;
    const int64_t r0 = (int64_t)R * kTile, c0 = (int64_t)C * kTile;
    f64x4 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
    const double* P = w.A + q0 * d;
    tile_gemm_f64<kLdlKT>(P + r0, d, kTile, P + c0, d, kTile, K, acc, sm);
    // this tile's turn
    if (threadIdx.x == 0) ok = sched_wait(a, w, &w.cnt[R * nb + C], k.ord);
    if (!sched_share(ok, s_ok)) return;
    double old[2][2][4];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t gi = r0 + acc64_row(bi, r), gj = c0 + acc64_col(bj);
                old[bi][bj][r] = gj <= gi ? w.A[gi * d + gj] : 0.0;
            }
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t gi = r0 + acc64_row(bi, r), gj = c0 + acc64_col(bj);
                if (gj <= gi) st_coherent(&w.A[gi * d + gj], old[bi][bj][r] - acc[bi][bj][r]);
            }
    vm_wait_all();
    __syncthreads();
    if (threadIdx.x == 0) st_flag(&w.cnt[R * nb + C], k.ord + 1);
}

// One or two factorisations (nf) in one launch: tickets 0 .. nf-1 are the
// chains, the rest the two task tables merged phase by phase (factor 0's phase
// nb-1-j, then factor 1's), so both chains are served alike. Each factor keeps
// its own counters, abort flag and status; the ticket counter is factor 0's.
struct SchedLaunch {
    LdlWs w[2];
    SchedArgs a[2];
    int nf;
};

__global__ __launch_bounds__(kThreads, 2) void k_ldl_sched(SchedLaunch L) {
    __shared__ union {
        DiagSmem diag;
        GemmSmemF64<kLdlKT> g;
    } sm;
    __shared__ int s_tk, s_ok;
    // s_ps[m]: first task of merged slot m = nf j + f, factor f's phase nb_f - 1 - j
    __shared__ int s_ps[2 * kSchedMaxBlocks + 1];
    const int nf = L.nf;
    const int nbmax = nf == 2 ? max(L.a[0].nb, L.a[1].nb) : L.a[0].nb;
    for (int m = threadIdx.x; m < nf * nbmax; m += kThreads) {
        const int j = m / nf, nb = (m % nf) ? L.a[1].nb : L.a[0].nb;
        s_ps[m + 1] = j < nb ? sched_phase_tasks(nb - 1 - j, nb) : 0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        s_ps[0] = 0;
        for (int m = 0; m < nf * nbmax; ++m) s_ps[m + 1] += s_ps[m];
    }
    __syncthreads();
    const int ntask = s_ps[nf * nbmax];
    int m = 0;  // slot cursor: a workgroup's tickets only grow
    for (;;) {
        if (threadIdx.x == 0) s_tk = atomicAdd(L.w[0].ticket, 1);
        __syncthreads();
        const int tk = s_tk;
        __syncthreads();
        if (tk >= nf + ntask) return;
        // the factor's arguments by selection (an indexed kernel argument would be copied
        // to scratch memory)
        int f;
        if (tk < nf) {
            f = tk;
        } else {
            while (s_ps[m + 1] <= tk - nf) ++m;
            f = m % nf;
        }
        const LdlWs w = f ? L.w[1] : L.w[0];
        const SchedArgs a = f ? L.a[1] : L.a[0];
        if (tk < nf) {
            // the chain's waves issue first on their SIMDs: workgroups of other
            // work may share its compute unit
            __builtin_amdgcn_s_setprio(3);
            sched_chain(w, a, sm.diag, s_ok);
            __builtin_amdgcn_s_setprio(0);
            continue;
        }
        const SchedTask k = sched_decode(a.nb - 1 - m / nf, tk - nf - s_ps[m], a.nb);
        if (k.panel) sched_panel(w, a, k.lo, k.C, sm.g, s_ok);
        else sched_update(w, a, k, sm.g, s_ok);
    }
}

// H[i][j] = C[i][j] / C[j][j] (i < j), C[j][j]^2 (i = j), 0 (i > j), with
// C[i][j] = A[j][i]; D[j] = C[j][j]^2 if requested. Tiles below the diagonal are
// zeros and read nothing; whole tiles of an H with 16-byte aligned rows (and an
// even order) move in 16-byte pieces, every load in flight; others go element by
// element.
__global__ __launch_bounds__(kThreads) void k_ldl_store(float* __restrict__ H, int64_t d,
                                                        int64_t ldh, float* __restrict__ D,
                                                        LdlWs w) {
    const int64_t rt = blockIdx.y, ct = blockIdx.x;  // tile of H: rows rt, cols ct
    const int t = threadIdx.x;
    __shared__ float tile[kTile][kTile + 1];
    __shared__ double dj[kTile];
    const int64_t i0 = rt * kTile, j0 = ct * kTile;
    const bool vec = i0 + kTile <= d && j0 + kTile <= d && (ldh & 3) == 0 && (d & 1) == 0 &&
                     (reinterpret_cast<uintptr_t>(H) & 15) == 0;
    constexpr int kV4 = kTile * kTile / 4 / kThreads, kV2 = kTile * kTile / 2 / kThreads;
    if (rt > ct) {
        if (vec) {
#pragma unroll
            for (int u = 0; u < kV4; ++u) {
                const int q = t + u * kThreads;
                *reinterpret_cast<f32x4*>(H + (i0 + (q >> 4)) * ldh + j0 + ((q & 15) << 2)) =
                    f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        } else {
            for (int e = t; e < kTile * kTile; e += kThreads) {
                const int64_t i = i0 + e / kTile, j = j0 + e % kTile;
                if (i < d && j < d) H[i * ldh + j] = 0.0f;
            }
        }
        return;
    }
    if (t < kTile) {
        const int64_t j = j0 + t;
        dj[t] = (j < d) ? w.A[j * d + j] : 1.0;
    }
    __syncthreads();
    if (vec) {
        // A rows j0 + b, columns i0 + a2, +1
        f64x2 x[kV2];
#pragma unroll
        for (int u = 0; u < kV2; ++u) {
            const int q = t + u * kThreads;
            x[u] = *reinterpret_cast<const f64x2*>(w.A + (j0 + (q >> 5)) * d + i0 + ((q & 31) << 1));
        }
#pragma unroll
        for (int u = 0; u < kV2; ++u) {
            const int q = t + u * kThreads;
            const int b = q >> 5, a2 = (q & 31) << 1;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int64_t i = i0 + a2 + e, j = j0 + b;
                float v = 0.0f;
                if (i < j) v = (float)(x[u][e] / dj[b]);
                else if (i == j) v = (float)(dj[b] * dj[b]);
                tile[a2 + e][b] = v;
            }
        }
    } else {
        for (int e = t; e < kTile * kTile; e += kThreads) {
            const int b = e / kTile, a = e % kTile;  // A row j0 + b, col i0 + a
            const int64_t j = j0 + b, i = i0 + a;
            float v = 0.0f;
            if (i < d && j < d) {
                if (i < j) v = (float)(w.A[j * d + i] / dj[b]);
                else if (i == j) v = (float)(dj[b] * dj[b]);
            }
            tile[a][b] = v;
        }
    }
    __syncthreads();
    if (vec) {
#pragma unroll
        for (int u = 0; u < kV4; ++u) {
            const int q = t + u * kThreads;
            const int a = q >> 4, b4 = (q & 15) << 2;
            const f32x4 v = {tile[a][b4], tile[a][b4 + 1], tile[a][b4 + 2], tile[a][b4 + 3]};
            *reinterpret_cast<f32x4*>(H + (i0 + a) * ldh + j0 + b4) = v;
        }
        if (D && rt == ct && t < kTile) D[j0 + t] = tile[t][t];
    } else {
        for (int e = t; e < kTile * kTile; e += kThreads) {
            const int a = e / kTile, b = e % kTile;  // H row i0 + a, col j0 + b
            const int64_t i = i0 + a, j = j0 + b;
            if (i >= d || j >= d) continue;
            H[i * ldh + j] = tile[a][b];
            if (D && i == j) D[j] = tile[a][b];
        }
    }
}

// status word out: -1, or the first failing pivot
__global__ void k_ldl_info_out(LdlWs w, int64_t* out) { *out = *w.info; }

// The scheduled path for orders up to kSchedMaxBlocks blocks, else the launch
// chain; BAKRON_LDL_PATH = "launch" or "scheduled" (read at each call) picks one
// where both apply, for tests.
static bool use_sched(int64_t nbt) {
    if (nbt > kSchedMaxBlocks) return false;
    const char* e = std::getenv("BAKRON_LDL_PATH");
    return !(e && std::strcmp(e, "launch") == 0);
}

static SchedArgs sched_args(int64_t d, uint64_t spin_limit) {
    SchedArgs a;
    a.d = d;
    a.nb = (int)ldl_blocks(d);
    a.ntask = 0;
    for (int p = 0; p < a.nb; ++p) a.ntask += sched_phase_tasks(p, a.nb);
    a.spin_limit = spin_limit;
    return a;
}

// the scheduled factorisation of nf (1 or 2) matrices, already loaded, in one launch
static void enqueue_sched(int nf, const int64_t* d, const LdlWs* w, hipStream_t stream) {
    // 10 s, or BAKRON_LDL_WAIT_LIMIT_US (a test hook that makes the waits expire)
    uint64_t limit_us = 10ull * 1000 * 1000;
    if (const char* e = std::getenv("BAKRON_LDL_WAIT_LIMIT_US")) {
        const long long v = std::atoll(e);
        if (v > 0) limit_us = (uint64_t)v;
    }
    const DeviceInfo di = device_info();
    const uint64_t spin = (uint64_t)di.clock_khz * limit_us / 1000ull;
    SchedLaunch L;
    L.nf = nf;
    int64_t total = 0, nbmax = 0, cube = 0;
    for (int f = 0; f < 2; ++f) {
        const int g = f < nf ? f : 0;
        L.w[f] = w[g];
        L.a[f] = sched_args(d[g], spin);
        if (f < nf) {
            total += L.a[f].ntask + 1;
            nbmax = std::max<int64_t>(nbmax, L.a[f].nb);
            cube += (int64_t)L.a[f].nb * L.a[f].nb * L.a[f].nb;
        }
    }
    // One workgroup per compute unit while the chains set the pace: more take tickets
    // further ahead of them and mostly wait. Two per compute unit (what the kernel's
    // registers and LDS allow) once the tile updates per diagonal block, sum nb^3 / nb_max
    // in tile products, reach 14000: measured faster from a pair of order 6144 (18432)
    // and a single factor of 8192 (16384), slower for a single 7168 (12544), even for a
    // pair of 5120 (12800).
    const int per_cu = cube / std::max<int64_t>(nbmax, 1) >= 14000 ? 2 : 1;
    const int grid = (int)std::min<int64_t>((int64_t)per_cu * di.cus, total);
    hipLaunchKernelGGL(k_ldl_sched, dim3((unsigned)grid), dim3(kThreads), 0, stream, L);
}

int enqueue_ldl(float* H, int64_t d, int64_t ldh, double damp_rel, float* D, void* ws,
                hipStream_t stream, int64_t* info_dev, bool allow_sched) {
    LdlWs w = carve(ws, d);
    const int64_t nbt = ldl_blocks(d);
    if (nbt > 65535) return BAKRON_E_INVALID_ARG;
    hipLaunchKernelGGL(k_ldl_init, dim3(1), dim3(kThreads), 0, stream, H, d, ldh, damp_rel, w);
    hipLaunchKernelGGL(k_ldl_load, dim3((unsigned)nbt, (unsigned)nbt), dim3(kThreads), 0, stream,
                       H, d, ldh, w);
    if (allow_sched && use_sched(nbt)) {
        enqueue_sched(1, &d, &w, stream);
    } else {
        // Per 64-wide block k0 (last to first) of each 512-wide super-panel [s0, s1):
        //   panel(k0)
        //   diag(k0 - 64) + inner(k0)      -- one launch: the next diagonal block takes this
        //                                     block's update and is factored beside the rest
        //                                     of this block's inner update
        // and after the super-panel the outer update, then the next super-panel's first
        // diagonal block on its own.
        const int64_t nsuper = (d + kSuper - 1) / kSuper;
        for (int64_t s = nsuper - 1; s >= 0; --s) {
            const int64_t s0 = s * kSuper, s1 = std::min<int64_t>(s0 + kSuper, d);
            const int64_t top = ((s1 - 1) / 64) * 64;
            hipLaunchKernelGGL(k_ldl_diag, dim3(1), dim3(kThreads), 0, stream, d, top,
                               (int)std::min<int64_t>(64, d - top), w);
            for (int64_t k0 = top; k0 >= s0; k0 -= 64) {
                const int nb = (int)std::min<int64_t>(64, d - k0);
                if (k0 > 0) {
                    hipLaunchKernelGGL(k_ldl_panel, dim3((unsigned)((k0 + 63) / 64)), dim3(kThreads),
                                       0, stream, d, k0, nb, w);
                }
                if (k0 > s0) {  // rows [s0, k0) of the super-panel, every column < k0
                    const int64_t rt = (k0 - s0 + kTile - 1) / kTile, ct = (k0 + kTile - 1) / kTile;
                    hipLaunchKernelGGL(k_ldl_diag_update, dim3((unsigned)(1 + rt * ct)), dim3(kThreads),
                                       0, stream, d, k0 - 64, s0, k0, k0, k0, (int64_t)nb, (int)ct, w);
                }
            }
            if (s0 > 0) {
                const int64_t ns = (s0 + kSqR * kOutM - 1) / (kSqR * kOutM), nsq = ns * (ns + 1) / 2;
                const int64_t grid = kXcds * ((nsq + kXcds - 1) / kXcds) * kSqR * kSqC;
                hipLaunchKernelGGL(k_ldl_outer, dim3((unsigned)grid), dim3(kOutThreads), 0, stream, d, s0, s0,
                                   s1 - s0, (int)nsq, w);
            }
        }
    }
    hipLaunchKernelGGL(k_ldl_store, dim3((unsigned)nbt, (unsigned)nbt), dim3(kThreads), 0, stream,
                       H, d, ldh, D, w);
    if (info_dev) hipLaunchKernelGGL(k_ldl_info_out, dim3(1), dim3(1), 0, stream, w, info_dev);
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

int enqueue_ldl_pair(float* HA, int64_t dA, int64_t ldha, float* DA, void* wsA, int64_t* infoA,
                     float* HB, int64_t dB, int64_t ldhb, float* DB, void* wsB, int64_t* infoB,
                     double damp_rel, hipStream_t stream, hipStream_t stream_b) {
    const int64_t nbA = ldl_blocks(dA), nbB = ldl_blocks(dB);
    if (!use_sched(nbA) || !use_sched(nbB)) {
        // Side by side on the two streams, both by the chain of launches: a persistent
        // launch for the smaller one would hold a slot on every compute unit for the
        // whole of its run, which the larger one's wide updates need.
        const int st = enqueue_ldl(HA, dA, ldha, damp_rel, DA, wsA, stream, infoA, false);
        if (st != BAKRON_OK) return st;
        return enqueue_ldl(HB, dB, ldhb, damp_rel, DB, wsB, stream_b, infoB, false);
    }
    const LdlWs w[2] = {carve(wsA, dA), carve(wsB, dB)};
    const int64_t d[2] = {dA, dB};
    float* H[2] = {HA, HB};
    float* D[2] = {DA, DB};
    const int64_t ldh[2] = {ldha, ldhb};
    int64_t* info[2] = {infoA, infoB};
    for (int f = 0; f < 2; ++f) {
        const int64_t nbt = ldl_blocks(d[f]);
        hipLaunchKernelGGL(k_ldl_init, dim3(1), dim3(kThreads), 0, stream, H[f], d[f], ldh[f], damp_rel, w[f]);
        hipLaunchKernelGGL(k_ldl_load, dim3((unsigned)nbt, (unsigned)nbt), dim3(kThreads), 0, stream, H[f],
                           d[f], ldh[f], w[f]);
    }
    enqueue_sched(2, d, w, stream);
    for (int f = 0; f < 2; ++f) {
        const int64_t nbt = ldl_blocks(d[f]);
        hipLaunchKernelGGL(k_ldl_store, dim3((unsigned)nbt, (unsigned)nbt), dim3(kThreads), 0, stream, H[f],
                           d[f], ldh[f], D[f], w[f]);
        hipLaunchKernelGGL(k_ldl_info_out, dim3(1), dim3(1), 0, stream, w[f], info[f]);
    }
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

int run_ldl(float* H, int64_t d, int64_t ldh, double damp_rel, float* D, int64_t* bad_pivot,
            void* ws, hipStream_t stream) {
    const int st = enqueue_ldl(H, d, ldh, damp_rel, D, ws, stream, nullptr, true);
    if (st != BAKRON_OK) return st;
    const LdlWs w = carve(ws, d);
    int64_t info = -1;
    if (hipMemcpyAsync(&info, w.info, sizeof(int64_t), hipMemcpyDeviceToHost, stream) !=
        hipSuccess)
        return BAKRON_E_DEVICE;
    if (hipStreamSynchronize(stream) != hipSuccess) return BAKRON_E_DEVICE;
    if (bad_pivot) *bad_pivot = info;
    if (info == -2) return BAKRON_E_DEVICE;  // a wait between workgroups ran past its limit
    return info >= 0 ? BAKRON_E_NOT_SPD : BAKRON_OK;
}

}  // namespace bk
