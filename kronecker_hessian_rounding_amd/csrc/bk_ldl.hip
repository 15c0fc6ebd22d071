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
//   inner : A[s0:k0, 0:k0] -= C12 C12^T restricted to the current 256-wide
//           super-panel's rows                        (MFMA, lower part)
//   outer : after each super-panel, A[0:s0, 0:s0] -= C_S C_S^T with
//           K = the super-panel width                 (MFMA, lower part)
#include <algorithm>

#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

constexpr int kSuper = 256;  // super-panel width (K of the big trailing updates)
constexpr int kLdlKT = 32;   // k-slice depth of the fp64 panel / inner-update GEMMs (K = 64);
                             // the wide outer updates use 16 (half the LDS, more workgroups per CU)

struct LdlWs {
    double* A;     // d x d working copy, lower triangle used, ld = d
    double* Wt;    // 64 x 64: Wt[q][p] = (C22^-1)[p][q] of the current diagonal block
    double* lam;   // damping lambda
    int64_t* info; // -1, or the first failing pivot index
};

static LdlWs carve(void* ws, int64_t d) {
    char* p = (char*)ws;
    LdlWs w;
    w.A = (double*)p;
    p += align256(sizeof(double) * (size_t)d * (size_t)d);
    w.Wt = (double*)p;
    p += align256(sizeof(double) * 64 * 64);
    w.lam = (double*)p;
    p += 256;
    w.info = (int64_t*)p;
    return w;
}

size_t ldl_workspace_bytes(int64_t d) {
    return align256(sizeof(double) * (size_t)d * (size_t)d) + align256(sizeof(double) * 4096) +
           256 + 256;
}

// lambda = damp_rel * mean(diag H) in fp64; info = -1.
__global__ __launch_bounds__(kThreads) void k_ldl_init(const float* __restrict__ H, int64_t d,
                                                       int64_t ldh, double damp_rel, LdlWs w) {
    __shared__ double red[kThreads];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < d; i += kThreads) s += (double)H[i * ldh + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        *w.lam = damp_rel * (red[0] / (double)d);
        *w.info = -1;
    }
}

// A[r][c] = H[c][r] (upper triangle of H read, lower triangle of A written),
// plus lambda on the diagonal; 64x64 tiles transposed through LDS.
__global__ __launch_bounds__(kThreads) void k_ldl_load(const float* __restrict__ H, int64_t d,
                                                       int64_t ldh, LdlWs w) {
    const int64_t rt = blockIdx.y, ct = blockIdx.x;  // tile of A: rows rt, cols ct, rt >= ct
    if (ct > rt) return;
    __shared__ float tile[kTile][kTile + 1];
    const int64_t r0 = rt * kTile, c0 = ct * kTile;
    for (int e = threadIdx.x; e < kTile * kTile; e += kThreads) {
        const int a = e / kTile, b = e % kTile;  // H row c0 + a, col r0 + b
        const int64_t hr = c0 + a, hc = r0 + b;
        tile[a][b] = (hr < d && hc < d && hr <= hc) ? H[hr * ldh + hc] : 0.0f;
    }
    __syncthreads();
    const double lam = *w.lam;
    for (int e = threadIdx.x; e < kTile * kTile; e += kThreads) {
        const int a = e / kTile, b = e % kTile;  // A row r0 + a, col c0 + b
        const int64_t r = r0 + a, c = c0 + b;
        if (r >= d || c > r) continue;
        double v = (double)tile[b][a];
        if (r == c) v += lam;
        w.A[r * d + c] = v;
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
        // 32x32 quadrants on or above the diagonal, one wave each, K = 64 panel rows
        const int qi = wv >> 1, qj = wv & 1;
        if (qi <= qj) {
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
        __syncthreads();
    }

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
    if (s.badj >= 0) {  // uniform after the barrier
        if (t == 0) *w.info = k0 + s.badj;
        return;
    }
    // X[0][1], X[0][2], X[0][3]
    if (wv > 0) ldl_inv_off(s, 0, wv, lane);
    __syncthreads();

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

// A[r][c] -= sum_{q < K} A[q0 + q][r] A[q0 + q][c] over rows [r_lo, r_hi),
// columns [0, c_hi), lower triangle only (c <= r).
template <int KT>
__global__ __launch_bounds__(kThreads) void k_ldl_update(int64_t d, int64_t r_lo, int64_t r_hi,
                                                         int64_t c_hi, int64_t q0, int64_t K,
                                                         LdlWs w) {
    if (*w.info >= 0) return;
    const int64_t r0 = r_lo + (int64_t)blockIdx.y * kTile;
    const int64_t c0 = (int64_t)blockIdx.x * kTile;
    if (c0 > r0 + kTile - 1) return;  // tile entirely above the diagonal
    __shared__ GemmSmemF64<KT> sm;
    update_tile<KT>(d, r0, r_hi, c0, c_hi, q0, K, w, sm);
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

// H[i][j] = C[i][j] / C[j][j] (i < j), C[j][j]^2 (i = j), 0 (i > j), with
// C[i][j] = A[j][i]; D[j] = C[j][j]^2 if requested.
__global__ __launch_bounds__(kThreads) void k_ldl_store(float* __restrict__ H, int64_t d,
                                                        int64_t ldh, float* __restrict__ D,
                                                        LdlWs w) {
    const int64_t rt = blockIdx.y, ct = blockIdx.x;  // tile of H: rows rt, cols ct
    __shared__ float tile[kTile][kTile + 1];
    __shared__ double dj[kTile];
    const int64_t i0 = rt * kTile, j0 = ct * kTile;
    if (threadIdx.x < kTile) {
        const int64_t j = j0 + threadIdx.x;
        dj[threadIdx.x] = (j < d) ? w.A[j * d + j] : 1.0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kTile * kTile; e += kThreads) {
        const int b = e / kTile, a = e % kTile;  // A row j0 + b, col i0 + a
        const int64_t j = j0 + b, i = i0 + a;
        float v = 0.0f;
        if (i < d && j < d) {
            if (i < j) v = (float)(w.A[j * d + i] / dj[b]);
            else if (i == j) v = (float)(dj[b] * dj[b]);
        }
        tile[a][b] = v;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kTile * kTile; e += kThreads) {
        const int a = e / kTile, b = e % kTile;  // H row i0 + a, col j0 + b
        const int64_t i = i0 + a, j = j0 + b;
        if (i >= d || j >= d) continue;
        H[i * ldh + j] = tile[a][b];
        if (D && i == j) D[j] = tile[a][b];
    }
}

// status word out: -1, or the first failing pivot
__global__ void k_ldl_info_out(LdlWs w, int64_t* out) { *out = *w.info; }

int enqueue_ldl(float* H, int64_t d, int64_t ldh, double damp_rel, float* D, void* ws,
                hipStream_t stream, int64_t* info_dev) {
    LdlWs w = carve(ws, d);
    const int64_t nbt = (d + kTile - 1) / kTile;
    if (nbt > 65535) return BAKRON_E_INVALID_ARG;
    hipLaunchKernelGGL(k_ldl_init, dim3(1), dim3(kThreads), 0, stream, H, d, ldh, damp_rel, w);
    hipLaunchKernelGGL(k_ldl_load, dim3((unsigned)nbt, (unsigned)nbt), dim3(kThreads), 0, stream,
                       H, d, ldh, w);
    // Per 64-wide block k0 (last to first) of each 256-wide super-panel [s0, s1):
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
            const int64_t tt = (s0 + kTile - 1) / kTile;
            hipLaunchKernelGGL(k_ldl_update<16>, dim3((unsigned)tt, (unsigned)tt), dim3(kThreads), 0,
                               stream, d, (int64_t)0, s0, s0, s0, s1 - s0, w);
        }
    }
    hipLaunchKernelGGL(k_ldl_store, dim3((unsigned)nbt, (unsigned)nbt), dim3(kThreads), 0, stream,
                       H, d, ldh, D, w);
    if (info_dev) hipLaunchKernelGGL(k_ldl_info_out, dim3(1), dim3(1), 0, stream, w, info_dev);
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

int run_ldl(float* H, int64_t d, int64_t ldh, double damp_rel, float* D, int64_t* bad_pivot,
            void* ws, hipStream_t stream) {
    const int st = enqueue_ldl(H, d, ldh, damp_rel, D, ws, stream, nullptr);
    if (st != BAKRON_OK) return st;
    const LdlWs w = carve(ws, d);
    int64_t info = -1;
    if (hipMemcpyAsync(&info, w.info, sizeof(int64_t), hipMemcpyDeviceToHost, stream) !=
        hipSuccess)
        return BAKRON_E_DEVICE;
    if (hipStreamSynchronize(stream) != hipSuccess) return BAKRON_E_DEVICE;
    if (bad_pivot) *bad_pivot = info;
    return info >= 0 ? BAKRON_E_NOT_SPD : BAKRON_OK;
}

}  // namespace bk
