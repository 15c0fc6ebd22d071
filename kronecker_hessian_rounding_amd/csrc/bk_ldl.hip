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
// The block is held as the upper matrix a[i][j] = A[k0 + j][k0 + i] (i <= j),
// padded with the identity beyond nb. Thread t owns rows ti + 16 x and columns
// tj + 16 y (x, y = 0..3) in registers, with tj = t / 16 and ti = t % 16, so
// the 16 owners of a column (and its pivot) sit in one wave: the pivot is
// broadcast with readlane and each column costs one workgroup barrier.
__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const long long b = __builtin_bit_cast(long long, v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), lane);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

__global__ __launch_bounds__(kThreads) void k_ldl_diag(int64_t d, int64_t k0, int nb, LdlWs w) {
    if (*w.info >= 0) return;
    __shared__ double col[2][64];   // scaled column jj of C (rows < jj)
    __shared__ double cst[64][65];  // C, column-major: cst[j][i] = C[i][j]
    __shared__ double rcd[64];      // 1 / C[j][j]
    __shared__ double xrow[2][64];  // row m of X = C^-1
    __shared__ int bad;
    const int t = threadIdx.x;
    const int tj = t >> 4, ti = t & 15;
    const int wv = t >> 6;
    double a[4][4];
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int i = ti + 16 * x, j = tj + 16 * y;
            double v = 0.0;
            if (i <= j) {
                if (j < nb) v = w.A[(k0 + j) * d + k0 + i];
                else if (i == j) v = 1.0;
            }
            a[x][y] = v;
        }
    if (t == 0) bad = 0;
    __syncthreads();

    // columns jj = 16 yj + bj from the last; yj is a compile-time index into a[][]
#pragma unroll
    for (int yj = 3; yj >= 0; --yj) {
        for (int bj = 15; bj >= 0; --bj) {
            const int jj = 16 * yj + bj;
            if (wv == (bj >> 2)) {  // the wave holding column jj
                const double pv = readlane_f64(a[yj][yj], (16 * bj + bj) & 63);
                if (!(pv > 0.0) || !(pv < INFINITY)) {
                    if ((t & 63) == 0) bad = 1;
                } else if (tj == bj) {  // its 16 owners scale the column
                    const double rc = rsqrt(pv);
                    const double c = pv * rc;
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int i = ti + 16 * x;
                        if (i < jj) {
                            a[x][yj] *= rc;
                            col[jj & 1][i] = a[x][yj];
                            cst[jj][i] = a[x][yj];
                        } else if (i == jj) {
                            a[x][yj] = c;
                            cst[jj][i] = c;
                            rcd[jj] = rc;
                        }
                    }
                }
            }
            __syncthreads();
            if (bad) {  // uniform after the barrier
                if (t == 0 && jj < nb) *w.info = k0 + jj;
                return;
            }
            // a[i][k] -= C[i][jj] C[k][jj] for i <= k < jj
            double ci[4], ck[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) ci[x] = col[jj & 1][ti + 16 * x];
#pragma unroll
            for (int y = 0; y < 4; ++y) ck[y] = col[jj & 1][tj + 16 * y];
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y <= yj; ++y) {
                    const int i = ti + 16 * x, k = tj + 16 * y;
                    if (i <= k && k < jj) a[x][y] = fma(-ci[x], ck[y], a[x][y]);
                }
        }
    }
    // C22 back into A (lower storage: A[k0 + j][k0 + i] = C[i][j])
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int i = ti + 16 * x, j = tj + 16 * y;
            if (i <= j && j < nb) w.A[(k0 + j) * d + k0 + i] = a[x][y];
        }
    // X = C^-1 (upper), right-looking from the last row: s[i][k] accumulates
    // sum_{m > current} C[i][m] X[m][k]; row m is final once every m' > m is in.
    double s[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) s[x][y] = 0.0;
#pragma unroll
    for (int xm = 3; xm >= 0; --xm) {
        for (int bm = 15; bm >= 0; --bm) {
            const int m = 16 * xm + bm;
            if (ti == bm) {  // owners of row m finish it
                const double inv = rcd[m];
#pragma unroll
                for (int y = 0; y < 4; ++y) {
                    const int k = tj + 16 * y;
                    double v = 0.0;
                    if (k >= m) v = ((k == m ? 1.0 : 0.0) - s[xm][y]) * inv;
                    xrow[m & 1][k] = v;
                    w.Wt[k * 64 + m] = v;  // Wt[q][p] = X[p][q]
                }
            }
            __syncthreads();
            double cm[4], xk[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) cm[x] = cst[m][ti + 16 * x];  // C[i][m]
#pragma unroll
            for (int y = 0; y < 4; ++y) xk[y] = xrow[m & 1][tj + 16 * y];
#pragma unroll
            for (int x = 0; x <= xm; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) {
                    const int i = ti + 16 * x, k = tj + 16 * y;
                    if (i < m && k >= m) s[x][y] = fma(cm[x], xk[y], s[x][y]);
                }
        }
    }
}

// C12^T[p][r] = sum_q (C22^-1)[p][q] A[k0 + q][r] for r in this workgroup's 64
// columns (r < k0), written back in place into A[k0 + p][r].
__global__ __launch_bounds__(kThreads) void k_ldl_panel(int64_t d, int64_t k0, int nb, LdlWs w) {
    if (*w.info >= 0) return;
    __shared__ GemmSmem<double> sm;
    const int64_t r0 = (int64_t)blockIdx.x * kTile;
    const int Cn = (int)min<int64_t>(kTile, k0 - r0);
    f64x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    tile_gemm_f64(w.Wt, 64, nb, w.A + k0 * d + r0, d, Cn, nb, acc, sm);
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

// A[r][c] -= sum_{q < K} A[q0 + q][r] A[q0 + q][c] over rows [r_lo, r_hi),
// columns [0, c_hi), lower triangle only (c <= r).
__global__ __launch_bounds__(kThreads) void k_ldl_update(int64_t d, int64_t r_lo, int64_t r_hi,
                                                         int64_t c_hi, int64_t q0, int64_t K,
                                                         LdlWs w) {
    if (*w.info >= 0) return;
    const int64_t r0 = r_lo + (int64_t)blockIdx.y * kTile;
    const int64_t c0 = (int64_t)blockIdx.x * kTile;
    if (c0 > r0 + kTile - 1) return;  // tile entirely above the diagonal
    __shared__ GemmSmem<double> sm;
    const int R = (int)min<int64_t>(kTile, r_hi - r0);
    const int Cn = (int)min<int64_t>(kTile, c_hi - c0);
    f64x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    const double* P = w.A + q0 * d;
    tile_gemm_f64(P + r0, d, R, P + c0, d, Cn, K, acc, sm);
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

int run_ldl(float* H, int64_t d, int64_t ldh, double damp_rel, float* D, int64_t* bad_pivot,
            void* ws, hipStream_t stream) {
    LdlWs w = carve(ws, d);
    const int64_t nbt = (d + kTile - 1) / kTile;
    if (nbt > 65535) return BAKRON_E_INVALID_ARG;
    hipLaunchKernelGGL(k_ldl_init, dim3(1), dim3(kThreads), 0, stream, H, d, ldh, damp_rel, w);
    hipLaunchKernelGGL(k_ldl_load, dim3((unsigned)nbt, (unsigned)nbt), dim3(kThreads), 0, stream,
                       H, d, ldh, w);
    const int64_t nsuper = (d + kSuper - 1) / kSuper;
    for (int64_t s = nsuper - 1; s >= 0; --s) {
        const int64_t s0 = s * kSuper, s1 = std::min<int64_t>(s0 + kSuper, d);
        for (int64_t k0 = ((s1 - 1) / 64) * 64; k0 >= s0; k0 -= 64) {
            const int nb = (int)std::min<int64_t>(64, d - k0);
            hipLaunchKernelGGL(k_ldl_diag, dim3(1), dim3(kThreads), 0, stream, d, k0, nb, w);
            if (k0 > 0) {
                hipLaunchKernelGGL(k_ldl_panel, dim3((unsigned)((k0 + 63) / 64)), dim3(kThreads),
                                   0, stream, d, k0, nb, w);
            }
            if (k0 > s0) {  // rows [s0, k0) of the super-panel, every column < k0
                const int64_t rt = (k0 - s0 + kTile - 1) / kTile, ct = (k0 + kTile - 1) / kTile;
                hipLaunchKernelGGL(k_ldl_update, dim3((unsigned)ct, (unsigned)rt), dim3(kThreads),
                                   0, stream, d, s0, k0, k0, k0, (int64_t)nb, w);
            }
        }
        if (s0 > 0) {
            const int64_t tt = (s0 + kTile - 1) / kTile;
            hipLaunchKernelGGL(k_ldl_update, dim3((unsigned)tt, (unsigned)tt), dim3(kThreads), 0,
                               stream, d, (int64_t)0, s0, s0, s0, s1 - s0, w);
        }
    }
    hipLaunchKernelGGL(k_ldl_store, dim3((unsigned)nbt, (unsigned)nbt), dim3(kThreads), 0, stream,
                       H, d, ldh, D, w);
    if (hipGetLastError() != hipSuccess) return BAKRON_E_DEVICE;
    int64_t info = -1;
    if (hipMemcpyAsync(&info, w.info, sizeof(int64_t), hipMemcpyDeviceToHost, stream) !=
        hipSuccess)
        return BAKRON_E_DEVICE;
    if (hipStreamSynchronize(stream) != hipSuccess) return BAKRON_E_DEVICE;
    if (bad_pivot) *bad_pivot = info;
    return info >= 0 ? BAKRON_E_NOT_SPD : BAKRON_OK;
}

}  // namespace bk
