// bk_ldl.hip -- damped LDL factorisation H + lambda I = (L + I) diag(D) (L + I)^T,
// L strictly upper (YAQA article, section 4, the factorisation paragraph;
// damping lambda = damp_rel * mean(diag H) as the factor estimates carry it,
// K-FAC tutorial on mlqm.cn, section 5).
//
// With J the index reversal, J H J = C' C'^T (lower Cholesky) gives H = C C^T
// with C = J C' J upper triangular; then L + I = C diag(C)^-1 and D = diag(C)^2.
// C is computed by a right-looking blocked Cholesky that runs from the LAST
// index block to the first, in fp64 on the device:
//   for each 64-wide block [k0, k1), last first:
//     diag   : C22 = reverse Cholesky of A[k0:k1, k0:k1] (one workgroup, LDS),
//              plus C22^-1 for the panel solve
//     panel  : C12 = A[0:k0, k0:k1] C22^-T  (rows independent)
//     update : A[0:k0, s0:k0] -= C12 C12[s0:k0]^T inside the current 256-wide
//              super-panel [s0, s1) (fp64 MFMA tiles)
//   and after each super-panel one trailing update of A[0:s0, 0:s0] with
//   K = s1 - s0 (fp64 MFMA tiles, upper triangle only).
// Only the upper triangle of the working copy is ever read or written.
#include <algorithm>

#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

constexpr int kSuper = 256;  // super-panel width (K of the big trailing updates)

struct LdlWs {
    double* A;     // d x d working copy (upper triangle used), ld = d
    double* CT;    // kSuper x d: CT[q][r] = C[r][s0 + q] of the current super-panel
    double* Cinv;  // 64 x 64 inverse of the current diagonal block's C22
    double* lam;   // damping lambda
    int64_t* info; // -1, or the first failing pivot index
};

static LdlWs carve(void* ws, int64_t d) {
    char* p = (char*)ws;
    LdlWs w;
    w.A = (double*)p;
    p += align256(sizeof(double) * (size_t)d * (size_t)d);
    w.CT = (double*)p;
    p += align256(sizeof(double) * (size_t)kSuper * (size_t)d);
    w.Cinv = (double*)p;
    p += align256(sizeof(double) * 64 * 64);
    w.lam = (double*)p;
    p += 256;
    w.info = (int64_t*)p;
    return w;
}

size_t ldl_workspace_bytes(int64_t d) {
    return align256(sizeof(double) * (size_t)d * (size_t)d) +
           align256(sizeof(double) * (size_t)kSuper * (size_t)d) + align256(sizeof(double) * 4096) +
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

// A = upper triangle of H (fp64) + lambda on the diagonal.
__global__ __launch_bounds__(kThreads) void k_ldl_load(const float* __restrict__ H, int64_t d,
                                                       int64_t ldh, LdlWs w) {
    const int64_t rt = blockIdx.y, ct = blockIdx.x;
    if (rt > ct) return;
    const double lam = *w.lam;
    for (int e = threadIdx.x; e < kTile * kTile; e += kThreads) {
        const int64_t i = rt * kTile + e / kTile, j = ct * kTile + e % kTile;
        if (i >= d || j >= d || i > j) continue;
        double v = (double)H[i * ldh + j];
        if (i == j) v += lam;
        w.A[i * d + j] = v;
    }
}

// Reverse Cholesky of the diagonal block A[k0:k0+nb, k0:k0+nb] (upper) in LDS,
// written back as C22, and C22^-1 into w.Cinv.
__global__ __launch_bounds__(kThreads) void k_ldl_diag(int64_t d, int64_t k0, int nb, LdlWs w) {
    if (*w.info >= 0) return;
    __shared__ double a[64][65];
    __shared__ double inv[64][65];
    const int t = threadIdx.x;
    for (int e = t; e < 64 * 64; e += kThreads) {
        const int i = e / 64, j = e % 64;
        a[i][j] = (i <= j && j < nb) ? w.A[(k0 + i) * d + k0 + j] : 0.0;
        inv[i][j] = 0.0;
    }
    __syncthreads();
    for (int jj = nb - 1; jj >= 0; --jj) {
        const double piv = a[jj][jj];
        if (!(piv > 0.0) || !(piv < INFINITY)) {  // uniform: every thread read the same value
            if (t == 0) *w.info = k0 + jj;
            return;
        }
        const double c = sqrt(piv);
        __syncthreads();
        if (t < jj) a[t][jj] /= c;
        if (t == 0) a[jj][jj] = c;
        __syncthreads();
        // a[ii][kk] -= a[ii][jj] * a[kk][jj] for ii <= kk < jj
        for (int e = t; e < jj * jj; e += kThreads) {
            const int ii = e / jj, kk = e % jj;
            if (ii <= kk) a[ii][kk] -= a[ii][jj] * a[kk][jj];
        }
        __syncthreads();
    }
    // inverse of the upper triangular C22, one column per thread
    if (t < nb) {
        const int j = t;
        inv[j][j] = 1.0 / a[j][j];
        for (int p = j - 1; p >= 0; --p) {
            double s = 0.0;
            for (int qq = p + 1; qq <= j; ++qq) s += a[p][qq] * inv[qq][j];
            inv[p][j] = -s / a[p][p];
        }
    }
    __syncthreads();
    for (int e = t; e < 64 * 64; e += kThreads) {
        const int i = e / 64, j = e % 64;
        if (i <= j && j < nb) w.A[(k0 + i) * d + k0 + j] = a[i][j];
        w.Cinv[e] = inv[i][j];
    }
}

// C12 = A[r0:r0+64, k0:k0+nb] C22^-T for rows r < k0; written back into A and,
// transposed, into CT rows (k0 - s0) .. (k0 - s0 + nb).
__global__ __launch_bounds__(kThreads) void k_ldl_panel(int64_t d, int64_t k0, int nb,
                                                        int64_t s0, LdlWs w) {
    if (*w.info >= 0) return;
    __shared__ double a[64][65];
    __shared__ double ci[64][65];
    __shared__ double out[64][65];
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    const int rows = (int)min<int64_t>(64, k0 - r0);
    for (int e = t; e < 64 * 64; e += kThreads) {
        const int i = e / 64, j = e % 64;
        a[i][j] = (i < rows && j < nb) ? w.A[(r0 + i) * d + k0 + j] : 0.0;
        ci[i][j] = w.Cinv[e];
    }
    __syncthreads();
    {
        const int rr = t >> 2;
        for (int p = t & 3; p < 64; p += 4) {
            double s = 0.0;
            for (int qq = p; qq < nb; ++qq) s += a[rr][qq] * ci[p][qq];
            out[rr][p] = s;
        }
    }
    __syncthreads();
    for (int e = t; e < 64 * 64; e += kThreads) {
        const int i = e / 64, j = e % 64;  // row-major write into A
        if (i < rows && j < nb) w.A[(r0 + i) * d + k0 + j] = out[i][j];
        const int p = e / 64, rr = e % 64;  // transposed write into CT
        if (rr < rows && p < nb) w.CT[(k0 - s0 + p) * d + r0 + rr] = out[rr][p];
    }
}

// A[r][c] -= sum_q CT[q0 + q][r] CT[q0 + q][c], q < K, over rows [0, rmax) and
// columns [c_lo, c_hi), upper triangle only (r <= c).
__global__ __launch_bounds__(kThreads) void k_ldl_update(int64_t d, int64_t rmax, int64_t c_lo,
                                                         int64_t c_hi, int64_t q0, int64_t K,
                                                         LdlWs w) {
    if (*w.info >= 0) return;
    const int64_t r0 = (int64_t)blockIdx.y * kTile;
    const int64_t c0 = c_lo + (int64_t)blockIdx.x * kTile;
    if (r0 > c0 + kTile - 1) return;  // tile entirely below the diagonal
    __shared__ GemmSmem<double> sm;
    const int R = (int)min<int64_t>(kTile, rmax - r0);
    const int Cn = (int)min<int64_t>(kTile, c_hi - c0);
    f64x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    const double* CT = w.CT + q0 * d;
    tile_gemm_f64(CT + r0, d, R, CT + c0, d, Cn, K, acc, sm);
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lr = acc64_row(bi, r), lc = acc64_col(bj);
                const int64_t gi = r0 + lr, gj = c0 + lc;
                if (lr < R && lc < Cn && gi <= gj) w.A[gi * d + gj] -= acc[bi][bj][r];
            }
}

// H <- L (strict upper, fp32), D on the diagonal, 0 below; D[] if requested.
__global__ __launch_bounds__(kThreads) void k_ldl_store(float* __restrict__ H, int64_t d,
                                                        int64_t ldh, float* __restrict__ D,
                                                        LdlWs w) {
    const int64_t rt = blockIdx.y, ct = blockIdx.x;
    for (int e = threadIdx.x; e < kTile * kTile; e += kThreads) {
        const int64_t i = rt * kTile + e / kTile, j = ct * kTile + e % kTile;
        if (i >= d || j >= d) continue;
        float v = 0.0f;
        if (i < j) {
            v = (float)(w.A[i * d + j] / w.A[j * d + j]);
        } else if (i == j) {
            const double c = w.A[j * d + j];
            v = (float)(c * c);
            if (D) D[j] = v;
        }
        H[i * ldh + j] = v;
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
                                   0, stream, d, k0, nb, s0, w);
            }
            if (k0 > s0) {
                const int64_t ct = (k0 - s0 + kTile - 1) / kTile, rt = (k0 + kTile - 1) / kTile;
                hipLaunchKernelGGL(k_ldl_update, dim3((unsigned)ct, (unsigned)rt), dim3(kThreads),
                                   0, stream, d, k0, s0, k0, k0 - s0, (int64_t)nb, w);
            }
        }
        if (s0 > 0) {
            const int64_t tt = (s0 + kTile - 1) / kTile;
            hipLaunchKernelGGL(k_ldl_update, dim3((unsigned)tt, (unsigned)tt), dim3(kThreads), 0,
                               stream, d, s0, (int64_t)0, s0, (int64_t)0, s1 - s0, w);
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
