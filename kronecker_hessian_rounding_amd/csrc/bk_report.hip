// bk_report.hip -- per-layer bound and sensitivity report.
//
// The YAQA article (section 4) bounds the proxy loss of the rule by
// tr(D_I) tr(D_O) sigma^2, with D_I and D_O the LDL pivots of the damped
// factors and sigma^2 the rounding noise; for nearest rounding without
// clamping |eta_ij| <= s_i / 2, which gives the sharp form
// sum_i D_O,i s_i^2 / 4 * tr(D_I) and the page's form with sigma = max_i s_i / 2.
// The KronQ page (sensitivity) scores a layer by tr(A) tr(G), the traces of
// the two undamped factors. One workgroup sums everything in fp64.
#include <cmath>

#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

__device__ __forceinline__ double block_sum(double v, double* red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double s = 0.0;
    for (int i = 0; i < kThreads / 64; ++i) s += red[i];
    __syncthreads();
    return s;
}

__global__ __launch_bounds__(kThreads) void k_layer_report(int64_t m, int64_t n, const float* __restrict__ DO,
                                                           const float* __restrict__ DI,
                                                           const float* __restrict__ scales,
                                                           const float* __restrict__ HI, int64_t ldhi,
                                                           const float* __restrict__ HO, int64_t ldho,
                                                           double* __restrict__ out) {
    __shared__ double red[kThreads / 64];
    double tdo = 0.0, tdi = 0.0, sharp = 0.0, thi = 0.0, tho = 0.0, smax = 0.0;
    for (int64_t i = threadIdx.x; i < m; i += kThreads) {
        const double d = DO ? (double)DO[i] : 1.0;
        const double s = (double)scales[i];
        tdo += d;
        sharp += d * s * s * 0.25;
        smax = fmax(smax, fabs(s));
        if (HO) tho += (double)HO[i * (ldho + 1)];
    }
    for (int64_t j = threadIdx.x; j < n; j += kThreads) {
        tdi += (double)DI[j];
        if (HI) thi += (double)HI[j * (ldhi + 1)];
    }
    tdo = block_sum(tdo, red);
    tdi = block_sum(tdi, red);
    sharp = block_sum(sharp, red);
    thi = block_sum(thi, red);
    tho = block_sum(tho, red);
    for (int o = 32; o > 0; o >>= 1) smax = fmax(smax, __shfl_xor(smax, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = smax;
    __syncthreads();
    if (threadIdx.x == 0) {
        double mx = 0.0;
        for (int i = 0; i < kThreads / 64; ++i) mx = fmax(mx, red[i]);
        out[0] = tdo;
        out[1] = tdi;
        out[2] = sharp * tdi;
        out[3] = tdi * tdo * mx * mx * 0.25;
        out[4] = HI ? thi : NAN;
        out[5] = HO ? tho : NAN;
        out[6] = out[4] * out[5];
    }
}

int launch_layer_report(int64_t m, int64_t n, const float* DO, const float* DI, const float* scales,
                        const float* HI, int64_t ldhi, const float* HO, int64_t ldho, double* out,
                        hipStream_t stream) {
    hipLaunchKernelGGL(k_layer_report, dim3(1), dim3(kThreads), 0, stream, m, n, DO, DI, scales, HI, ldhi, HO,
                       ldho, out);
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

}  // namespace bk
