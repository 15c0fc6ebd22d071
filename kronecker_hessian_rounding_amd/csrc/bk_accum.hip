// bk_accum.hip -- Hessian factor accumulation H <- beta H + alpha X^T X (fp32 MFMA).
//
// The Kronecker factors are second moments over tokens: H_I = E[x^T x] of the
// layer inputs and H_O = E[g^T g] of the output gradients (YAQA article,
// section 3; K-FAC tutorial on mlqm.cn, section 5). With X stored as T x d
// (one token per row), X^T X is a contraction over T whose operands are both
// K-major, so each 64x64 tile of H is one TN tile GEMM. Only tiles on or above
// the diagonal are computed; each writes its tile and the mirrored tile, and a
// diagonal tile writes its upper half and mirrors it, so H is exactly
// symmetric.
#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

__global__ __launch_bounds__(kThreads) void k_syrk(const float* __restrict__ X, int64_t T,
                                                   int64_t d, int64_t ldx, float alpha,
                                                   float beta, float* __restrict__ H,
                                                   int64_t ldh, int64_t nb) {
    __shared__ GemmSmem<float> sm;
    // tile id -> (bi, bj), bi <= bj, row-major over the upper triangle
    const int64_t id = blockIdx.x;
    auto start = [nb](int64_t b) { return b * (2 * nb - b + 1) / 2; };
    const double q = (double)(2 * nb + 1);
    int64_t bi = (int64_t)((q - sqrt(q * q - 8.0 * (double)id)) * 0.5);
    if (bi < 0) bi = 0;
    while (bi + 1 < nb && start(bi + 1) <= id) ++bi;
    while (bi > 0 && start(bi) > id) --bi;
    const int64_t bj = bi + (id - start(bi));

    const int64_t r0 = bi * kTile, c0 = bj * kTile;
    const int R = (int)min<int64_t>(kTile, d - r0);
    const int Cn = (int)min<int64_t>(kTile, d - c0);
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    tile_gemm_f32(X + r0, ldx, R, X + c0, ldx, Cn, T, acc, sm);

    const int c = acc32_col();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int r = acc32_row(v);
        if (r >= R || c >= Cn) continue;
        if (bi == bj && r > c) continue;
        const int64_t gi = r0 + r, gj = c0 + c;
        float val = alpha * acc[v];
        if (beta != 0.0f) val = fmaf(beta, H[gi * ldh + gj], val);
        H[gi * ldh + gj] = val;
        if (gi != gj) H[gj * ldh + gi] = val;
    }
}

int launch_hessian_accum(const float* X, int64_t T, int64_t d, int64_t ldx, float alpha,
                         float beta, float* H, int64_t ldh, hipStream_t stream) {
    const int64_t nb = (d + kTile - 1) / kTile;
    const int64_t tiles = nb * (nb + 1) / 2;
    if (tiles > 0x7fffffff) return BAKRON_E_INVALID_ARG;
    hipLaunchKernelGGL(k_syrk, dim3((unsigned)tiles), dim3(kThreads), 0, stream, X, T, d, ldx,
                       alpha, beta, H, ldh, nb);
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

}  // namespace bk
