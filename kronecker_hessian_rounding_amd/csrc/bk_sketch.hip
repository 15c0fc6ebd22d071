// bk_sketch.hip -- per-token weights of the Sketch A factor estimate.
//
// Sketch A (YAQA article, section 3) takes the tokens of a sequence as
// independent and updates the two factors in turn, each token weighted by the
// other factor's quadratic form:
//   (H_I)_i = E_t[x_t^T x_t w_t],  w_t = g_t (H_O)_{i-1} g_t^T / ||(H_O)_{i-1}||_F^2,
// and the same with the roles of x and g exchanged. This file computes the
// weights w_t = y_t H y_t^T / ||H||_F^2 for the rows y_t of Y (T x d); the
// weighted accumulation itself is the Hessian SYRK with every token scaled by
// sqrt(w_t) in its pre-pass (bk_accum.hip).
//
// The quadratic forms are the row sums of (Y H) o Y. H is symmetric, so with
// 64-wide index blocks C, C' the form is
//   y H y^T = sum_C y_C (H_CC y_C^T + 2 sum_{C' > C} H_CC' y_C'^T),
// half the products of the dense form. H_CC' for C' > C is read as the rows
// C' of column block C (H_C'C, the lower triangle), so every product is a TN
// product of H and Y^T (both K-major): Y is first transposed into the
// workspace, then tile (C, t) is two fp32 MFMA tile GEMMs, over K = C (the
// diagonal block) and over K = the blocks below it, whose epilogue multiplies
// by Y^T and sums the tile's 64 rows, giving one partial per token and column
// tile. A last kernel adds the partials in tile order (deterministic) and
// divides by ||H||_F^2, itself summed in fp64 in a fixed order.
#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

constexpr int kQKT = 32;  // k-slice depth of the quadratic-form tile GEMM

struct TokenWs {
    float* yt;    // d x T, Y transposed
    float* part;  // ceil(d / 64) x T partial quadratic forms
    double* fro;  // 256 partial sums of H^2, then the total at [256]
};

inline size_t tw_yt_bytes(int64_t T, int64_t d) { return align256(sizeof(float) * (size_t)T * (size_t)d); }
inline size_t tw_part_bytes(int64_t T, int64_t d) {
    return align256(sizeof(float) * (size_t)((d + kTile - 1) / kTile) * (size_t)T);
}
size_t token_weights_workspace_bytes(int64_t T, int64_t d) {
    return tw_yt_bytes(T, d) + tw_part_bytes(T, d) + align256(sizeof(double) * 257);
}

// Y (T x d, ldy) -> Yt (d x T): 64 x 64 tiles through LDS, both sides coalesced.
__global__ __launch_bounds__(kThreads) void k_tw_transpose(const float* __restrict__ Y, int64_t T, int64_t d,
                                                           int64_t ldy, float* __restrict__ Yt) {
    __shared__ float tile[64][65];
    const int64_t t0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += kThreads / 64) {
        const int64_t t = t0 + r, c = c0 + tx;
        tile[r][tx] = (t < T && c < d) ? Y[t * ldy + c] : 0.0f;
    }
    __syncthreads();
    for (int r = ty; r < 64; r += kThreads / 64) {
        const int64_t c = c0 + r, t = t0 + tx;
        if (c < d && t < T) Yt[c * T + t] = tile[tx][r];
    }
}

// Block b: sum of H_ij^2 over the elements b, b + 256, ... (row-major order).
__global__ __launch_bounds__(kThreads) void k_tw_fro(const float* __restrict__ H, int64_t d, int64_t ldh,
                                                     double* __restrict__ fro) {
    __shared__ double red[kThreads / 64];
    double s = 0.0;
    const int64_t total = d * d;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += (int64_t)gridDim.x * kThreads) {
        const double h = (double)H[(e / d) * ldh + e % d];
        s += h * h;
    }
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int i = 0; i < kThreads / 64; ++i) t += red[i];
        fro[blockIdx.x] = t;
    }
}

// Tile (t-tile, c-tile) = (blockIdx.x, blockIdx.y):
//   part[ct][t] = sum_{c in tile} Y^T[c][t] ((H_CC Y_C^T)[c][t] + 2 sum_{C' > C} (H_CC' Y_C'^T)[c][t]).
// Column tiles are blockIdx.y, so the tiles with the longest K (C = 0) start first.
__global__ __launch_bounds__(kThreads) void k_tw_qform(const float* __restrict__ H, int64_t ldh,
                                                       const float* __restrict__ Yt, int64_t T, int64_t d,
                                                       float* __restrict__ part) {
    __shared__ GemmSmemF32<kQKT> sm;
    __shared__ float red[2][2][64];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kTile, c0 = (int64_t)blockIdx.y * kTile;
    const int R = (int)min<int64_t>(kTile, d - c0), Cn = (int)min<int64_t>(kTile, T - t0);
    f32x16 accd, acco;
#pragma unroll
    for (int v = 0; v < 16; ++v) accd[v] = acco[v] = 0.0f;
    // C[r][c] = sum_k A[k][r] B[k][c] with A = rows k of H's column block c0 and B = rows k
    // of Y^T (token block t0): k in the diagonal block, then k below it
    tile_gemm_f32<kQKT>(H + c0 * ldh + c0, ldh, R, Yt + c0 * T + t0, T, Cn, R, accd, sm, true, tid);
    const int64_t kb = c0 + kTile;
    if (kb < d) {
        __syncthreads();  // the shared memory is reused
        tile_gemm_f32<kQKT>(H + kb * ldh + c0, ldh, R, Yt + kb * T + t0, T, Cn, d - kb, acco, sm, true, tid);
    }
    const int col = acc32_col(tid);
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int row = acc32_row(v, tid);
        if (row < R && col < Cn) s = fmaf(fmaf(2.0f, acco[v], accd[v]), Yt[(c0 + row) * T + t0 + col], s);
    }
    const int w = tid >> 6, lane = tid & 63;
    red[w >> 1][lane >> 5][col] = s;
    __syncthreads();
    if (tid < 64 && tid < Cn)
        part[(int64_t)blockIdx.y * T + t0 + tid] = (red[0][0][tid] + red[0][1][tid]) + (red[1][0][tid] + red[1][1][tid]);
}

// w_t = (sum over column tiles of part[.][t], in order) / ||H||_F^2; with H = I
// (part == nullptr) w_t = sum_k y_tk^2 / d.
__global__ __launch_bounds__(kThreads) void k_tw_finish(const float* __restrict__ Y, int64_t T, int64_t d,
                                                        int64_t ldy, const float* __restrict__ part,
                                                        int64_t nct, const double* __restrict__ fro,
                                                        int nfro, float* __restrict__ w) {
    __shared__ double inv;
    if (threadIdx.x == 0 && part) {
        double s = 0.0;
        for (int i = 0; i < nfro; ++i) s += fro[i];
        inv = 1.0 / s;
    }
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= T) return;
    if (part) {
        double q = 0.0;
        for (int64_t ct = 0; ct < nct; ++ct) q += (double)part[ct * T + t];
        w[t] = (float)(q * inv);
    } else {
        double q = 0.0;
        for (int64_t k = 0; k < d; ++k) {
            const double y = (double)Y[t * ldy + k];
            q += y * y;
        }
        w[t] = (float)(q / (double)d);
    }
}

int launch_token_weights(const float* Y, int64_t T, int64_t d, int64_t ldy, const float* H, int64_t ldh,
                         float* w, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (T == 0) return BAKRON_OK;
    if (!H) {
        hipLaunchKernelGGL(k_tw_finish, dim3((unsigned)((T + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                           stream, Y, T, d, ldy, (const float*)nullptr, (int64_t)0, (const double*)nullptr, 0, w);
        return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
    }
    if (!ws || ws_bytes < token_weights_workspace_bytes(T, d)) return BAKRON_E_WORKSPACE;
    char* base = (char*)ws;
    TokenWs tw;
    tw.yt = (float*)base;
    tw.part = (float*)(base + tw_yt_bytes(T, d));
    tw.fro = (double*)(base + tw_yt_bytes(T, d) + tw_part_bytes(T, d));
    const int64_t nct = (d + kTile - 1) / kTile, ntt = (T + kTile - 1) / kTile;
    if (nct > 65535 || ntt > 0x7fffffff) return BAKRON_E_INVALID_ARG;
    hipLaunchKernelGGL(k_tw_transpose, dim3((unsigned)ntt, (unsigned)nct), dim3(kThreads), 0, stream, Y, T, d,
                       ldy, tw.yt);
    hipLaunchKernelGGL(k_tw_fro, dim3(256), dim3(kThreads), 0, stream, H, d, ldh, tw.fro);
    hipLaunchKernelGGL(k_tw_qform, dim3((unsigned)ntt, (unsigned)nct), dim3(kThreads), 0, stream, H, ldh, tw.yt,
                       T, d, tw.part);
    hipLaunchKernelGGL(k_tw_finish, dim3((unsigned)((T + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                       Y, T, d, ldy, (const float*)tw.part, nct, (const double*)tw.fro, 256, w);
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

}  // namespace bk
