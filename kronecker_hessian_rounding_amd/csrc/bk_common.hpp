// bk_common.hpp -- device building blocks shared by the libbakron kernels (gfx950).
//
//  * 64x64 output tiles of C[r][c] (+)= sum_k A[k][r] * B[k][c] ("TN" form: both
//    operands stored K-major, so the rows of A and B are contiguous along the
//    output index). Every contraction in the library has this shape: the
//    Hessian factor X^T X, the far-field feedback products of the rounding
//    solve, and the trailing updates of the LDL factorisation.
//    fp32 tiles use v_mfma_f32_32x32x2_f32, fp64 tiles v_mfma_f64_16x16x4_f64.
//    A workgroup of 256 threads (4 waves) owns one 64x64 tile; wave w owns the
//    32x32 quadrant (w/2, w%2). Operand k-slices are staged in LDS, double
//    buffered, with the next slice fetched into registers during the MFMAs.
//  * the base quantiser and the counter-based uniform draw.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;      // output tile edge (also the rounding leaf edge)
constexpr int kThreads = 256;  // threads per workgroup for tile kernels
constexpr int kKT = 16;        // k-slice staged in LDS per step

// ---------------------------------------------------------------------------
// LDS staging for a tile GEMM (double buffered k-slices of A and B)
// ---------------------------------------------------------------------------
template <typename T>
struct GemmSmem {
    T a[2][kKT][kTile];
    T b[2][kKT][kTile];
};

// Load one k-slice element set for this thread: rows k0 + lk, 4 consecutive
// output columns lc..lc+3 (fp32) or 2 sets of 2 (fp64 uses 4 scalars too).
template <typename T>
__device__ __forceinline__ void gemm_load_slice(const T* __restrict__ A, int64_t lda, int R,
                                                int64_t K, int64_t k0, int lk, int lc, T (&ra)[4]) {
    const int64_t k = k0 + lk;
    if (k < K) {
        const T* p = A + k * lda + lc;
        if (lc + 3 < R) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ra[e] = p[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) ra[e] = (lc + e < R) ? p[e] : T(0);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ra[e] = T(0);
    }
}

// ---------------------------------------------------------------------------
// fp32 64x64 tile over KT-deep k-slices kept in LDS as loaded ([k][column]):
// 16-byte stores of consecutive columns, and per MFMA each half-wave reads 32
// consecutive columns of one k-row, so neither side has bank conflicts. The
// next slice is fetched into registers while the current one feeds the MFMAs,
// and the MFMA operands are read from LDS two k-steps ahead.
// ---------------------------------------------------------------------------
template <int KT>
struct GemmSmemF32 {
    float a[2][KT][kTile];
    float b[2][KT][kTile];
};

// Thread t loads rows k0 + (t >> 4) + 16 h (h < KT / 16), columns 4 (t & 15)..+3,
// of a K-major operand; zeros outside [0, K) x [0, R). fast: the tile is 64
// columns wide and 16-byte aligned, so each row is one vector load (rows past
// K are clamped here and zeroed by the store, which keeps the loads in flight).
template <int KT, bool kFast>
__device__ __forceinline__ void slice_load_f32(const float* __restrict__ A, int64_t lda, int R,
                                               int64_t K, int64_t k0, f32x4 (&v)[KT / 16]) {
    const int t = threadIdx.x;
    const int c4 = (t & 15) << 2;
#pragma unroll
    for (int h = 0; h < KT / 16; ++h) {
        const int64_t k = k0 + (t >> 4) + 16 * h;
        if (kFast) {
            v[h] = *reinterpret_cast<const f32x4*>(A + min(k, K - 1) * lda + c4);
        } else {
            const float* p = A + k * lda + c4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[h][e] = (k < K && c4 + e < R) ? p[e] : 0.0f;
        }
    }
}

// stores a loaded slice; rows k0 + r >= K are written as zeros
template <int KT>
__device__ __forceinline__ void slice_store_f32(float (&dst)[KT][kTile], const f32x4 (&v)[KT / 16],
                                                int64_t K, int64_t k0) {
    const int t = threadIdx.x;
    const int c4 = (t & 15) << 2;
#pragma unroll
    for (int h = 0; h < KT / 16; ++h) {
        const int r = (t >> 4) + 16 * h;
        *reinterpret_cast<f32x4*>(&dst[r][c4]) = k0 + r < K ? v[h] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
}

template <int KT, bool kFast>
__device__ __forceinline__ void tile_gemm_f32_impl(const float* __restrict__ A, int64_t lda, int R,
                                                   const float* __restrict__ B, int64_t ldb, int Cn,
                                                   int64_t K, f32x16& acc, GemmSmemF32<KT>& sm,
                                                   bool active) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int ra = (w >> 1) * 32 + (lane & 31);
    const int rb = (w & 1) * 32 + (lane & 31);
    const int kh = lane >> 5;
    const int64_t nk = (K + KT - 1) / KT;
    f32x4 va[KT / 16], vb[KT / 16];
    if (active) {
        slice_load_f32<KT, kFast>(A, lda, R, K, 0, va);
        slice_load_f32<KT, kFast>(B, ldb, Cn, K, 0, vb);
        slice_store_f32<KT>(sm.a[0], va, K, 0);
        slice_store_f32<KT>(sm.b[0], vb, K, 0);
    }
    __syncthreads();
    for (int64_t it = 0; it < nk; ++it) {
        const int cur = (int)(it & 1);
        const bool more = active && it + 1 < nk;
        if (!active) {
            __syncthreads();
            continue;
        }
        if (more) {
            slice_load_f32<KT, kFast>(A, lda, R, K, (it + 1) * KT, va);
            slice_load_f32<KT, kFast>(B, ldb, Cn, K, (it + 1) * KT, vb);
        }
        float fa[3], fb[3];
        fa[0] = sm.a[cur][kh][ra];
        fb[0] = sm.b[cur][kh][rb];
        fa[1] = sm.a[cur][2 + kh][ra];
        fb[1] = sm.b[cur][2 + kh][rb];
#pragma unroll
        for (int s = 0; s < KT / 2; ++s) {
            if (s + 2 < KT / 2) {
                fa[(s + 2) % 3] = sm.a[cur][2 * (s + 2) + kh][ra];
                fb[(s + 2) % 3] = sm.b[cur][2 * (s + 2) + kh][rb];
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the reads two steps ahead of the MFMAs
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s % 3], fb[s % 3], acc, 0, 0, 0);
        }
        if (more) {
            slice_store_f32<KT>(sm.a[cur ^ 1], va, K, (it + 1) * KT);
            slice_store_f32<KT>(sm.b[cur ^ 1], vb, K, (it + 1) * KT);
        }
        __syncthreads();
    }
}

// acc += A^T B over K for the 64x64 tile: A element (k, r) at A[k*lda + r]
// with r < R valid (others read as 0), B (k, c) at B[k*ldb + c] with c < Cn;
// wave w owns the 32x32 quadrant (w / 2, w % 2). Threads 0..255 compute; with
// active = false a thread (of a larger workgroup) only takes part in the
// barriers. Every thread of the workgroup must call it.
template <int KT>
__device__ __forceinline__ void tile_gemm_f32(const float* __restrict__ A, int64_t lda, int R,
                                              const float* __restrict__ B, int64_t ldb, int Cn,
                                              int64_t K, f32x16& acc, GemmSmemF32<KT>& sm,
                                              bool active = true) {
    if (K <= 0) return;
    const bool fast = R == kTile && Cn == kTile && (lda & 3) == 0 && (ldb & 3) == 0 &&
                      ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    if (fast) tile_gemm_f32_impl<KT, true>(A, lda, R, B, ldb, Cn, K, acc, sm, active);
    else tile_gemm_f32_impl<KT, false>(A, lda, R, B, ldb, Cn, K, acc, sm, active);
}

// Position (row, col) inside the 64x64 tile of element v (0..15) of this
// lane's fp32 accumulator (32x32x2 output layout: col = lane % 32,
// row = 8*(v/4) + 4*(lane/32) + v%4 within the wave's quadrant).
__device__ __forceinline__ int acc32_row(int v) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    return (w >> 1) * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int acc32_col() {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    return (w & 1) * 32 + (lane & 31);
}

// fp64: acc[4] (2x2 blocks of 16x16 per wave quadrant) += A^T B over K.
__device__ __forceinline__ void tile_gemm_f64(const double* __restrict__ A, int64_t lda, int R,
                                              const double* __restrict__ B, int64_t ldb, int Cn,
                                              int64_t K, f64x4 (&acc)[2][2], GemmSmem<double>& sm) {
    if (K <= 0) return;
    const int t = threadIdx.x;
    const int lk = t >> 4;
    const int lc = (t & 15) << 2;
    const int lane = t & 63;
    const int w = t >> 6;
    const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
    double ra[4], rb[4];
    const int64_t nk = (K + kKT - 1) / kKT;
    gemm_load_slice<double>(A, lda, R, K, 0, lk, lc, ra);
    gemm_load_slice<double>(B, ldb, Cn, K, 0, lk, lc, rb);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        sm.a[0][lk][lc + e] = ra[e];
        sm.b[0][lk][lc + e] = rb[e];
    }
    __syncthreads();
    for (int64_t it = 0; it < nk; ++it) {
        const int cur = (int)(it & 1);
        const bool more = (it + 1 < nk);
        if (more) {
            gemm_load_slice<double>(A, lda, R, K, (it + 1) * kKT, lk, lc, ra);
            gemm_load_slice<double>(B, ldb, Cn, K, (it + 1) * kKT, lk, lc, rb);
        }
#pragma unroll
        for (int kk = 0; kk < kKT; kk += 4) {
            const int kr = kk + (lane >> 4);
            const double a0 = sm.a[cur][kr][wr + (lane & 15)];
            const double a1 = sm.a[cur][kr][wr + 16 + (lane & 15)];
            const double b0 = sm.b[cur][kr][wc + (lane & 15)];
            const double b1 = sm.b[cur][kr][wc + 16 + (lane & 15)];
            acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (more) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sm.a[cur ^ 1][lk][lc + e] = ra[e];
                sm.b[cur ^ 1][lk][lc + e] = rb[e];
            }
        }
        __syncthreads();
    }
}

// Position of element r (0..3) of block (bi, bj) of this lane's fp64 accumulator
// (v_mfma_f64_16x16x4_f64 output layout, checked on gfx950: col = lane % 16,
// row = lane / 16 + 4 r).
__device__ __forceinline__ int acc64_row(int bi, int r) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    return (w >> 1) * 32 + bi * 16 + (lane >> 4) + 4 * r;
}
__device__ __forceinline__ int acc64_col(int bj) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    return (w & 1) * 32 + bj * 16 + (lane & 15);
}

// ---------------------------------------------------------------------------
// Counter-based uniform draw: SplitMix64 (Steele, Lea, Flood 2014) output
// number idx+1 of a stream seeded with `seed`; the top 24 bits as u in [0, 1).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float uniform24(uint64_t seed, uint64_t idx) {
    uint64_t z = seed + (idx + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (float)(uint32_t)(z >> 40) * (1.0f / 16777216.0f);
}

// Sum over the 4 lanes of a quad (lanes 4k..4k+3), result in every lane.
__device__ __forceinline__ float quad_sum(float x) {
    // quad_perm [1,0,3,2] then [2,3,0,1]
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1,
                                                                0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E,
                                                                0xF, 0xF, false));
    return x;
}

}  // namespace bk
