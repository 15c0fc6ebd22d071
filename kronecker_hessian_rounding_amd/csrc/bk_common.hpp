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
//  * the base quantiser and the counter-based draws (SplitMix64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kTile = 64;      // output tile edge (also the rounding leaf edge)
constexpr int kThreads = 256;  // threads per workgroup for tile kernels

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
                                               int64_t K, int64_t k0, f32x4 (&v)[KT / 16], int t) {
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
                                                int64_t K, int64_t k0, int t) {
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
                                                   bool active, int tid) {
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int ra = (w >> 1) * 32 + (lane & 31);
    const int rb = (w & 1) * 32 + (lane & 31);
    const int kh = lane >> 5;
    const int64_t nk = (K + KT - 1) / KT;
    f32x4 va[KT / 16], vb[KT / 16];
    if (active) {
        slice_load_f32<KT, kFast>(A, lda, R, K, 0, va, tid);
        slice_load_f32<KT, kFast>(B, ldb, Cn, K, 0, vb, tid);
        slice_store_f32<KT>(sm.a[0], va, K, 0, tid);
        slice_store_f32<KT>(sm.b[0], vb, K, 0, tid);
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
            slice_load_f32<KT, kFast>(A, lda, R, K, (it + 1) * KT, va, tid);
            slice_load_f32<KT, kFast>(B, ldb, Cn, K, (it + 1) * KT, vb, tid);
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
            slice_store_f32<KT>(sm.a[cur ^ 1], va, K, (it + 1) * KT, tid);
            slice_store_f32<KT>(sm.b[cur ^ 1], vb, K, (it + 1) * KT, tid);
        }
        __syncthreads();
    }
}

// acc += A^T B over K for the 64x64 tile: A element (k, r) at A[k*lda + r]
// with r < R valid (others read as 0), B (k, c) at B[k*ldb + c] with c < Cn;
// wave w owns the 32x32 quadrant (w / 2, w % 2). Threads 0..255 compute; with
// active = false a thread (of a larger workgroup) only takes part in the
// barriers. Every thread of the workgroup must call it; tid is its thread
// index (passed in so that a caller looping over tasks can keep the index
// arithmetic inside the loop).
template <int KT>
__device__ __forceinline__ void tile_gemm_f32(const float* __restrict__ A, int64_t lda, int R,
                                              const float* __restrict__ B, int64_t ldb, int Cn,
                                              int64_t K, f32x16& acc, GemmSmemF32<KT>& sm,
                                              bool active, int tid) {
    if (K <= 0) return;
    const bool fast = R == kTile && Cn == kTile && (lda & 3) == 0 && (ldb & 3) == 0 &&
                      ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    if (fast) tile_gemm_f32_impl<KT, true>(A, lda, R, B, ldb, Cn, K, acc, sm, active, tid);
    else tile_gemm_f32_impl<KT, false>(A, lda, R, B, ldb, Cn, K, acc, sm, active, tid);
}

// Position (row, col) inside the 64x64 tile of element v (0..15) of this
// lane's fp32 accumulator (32x32x2 output layout: col = lane % 32,
// row = 8*(v/4) + 4*(lane/32) + v%4 within the wave's quadrant).
__device__ __forceinline__ int acc32_row(int v, int tid) {
    const int lane = tid & 63, w = tid >> 6;
    return (w >> 1) * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int acc32_col(int tid) {
    const int lane = tid & 63, w = tid >> 6;
    return (w & 1) * 32 + (lane & 31);
}

// ---------------------------------------------------------------------------
// fp64 64x64 tile over KT-deep k-slices (double buffered, [k][column] as
// loaded); same structure as the fp32 tile: loads of the next slice in
// flight during the MFMAs, MFMA operands read one k-step ahead.
// ---------------------------------------------------------------------------
// threadIdx.x through an opaque move: what is derived from it is computed where
// it is used, not hoisted out of a persistent kernel's task loop (where it would
// hold registers across every task)
__device__ __forceinline__ int tid_opaque() {
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"((int)threadIdx.x));
    return r;
}

template <int KT>
struct GemmSmemF64 {
    double a[2][KT][kTile];
    double b[2][KT][kTile];
};

// Thread t loads 16-byte pairs: rows k0 + (t >> 5) + 8 u (u < KT / 8), columns
// 2 (t & 31), +1; zeros outside [0, K) x [0, R). kFast: 64 columns, 16-byte
// aligned rows (rows past K clamped here, zeroed by the store).
template <int KT, bool kFast>
__device__ __forceinline__ void slice_load_f64(const double* __restrict__ A, int64_t lda, int R,
                                               int64_t K, int64_t k0, f64x2 (&v)[KT / 8], int t) {
    const int c2 = (t & 31) << 1;
#pragma unroll
    for (int u = 0; u < KT / 8; ++u) {
        const int64_t k = k0 + (t >> 5) + 8 * u;
        if (kFast) {
            v[u] = *reinterpret_cast<const f64x2*>(A + min(k, K - 1) * lda + c2);
        } else {
            const double* p = A + k * lda + c2;
#pragma unroll
            for (int e = 0; e < 2; ++e) v[u][e] = (k < K && c2 + e < R) ? p[e] : 0.0;
        }
    }
}

template <int KT>
__device__ __forceinline__ void slice_store_f64(double (&dst)[KT][kTile], const f64x2 (&v)[KT / 8],
                                                int64_t K, int64_t k0, int t) {
    const int c2 = (t & 31) << 1;
#pragma unroll
    for (int u = 0; u < KT / 8; ++u) {
        const int r = (t >> 5) + 8 * u;
        *reinterpret_cast<f64x2*>(&dst[r][c2]) = k0 + r < K ? v[u] : f64x2{0.0, 0.0};
    }
}

template <int KT, bool kFast>
__device__ __forceinline__ void tile_gemm_f64_impl(const double* __restrict__ A, int64_t lda, int R,
                                                   const double* __restrict__ B, int64_t ldb, int Cn,
                                                   int64_t K, f64x4 (&acc)[2][2], GemmSmemF64<KT>& sm) {
    const int tid = tid_opaque();
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int ra = (w >> 1) * 32 + (lane & 15);
    const int rb = (w & 1) * 32 + (lane & 15);
    const int kq = lane >> 4;
    const int64_t nk = (K + KT - 1) / KT;
    f64x2 va[KT / 8], vb[KT / 8];
    slice_load_f64<KT, kFast>(A, lda, R, K, 0, va, tid);
    slice_load_f64<KT, kFast>(B, ldb, Cn, K, 0, vb, tid);
    slice_store_f64<KT>(sm.a[0], va, K, 0, tid);
    slice_store_f64<KT>(sm.b[0], vb, K, 0, tid);
    __syncthreads();
    for (int64_t it = 0; it < nk; ++it) {
        const int cur = (int)(it & 1);
        const bool more = it + 1 < nk;
        if (more) {
            slice_load_f64<KT, kFast>(A, lda, R, K, (it + 1) * KT, va, tid);
            slice_load_f64<KT, kFast>(B, ldb, Cn, K, (it + 1) * KT, vb, tid);
        }
        double fa[2][2], fb[2][2];
        fa[0][0] = sm.a[cur][kq][ra];
        fa[0][1] = sm.a[cur][kq][ra + 16];
        fb[0][0] = sm.b[cur][kq][rb];
        fb[0][1] = sm.b[cur][kq][rb + 16];
#pragma unroll
        for (int s = 0; s < KT / 4; ++s) {
            const int c = s & 1;
            if (s + 1 < KT / 4) {
                const int kr = 4 * (s + 1) + kq;
                fa[c ^ 1][0] = sm.a[cur][kr][ra];
                fa[c ^ 1][1] = sm.a[cur][kr][ra + 16];
                fb[c ^ 1][0] = sm.b[cur][kr][rb];
                fb[c ^ 1][1] = sm.b[cur][kr][rb + 16];
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the reads one step ahead of the MFMAs
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 2; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[c][bi], fb[c][bj], acc[bi][bj], 0, 0, 0);
        }
        if (more) {
            slice_store_f64<KT>(sm.a[cur ^ 1], va, K, (it + 1) * KT, tid);
            slice_store_f64<KT>(sm.b[cur ^ 1], vb, K, (it + 1) * KT, tid);
        }
        __syncthreads();
    }
}

// fp64: acc[bi][bj] (2x2 blocks of 16x16 per wave quadrant) += A^T B over K,
// A element (k, r) at A[k*lda + r] (r < R), B (k, c) at B[k*ldb + c] (c < Cn).
// All 256 threads of the workgroup must call it.
template <int KT>
__device__ __forceinline__ void tile_gemm_f64(const double* __restrict__ A, int64_t lda, int R,
                                              const double* __restrict__ B, int64_t ldb, int Cn,
                                              int64_t K, f64x4 (&acc)[2][2], GemmSmemF64<KT>& sm) {
    if (K <= 0) return;
    const bool fast = R == kTile && Cn == kTile && (lda & 1) == 0 && (ldb & 1) == 0 &&
                      ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    if (fast) tile_gemm_f64_impl<KT, true>(A, lda, R, B, ldb, Cn, K, acc, sm);
    else tile_gemm_f64_impl<KT, false>(A, lda, R, B, ldb, Cn, K, acc, sm);
}

// Position of element r (0..3) of block (bi, bj) of this lane's fp64 accumulator
// (v_mfma_f64_16x16x4_f64 output layout, checked on gfx950: col = lane % 16,
// row = lane / 16 + 4 r).
__device__ __forceinline__ int acc64_row(int bi, int r) {
    const int tid = tid_opaque(), lane = tid & 63, w = tid >> 6;
    return (w >> 1) * 32 + bi * 16 + (lane >> 4) + 4 * r;
}
__device__ __forceinline__ int acc64_col(int bj) {
    const int tid = tid_opaque(), lane = tid & 63, w = tid >> 6;
    return (w & 1) * 32 + bj * 16 + (lane & 15);
}

// ---------------------------------------------------------------------------
// Counter-based draws: SplitMix64 (Steele, Lea, Flood 2014) output number
// idx+1 of a stream seeded with `seed`. uniform24 takes its top 24 bits as u in
// [0, 1) (stochastic rounding); the incoherence rotation takes its top bit as a
// sign.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t splitmix64_out(uint64_t seed, uint64_t idx) {
    uint64_t z = seed + (idx + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
__device__ __forceinline__ float uniform24(uint64_t seed, uint64_t idx) {
    return (float)(uint32_t)(splitmix64_out(seed, idx) >> 40) * (1.0f / 16777216.0f);
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

// max that lets a NaN through
__device__ __forceinline__ float nan_max(float m, float a) { return (a > m || a != a) ? a : m; }

// The two fp16 pieces of x' = x 2^e (hi = fp16(x'), lo = fp16(x' - hi)), as fp16
// bits: with |x'| < 2^15 the pair holds x' to about 22 bits, and hi lo' + lo hi' +
// hi hi' gives a product to about fp32 accuracy.
__device__ __forceinline__ void split2_value(float x, int e, uint32_t& h, uint32_t& l) {
    const float xs = ldexpf(x, e);
    const _Float16 hv = (_Float16)xs;
    const _Float16 lv = (_Float16)(xs - (float)hv);
    h = (uint32_t)__builtin_bit_cast(uint16_t, hv);
    l = (uint32_t)__builtin_bit_cast(uint16_t, lv);
}

// ---------------------------------------------------------------------------
// Hand-over primitives for persistent kernels. Each XCD has its own L2, so
// data passed between workgroups is written with device-coherent (agent-scope)
// stores, which go through to memory, and a producer raises its counter (also
// agent scope) only once those stores have completed (s_waitcnt vmcnt(0)): no
// cache-wide write-back is needed. A consumer that then reads through the
// caches first invalidates them (acquire fence at agent scope).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int ld_flag(const int* f) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(int* f, int v) {
    __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(float* q, float v) {
    __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(double* q, double v) {
    __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes as two device-coherent 8-byte stores
__device__ __forceinline__ void st_coherent16(f16x8* q, const uint32_t (&v)[4]) {
    uint64_t* q64 = reinterpret_cast<uint64_t*>(q);
    __hip_atomic_store(q64, (uint64_t)v[0] | ((uint64_t)v[1] << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q64 + 1, (uint64_t)v[2] | ((uint64_t)v[3] << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
// keeps the compiler from moving the data loads above the counter check
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// the wave's own memory operations, cache maintenance included, have completed
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace bk
