// bk_accum.hip -- Hessian factor accumulation H <- beta H + alpha X^T X.
//
// The Kronecker factors are second moments over tokens: H_I = E[x^T x] of the
// layer inputs and H_O = E[g^T g] of the output gradients (YAQA article,
// section 3; K-FAC tutorial on mlqm.cn, section 5). With X stored as T x d
// (one token per row), X^T X is a contraction over T whose operands are both
// K-major, so each 128x128 tile of H is one TN tile GEMM. Only tiles on or
// above the diagonal are computed; each writes its tile and the mirrored
// tile, and a diagonal tile writes its upper half and mirrors it, so H is
// exactly symmetric.
//
// Two arithmetic paths, picked by the workspace the caller passes:
//  * two fp16 pieces per element, of columns scaled by powers of two, on the
//    fp16 matrix cores (the piece path, below k_syrk_reduce), when the
//    workspace holds the pieces;
//  * fp32 MFMA otherwise.
// Both keep the product to fp32 accuracy.
//
// Work balance (both paths): with P workgroups resident at once (two per CU),
// whole rounds of P tiles run over the full K; the tiles left over after the
// last whole round (or all tiles, when there are fewer than P) are split over
// K into partials that a second kernel adds in a fixed order, so the result
// does not depend on scheduling.
//
// fp32 path: whole 128x128 tiles stream their 32-deep k-slices straight from
// global memory into LDS (direct-to-LDS loads, one slice ahead); ragged tiles
// go through registers with zero fill.
#include <algorithm>

#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

constexpr int kT128 = 128;
constexpr int kSyKT = 32;   // k-slice depth of the register-staged path (ragged tiles)
constexpr int kRingKT = 32; // k-slice depth of the direct-to-LDS ring (whole 128x128 tiles)
constexpr int kRingNS = 2;  // slices in the ring: loads run kRingNS - 1 slices ahead
                            // (measured against 16 x 3, 16 x 4, 24 x 2, 40 x 2 and the deeper
                            // one-workgroup-per-CU rings; 32 x 2 keeps two workgroups per CU)

// k-slices stored as loaded ([k][column]): 16-byte stores of consecutive columns
// and, for each MFMA, 32 consecutive columns of one k-row per half-wave, both
// free of bank conflicts
struct SyrkSmem {
    float a[2][kSyKT][kT128];
    float b[2][kSyKT][kT128];
};

// Whole tiles: a ring of kRingNS slices, each filled by direct global-to-LDS loads
// (global_load_lds_dwordx4: a wave's 64 lanes write two consecutive 128-float rows).
struct SyrkRing {
    float a[kRingNS][kRingKT][kT128];
    float b[kRingNS][kRingKT][kT128];
};

union SyrkShared {
    SyrkSmem staged;
    SyrkRing ring;
};

// Tile order. The upper triangle of nb x nb tiles is cut into g x g super-tiles
// (g = kSuper128), taken super-row by super-row, each super-row starting with its
// diagonal super-tile; inside a super-tile the tiles go row by row. Tiles that are
// close in this order share their operand panels (columns of X), so a run of them
// on one XCD reads about 2g panels per k-slice through that XCD's L2 instead of
// all nb.
constexpr int64_t kSuper128 = 8;
constexpr int kXcds = 8;  // workgroup b of a launch is placed on XCD b mod 8

// tile id -> (bi, bj), bi <= bj
__device__ __forceinline__ void upper_tile(int64_t id, int64_t nb, int64_t& bi, int64_t& bj) {
    constexpr int64_t g = kSuper128;
    int64_t s0 = 0;  // first tile-row of the super-row
    for (;;) {
        const int64_t r = min(g, nb - s0);
        const int64_t tri = r * (r + 1) / 2;
        const int64_t row = tri + r * (nb - s0 - r);
        if (id < row || s0 + r >= nb) {
            if (id < tri) {  // the diagonal super-tile, row by row
                int64_t i = 0;
                while (id >= r - i) {
                    id -= r - i;
                    ++i;
                }
                bi = s0 + i;
                bj = bi + id;
            } else {  // an off-diagonal super-tile of r rows and c columns
                id -= tri;
                int64_t c0 = s0 + r;
                for (;;) {
                    const int64_t c = min(g, nb - c0);
                    if (id < r * c) {
                        bi = s0 + id / c;
                        bj = c0 + id % c;
                        break;
                    }
                    id -= r * c;
                    c0 += c;
                }
            }
            return;
        }
        id -= row;
        s0 += r;
    }
}

// Workgroup b of an n-workgroup launch -> its place in [0, n): XCD x takes the
// x-th contiguous run of the order, so the workgroups resident on one XCD at a
// time hold neighbouring tiles.
__device__ __forceinline__ int64_t xcd_rank(int64_t b, int64_t n) {
    const int64_t x = b % kXcds;
    const int64_t q = n / kXcds, rr = n % kXcds;
    return x * q + min(x, rr) + b / kXcds;
}

// Thread t loads rows k0 + (t >> 5) + 8 h (h = 0..3), columns 4 (t & 31)..+3
// of the ncol columns starting at X + c0; zeros outside [0, K) x [0, ncol).
__device__ __forceinline__ void syrk_load(const float* __restrict__ X, int64_t ldx, int ncol,
                                          int64_t K, int64_t k0, f32x4 (&v)[4]) {
    const int t = threadIdx.x;
    const int c4 = (t & 31) << 2;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int64_t k = k0 + (t >> 5) + 8 * h;
        const float* p = X + k * ldx + c4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[h][e] = (k < K && c4 + e < ncol) ? p[e] : 0.0f;
    }
}

// stores a loaded slice; rows k0 + r >= K are written as zeros
__device__ __forceinline__ void syrk_store(float (&dst)[kSyKT][kT128], const f32x4 (&v)[4], int64_t K,
                                           int64_t k0) {
    const int t = threadIdx.x;
    const int c4 = (t & 31) << 2;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int r = (t >> 5) + 8 * h;
        *reinterpret_cast<f32x4*>(&dst[r][c4]) = k0 + r < K ? v[h] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
}

// The MFMAs of one 32-deep slice: wave quadrant rows wr.., columns wc..; the
// operands of k-step s + 1 are read from LDS before the MFMAs of step s issue.
template <int KT>
__device__ __forceinline__ void syrk_slice(const float (&a)[KT][kT128], const float (&b)[KT][kT128],
                                           int wr, int wc, f32x16 (&acc)[2][2]) {
    const int lane = threadIdx.x & 63;
    const int kh = lane >> 5, l31 = lane & 31;
    float fa[2][2], fb[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        fa[0][h] = a[kh][wr + 32 * h + l31];
        fb[0][h] = b[kh][wc + 32 * h + l31];
    }
#pragma unroll
    for (int s = 0; s < KT / 2; ++s) {
        const int cur = s & 1;
        if (s + 1 < KT / 2) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                fa[cur ^ 1][h] = a[2 * (s + 1) + kh][wr + 32 * h + l31];
                fb[cur ^ 1][h] = b[2 * (s + 1) + kh][wc + 32 * h + l31];
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this step's MFMAs
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[cur][rb], fb[cur][cb], acc[rb][cb], 0, 0, 0);
    }
}

// acc[rb][cb] (32x32 blocks of this wave's 64x64 quadrant) += sum_{k in [kb, ke)}
// X[k][r0 + r] X[k][c0 + c] for a ragged tile; the next slice is loaded into
// registers while the current one feeds the MFMAs.
__device__ __forceinline__ void syrk_tile_staged(const float* __restrict__ A, const float* __restrict__ B,
                                               int64_t ldx, int R, int Cn, int64_t kb, int64_t ke,
                                               f32x16 (&acc)[2][2], SyrkSmem& sm) {
    const int w = threadIdx.x >> 6;
    const int wr = (w >> 1) * 64, wc = (w & 1) * 64;
    const int64_t nk = (ke - kb + kSyKT - 1) / kSyKT;
    f32x4 va[4], vb[4];
    syrk_load(A, ldx, R, ke, kb, va);
    syrk_load(B, ldx, Cn, ke, kb, vb);
    syrk_store(sm.a[0], va, ke, kb);
    syrk_store(sm.b[0], vb, ke, kb);
    __syncthreads();
    for (int64_t it = 0; it < nk; ++it) {
        const int cur = (int)(it & 1);
        const bool more = it + 1 < nk;
        if (more) {
            const int64_t k0 = kb + (it + 1) * kSyKT;
            syrk_load(A, ldx, R, ke, k0, va);
            syrk_load(B, ldx, Cn, ke, k0, vb);
        }
        syrk_slice<kSyKT>(sm.a[cur], sm.b[cur], wr, wc, acc);
        if (more) {
            syrk_store(sm.a[cur ^ 1], va, ke, kb + (it + 1) * kSyKT);
            syrk_store(sm.b[cur ^ 1], vb, ke, kb + (it + 1) * kSyKT);
        }
        __syncthreads();
    }
}

// Wait until at most N of this wave's vector-memory operations are outstanding, then
// meet the other waves. Direct-to-LDS loads complete in issue order with the wave's
// other vector loads, so with N = the loads issued after slice s, slice s is in LDS
// once every wave has passed. No compiler fence is involved: the ring's later loads
// stay in flight across the barrier.
// N counts only the ring's own loads, so this holds only while the kernel keeps every
// value in registers: a spill would add scratch loads and stores to the count (the
// build rejects any kernel with scratch for that reason).
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// The whole-tile case (128 x 128, 16-byte aligned rows): slice s of the K-range goes to
// ring slot s mod kRingNS; at the top of slice s the loads of slice s + kRingNS - 1 go
// out into the slot every wave finished reading in slice s - 1. A K-range that is not
// a whole number of slices ends with one register-staged, zero-filled slice.
__device__ __forceinline__ void syrk_tile_ring(const float* __restrict__ A, const float* __restrict__ B,
                                               int64_t ldx, int64_t kb, int64_t ke,
                                               f32x16 (&acc)[2][2], SyrkRing& sm) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = (w >> 1) * 64, wc = (w & 1) * 64;
    const int c4 = (lane & 31) << 2;
    constexpr int kLoads = 2 * (kRingKT / 8);  // direct loads per wave per slice
    const int64_t nf = (ke - kb) / kRingKT;    // whole slices
    auto issue = [&](int64_t s) {
        const int slot = (int)(s % kRingNS);
        const int64_t k0 = kb + s * kRingKT;
#pragma unroll
        for (int h = 0; h < kRingKT / 8; ++h) {
            const int r = 2 * w + 8 * h;  // this wave's two rows
            const int64_t k = k0 + r + (lane >> 5);
            __builtin_amdgcn_global_load_lds(A + k * ldx + c4, &sm.a[slot][r][0], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(B + k * ldx + c4, &sm.b[slot][r][0], 16, 0, 0);
        }
    };
    for (int s = 0; s < kRingNS - 1; ++s)
        if (s < nf) issue(s);
    for (int64_t it = 0; it < nf; ++it) {
        if (it + kRingNS - 2 < nf) vm_wait_barrier<(kRingNS - 2) * kLoads>();
        else vm_wait_barrier<0>();
        if (it + kRingNS - 1 < nf) issue(it + kRingNS - 1);
        const int slot = (int)(it % kRingNS);
        syrk_slice<kRingKT>(sm.a[slot], sm.b[slot], wr, wc, acc);
    }
    const int64_t kt = kb + nf * kRingKT;
    if (kt < ke) {
        __syncthreads();  // every wave is done with the ring
        const int t = threadIdx.x;
        f32x4 va[kRingKT / 8], vb[kRingKT / 8];
#pragma unroll
        for (int h = 0; h < kRingKT / 8; ++h) {
            const int64_t k = kt + (t >> 5) + 8 * h;
            const int64_t kc = min(k, ke - 1);
            va[h] = *reinterpret_cast<const f32x4*>(A + kc * ldx + c4);
            vb[h] = *reinterpret_cast<const f32x4*>(B + kc * ldx + c4);
        }
#pragma unroll
        for (int h = 0; h < kRingKT / 8; ++h) {
            const int r = (t >> 5) + 8 * h;
            const bool in = kt + r < ke;
            *reinterpret_cast<f32x4*>(&sm.a[0][r][c4]) = in ? va[h] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            *reinterpret_cast<f32x4*>(&sm.b[0][r][c4]) = in ? vb[h] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        __syncthreads();
        syrk_slice<kRingKT>(sm.a[0], sm.b[0], wr, wc, acc);
    }
}

__device__ __forceinline__ void syrk_tile(const float* __restrict__ X, int64_t ldx, int64_t r0,
                                          int R, int64_t c0, int Cn, int64_t kb, int64_t ke,
                                          f32x16 (&acc)[2][2], SyrkShared& sm) {
    if (ke <= kb) return;
    const float* A = X + r0;
    const float* B = X + c0;
    const bool full = R == kT128 && Cn == kT128 && (ldx & 3) == 0 &&
                      ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    if (full) syrk_tile_ring(A, B, ldx, kb, ke, acc, sm.ring);
    else syrk_tile_staged(A, B, ldx, R, Cn, kb, ke, acc, sm.staged);
}

// row / column inside the 128x128 tile of element v of block (rb, cb)
__device__ __forceinline__ int syrk_row(int rb, int v) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    return (w >> 1) * 64 + 32 * rb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int syrk_col(int cb) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    return (w & 1) * 64 + 32 * cb + (lane & 31);
}

// Write alpha * acc (+ beta H) into tile (bi, bj) of H and its mirror. With exps
// (the piece path's column exponents), acc holds the product of the scaled columns
// and is first scaled back by 2^-(e_i + e_j), exactly.
__device__ __forceinline__ void syrk_write(float* __restrict__ H, int64_t ldh, int64_t d,
                                           int64_t bi, int64_t bj, float alpha, float beta,
                                           const f32x16 (&acc)[2][2], const int* __restrict__ exps) {
    const int64_t r0 = bi * kT128, c0 = bj * kT128;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int c = syrk_col(cb);
            const int ec = exps ? exps[c0 + c] : 0;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = syrk_row(rb, v);
                const int64_t gi = r0 + r, gj = c0 + c;
                if (gi >= d || gj >= d) continue;
                if (bi == bj && r > c) continue;
                const float a = exps ? ldexpf(acc[rb][cb][v], -(exps[gi] + ec)) : acc[rb][cb][v];
                float val = alpha * a;
                if (beta != 0.0f) val = fmaf(beta, H[gi * ldh + gj], val);
                H[gi * ldh + gj] = val;
                if (gi != gj) H[gj * ldh + gi] = val;
            }
        }
}

// Whole tiles [tile_beg, tile_beg + gridDim.x) over the full K.
__global__ __launch_bounds__(kThreads) void k_syrk_full(const float* __restrict__ X, int64_t T,
                                                        int64_t d, int64_t ldx, float alpha,
                                                        float beta, float* __restrict__ H,
                                                        int64_t ldh, int64_t nb, int64_t tile_beg) {
    __shared__ SyrkShared sm;
    int64_t bi, bj;
    upper_tile(tile_beg + xcd_rank(blockIdx.x, gridDim.x), nb, bi, bj);
    const int R = (int)min<int64_t>(kT128, d - bi * kT128);
    const int Cn = (int)min<int64_t>(kT128, d - bj * kT128);
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
    syrk_tile(X, ldx, bi * kT128, R, bj * kT128, Cn, 0, T, acc, sm);
    syrk_write(H, ldh, d, bi, bj, alpha, beta, acc, nullptr);
}

// Tiles [tile_beg, tile_beg + ntiles), each split into nsplit K-ranges; block
// (tile u, split s) writes its raw 128x128 partial to part[(u * nsplit + s)].
__global__ __launch_bounds__(kThreads) void k_syrk_split(const float* __restrict__ X, int64_t T,
                                                         int64_t d, int64_t ldx, int64_t nb,
                                                         int64_t tile_beg, int nsplit,
                                                         float* __restrict__ part) {
    __shared__ SyrkShared sm;
    const int u = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
    int64_t bi, bj;
    upper_tile(tile_beg + u, nb, bi, bj);
    const int R = (int)min<int64_t>(kT128, d - bi * kT128);
    const int Cn = (int)min<int64_t>(kT128, d - bj * kT128);
    // K-ranges in whole slices
    const int64_t nsl = (T + kSyKT - 1) / kSyKT;
    const int64_t per = (nsl + nsplit - 1) / nsplit;
    const int64_t kb = std::min<int64_t>(T, (int64_t)sp * per * kSyKT);
    const int64_t ke = std::min<int64_t>(T, kb + per * kSyKT);
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
    syrk_tile(X, ldx, bi * kT128, R, bj * kT128, Cn, kb, ke, acc, sm);
    float* out = part + (size_t)blockIdx.x * kT128 * kT128;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int c = syrk_col(cb);
#pragma unroll
            for (int v = 0; v < 16; ++v) out[syrk_row(rb, v) * kT128 + c] = acc[rb][cb][v];
        }
}

// Sum the nsplit partials of each split tile in order and write H; block
// (u, g) handles rows 8 g .. 8 g + 7 of tile u.
__global__ __launch_bounds__(kThreads) void k_syrk_reduce(int64_t d, float alpha, float beta,
                                                          float* __restrict__ H, int64_t ldh,
                                                          int64_t nb, int64_t tile_beg, int nsplit,
                                                          const float* __restrict__ part,
                                                          const int* __restrict__ exps) {
    const int u = blockIdx.x;
    int64_t bi, bj;
    upper_tile(tile_beg + u, nb, bi, bj);
    const float* base = part + (size_t)u * nsplit * kT128 * kT128;
    const int e = blockIdx.y * 8 * kT128 + threadIdx.x * 4;
    f32x4 s = *reinterpret_cast<const f32x4*>(base + e);
    for (int q = 1; q < nsplit; ++q) s += *reinterpret_cast<const f32x4*>(base + (size_t)q * kT128 * kT128 + e);
    const int r = e / kT128, c0 = e % kT128;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = c0 + k;
        const int64_t gi = bi * kT128 + r, gj = bj * kT128 + c;
        if (gi >= d || gj >= d) continue;
        if (bi == bj && r > c) continue;
        float val = alpha * (exps ? ldexpf(s[k], -(exps[gi] + exps[gj])) : s[k]);
        if (beta != 0.0f) val = fmaf(beta, H[gi * ldh + gj], val);
        H[gi * ldh + gj] = val;
        if (gi != gj) H[gj * ldh + gi] = val;
    }
}

// ---------------------------------------------------------------------------
// The two-piece fp16 path.
//
// The gfx950 matrix cores multiply fp16 pairs at sixteen times their fp32
// rate. Column c of X is first scaled by a power of two, x' = x 2^e_c, chosen
// so that the column's largest magnitude lies in [2^14, 2^15) (well inside the
// fp16 range; e_c = 0 for a zero or non-finite column). Each x' is cut into two
// fp16 pieces, h = fp16(x') and l = fp16(x' - h), rounding to nearest even;
// x' - h is exact in fp32, |x' - h| <= 2^-11 |x'| and |x' - h - l| <= 2^-22 |x'|
// while l is a normal fp16, i.e. for |x'| >= 2^-3, within 2^17 of the column's
// largest magnitude; below that l carries an absolute error of at most 2^-25
// (half the smallest fp16 step), 2^-39 of the column's largest magnitude. A
// product x'y' is taken as hh' + hl' + lh'; the term left out (ll') is below
// 2^-22 |x'y'|. The fp16 products are exact in fp32 and add into fp32
// accumulators, so a 128 x 128 tile of H costs three matrix-core passes at a
// sixteenth of the fp32 cost each, and the pieces take 4 bytes per element.
// The tile's result is scaled back by 2^-(e_i + e_j), which is exact.
//
// The pre-pass: per-column maxima over chunks of tokens (k_colmax /
// k_colmax_t), their reduction to the exponents (k_colexp), then the split
// (k_split2 / k_split2_t), which writes the pieces in the order the MFMA reads
// them: for each group g of 8 consecutive tokens and each column c, the 8 fp16
// values of that column (16 bytes), piece planes apart: Xs[piece][g][c][0..7].
// The tokens are padded with zeros to a whole number of stages and the columns
// to whole 128-wide tiles, so every tile streams whole 2 KB rows of Xs straight
// into LDS.
// ---------------------------------------------------------------------------

#ifndef BK_S2_NS
#define BK_S2_NS 4
#endif
#ifndef BK_S2_KB
#define BK_S2_KB 1
#endif
constexpr int kNP = 2;           // fp16 pieces per element
constexpr int kS2NS = BK_S2_NS;  // stages in the ring: loads run kS2NS - 1 stages ahead
constexpr int kS2KB = BK_S2_KB;  // 16-token blocks per stage
constexpr int64_t kS2Pad = 32;   // tokens are padded to a multiple of this (whole stages)
static_assert(kS2Pad % (16 * kS2KB) == 0, "whole stages");
constexpr int kMaxChunks = 256;  // token chunks of the column-maximum pass

struct Split2Shape {
    int64_t ng;  // groups of 8 tokens (padded)
    int64_t dp;  // columns (padded to whole tiles)
    int64_t nstage;
    int nchunk;       // token chunks of the column-maximum pass
    size_t exps_off;  // int32 [dp] column exponents
    size_t cmax_off;  // fp32 [nchunk][dp] partial column maxima
    size_t bytes;
};
inline Split2Shape split2_shape(int64_t T, int64_t d) {
    Split2Shape s;
    const int64_t Tp = (T + kS2Pad - 1) / kS2Pad * kS2Pad;
    s.ng = Tp / 8;
    s.dp = (d + kT128 - 1) / kT128 * kT128;
    s.nstage = Tp / (16 * kS2KB);
    s.nchunk = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxChunks, (T + 127) / 128));
    size_t o = align256((size_t)kNP * (size_t)Tp * (size_t)s.dp * 2);
    s.exps_off = o;
    o += align256(sizeof(int) * (size_t)s.dp);
    s.cmax_off = o;
    o += align256(sizeof(float) * (size_t)s.nchunk * (size_t)s.dp);
    s.bytes = o;
    return s;
}


// Partial maxima of |x| (|x sqrt(w)| with token weights) for columns 4 t .. 4 t + 3 of
// block x over the tokens of chunk blockIdx.y; columns in [d, dp) get 0.
template <bool kVec>
__global__ __launch_bounds__(kThreads) void k_colmax(const float* __restrict__ X, int64_t T, int64_t d,
                                                     int64_t ldx, int64_t dp, int nchunk,
                                                     const float* __restrict__ wt, float* __restrict__ part) {
    const int64_t c4 = (int64_t)blockIdx.x * (4 * kThreads) + 4 * threadIdx.x;
    if (c4 >= dp) return;
    const int64_t per = (T + nchunk - 1) / nchunk;
    const int64_t k0 = std::min<int64_t>(T, (int64_t)blockIdx.y * per), k1 = std::min<int64_t>(T, k0 + per);
    f32x4 m = {0.0f, 0.0f, 0.0f, 0.0f};
    const bool vec = kVec && c4 + 4 <= d;
    constexpr int kU = 4;  // rows in flight per thread
    for (int64_t kb = k0; kb < k1; kb += kU) {
        f32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t k = kb + u;
            const float* row = X + k * ldx + c4;
            v[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (k < k1) {
                if (vec) {
                    v[u] = *reinterpret_cast<const f32x4*>(row);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (c4 + j < d) v[u][j] = row[j];
                }
                if (wt) v[u] *= sqrtf(fmaxf(wt[k], 0.0f));
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) m[j] = nan_max(m[j], fabsf(v[u][j]));
    }
    float* out = part + (size_t)blockIdx.y * dp + c4;
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = m[j];
}

// The same for X stored d x T (one row per column of the product; a batch of S
// matrices of tin tokens, bs floats apart): wave w of block x takes row 4 x + w.
__global__ __launch_bounds__(kThreads) void k_colmax_t(const float* __restrict__ X, int64_t T, int64_t d,
                                                       int64_t ldx, int64_t tin, int64_t bs, int64_t dp,
                                                       int nchunk, float* __restrict__ part) {
    const int lane = threadIdx.x & 63;
    const int64_t c = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (c >= dp) return;
    const int64_t per = (T + nchunk - 1) / nchunk;
    const int64_t k0 = std::min<int64_t>(T, (int64_t)blockIdx.y * per), k1 = std::min<int64_t>(T, k0 + per);
    float m = 0.0f;
    if (c < d)
        for (int64_t k = k0 + lane; k < k1; k += 64) m = nan_max(m, fabsf(X[(k / tin) * bs + c * ldx + k % tin]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = nan_max(m, __shfl_xor(m, o));
    if (lane == 0) part[(size_t)blockIdx.y * dp + c] = m;
}

// e_c = 15 - E for a column maximum f 2^E (f in [1/2, 1)), so the scaled column's
// largest magnitude lies in [2^14, 2^15); 0 for a zero or non-finite maximum.
// Workgroup x reduces columns 16 x .. 16 x + 15: thread (c, r) takes chunks r, r + 16,
// .. of column c (every load in flight at once), then the 16 partial maxima of a
// column are combined through LDS.
constexpr int kExpCols = 16;
__global__ __launch_bounds__(kThreads) void k_colexp(const float* __restrict__ part, int64_t dp, int nchunk,
                                                     int* __restrict__ exps) {
    constexpr int kRowsPer = kThreads / kExpCols;  // 16 chunk groups
    constexpr int kU = kMaxChunks / kRowsPer;      // chunks per thread at most
    __shared__ float red[kRowsPer][kExpCols];
    const int cl = threadIdx.x % kExpCols, rg = threadIdx.x / kExpCols;
    const int64_t c = (int64_t)blockIdx.x * kExpCols + cl;
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int q = rg + kRowsPer * u;
        v[u] = (c < dp && q < nchunk) ? part[(size_t)q * dp + c] : 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int u = 0; u < kU; ++u) m = nan_max(m, v[u]);
    red[rg][cl] = m;
    __syncthreads();
    if (rg != 0 || c >= dp) return;
#pragma unroll
    for (int r = 1; r < kRowsPer; ++r) m = nan_max(m, red[r][cl]);
    int e = 0;
    if (m > 0.0f && m < INFINITY) {
        int E;
        frexpf(m, &E);
        e = 15 - E;
    }
    exps[c] = e;
}


// Block (x, g): columns 1024 x .. 1024 x + 1023 of tokens 8 g .. 8 g + 7 into the
// two planes, through LDS. Each row is read as 16-byte vectors where four
// columns lie inside [0, d) and X allows it (kVec), element by element
// otherwise; thread t then splits columns t, t + 256, t + 512, t + 768, so each
// store instruction writes 1 KB of consecutive 16-byte units of a plane.
constexpr int kSplitCols = 4 * kThreads;
// wt (optional): token weights; row k is scaled by sqrt(max(wt[k], 0)) before the
// split, which turns the SYRK into sum_k wt[k] x_k^T x_k.
template <bool kVec>
__global__ __launch_bounds__(kThreads) void k_split2(const float* __restrict__ X, int64_t T,
                                                     int64_t d, int64_t ldx, int64_t ng,
                                                     int64_t dp, uint4* __restrict__ Xs,
                                                     const float* __restrict__ wt, const int* __restrict__ exps) {
    __shared__ float tile[8][kSplitCols];
    const int t = threadIdx.x;
    const int64_t cb = (int64_t)blockIdx.x * kSplitCols;
    const int64_t c4 = cb + 4 * t;  // this thread's four columns on the read side
    const bool vec = kVec && c4 + 4 <= d;
    int ex[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ex[q] = cb + t + kThreads * q < dp ? exps[cb + t + kThreads * q] : 0;
    for (int64_t g = blockIdx.y; g < ng; g += gridDim.y) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t k = 8 * g + e;
            const float* row = X + k * ldx + c4;
            f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (k < T) {
                if (vec) {
                    v = *reinterpret_cast<const f32x4*>(row);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (c4 + j < d) v[j] = row[j];
                }
            }
            if (wt && k < T) v *= sqrtf(fmaxf(wt[k], 0.0f));
            *reinterpret_cast<f32x4*>(&tile[e][4 * t]) = v;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int cl = t + kThreads * q;
            const int64_t c = cb + cl;
            uint32_t pk[kNP][4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                uint32_t h0, l0, h1, l1;
                split2_value(tile[e][cl], ex[q], h0, l0);
                split2_value(tile[e + 1][cl], ex[q], h1, l1);
                pk[0][e >> 1] = h0 | (h1 << 16);
                pk[1][e >> 1] = l0 | (l1 << 16);
            }
            if (c < dp) {
#pragma unroll
                for (int p = 0; p < kNP; ++p)
                    Xs[((int64_t)p * ng + g) * dp + c] = uint4{pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
            }
        }
        __syncthreads();
    }
}

// The same planes from X stored d x T (one row per output column, the tokens
// along the row), for H = X X^T: thread (c, q) splits tokens 32 q .. 32 q + 31 of
// row c, one whole 128-byte line, into four groups of 8; a wave writes 1 KB of
// consecutive 16-byte units of each plane per group. A batch of S such matrices
// of tin tokens each, bs floats apart, reads as one with T = S tin: token k of
// row c is X[(k / tin) bs + c ldx + k % tin].
template <bool kVec>
__global__ __launch_bounds__(kThreads) void k_split2_t(const float* __restrict__ X, int64_t T,
                                                       int64_t d, int64_t ldx, int64_t tin, int64_t bs,
                                                       int64_t ng, int64_t dp, uint4* __restrict__ Xs,
                                                       const int* __restrict__ exps) {
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c >= dp) return;
    const int ec = exps[c];
    for (int64_t q = blockIdx.y; q < ng / 4; q += gridDim.y) {
        const int64_t k0 = 32 * q;
        const int64_t j0 = k0 % tin;
        const float* row = X + (k0 / tin) * bs + c * ldx + j0;
        float v[32];
        if (kVec && c < d && k0 + 32 <= T && j0 + 32 <= tin) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(row + 4 * e);
#pragma unroll
                for (int j = 0; j < 4; ++j) v[4 * e + j] = t[j];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const int64_t k = k0 + e;
                v[e] = (c < d && k < T) ? X[(k / tin) * bs + c * ldx + k % tin] : 0.0f;
            }
        }
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            uint32_t pk[kNP][4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                uint32_t h0, l0, h1, l1;
                split2_value(v[8 * gi + e], ec, h0, l0);
                split2_value(v[8 * gi + e + 1], ec, h1, l1);
                pk[0][e >> 1] = h0 | (h1 << 16);
                pk[1][e >> 1] = l0 | (l1 << 16);
            }
            const int64_t g = 4 * q + gi;
#pragma unroll
            for (int p = 0; p < kNP; ++p)
                Xs[((int64_t)p * ng + g) * dp + c] = uint4{pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
        }
    }
}

// One ring stage of both operands: [piece][16-token block][token half][column].
struct Split2Stage {
    f16x8 v[kNP][kS2KB][2][kT128];
};
struct Split2Ring {
    Split2Stage a[kS2NS];
    Split2Stage b[kS2NS];
};

// The 12 MFMAs of one 16-token block, per wave quadrant: the three piece products
// of each of the four 32 x 32 blocks, smallest first, the four blocks interleaved
// so that no MFMA waits on the one before it.
__device__ __forceinline__ void split2_block(const f16x8 (&fa)[kNP][2], const f16x8 (&fb)[kNP][2],
                                             f32x16 (&acc)[2][2]) {
    constexpr int kPa[3] = {0, 1, 0};
    constexpr int kPb[3] = {1, 0, 0};
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[kPa[t]][rb], fb[kPb[t]][cb], acc[rb][cb],
                                                                     0, 0, 0);
}

// The MFMAs of one stage (rows wr.., columns wc.. of the tile); the operands of
// block kb + 1 are read from LDS before the MFMAs of block kb issue.
__device__ __forceinline__ void split2_stage(const Split2Stage& a, const Split2Stage& b, int wr, int wc,
                                             int lane, f32x16 (&acc)[2][2]) {
    const int kh = lane >> 5, l31 = lane & 31;
    f16x8 fa[2][kNP][2], fb[2][kNP][2];
#pragma unroll
    for (int p = 0; p < kNP; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            fa[0][p][h] = a.v[p][0][kh][wr + 32 * h + l31];
            fb[0][p][h] = b.v[p][0][kh][wc + 32 * h + l31];
        }
#pragma unroll
    for (int kb = 0; kb < kS2KB; ++kb) {
        const int cur = kb & 1;
        if (kb + 1 < kS2KB) {
#pragma unroll
            for (int p = 0; p < kNP; ++p)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    fa[cur ^ 1][p][h] = a.v[p][kb + 1][kh][wr + 32 * h + l31];
                    fb[cur ^ 1][p][h] = b.v[p][kb + 1][kh][wc + 32 * h + l31];
                }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this block's MFMAs
        split2_block(fa[cur], fb[cur], acc);
    }
}

// Stages [s_beg, s_end) of tile columns (ca.., cb..): stage s goes to ring slot
// s mod kS2NS; at the top of stage s the loads of stage s + kS2NS - 1 go out into
// the slot every wave finished reading in stage s - 1 (as in syrk_tile_ring).
__device__ __forceinline__ void split2_tile(const uint4* __restrict__ Xs, int64_t ng, int64_t dp,
                                            int64_t ca, int64_t cb, int64_t s_beg, int64_t s_end,
                                            f32x16 (&acc)[2][2], Split2Ring& sm) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = (w >> 1) * 64, wc = (w & 1) * 64;
    constexpr int kRows = kNP * kS2KB * 2 * 2;  // 1 KB rows per operand per stage
    constexpr int kPerWave = kRows / 4;
    constexpr int kLoads = 2 * kPerWave;        // direct loads per wave per stage
    const int64_t ns = s_end - s_beg;
    auto issue = [&](int64_t s) {
        const int slot = (int)(s % kS2NS);
        const int64_t kb0 = (s_beg + s) * kS2KB;
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int q = w + 4 * i;
            const int half = q & 1, th = (q >> 1) & 1, kbl = (q >> 2) % kS2KB, p = (q >> 2) / kS2KB;
            const int64_t g = 2 * (kb0 + kbl) + th;
            const uint4* row = Xs + ((int64_t)p * ng + g) * dp + 64 * half + lane;
            __builtin_amdgcn_global_load_lds(row + ca, &sm.a[slot].v[p][kbl][th][64 * half], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(row + cb, &sm.b[slot].v[p][kbl][th][64 * half], 16, 0, 0);
        }
    };
    for (int s = 0; s < kS2NS - 1; ++s)
        if (s < ns) issue(s);
    for (int64_t it = 0; it < ns; ++it) {
        if (it + kS2NS - 2 < ns) vm_wait_barrier<(kS2NS - 2) * kLoads>();
        else vm_wait_barrier<0>();
        const int slot = (int)(it % kS2NS);
        if (it + kS2NS - 1 < ns) issue(it + kS2NS - 1);
        split2_stage(sm.a[slot], sm.b[slot], wr, wc, lane, acc);
    }
}

// Whole tiles [tile_beg, tile_beg + gridDim.x) over all stages.
__global__ __launch_bounds__(kThreads) void k_syrk2_full(const uint4* __restrict__ Xs, int64_t ng,
                                                         int64_t dp, int64_t nstage, int64_t d,
                                                         float alpha, float beta, float* __restrict__ H,
                                                         int64_t ldh, int64_t nb, int64_t tile_beg,
                                                         const int* __restrict__ exps) {
    __shared__ Split2Ring sm;
    int64_t bi, bj;
    upper_tile(tile_beg + xcd_rank(blockIdx.x, gridDim.x), nb, bi, bj);
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
    split2_tile(Xs, ng, dp, bi * kT128, bj * kT128, 0, nstage, acc, sm);
    syrk_write(H, ldh, d, bi, bj, alpha, beta, acc, exps);
}

// Tiles [tile_beg, tile_beg + ntiles), each split into nsplit stage ranges; block
// (tile u, split s) writes its raw 128x128 partial to part[(u * nsplit + s)].
__global__ __launch_bounds__(kThreads) void k_syrk2_split(const uint4* __restrict__ Xs, int64_t ng,
                                                          int64_t dp, int64_t nstage, int64_t nb,
                                                          int64_t tile_beg, int nsplit,
                                                          float* __restrict__ part) {
    __shared__ Split2Ring sm;
    const int u = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
    int64_t bi, bj;
    upper_tile(tile_beg + u, nb, bi, bj);
    const int64_t per = (nstage + nsplit - 1) / nsplit;
    const int64_t sb = std::min<int64_t>(nstage, (int64_t)sp * per);
    const int64_t se = std::min<int64_t>(nstage, sb + per);
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
    split2_tile(Xs, ng, dp, bi * kT128, bj * kT128, sb, se, acc, sm);
    float* out = part + (size_t)blockIdx.x * kT128 * kT128;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int c = syrk_col(cb);
#pragma unroll
            for (int v = 0; v < 16; ++v) out[syrk_row(rb, v) * kT128 + c] = acc[rb][cb][v];
        }
}

namespace {
// workgroups resident at once: LDS-limited per CU (160 KB)
int resident_slots(size_t lds_bytes) {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus = n;
    }
    return cus * std::max<int>(1, (int)((160 * 1024) / lds_bytes));
}

// Whole rounds of P tiles over the full K; a short last round is split over K
// into at most P workgroups (at least 8 K-units each), if the partials fit in
// `room` bytes; otherwise it runs whole.
struct SyrkPlan {
    int64_t full, rem;
    int nsplit;
};
SyrkPlan plan_tiles(int64_t tiles, int64_t P, int64_t kunits, size_t room) {
    SyrkPlan pl;
    pl.full = (tiles / P) * P;
    pl.rem = tiles - pl.full;
    pl.nsplit = 1;
    if (pl.rem > P / 2) {  // a well-filled last round: run it whole too
        pl.full = tiles;
        pl.rem = 0;
    }
    if (pl.rem > 0) {
        pl.nsplit = (int)std::min<int64_t>(P / pl.rem, kunits / 8);
        const size_t need = sizeof(float) * (size_t)pl.rem * (size_t)std::max(pl.nsplit, 1) * kT128 * kT128;
        if (pl.nsplit < 2 || room < need) {  // no split possible
            pl.full = tiles;
            pl.rem = 0;
            pl.nsplit = 1;
        }
    }
    return pl;
}
}  // namespace

size_t hessian_workspace_bytes(int64_t T, int64_t d) {
    const size_t part = sizeof(float) * kT128 * kT128 *
                        (size_t)std::max(resident_slots(sizeof(SyrkShared)), resident_slots(sizeof(Split2Ring)));
    return split2_shape(T, d).bytes + part;
}

int launch_hessian_accum(const float* X, int64_t T, int64_t d, int64_t ldx, float alpha,
                         float beta, float* H, int64_t ldh, void* ws, size_t ws_bytes,
                         hipStream_t stream, bool trans, const float* wt, int64_t tin, int64_t bs) {
    const int64_t nb = (d + kT128 - 1) / kT128;
    const int64_t tiles = nb * (nb + 1) / 2;
    if (tiles > 0x7fffffff) return BAKRON_E_INVALID_ARG;
    const Split2Shape sh = split2_shape(T, d);
    if (ws != nullptr && ws_bytes >= sh.bytes) {
        // the two-piece fp16 path: column exponents, then the pieces
        uint4* Xs = (uint4*)ws;
        int* exps = (int*)((char*)ws + sh.exps_off);
        float* cmax = (float*)((char*)ws + sh.cmax_off);
        if (tin <= 0) tin = T;  // one matrix
        if (trans) {
            const dim3 grid((unsigned)((sh.dp + kThreads / 64 - 1) / (kThreads / 64)), (unsigned)sh.nchunk);
            hipLaunchKernelGGL(k_colmax_t, grid, dim3(kThreads), 0, stream, X, T, d, ldx, tin, bs, sh.dp, sh.nchunk,
                               cmax);
        } else {
            const dim3 grid((unsigned)((sh.dp + 4 * kThreads - 1) / (4 * kThreads)), (unsigned)sh.nchunk);
            const bool vec = (ldx & 3) == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0;
            if (vec)
                hipLaunchKernelGGL(k_colmax<true>, grid, dim3(kThreads), 0, stream, X, T, d, ldx, sh.dp, sh.nchunk,
                                   wt, cmax);
            else
                hipLaunchKernelGGL(k_colmax<false>, grid, dim3(kThreads), 0, stream, X, T, d, ldx, sh.dp, sh.nchunk,
                                   wt, cmax);
        }
        hipLaunchKernelGGL(k_colexp, dim3((unsigned)((sh.dp + kExpCols - 1) / kExpCols)), dim3(kThreads), 0, stream,
                           (const float*)cmax, sh.dp, sh.nchunk, exps);
        if (sh.ng > 0 && trans) {
            const unsigned gy = (unsigned)std::min<int64_t>(sh.ng / 4, 65535);
            const dim3 grid((unsigned)((sh.dp + kThreads - 1) / kThreads), gy);
            const bool vec = (ldx & 3) == 0 && (tin & 3) == 0 && (bs & 3) == 0 &&
                             (reinterpret_cast<uintptr_t>(X) & 15) == 0;
            if (vec)
                hipLaunchKernelGGL(k_split2_t<true>, grid, dim3(kThreads), 0, stream, X, T, d, ldx, tin, bs, sh.ng,
                                   sh.dp, Xs, (const int*)exps);
            else
                hipLaunchKernelGGL(k_split2_t<false>, grid, dim3(kThreads), 0, stream, X, T, d, ldx, tin, bs, sh.ng,
                                   sh.dp, Xs, (const int*)exps);
        } else if (sh.ng > 0) {
            const unsigned gy = (unsigned)std::min<int64_t>(sh.ng, 65535);
            const dim3 grid((unsigned)((sh.dp + kSplitCols - 1) / kSplitCols), gy);
            const bool vec = (ldx & 3) == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0;
            if (vec)
                hipLaunchKernelGGL(k_split2<true>, grid, dim3(kThreads), 0, stream, X, T, d, ldx, sh.ng, sh.dp, Xs,
                                   wt, (const int*)exps);
            else
                hipLaunchKernelGGL(k_split2<false>, grid, dim3(kThreads), 0, stream, X, T, d, ldx, sh.ng, sh.dp, Xs,
                                   wt, (const int*)exps);
        }
        const SyrkPlan pl = plan_tiles(tiles, resident_slots(sizeof(Split2Ring)), sh.nstage,
                                       ws_bytes - sh.bytes);
        if (pl.full > 0)
            hipLaunchKernelGGL(k_syrk2_full, dim3((unsigned)pl.full), dim3(kThreads), 0, stream, Xs,
                               sh.ng, sh.dp, sh.nstage, d, alpha, beta, H, ldh, nb, (int64_t)0, (const int*)exps);
        if (pl.rem > 0) {
            float* part = (float*)((char*)ws + sh.bytes);
            hipLaunchKernelGGL(k_syrk2_split, dim3((unsigned)(pl.rem * pl.nsplit)), dim3(kThreads), 0,
                               stream, Xs, sh.ng, sh.dp, sh.nstage, nb, pl.full, pl.nsplit, part);
            hipLaunchKernelGGL(k_syrk_reduce, dim3((unsigned)pl.rem, kT128 / 8), dim3(kThreads), 0, stream,
                               d, alpha, beta, H, ldh, nb, pl.full, pl.nsplit, (const float*)part, (const int*)exps);
        }
        return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
    }
    // the fp32-MFMA path (no room for the pieces); it reads X as T x d only
    if (trans || wt) return BAKRON_E_WORKSPACE;
    const int64_t nsl = (T + kSyKT - 1) / kSyKT;
    const SyrkPlan pl = plan_tiles(tiles, resident_slots(sizeof(SyrkShared)), nsl,
                                   ws != nullptr ? ws_bytes : 0);
    if (pl.full > 0) {
        hipLaunchKernelGGL(k_syrk_full, dim3((unsigned)pl.full), dim3(kThreads), 0, stream, X, T, d,
                           ldx, alpha, beta, H, ldh, nb, (int64_t)0);
    }
    if (pl.rem > 0) {
        float* part = (float*)ws;
        hipLaunchKernelGGL(k_syrk_split, dim3((unsigned)(pl.rem * pl.nsplit)), dim3(kThreads), 0, stream,
                           X, T, d, ldx, nb, pl.full, pl.nsplit, part);
        hipLaunchKernelGGL(k_syrk_reduce, dim3((unsigned)pl.rem, kT128 / 8), dim3(kThreads), 0, stream, d, alpha,
                           beta, H, ldh, nb, pl.full, pl.nsplit, (const float*)part, (const int*)nullptr);
    }
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

}  // namespace bk
