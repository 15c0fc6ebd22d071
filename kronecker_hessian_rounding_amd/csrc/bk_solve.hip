// bk_solve.hip -- the BaKron rounding solve on gfx950.
//
// Rule (YAQA article, section 4): entry (i, j) of W* is rounded as
//   W_ij = Q(W*_ij + a_i^T D[:i,:j] b_j + a_i^T D[:i,j] + D[i,:j] b_j)
// with a_i, b_j columns of the strictly upper L_O, L_I and D = W* - W. With
// A = L + I (unit upper) and C = A_O^T D (so C_ij = P_ij + D_ij, where
// P_ij = sum_{k<i} L_O[k,i] D_kj), the pre-rounding value is
//   t_ij = W*_ij + P_ij + sum_{l<j} C_il L_I[l,j].
// Entry (i, j) depends on every (k, l) with k <= i, l <= j, so all entries of
// one anti-diagonal are independent (BaKron Abstract, anti-diagonal
// parallelism). The work is cut into 64x64 leaves; leaf (I, J), with row block
// R_I and column block S_J, sits on leaf-diagonal d = I + J. Its feedback
//   p = sum_{I'<I} L_O[R_I', R_I]^T D[R_I', S_J]   (column far field)
//   o = sum_{J'<J} C[R_I, S_J'] L_I[S_J', S_J]      (row far field)
// is split by how far back the source block lies:
//  * three or more blocks back: MFMA GEMMs over K, split into partials, run by
//    other workgroups once those leaves are done (O(mn(m+n)) flops in all, the
//    bound of the BaKron Abstract);
//  * two blocks back: multiplied by the leaf's own workgroup before its sweep;
//  * the adjacent block: handed over 16 columns (rows) at a time while the
//    neighbour is still sweeping, and multiplied as it arrives.
// The leaf then runs its in-leaf sums as a 127-step anti-diagonal wavefront.
// Column x of a leaf's D and row x of its C are final 63 + x steps into that
// sweep, so a leaf can start about 64 steps (plus the hand-over latency) after
// its neighbours rather than a whole sweep after them.
//
// Everything runs in one persistent launch. Workgroups take tasks in a fixed
// order: the leaves of diagonal k, then the far fields of diagonal k + 1. A
// task waits only on tasks earlier in that order, so the earliest unfinished
// task can always proceed. Progress counters in global memory carry the
// hand-overs; every wait is bounded in time, and an expired wait stops the
// solve and is reported.
#include <limits.h>

#include <algorithm>
#include <cstdlib>

#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

constexpr int kB = kTile;        // leaf edge
constexpr int kNch = 4;          // maximum K-chunks per far-field product
constexpr int kRing = 4;         // diagonals whose far-field partials are held at once
constexpr int kTargetWg = 1024;  // far-field tasks aimed for per diagonal
constexpr int kFarKT = 64;       // k-slice depth of the far-field GEMMs
constexpr int kSweep = 2 * kB - 1;  // steps of one leaf's wavefront
constexpr int kStrip = 16;       // columns (rows) per hand-over
constexpr int kStrips = kB / kStrip;

struct SolveParams {
    const float* W;
    int64_t ldw;
    const float* LO;
    int64_t ldlo;
    const float* LI;
    int64_t ldli;
    int64_t m, n;
    int M, N;  // leaf grid
    int bits, stochastic;
    uint64_t seed;
    const float* scales;
    uint8_t* codes;
    int64_t ldc;
    float* delta;
    int64_t ldd;
    float* ct;  // n x m, C^T, ld = m
    float* parts;
    double* leaf_loss;
    int* leaf_clamp;
    const float* DO;
    const float* DI;
    int want_loss;
    int* info;
    int maxleaf;
    // schedule
    int* ticket;     // next task to take
    int* abort;      // set once a wait has expired
    int* prog_d;     // per leaf: strips of D published (0..4)
    int* prog_c;     // per leaf: strips of C published (0..4)
    int* setup;      // per leaf: 1 once its far-field partials are consumed
    int* fardone;    // per leaf: far-field tasks finished
    int* seg;        // first task of each group k (ND + 1 entries)
    int* nchd;       // K-chunks of the far-field products, per diagonal
    int ND;          // leaf-diagonals
    int ntask;
    uint64_t spin_limit;  // wall-clock ticks a single wait may take
};

__host__ __device__ __forceinline__ int diag_lo(int N, int d) { return d - (N - 1) > 0 ? d - (N - 1) : 0; }
__host__ __device__ __forceinline__ int diag_hi(int M, int d) { return d < M - 1 ? d : M - 1; }
__host__ __device__ __forceinline__ int diag_leaves(int M, int N, int d) {
    return diag_hi(M, d) - diag_lo(N, d) + 1;
}
// K-chunks per far-field product on diagonal d: enough tasks to fill the chip,
// chunks of at least 4 blocks
__host__ __device__ __forceinline__ int diag_nch(int M, int N, int d) {
    const int lo = diag_lo(N, d), hi = diag_hi(M, d), nl = hi - lo + 1;
    const int kmax = (hi > d - lo ? hi : d - lo) - 2;  // blocks three or more back
    int nch = (kTargetWg + 2 * nl - 1) / (2 * nl);
    const int cap = kmax / 4 > 1 ? kmax / 4 : 1;
    nch = nch < cap ? nch : cap;
    nch = nch < kNch ? nch : kNch;
    return nch > 1 ? nch : 1;
}
// tasks of group k: the leaves of diagonal k, then the far fields of diagonal k + 1
// (those exist from diagonal 3 on: they need blocks three or more back). A far
// task reads leaves two or more groups back, so it rarely waits; the leaves of
// its diagonal come right after it in the order.
__host__ __device__ __forceinline__ int group_far(int ND, int k) { return (k + 1 >= 3 && k + 1 < ND) ? k + 1 : -1; }
__host__ __device__ __forceinline__ int group_tasks(int M, int N, int ND, int k) {
    int s = diag_leaves(M, N, k);
    const int df = group_far(ND, k);
    if (df >= 0) s += diag_leaves(M, N, df) * 2 * diag_nch(M, N, df);
    return s;
}

__device__ __forceinline__ int leaf_lo(const SolveParams& p, int d) { return diag_lo(p.N, d); }

// far-field partials: ring slot of the diagonal, leaf slot on it, kind (0: p, 1: o^T), K-chunk
__device__ __forceinline__ float* part_ptr(const SolveParams& p, int d, int slot, int kind, int c) {
    return p.parts + ((((size_t)(d % kRing) * p.maxleaf + slot) * 2 + kind) * kNch + c) * (kB * kB);
}

// ---------------------------------------------------------------------------
// hand-over primitives. Each XCD has its own L2, so data passed between
// workgroups is written with device-coherent (agent-scope) stores, which go
// through to memory, and a producer raises its counter (also agent scope)
// only once those stores have completed (s_waitcnt vmcnt(0)): no cache-wide
// write-back is needed. A consumer that then reads through the caches first
// invalidates them (acquire fence at agent scope); the hand-overs inside a
// leaf's sweep read with device-coherent loads instead, so the sweep never
// waits on cache maintenance.
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
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
// keeps the compiler from moving the data loads above the counter check
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// the wave's own memory operations, cache maintenance included, have completed
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Waits until *f >= v. Returns false if this wait ran past the time limit (it
// then stops every other wait of the solve) or another one already did.
__device__ __forceinline__ bool wait_flag(const SolveParams& p, const int* f, int v) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        if (ld_flag(f) >= v) return true;
        if (ld_flag(p.abort)) return false;
        if (__builtin_amdgcn_s_memrealtime() - t0 > p.spin_limit) {
            st_flag(p.abort, 1);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// ---------------------------------------------------------------------------
// scales: s_i = fp32(2 max_j |W*_ij|) / fp32(Lq), or the caller's scale
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_scales(const float* __restrict__ W, int64_t n,
                                                     int64_t ldw, int bits,
                                                     const float* __restrict__ row_scale,
                                                     float* __restrict__ scales, int* info) {
    const int64_t i = blockIdx.x;
    float s;
    if (row_scale) {
        s = row_scale[i];
    } else {
        __shared__ float red[kThreads];
        float a = 0.0f;
        const float* w = W + i * ldw;
        for (int64_t j = threadIdx.x; j < n; j += kThreads) {
            const float v = fabsf(w[j]);
            a = (v > a || v != v) ? v : a;  // NaN propagates
        }
        red[threadIdx.x] = a;
        __syncthreads();
        for (int o = kThreads / 2; o > 0; o >>= 1) {
            if ((int)threadIdx.x < o) {
                const float b = red[threadIdx.x + o];
                const float c = red[threadIdx.x];
                red[threadIdx.x] = (b > c || b != b) ? b : c;
            }
            __syncthreads();
        }
        s = (2.0f * red[0]) / (float)((1 << bits) - 1);
    }
    if (threadIdx.x == 0) {
        scales[i] = s;
        if (!(s > 0.0f) || !(s < INFINITY)) atomicMin(info, (int)min<int64_t>(i + 1, INT_MAX - 1));
    }
}


// Clears the schedule state and builds the task table: workgroup 0 scans the
// per-group task counts 256 diagonals at a time; the counters are cleared by the
// whole grid.
__global__ __launch_bounds__(kThreads) void k_solve_init(SolveParams p) {
    const int64_t nl = (int64_t)p.M * p.N;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < nl; e += (int64_t)gridDim.x * kThreads) {
        p.prog_d[e] = 0;
        p.prog_c[e] = 0;
        p.setup[e] = 0;
        p.fardone[e] = 0;
    }
    if (blockIdx.x != 0) return;
    __shared__ int sc[kThreads];
    const int t = threadIdx.x;
    int carry = 0;
    for (int base = 0; base < p.ND; base += kThreads) {
        const int k = base + t;
        int v = 0;
        if (k < p.ND) {
            p.nchd[k] = diag_nch(p.M, p.N, k);
            v = group_tasks(p.M, p.N, p.ND, k);
        }
        sc[t] = v;
        __syncthreads();
        for (int o = 1; o < kThreads; o <<= 1) {  // inclusive scan
            const int x = t >= o ? sc[t - o] : 0;
            __syncthreads();
            sc[t] += x;
            __syncthreads();
        }
        if (k < p.ND) p.seg[k] = carry + sc[t] - v;
        carry += sc[kThreads - 1];
        __syncthreads();
    }
    if (t == 0) {
        p.seg[p.ND] = carry;
        *p.info = INT_MAX;
        *p.ticket = 0;
        *p.abort = 0;
    }
}

// ---------------------------------------------------------------------------
// far field of diagonal d: chunk c (of nch) of p (kind 0) or o^T (kind 1) of
// one leaf, over the blocks three or more above (p) or to the left (o) of the
// leaf. It starts once the last leaf of its K range has published all of its
// D (C); the leaves before it in that column (row) finished earlier, since
// each waited on its predecessor. Each chunk writes its own 64x64 partial (an
// empty chunk writes zeros); the leaf adds them in chunk order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void chunk_range(int kblk, int nch, int c, int& b0, int& b1) {
    const int len = (kblk + nch - 1) / nch;
    b0 = min(c * len, kblk);
    b1 = min(b0 + len, kblk);
}

// Whole 64x64 far-field tiles with 16-byte aligned rows: k-slices of kFarRingKT
// rows fill a ring of kFarRingNS slots in LDS by direct global-to-LDS loads
// (global_load_lds_dwordx4: one instruction of a wave fills four 64-float rows),
// kFarRingNS - 1 slices ahead of the MFMAs, so several slices of loads are in
// flight while the tile is computed. Waves 0-3 load and compute (32x32 quadrant
// each); the others only join the barriers.
constexpr int kFarRingKT = 32;
constexpr int kFarRingNS = 4;
struct FarRing {
    float a[kFarRingNS][kFarRingKT][kB];
    float b[kFarRingNS][kFarRingKT][kB];
};

// Wait until at most N of this wave's vector-memory operations are outstanding, then
// meet the other waves. Direct-to-LDS loads complete in issue order, so with N = the
// loads issued after slice s, slice s is in LDS once every wave has passed; the later
// loads stay in flight across the barrier.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// acc += A^T B over K (a multiple of kFarRingKT) for a whole 64x64 tile: A (k, r) at
// A[k*lda + r], B (k, c) at B[k*ldb + c]; every thread of the workgroup calls it.
__device__ __forceinline__ void far_gemm_ring(const float* __restrict__ A, int64_t lda,
                                              const float* __restrict__ B, int64_t ldb, int64_t K,
                                              f32x16& acc, FarRing& sm, int tid) {
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool active = w < 4;
    const int ra = (w >> 1) * 32 + (lane & 31);
    const int rb = (w & 1) * 32 + (lane & 31);
    const int kh = lane >> 5;
    const int c4 = (lane & 15) << 2;
    constexpr int kLoads = 2 * (kFarRingKT / 16);  // direct loads per active wave per slice
    const int64_t ns = K / kFarRingKT;
    auto issue = [&](int64_t s) {
        const int slot = (int)(s % kFarRingNS);
        const int64_t k0 = s * kFarRingKT;
#pragma unroll
        for (int h = 0; h < kFarRingKT / 16; ++h) {
            const int r = 4 * (2 * w + h);  // rows r .. r+3 of the slice
            const int64_t k = k0 + r + (lane >> 4);
            __builtin_amdgcn_global_load_lds(A + k * lda + c4, &sm.a[slot][r][0], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(B + k * ldb + c4, &sm.b[slot][r][0], 16, 0, 0);
        }
    };
    if (active)
        for (int s = 0; s < kFarRingNS - 1; ++s)
            if (s < ns) issue(s);
    for (int64_t it = 0; it < ns; ++it) {
        if (it + kFarRingNS - 2 < ns) vm_wait_barrier<(kFarRingNS - 2) * kLoads>();
        else vm_wait_barrier<0>();
        if (!active) continue;
        if (it + kFarRingNS - 1 < ns) issue(it + kFarRingNS - 1);
        const int slot = (int)(it % kFarRingNS);
        float fa[3], fb[3];
        fa[0] = sm.a[slot][kh][ra];
        fb[0] = sm.b[slot][kh][rb];
        fa[1] = sm.a[slot][2 + kh][ra];
        fb[1] = sm.b[slot][2 + kh][rb];
#pragma unroll
        for (int s = 0; s < kFarRingKT / 2; ++s) {
            if (s + 2 < kFarRingKT / 2) {
                fa[(s + 2) % 3] = sm.a[slot][2 * (s + 2) + kh][ra];
                fb[(s + 2) % 3] = sm.b[slot][2 * (s + 2) + kh][rb];
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the reads two steps ahead of the MFMAs
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s % 3], fb[s % 3], acc, 0, 0, 0);
        }
    }
}

union FarSmem {
    GemmSmemF32<kFarKT> staged;  // ragged tiles
    FarRing ring;
};

__device__ __forceinline__ void far_task(const SolveParams& p, int d, int task, FarSmem& sm, int tid) {
    const int nch = p.nchd[d];
    const int slot = task / (2 * nch);
    const int kind = (task / nch) & 1;
    const int c = task % nch;
    const int I = leaf_lo(p, d) + slot;
    const int J = d - I;
    const bool has = kind == 0 ? (p.LO != nullptr && I > 2) : (p.LI != nullptr && J > 2);
    if (has) {
        int kb0, kb1;
        chunk_range((kind == 0 ? I : J) - 2, nch, c, kb0, kb1);
        if (tid == 0) {
            if (kb1 > kb0) {
                if (kind == 0) wait_flag(p, &p.prog_d[(int64_t)(kb1 - 1) * p.N + J], kStrips);
                else wait_flag(p, &p.prog_c[(int64_t)I * p.N + kb1 - 1], kStrips);
            }
            if (d >= kRing) {  // the leaf that last used this ring slot has read it
                const int dp = d - kRing;
                if (slot < diag_leaves(p.M, p.N, dp)) {
                    const int Ip = leaf_lo(p, dp) + slot;
                    wait_flag(p, &p.setup[(int64_t)Ip * p.N + (dp - Ip)], 1);
                }
            }
            acquire_agent();
            vm_wait_all();
        }
        __syncthreads();
        const int64_t i0 = (int64_t)I * kB, j0 = (int64_t)J * kB;
        const int R = (int)min<int64_t>(kB, p.m - i0), Cc = (int)min<int64_t>(kB, p.n - j0);
        const int64_t k0 = (int64_t)kb0 * kB, K = (int64_t)(kb1 - kb0) * kB;
        f32x16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
        const bool active = tid < kThreads;  // the other waves only join the barriers
        // p[ii][jj] = sum_k L_O[k][i0+ii] D[k][j0+jj];  o^T[jj][ii] = sum_l L_I[l][j0+jj] C^T[l][i0+ii]
        const float* A = kind == 0 ? p.LO + k0 * p.ldlo + i0 : p.LI + k0 * p.ldli + j0;
        const float* Bm = kind == 0 ? p.delta + k0 * p.ldd + j0 : p.ct + k0 * p.m + i0;
        const int64_t lda = kind == 0 ? p.ldlo : p.ldli, ldb = kind == 0 ? p.ldd : p.m;
        const int ra_lim = kind == 0 ? R : Cc, cb_lim = kind == 0 ? Cc : R;
        const bool whole = R == kB && Cc == kB && ((lda | ldb) & 3) == 0 &&
                           ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(Bm)) & 15) == 0;
        if (whole) far_gemm_ring(A, lda, Bm, ldb, K, acc, sm.ring, tid);
        else tile_gemm_f32<kFarKT>(A, lda, ra_lim, Bm, ldb, cb_lim, K, acc, sm.staged, active, tid);
        if (active) {
            float* part = part_ptr(p, d, slot, kind, c);
            const int cc = acc32_col(tid);
#pragma unroll
            for (int v = 0; v < 16; ++v) st_coherent(&part[acc32_row(v, tid) * kB + cc], acc[v]);
        }
        vm_wait_all();  // every wave's device-coherent partial stores have completed
        __syncthreads();
    }
    if (tid == 0) {
        __hip_atomic_fetch_add(&p.fardone[(int64_t)I * p.N + J], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// leaf solve: the 64x64 leaf (I, J) of diagonal d.
//
// Entry (i, j) is finalised at step i + j. Its in-leaf sums
//   pn = sum_{k<i} L_O[k][i] D[k][j],   rn = sum_{l<j} g[i][l] L_I[l][j]
// (g = C, the column feedback plus error of the row) are split into a bulk,
// which only uses entries finalised three or more steps earlier, and the two
// newest terms of each (k = i-1, i-2 and l = j-1, j-2). Four bulk waves compute
// the bulk of step st + 2 while the finaliser wave finalises step st, so the dependent chain
// of a step holds no LDS read: the finaliser takes D[i-1][j] and D[i-2][j]
// from the lanes above by DPP, g[i][j-1] and g[i][j-2] from its own previous
// steps, and the bulk sums and static inputs were read one step ahead.
//
// Bulk lanes are (a, quarter q) with lane = 4 a + q; quarter q owns the k / l
// range [16q, 16q + 16). Lane a sums P along row a of L_O^T and R along column
// a of L_I, both held in registers, against 16-float chunks of D and g read as
// four adjacent 16-byte words (68-float rows spread a row group over the
// banks); the factors are zero beyond the bulk's range, so no term needs a
// per-step mask.
//
// Waves 5 and 6 do the hand-overs, column-wise (5: D to the leaf below, and
// L_O[above, this]^T D[above, strip] into p) and row-wise (6: C to the leaf on
// the right, and C[strip, left] L_I[left, this] into o). Strip c (columns or
// rows 16c..16c+15) of this leaf is final after step 78 + 16c; it is stored a
// step later (storing each column as it became final, 64 scattered rows a
// store, measured slower) and its counter raised three steps after that, when
// the stores have landed. The neighbour's strip c (c >= 1) is taken in a window ending at
// step 16c - 2: counter read at 16c - 12, checked (and waited for, if late)
// at 16c - 10 and the strip loaded (device-coherent loads, which go to memory),
// multiplied with v_mfma_f32_16x16x4_f32 over steps 16c - 7 .. 16c - 3 (a
// dozen MFMAs a step, within what the other waves take for a step) and added
// to p (o) before the finaliser reads columns (rows) 16c.., at the end of step
// 16c - 1. Strip 0 is taken before the sweep.
// ---------------------------------------------------------------------------
constexpr int kLeafWaves = 7;
constexpr int kLeafThreads = kLeafWaves * 64;
// Roles in the sweep by wave index. Waves are spread over the four SIMDs by
// index (SIMD w mod 4): the finaliser, whose chain sets the pace, has SIMD 3 to
// itself (sharing it with a bulk wave cost a fifth of the sweep's speed); bulk
// waves 0, 1, 2 and 4 and hand-over waves 5 and 6 fill SIMDs 0-2. Putting both
// hand-over waves on one SIMD measured slower.
constexpr int kFinWave = 3;
constexpr int kColWave = 5;  // hand-over of columns of D (to the leaf below)
constexpr int kRowWave = 6;  // hand-over of rows of C (to the leaf on the right)
constexpr int kTs = 68;  // row stride of the 64x64 tiles: 16-byte aligned rows, 4 banks apart
constexpr int kPs = 66;  // row stride of the per-entry inputs: anti-diagonal walks hit distinct banks

struct LeafSmem {
    float DT[kB][kTs];     // D transposed: DT[j][k] = D[k][j] (0 until known)
    float Gs[kB][kTs];     // g = C of the leaf, row-major (0 until known)
    float bt[kB][kTs];     // W* + o, transposed: bt[j][i] for entry (i, j)
    float pt[kB][kTs];     // p, transposed: pt[j][i]
    float wst[kB][kPs];    // W*, overwritten by eta = t - q once the entry is final
    float pnb[3][kB];      // bulk sums, by step modulo 3 (written two steps ahead)
    float rnb[3][kB];
    float li1[kB];         // L_I[j-1][j], L_I[j-2][j]: the finaliser's terms
    float li2[kB];
    uint8_t code[kB][kB + 4];
    float DI[kB];
    double red[kLeafWaves];
    int red_i[kLeafWaves];
};

// acc += X^T Y over k = 0..63 for the 64x64 tile, X[k][r] at x[k * sx + r] and
// Y[k][c] at y[k * sy + c] in LDS; waves 0-3 each own a 32x32 quadrant
// (32x32x2 f32 MFMA operand and output layout of bk_common.hpp).
__device__ __forceinline__ void adj_gemm(const float* x, int sx, const float* y, int sy, f32x16& acc, int tid) {
    const int lane = tid & 63, w = tid >> 6;
    const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
#pragma unroll
    for (int k = 0; k < kB; k += 2) {
        const int kr = k + (lane >> 5);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x[kr * sx + wr + (lane & 31)], y[kr * sy + wc + (lane & 31)],
                                                   acc, 0, 0, 0);
    }
}

// A step ends with lds_wait_all() (the step's LDS stores are complete), the reads
// for the next step, then barrier_no_wait(): the reads stay in flight across the
// barrier, which needs only the stores. The memory clobbers keep the compiler from
// moving memory operations across either point.
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier_no_wait() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ float lane_above(float x) {
    // wave_shr:1 -- lane i receives lane i-1's value, lane 0 receives 0
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x138,
                                                                  0xF, 0xF, false));
}

__device__ __forceinline__ f32x4 lds4(const float* q) { return *reinterpret_cast<const f32x4*>(q); }

// ---- hand-overs (waves 5 and 6). Operand kk of lane l is row 4 kk + l / 16,
// column l % 16 of the neighbour's strip: D[i0-64+k][j0+16c+x] (column-wise) or
// C^T[j0-64+l][i0+16c+r] (row-wise). The product tile is 64 x 16 (16 x 64),
// four 16x16 blocks; element q of block t sits at row 4 (l / 16) + q, column
// l % 16 of the block (v_mfma_f32_16x16x4_f32 output layout).
struct Handover {
    float fa[64];  // the static factor block in operand order: element 4 kk + t is
                   // row 4 kk + l / 16, column 16 t + l % 16 of L_O[above, this] (L_I[left, this])
    float bv[16];
    f32x4 acc[4];
};

__device__ __forceinline__ void handover_factor(const SolveParams& p, bool col, int64_t i0, int64_t j0, int R,
                                                int Cc, Handover& h, int lane) {
    const float* src = col ? p.LO + (i0 - kB) * p.ldlo + i0 : p.LI + (j0 - kB) * p.ldli + j0;
    const int64_t ld = col ? p.ldlo : p.ldli;
    const int lim = col ? R : Cc;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
        const int64_t k = 4 * kk + (lane >> 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = 16 * t + (lane & 15);
            h.fa[4 * kk + t] = c < lim ? src[k * ld + c] : 0.0f;
        }
    }
}

__device__ __forceinline__ void handover_load(const SolveParams& p, bool col, int c, int64_t i0, int64_t j0,
                                              int R, int Cc, Handover& h, int lane) {
    const int s = kStrip * c + (lane & 15);
    // a wave-uniform base and stride, and a 32-bit lane offset
    const float* src = col ? p.delta + (i0 - kB) * p.ldd + j0 : p.ct + (j0 - kB) * p.m + i0;
    const int64_t ld = col ? p.ldd : p.m;
    const bool ok = s < (col ? Cc : R);
    const int64_t off = (lane >> 4) * ld + s;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
        const float* row = src + (int64_t)(4 * kk) * ld;
        h.bv[kk] = ok ? __hip_atomic_load(row + off, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) h.acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

template <int KK0, int KK1>
__device__ __forceinline__ void handover_mma(bool col, Handover& h) {
#pragma unroll
    for (int kk = KK0; kk < KK1; ++kk) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (col)  // p[a][x] += sum_k L_O[above k][a] D[above k][x]
                h.acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(h.fa[4 * kk + t], h.bv[kk], h.acc[t], 0, 0, 0);
            else  // o[r][j] += sum_l C[r][left l] L_I[left l][j]
                h.acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(h.bv[kk], h.fa[4 * kk + t], h.acc[t], 0, 0, 0);
        }
    }
}

// the four elements of a lane's block t are consecutive in the transposed p and
// o: one 16-byte read-modify-write each
__device__ __forceinline__ void handover_add(LeafSmem& sm, bool col, int c, const Handover& h, int lane) {
    const int r0 = 4 * (lane >> 4), cc = lane & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        // column-wise: entries (16t + r0 + q, 16c + cc); row-wise: (16c + r0 + q, 16t + cc)
        f32x4* q4 = col ? reinterpret_cast<f32x4*>(&sm.pt[kStrip * c + cc][16 * t + r0])
                        : reinterpret_cast<f32x4*>(&sm.bt[16 * t + cc][kStrip * c + r0]);
        *q4 += h.acc[t];
    }
}

// stores strip c of this leaf's D (column-wise) or C^T (row-wise), device-coherent.
// Lane (s, quarter) reads 16 consecutive k of row s of DT (Gs) as four 16-byte words;
// each store then covers 16 consecutive columns (strip entries s) of four rows k.
__device__ __forceinline__ void handover_publish(const SolveParams& p, const LeafSmem& sm, bool col, int c,
                                                 int64_t i0, int64_t j0, int R, int Cc, int lane) {
    const int si = lane & 15, qk = lane >> 4;  // strip entry, quarter of k
    const int s = kStrip * c + si;
    float* dst = col ? p.delta + i0 * p.ldd + j0 + s : p.ct + j0 * p.m + i0 + s;
    const int64_t ld = col ? p.ldd : p.m;
    const int klim = col ? R : Cc, slim = col ? Cc : R;
    const float* rowp = col ? &sm.DT[s][16 * qk] : &sm.Gs[s][16 * qk];  // D[k][s] = DT[s][k]; C[s][k] = Gs[s][k]
    f32x4 v[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) v[h] = lds4(rowp + 4 * h);  // every read first
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int k = 16 * qk + e;
        if (k < klim && s < slim) st_coherent(dst + (int64_t)k * ld, v[e >> 2][e & 3]);
    }
}

__device__ __forceinline__ void handover_flag(const SolveParams& p, bool col, int64_t leaf, int v, int lane) {
    vm_wait_all();  // the strip's device-coherent stores have completed
    if (lane == 0) st_flag(col ? &p.prog_d[leaf] : &p.prog_c[leaf], v);
}

__device__ __forceinline__ void leaf_task(const SolveParams& p, int d, int slot, LeafSmem& sm, int tid) {
    const int I = leaf_lo(p, d) + slot;
    const int J = d - I;
    const int64_t i0 = (int64_t)I * kB, j0 = (int64_t)J * kB;
    const int R = (int)min<int64_t>(kB, p.m - i0), Cc = (int)min<int64_t>(kB, p.n - j0);
    const int t = tid;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t leaf = (int64_t)I * p.N + J;
    const int nch = p.nchd[d];
    const bool far_p = p.LO && I > 2, far_o = p.LI && J > 2;  // far-field partials (blocks <= I-3, J-3)
    const bool two_p = p.LO && I > 1, two_o = p.LI && J > 1;  // the blocks two back
    const bool adj_p = p.LO && I > 0, adj_o = p.LI && J > 0;  // the adjacent blocks (handed over)
    if (t < 2) {  // no L_I[j-d][j] for j < d
        sm.li2[t] = 0.0f;
        if (t < 1) sm.li1[t] = 0.0f;
    }
    constexpr int kPer = (kB * kB + kLeafThreads - 1) / kLeafThreads;
    // ---- A: static inputs, every load of the thread in flight at once
    //   DT  <- L_O[i0-128+k][i0+c]  pt <- L_I[j0-128+k][j0+c]    (blocks two back: staging)
    //   wst <- W*[i0+k][j0+c]       li1, li2 <- the first two superdiagonals of L_I
    {
        float v1[kPer], v3[kPer], v5[kPer], v6[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            const int k = e >> 6, c = e & 63;
            const bool in = e < kB * kB;
            v1[u] = (in && two_p && c < R) ? p.LO[(i0 - 2 * kB + k) * p.ldlo + i0 + c] : 0.0f;
            v3[u] = (in && two_o && c < Cc) ? p.LI[(j0 - 2 * kB + k) * p.ldli + j0 + c] : 0.0f;
            v5[u] = (in && k < R && c < Cc) ? p.W[(i0 + k) * p.ldw + j0 + c] : 0.0f;
            v6[u] = (in && p.LI && (c - k == 1 || c - k == 2) && c < Cc) ? p.LI[(j0 + k) * p.ldli + j0 + c] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            if (e < kB * kB) {
                const int k = e >> 6, c = e & 63;
                sm.DT[k][c] = v1[u];
                sm.pt[k][c] = v3[u];
                sm.wst[k][c] = v5[u];
                if (c - k == 1) sm.li1[c] = v6[u];
                if (c - k == 2) sm.li2[c] = v6[u];
            }
        }
    }
    // ---- B: far fields from three or more blocks back: once their tasks are done,
    // the K-chunk partials are summed in chunk order into registers (every load
    // issued first; absent chunks read a valid address and are replaced by zero)
    if (t == 0) {
        if (d >= 3) wait_flag(p, &p.fardone[leaf], 2 * nch);
        acquire_agent();
        vm_wait_all();
    }
    __syncthreads();
    constexpr int kG = (kB * kB / 4 + kLeafThreads - 1) / kLeafThreads;
    const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 pvs[kG], ovs[kG];  // p and o^T, four consecutive entries per group
    {
        const bool any = far_p || far_o;
        f32x4 xp[kG][kNch], xo[kG][kNch];
        if (any) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int g = min(t + u * kLeafThreads, kB * kB / 4 - 1);
#pragma unroll
                for (int c = 0; c < kNch; ++c) {
                    const int cc = min(c, nch - 1);
                    xp[u][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, d, slot, 0, cc) + 4 * g);
                    xo[u][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, d, slot, 1, cc) + 4 * g);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            if (u == 2 && any) {
#pragma unroll
                for (int uu = 2; uu < kG; ++uu) {
                    const int gg = min(t + uu * kLeafThreads, kB * kB / 4 - 1);
#pragma unroll
                    for (int c = 0; c < kNch; ++c) {
                        const int cc = min(c, nch - 1);
                        xp[uu][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, d, slot, 0, cc) + 4 * gg);
                        xo[uu][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, d, slot, 1, cc) + 4 * gg);
                    }
                }
            }
            f32x4 pv = z4, ov = z4;
            if (any) {
#pragma unroll
                for (int c = 0; c < kNch; ++c) {
                    const bool up = far_p && c < nch, uo = far_o && c < nch;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        pv[k] += up ? xp[u][c][k] : 0.0f;
                        ov[k] += uo ? xo[u][c][k] : 0.0f;
                    }
                }
            }
            pvs[u] = pv;
            ovs[u] = ov;
        }
    }
    // the partials are read (their ring slot may be reused)
    __syncthreads();
    if (t == 0) st_flag(&p.setup[leaf], 1);
    // ---- the leaves two blocks up and to the left: once they are done, their
    // blocks are multiplied (K = 64)
    if (t == 0) {
        if (two_p) wait_flag(p, &p.prog_d[leaf - 2 * (int64_t)p.N], kStrips);
        if (two_o) wait_flag(p, &p.prog_c[leaf - 2], kStrips);
        acquire_agent();
        vm_wait_all();
    }
    __syncthreads();
    //   Gs <- D[i0-128+k][j0+c]     bt <- C^T[j0-128+k][i0+c]     (staging)
    {
        float v2[kPer], v4[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            const int k = e >> 6, c = e & 63;
            const bool in = e < kB * kB;
            v2[u] = (in && two_p && c < Cc) ? p.delta[(i0 - 2 * kB + k) * p.ldd + j0 + c] : 0.0f;
            v4[u] = (in && two_o && c < R) ? p.ct[(j0 - 2 * kB + k) * p.m + i0 + c] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            if (e < kB * kB) {
                const int k = e >> 6, c = e & 63;
                sm.Gs[k][c] = v2[u];
                sm.bt[k][c] = v4[u];
            }
        }
    }
    __syncthreads();
    f32x16 ap, ao;  // products with the blocks two back: p += L_O^T D, o^T += L_I^T C^T
#pragma unroll
    for (int v = 0; v < 16; ++v) ap[v] = ao[v] = 0.0f;
    if (w < 4) {
        if (two_p) adj_gemm(&sm.DT[0][0], kTs, &sm.Gs[0][0], kTs, ap, t);
        if (two_o) adj_gemm(&sm.pt[0][0], kTs, &sm.bt[0][0], kTs, ao, t);
    }
    __syncthreads();
    // ---- C: p = partials + ap, o = partials + ao, then W* added to o; D, g and
    // the codes cleared (the staging is consumed)
#pragma unroll
    for (int u = 0; u < kG; ++u) {
        const int g = t + u * kLeafThreads;
        if (g < kB * kB / 4) {
            const int k = g >> 4, c4 = (g & 15) << 2;
            *reinterpret_cast<f32x4*>(&sm.DT[k][c4]) = z4;
            *reinterpret_cast<f32x4*>(&sm.Gs[k][c4]) = z4;
            *reinterpret_cast<uint32_t*>(&sm.code[k][c4]) = 0u;
            const int e = 4 * g;
            const int r = e / kB, c0 = e % kB;  // p: row r, cols c0..c0+3; o^T: row (= leaf col) r, leaf rows c0..
#pragma unroll
            for (int q = 0; q < 4; ++q) sm.pt[c0 + q][r] = pvs[u][q];
            *reinterpret_cast<f32x4*>(&sm.bt[r][c0]) = ovs[u];
        }
    }
    __syncthreads();
    if (w < 4) {
        const int cc = acc32_col(t);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            sm.pt[cc][acc32_row(v, t)] += ap[v];  // entry (row, cc)
            sm.bt[acc32_row(v, t)][cc] += ao[v];  // entry (cc, row)
        }
    }
    __syncthreads();
    for (int e = t; e < kB * kB; e += kLeafThreads) {
        const int j = e / kB, i = e % kB;
        sm.bt[j][i] += sm.wst[i][j];
    }
    if (t < kB) {
        sm.DI[t] = (p.want_loss && t < Cc) ? p.DI[j0 + t] : 0.0f;
        sm.pnb[0][t] = sm.pnb[1][t] = sm.pnb[2][t] = 0.0f;
        sm.rnb[0][t] = sm.rnb[1][t] = sm.rnb[2][t] = 0.0f;
    }
    __syncthreads();
    // ---- D: the neighbours' first strips are taken before the sweep
    const bool hwave = w == kColWave || w == kRowWave;
    const bool hcol = w == kColWave;
    const bool hown = hcol ? adj_p : adj_o;  // this hand-over wave has a neighbour to take from
    const int* hflag = !hown ? p.prog_d : hcol ? p.prog_d + (leaf - p.N) : p.prog_c + (leaf - 1);
    Handover h;  // the factor block stays in registers for the whole sweep
    if (hwave && hown) {
        handover_factor(p, hcol, i0, j0, R, Cc, h, lane);
        wait_flag(p, hflag, 1);
        compiler_fence();
        handover_load(p, hcol, 0, i0, j0, R, Cc, h, lane);
        handover_mma<0, 16>(hcol, h);
        handover_add(sm, hcol, 0, h, lane);
    }

    double loss = 0.0;
    int nclamp = 0;
    const bool bulk = w != kFinWave && w != kColWave && w != kRowWave;
    if (bulk) {
        // ---------------- bulk waves ----------------
        // Lane (a, quarter q) sums the k / l range [16q, 16q + 16) of two bulk sums of
        // the entries finalised two steps later (x = st + 2 - a):
        //   P of entry (a, x): sum_k L_O[k][a] D[k][x],  k <= a - 3 (row a)
        //   R of entry (x, a): sum_l g[x][l] L_I[l][a],  l <= a - 3 (column a)
        // so both triangular factors stay in registers (row a of L_O^T, column a of
        // L_I) and a step reads two 16-float chunks per lane: column x of D and row x
        // of g. The newest terms (k, l = a - 3, final in the previous step) are read
        // on their own at the start of the step; the chunks (entries final a step
        // earlier) were read at the end of the previous step, so their LDS latency
        // overlaps the barrier and the finaliser's work.
        const int bt = (w == 4 ? kFinWave : w) * 64 + lane;  // bulk thread 0..255 (waves 0, 1, 2, 4)
        const int a = bt >> 2;
        const int q = bt & 3;
        const int k0 = 16 * q;
        float lo[16];  // L_O[i0 + k][i0 + a] for k <= a - 4, else 0
        float li[16];  // L_I[j0 + l][j0 + a] for l <= a - 4, else 0
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            lo[e] = (p.LO && k0 + e <= a - 4 && a < R) ? p.LO[(i0 + k0 + e) * p.ldlo + i0 + a] : 0.0f;
            li[e] = (p.LI && k0 + e <= a - 4 && a < Cc) ? p.LI[(j0 + k0 + e) * p.ldli + j0 + a] : 0.0f;
        }
        // L_O[a-3][a] and L_I[a-3][a], added by quarter 0 with the newest D and g
        const float lo3 = (p.LO && q == 0 && a >= 3 && a < R) ? p.LO[(i0 + a - 3) * p.ldlo + i0 + a] : 0.0f;
        const float li3 = (p.LI && q == 0 && a >= 3 && a < Cc) ? p.LI[(j0 + a - 3) * p.ldli + j0 + a] : 0.0f;
        // An entry written in the step the chunk is read meets a zero factor: L_O and
        // L_I are zero beyond a - 4.
        auto fetch = [&](int st, f32x4 (&c)[8]) {
            const int xc = min(max(st + 2 - a, 0), kB - 1);
            const float* dp = &sm.DT[xc][k0];
            const float* gp = &sm.Gs[xc][k0];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                c[h] = lds4(dp + 4 * h);
                c[4 + h] = lds4(gp + 4 * h);
            }
        };
        int slot3 = 2;  // (st + 2) mod 3
        auto step = [&](int st, const f32x4 (&cur)[8], f32x4 (&nxt)[8]) {
            const int x = st + 2 - a;
            const bool live = x >= 0 && x < kB;
            const int xc = min(max(x, 0), kB - 1);
            // the newest terms, read behind the chunks fetched in the previous step
            const int a3 = max(a - 3, 0);
            const float dnew = sm.DT[xc][a3];  // D[a-3][x]
            const float gnew = sm.Gs[xc][a3];  // g[x][a-3]
            float p0 = lo3 * dnew, p1 = 0.0f, r0 = li3 * gnew, r1 = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p0 = fmaf(lo[e], cur[0][e], p0);
                p1 = fmaf(lo[4 + e], cur[1][e], p1);
                r0 = fmaf(li[e], cur[4][e], r0);
                r1 = fmaf(li[4 + e], cur[5][e], r1);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p0 = fmaf(lo[8 + e], cur[2][e], p0);
                p1 = fmaf(lo[12 + e], cur[3][e], p1);
                r0 = fmaf(li[8 + e], cur[6][e], r0);
                r1 = fmaf(li[12 + e], cur[7][e], r1);
            }
            float pn = live ? p0 + p1 : 0.0f;
            float rn = live ? r0 + r1 : 0.0f;
            pn = quad_sum(pn);
            rn = quad_sum(rn);
            if (q == 0 && live) {
                sm.pnb[slot3][a] = pn;  // entry (a, x)
                sm.rnb[slot3][x] = rn;  // entry (x, a)
            }
            slot3 = slot3 == 2 ? 0 : slot3 + 1;
            // the next step's chunks go out after the stores and stay in flight across
            // the barrier: every entry they read with a nonzero factor was final a step
            // earlier, so later writes into the chunks meet a zero factor
            lds_wait_all();
            __builtin_amdgcn_sched_barrier(0);
            fetch(st + 1, nxt);
            __builtin_amdgcn_sched_barrier(0);
            barrier_no_wait();
        };
        f32x4 ca[8], cb[8];
        __syncthreads();
        fetch(0, ca);
        int st = 0;
        for (; st + 1 < 2 * kB - 1; st += 2) {
            step(st, ca, cb);
            step(st + 1, cb, ca);
        }
        step(st, ca, cb);  // 127 steps: the last one
    } else if (w == kFinWave) {
        // ---------------- finaliser wave: lane i owns row i ----------------
        // adds the two newest terms of each sum: D[i-1][j], D[i-2][j] (from the
        // lanes above, by DPP) and g[i][j-1], g[i][j-2] (its own previous results);
        // eta = t - q goes into W*'s slot (consumed one step earlier) for the loss
        const int i = t & 63;
        const float lo1 = (p.LO && i >= 1 && i < R) ? p.LO[(i0 + i - 1) * p.ldlo + i0 + i] : 0.0f;
        const float lo2 = (p.LO && i >= 2 && i < R) ? p.LO[(i0 + i - 2) * p.ldlo + i0 + i] : 0.0f;
        const int Lq = (1 << p.bits) - 1;
        const float half = 0.5f * (float)Lq;
        const float s = (i < R) ? p.scales[i0 + i] : 1.0f;
        const float rs = 1.0f / s;
        float d_last = 0.0f;   // D of this row's previous entry (read by the lane below)
        float dp1_last = 0.0f; // D[i-1][j] of the previous step (read by the lane below)
        float g_last = 0.0f, g_last2 = 0.0f;  // g of this row's previous two entries
        __syncthreads();
        // inputs of the next entry, read one step ahead: bulk sums and static data
        float n_pb = sm.pnb[0][i], n_rb = sm.rnb[0][i];
        float n_pin = 0.f, n_base = 0.f, n_w = 0.f, n_l1 = 0.f, n_l2 = 0.f;
        if (i == 0) {
            n_pin = sm.pt[0][0];
            n_base = sm.bt[0][0];
            n_w = sm.wst[0][0];
        }
        int slot3n = 1;  // (st + 1) mod 3
        for (int st = 0; st < 2 * kB - 1; ++st) {
            const int j = st - i;
            const float dprev1 = lane_above(d_last);    // D[i-1][j]
            const float dprev2 = lane_above(dp1_last);  // D[i-2][j]
            const float pb = n_pb, rb = n_rb;
            const float x_pin = n_pin, x_base = n_base, x_w = n_w, x_l1 = n_l1, x_l2 = n_l2;
            if (j >= 0 && j < Cc && i < R) {
                float u = 0.5f;
                if (p.stochastic)
                    u = uniform24(p.seed, (uint64_t)(i0 + i) * (uint64_t)p.n + (uint64_t)(j0 + j));
                const float P = x_pin + ((pb + lo2 * dprev2) + lo1 * dprev1);
                const float Rr = (rb + g_last2 * x_l2) + g_last * x_l1;
                const float tv = x_base + P + Rr;
                const float y = fmaf(tv, rs, half);
                float cf = floorf(y + u);
                nclamp += (cf < 0.0f || cf > (float)Lq) ? 1 : 0;
                cf = fminf(fmaxf(cf, 0.0f), (float)Lq);
                const float dl = fmaf(-s, cf - half, x_w);  // D = W* - s (c - Lq/2)
                const float g = P + dl;
                sm.DT[j][i] = dl;
                sm.Gs[i][j] = g;
                sm.code[i][j] = (uint8_t)cf;
                sm.wst[i][j] = fmaf(-s, cf - half, tv);  // eta
                d_last = dl;
                g_last2 = g_last;
                g_last = g;
            }
            dp1_last = dprev1;
            // inputs of the next entry (the bulk sums written in the previous step, static
            // data, this lane's own W* slot), read after the stores and left in flight
            // across the barrier; nothing writes them in the next step
            lds_wait_all();
            __builtin_amdgcn_sched_barrier(0);
            const int jn = min(max(j + 1, 0), kB - 1);
            n_pb = sm.pnb[slot3n][i];
            n_rb = sm.rnb[slot3n][i];
            n_pin = sm.pt[jn][i];
            n_base = sm.bt[jn][i];
            n_w = sm.wst[i][jn];
            n_l1 = sm.li1[jn];
            n_l2 = sm.li2[jn];
            slot3n = slot3n == 2 ? 0 : slot3n + 1;
            __builtin_amdgcn_sched_barrier(0);
            barrier_no_wait();
        }
    } else {
        // ---------------- hand-over waves (column-wise, row-wise) ----------------
        int seen = 0;  // neighbour's counter, read three steps before it is looked at
        __syncthreads();
#pragma nounroll
        for (int st = 0; st < kSweep; ++st) {
            // the lane index, opaque per step, so that the address arithmetic of the
            // loads and stores below is not hoisted out of the sweep and held across it
            int ln = lane;
            asm volatile("" : "+v"(ln));
            // the neighbour's strip c >= 1: window st = 16c - 12 .. 16c - 2
            const int cw = (st + 12) >> 4, ph = (st + 12) & 15;
            if (hown && cw >= 1 && cw < kStrips) {
                if (ph == 0) {
                    seen = ld_flag(hflag);
                } else if (ph == 2) {
                    if (seen < cw + 1) wait_flag(p, hflag, cw + 1);
                    compiler_fence();
                    handover_load(p, hcol, cw, i0, j0, R, Cc, h, ln);
                } else if (ph == 5) {
                    handover_mma<0, 3>(hcol, h);
                } else if (ph == 6) {
                    handover_mma<3, 6>(hcol, h);
                } else if (ph == 7) {
                    handover_mma<6, 9>(hcol, h);
                } else if (ph == 8) {
                    handover_mma<9, 12>(hcol, h);
                } else if (ph == 9) {
                    handover_mma<12, 16>(hcol, h);
                } else if (ph == 10) {
                    handover_add(sm, hcol, cw, h, ln);
                }
            }
            // this leaf's strip c <= 2: stored at st = 79 + 16c, counter raised 3 steps later
            if (st >= kB + kStrip - 1) {
                const int cp = (st - (kB + kStrip - 1)) >> 4, pp = (st - (kB + kStrip - 1)) & 15;
                if (cp < kStrips - 1) {
                    if (pp == 0) handover_publish(p, sm, hcol, cp, i0, j0, R, Cc, ln);
                    else if (pp == 3) handover_flag(p, hcol, leaf, cp + 1, ln);
                }
            }
            lds_wait_all();
            barrier_no_wait();
        }
    }
    // the last strips
    if (hwave) {
        handover_publish(p, sm, hcol, kStrips - 1, i0, j0, R, Cc, lane);
        handover_flag(p, hcol, leaf, kStrips, lane);
    }
    // loss partial: sum of D_O,i D_I,j eta_ij^2 over the leaf, in fp64
    if (p.want_loss) {
        for (int e = t; e < kB * kB; e += kLeafThreads) {
            const int i = e / kB, j = e % kB;
            if (i < R && j < Cc) {
                const float dO = p.DO ? p.DO[i0 + i] : 1.0f;
                const double eta = (double)sm.wst[i][j];
                loss += (double)(dO * sm.DI[j]) * eta * eta;
            }
        }
    }
    // ---- codes, along the leaf's rows (four per store where aligned); D and C^T
    // went out with the hand-overs
    {
        const bool ovec = (reinterpret_cast<uintptr_t>(p.codes) & 3) == 0 && (p.ldc & 3) == 0;
        for (int g = t; g < kB * kB / 4; g += kLeafThreads) {
            const int r = g >> 4, c4 = (g & 15) << 2;
            if (r >= R) continue;
            const uint32_t cv = *reinterpret_cast<const uint32_t*>(&sm.code[r][c4]);
            uint8_t* cp = p.codes + (i0 + r) * p.ldc + j0 + c4;
            if (ovec && c4 + 3 < Cc) {
                *reinterpret_cast<uint32_t*>(cp) = cv;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c4 + e < Cc) cp[e] = (uint8_t)(cv >> (8 * e));
            }
        }
    }
    // the leaf's loss and clamp count: within each wave by shuffles, then over the waves
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        loss += __shfl_xor(loss, o);
        nclamp += __shfl_xor(nclamp, o);
    }
    if ((t & 63) == 0) {
        sm.red[w] = loss;
        sm.red_i[w] = nclamp;
    }
    __syncthreads();
    if (t == 0) {
        double lsum = 0.0;
        int csum = 0;
#pragma unroll
        for (int k = 0; k < kLeafWaves; ++k) {
            lsum += sm.red[k];
            csum += sm.red_i[k];
        }
        p.leaf_loss[leaf] = lsum;
        p.leaf_clamp[leaf] = csum;
    }
}

// The whole solve: each workgroup takes the next task until none is left.
// Group k of the task order holds the leaves of diagonal k, then the far
// fields of diagonal k + 1.
union SolveSmem {
    LeafSmem leaf;
    FarSmem far;
};

__global__ __launch_bounds__(kLeafThreads, 1) void k_solve_run(SolveParams p) {
    __shared__ SolveSmem sm;
    __shared__ int s_task;
    if (*p.info != INT_MAX) return;  // a row scale was invalid
    for (;;) {
        // the thread index, opaque to the compiler once per task, so that index
        // arithmetic is not hoisted out of the loop and held across it
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        if (tid == 0) s_task = atomicAdd(p.ticket, 1);
        __syncthreads();
        const int tk = __builtin_amdgcn_readfirstlane(s_task);  // uniform: keeps the task's indices scalar
        if (tk >= p.ntask) break;
        int lo = 0, hi = p.ND - 1;  // the last group starting at or before tk
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.seg[mid] <= tk) lo = mid;
            else hi = mid - 1;
        }
        const int r = tk - p.seg[lo];
        const int nl = diag_leaves(p.M, p.N, lo);
        if (r < nl) leaf_task(p, lo, r, sm.leaf, tid);
        else far_task(p, lo + 1, r - nl, sm.far, tid);
        __syncthreads();  // the next task reuses the shared memory
    }
}

// loss = sum of leaf partials in a fixed order; clamped count; info.
__global__ __launch_bounds__(kThreads) void k_solve_finish(const double* leaf_loss,
                                                           const int* leaf_clamp, int64_t nleaves,
                                                           double* loss, int64_t* clamped,
                                                           const int* info_ws, const int* abort,
                                                           int32_t* info) {
    __shared__ double rl[kThreads];
    __shared__ long long rc[kThreads];
    double s = 0.0;
    long long c = 0;
    for (int64_t e = threadIdx.x; e < nleaves; e += kThreads) {
        s += leaf_loss[e];
        c += leaf_clamp[e];
    }
    rl[threadIdx.x] = s;
    rc[threadIdx.x] = c;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) {
            rl[threadIdx.x] += rl[threadIdx.x + o];
            rc[threadIdx.x] += rc[threadIdx.x + o];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (loss) *loss = rl[0];
        if (clamped) *clamped = (int64_t)rc[0];
        if (info) *info = (*info_ws != INT_MAX) ? *info_ws : (*abort ? -1 : 0);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {
struct Layout {
    int M, N, maxleaf, ND;
    size_t ct, delta, parts, leaf_loss, leaf_clamp, info, sched, flags, seg, nchd, total;
};

Layout layout(int64_t m, int64_t n) {
    Layout L;
    L.M = (int)((m + kB - 1) / kB);
    L.N = (int)((n + kB - 1) / kB);
    L.maxleaf = std::min(L.M, L.N);
    L.ND = L.M + L.N - 1;
    const size_t nl = (size_t)L.M * L.N;
    size_t o = 0;
    L.ct = o;
    o += align256(sizeof(float) * (size_t)m * (size_t)n);
    L.delta = o;
    o += align256(sizeof(float) * (size_t)m * (size_t)n);
    L.parts = o;  // kRing diagonals in flight
    o += align256(sizeof(float) * kRing * (size_t)L.maxleaf * 2 * kNch * kB * kB);
    L.leaf_loss = o;
    o += align256(sizeof(double) * nl);
    L.leaf_clamp = o;
    o += align256(sizeof(int) * nl);
    L.info = o;
    o += 256;
    L.sched = o;  // ticket, abort
    o += 256;
    L.flags = o;  // prog_d, prog_c, setup, fardone
    o += align256(sizeof(int) * 4 * nl);
    L.seg = o;
    o += align256(sizeof(int) * ((size_t)L.ND + 1));
    L.nchd = o;
    o += align256(sizeof(int) * (size_t)L.ND);
    L.total = o;
    return L;
}

struct DeviceInfo {
    int cus = 0;
    int clock_khz = 0;  // wall clock of s_memrealtime
};

DeviceInfo device_info() {
    static DeviceInfo cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    DeviceInfo& di = cache[dev];
    if (di.cus == 0) {
        int cus = 0, khz = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
            khz = 100000;
        di.clock_khz = khz;
        di.cus = cus;
    }
    return di;
}
}  // namespace

size_t solve_workspace_bytes(int64_t m, int64_t n) { return layout(m, n).total; }

int run_solve(const SolveArgs& a, void* ws, hipStream_t stream) {
    const Layout L = layout(a.m, a.n);
    int64_t ntask = 0;
    for (int k = 0; k < L.ND; ++k) ntask += group_tasks(L.M, L.N, L.ND, k);
    if (ntask >= INT_MAX / 2) return BAKRON_E_INVALID_ARG;
    const DeviceInfo di = device_info();
    char* base = (char*)ws;
    SolveParams p;
    p.W = a.W;
    p.ldw = a.ldw;
    p.LO = a.LO;
    p.ldlo = a.ldlo;
    p.LI = a.LI;
    p.ldli = a.ldli;
    p.m = a.m;
    p.n = a.n;
    p.M = L.M;
    p.N = L.N;
    p.bits = a.bits;
    p.stochastic = a.stochastic;
    p.seed = a.seed;
    p.scales = a.scales;
    p.codes = a.codes;
    p.ldc = a.ldc;
    p.delta = a.delta ? a.delta : (float*)(base + L.delta);
    p.ldd = a.delta ? a.ldd : a.n;
    p.ct = (float*)(base + L.ct);
    p.parts = (float*)(base + L.parts);
    p.leaf_loss = (double*)(base + L.leaf_loss);
    p.leaf_clamp = (int*)(base + L.leaf_clamp);
    p.DO = a.DO;
    p.DI = a.DI;
    p.want_loss = a.loss != nullptr;
    p.info = (int*)(base + L.info);
    p.maxleaf = L.maxleaf;
    const size_t nl = (size_t)L.M * L.N;
    p.ticket = (int*)(base + L.sched);
    p.abort = p.ticket + 1;
    p.prog_d = (int*)(base + L.flags);
    p.prog_c = p.prog_d + nl;
    p.setup = p.prog_c + nl;
    p.fardone = p.setup + nl;
    p.seg = (int*)(base + L.seg);
    p.nchd = (int*)(base + L.nchd);
    p.ND = L.ND;
    p.ntask = (int)ntask;
    // 10 s, or BAKRON_SOLVE_WAIT_LIMIT_US (a test hook that makes the waits expire)
    uint64_t limit_us = 10ull * 1000 * 1000;
    if (const char* e = std::getenv("BAKRON_SOLVE_WAIT_LIMIT_US")) {
        const long long v = std::atoll(e);
        if (v > 0) limit_us = (uint64_t)v;
    }
    p.spin_limit = (uint64_t)di.clock_khz * limit_us / 1000ull;

    const int init_blocks = (int)std::min<size_t>(1024, std::max<size_t>(1, (nl + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(k_solve_init, dim3((unsigned)init_blocks), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(k_scales, dim3((unsigned)a.m), dim3(kThreads), 0, stream, a.W, a.n, a.ldw,
                       a.bits, a.row_scale, a.scales, p.info);
    const int grid = (int)std::min<int64_t>(di.cus, ntask);
    hipLaunchKernelGGL(k_solve_run, dim3((unsigned)grid), dim3(kLeafThreads), 0, stream, p);
    hipLaunchKernelGGL(k_solve_finish, dim3(1), dim3(kThreads), 0, stream, p.leaf_loss,
                       p.leaf_clamp, (int64_t)nl, a.loss, a.clamped, p.info, p.abort, a.info);
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

}  // namespace bk
