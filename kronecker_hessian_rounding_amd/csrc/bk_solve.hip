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
//  * four or more blocks back: MFMA GEMMs over K (fp16 piece products), split
//    into partials, run by other workgroups once those leaves are done, two
//    leaves that share a factor panel at a time (O(mn(m+n)) flops in all, the
//    bound of the BaKron Abstract);
//  * two and three blocks back: multiplied by the leaf's own workgroup before
//    its sweep (fp32 MFMA);
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
constexpr int kNch = 4;          // far-field partials per leaf and kind: up to three K-chunks and a fringe
constexpr int kFringe = kNch - 1;  // the partial slot of the fringe (see far_tasks)
constexpr int kRing = 6;         // diagonals whose far-field partials are held at once
constexpr int kTargetWg = 512;   // far-field tasks aimed for per diagonal
constexpr int kFarMin = 3;       // first diagonal with far-field tasks (blocks four or more back)
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
    int* pdone;      // per leaf: 1 once its D and C pieces, and those of the leaves above and to its left, are written
    int* seg;        // first task of each group k (ND + 1 entries)
    int* nchd;       // K-chunks of the far-field products, per diagonal
    int ND;          // leaf-diagonals
    int ntask;
    uint64_t spin_limit;  // wall-clock ticks a single wait may take
    // far-field operands as fp16 piece planes (see the far-field section)
    int64_t Mp, Np;  // rows, columns padded to whole quads (an even number of leaves)
    int64_t Mc;      // columns of the C plane: a leaf of padding, the rows, whole quads
    const f16x8* lop;  // L_O: [2][Mp / 8][Mp]
    const f16x8* lip;  // L_I: [2][Np / 8][Np]
    f16x8* dpl;        // D:   [2][Mp / 8][Np]
    f16x8* cpl;        // C:   [2][Np / 8][Mc], row i at column i + 64
    const int* exd;    // eD per row of W (Mp)
    const int* exc;    // eC per row of W (Mp)
    const int* fexo;   // fO per column of L_O (Mp)
    const int* fexi;   // fI per column of L_I (Np)
};

__host__ __device__ __forceinline__ int diag_lo(int N, int d) { return d - (N - 1) > 0 ? d - (N - 1) : 0; }
__host__ __device__ __forceinline__ int diag_hi(int M, int d) { return d < M - 1 ? d : M - 1; }
__host__ __device__ __forceinline__ int diag_leaves(int M, int N, int d) {
    return diag_hi(M, d) - diag_lo(N, d) + 1;
}
// even indices in [lo, hi]
__host__ __device__ __forceinline__ int count_even(int lo, int hi) { return (hi >> 1) - ((lo + 1) >> 1) + 1; }
// K-chunks per far-field product on diagonal d: about kTargetWg tasks (one pair task
// per leaf on average), chunks of at least 4 blocks
__host__ __device__ __forceinline__ int diag_nch(int M, int N, int d) {
    const int lo = diag_lo(N, d), hi = diag_hi(M, d), nl = hi - lo + 1;
    const int kmax = (hi > d - lo ? hi : d - lo) - 3;  // blocks four or more back
    int nch = (kTargetWg + nl - 1) / nl;
    const int cap = kmax / 4 > 1 ? kmax / 4 : 1;
    nch = nch < cap ? nch : cap;
    nch = nch < kFringe ? nch : kFringe;
    return nch > 1 ? nch : 1;
}
// The far fields come in quads: the 2 x 2 leaves (I, J), (I, J + 1), (I + 1, J),
// (I + 1, J + 1) share two factor panels in each direction (the column far fields p:
// L_O panels I, I + 1 and D panels J, J + 1; the row far fields o: L_I panels J, J + 1
// and C panels I, I + 1), so one 128 x 128 tile gives all four. A quad covers the
// blocks four or more above (p) or left of (o) its first row (column): the second
// row's (column's) leaves take one more block during set-up. A quad is computed with
// its first leaf's diagonal d; its other leaves lie on d + 1 and d + 2. Column quads
// start at even I and J (even d), row quads at odd I (from -1: the first has row 0
// only) and even J (odd d), so every diagonal has quads of one kind.
__host__ __device__ __forceinline__ int quad_lo(int N, int d) {  // first row of a quad origin on d
    int lo = d - (N - 1) > -1 ? d - (N - 1) : -1;
    if ((d & 1) == 0) lo = lo < 0 ? 0 : lo;
    const int par = d & 1;  // origins have I of the parity of d (J is even)
    return ((lo & 1) == par) ? lo : lo + 1;
}
__host__ __device__ __forceinline__ int quad_count(int M, int N, int d) {
    const int lo = quad_lo(N, d), hi = d < M - 1 ? d : M - 1;
    return hi < lo ? 0 : (hi - lo) / 2 + 1;
}
__host__ __device__ __forceinline__ int far_tasks(int M, int N, int d, int nch) {
    return quad_count(M, N, d) * nch;
}
// The second row (column) of a quad needs one block more than the quad covers: its
// fringe, a 64 x 128 tile over that one block (K = 64) for the second row's two
// leaves, is one task per quad, run after the leaves of the quad's own diagonal; it
// writes partial slot kFringe. So every leaf multiplies the same two blocks during
// set-up.
__host__ __device__ __forceinline__ int fringe_tasks(int M, int N, int d) {
    return d >= kFarMin ? quad_count(M, N, d) : 0;
}
// tasks of group k: the leaves of diagonal k, then the far-field quads of diagonal
// k + 1 (those exist from diagonal kFarMin on), then the fringes of diagonal k. A quad
// task reads leaves three or more groups back and a fringe two, so they rarely wait;
// the leaves that take them come after them in the order.
__host__ __device__ __forceinline__ int group_far(int ND, int k) {
    return (k + 1 >= kFarMin && k + 1 < ND) ? k + 1 : -1;
}
__host__ __device__ __forceinline__ int group_tasks(int M, int N, int ND, int k) {
    int s = diag_leaves(M, N, k);
    const int df = group_far(ND, k);
    if (df >= 0) s += far_tasks(M, N, df, diag_nch(M, N, df));
    return s + fringe_tasks(M, N, k);
}

__device__ __forceinline__ int leaf_lo(const SolveParams& p, int d) { return diag_lo(p.N, d); }

// far-field partials: ring slot of the diagonal, leaf slot on it, kind (0: p, 1: o^T), K-chunk
__device__ __forceinline__ float* part_ptr(const SolveParams& p, int d, int slot, int kind, int c) {
    return p.parts + ((((size_t)(d % kRing) * p.maxleaf + slot) * 2 + kind) * kNch + c) * (kB * kB);
}

// Hand-overs between workgroups use the primitives of bk_common.hpp; those
// inside a leaf's sweep read with device-coherent loads instead, so the sweep
// never waits on cache maintenance.

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
// scales: s_i = fp32(2 max_j |W*_ij|) / fp32(Lq), or the caller's scale; also the
// bound b_i = max_j |W*_ij| + s_i Lq / 2 on row i of D and its exponent eD_i
// ---------------------------------------------------------------------------
// 2^e b below 2^14 (in [2^13, 2^14)); 0 for a zero or non-finite b
__device__ __forceinline__ int bound_exp(float b) {
    if (!(b > 0.0f) || !(b < INFINITY)) return 0;
    int E;
    frexpf(b, &E);
    return min(100, max(-100, 14 - E));
}
// 2^e m in [2^14, 2^15) for the largest magnitude m; 0 for a zero or non-finite m
__device__ __forceinline__ int max_exp(float m) {
    if (!(m > 0.0f) || !(m < INFINITY)) return 0;
    int E;
    frexpf(m, &E);
    return min(100, max(-100, 15 - E));
}

__global__ __launch_bounds__(kThreads) void k_scales(const float* __restrict__ W, int64_t n,
                                                     int64_t ldw, int bits,
                                                     const float* __restrict__ row_scale,
                                                     float* __restrict__ scales, float* __restrict__ bd,
                                                     int* __restrict__ ed, int* info) {
    const int64_t i = blockIdx.x;
    __shared__ float red[kThreads];
    float a = 0.0f;
    const float* w = W + i * ldw;
    // a batch of the row's entries in flight at once
    constexpr int kIn = 16;
    for (int64_t j0 = threadIdx.x; j0 < n; j0 += (int64_t)kIn * kThreads) {
        float v[kIn];
#pragma unroll
        for (int u = 0; u < kIn; ++u) {
            const int64_t j = j0 + (int64_t)u * kThreads;
            v[u] = j < n ? fabsf(w[j]) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kIn; ++u) a = nan_max(a, v[u]);
    }
    red[threadIdx.x] = a;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] = nan_max(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    const float Lq = (float)((1 << bits) - 1);
    const float s = row_scale ? row_scale[i] : (2.0f * red[0]) / Lq;
    if (threadIdx.x == 0) {
        scales[i] = s;
        if (!(s > 0.0f) || !(s < INFINITY)) atomicMin(info, (int)min<int64_t>(i + 1, INT_MAX - 1));
        const float b = red[0] + s * (0.5f * Lq);
        bd[i] = b;
        ed[i] = bound_exp(b);
    }
}

// ---------------------------------------------------------------------------
// pre-pass: the piece planes of L_O and L_I, and the exponents of the planes of C
// ---------------------------------------------------------------------------
constexpr int kPrepRows = 256;  // rows of a factor per pre-pass workgroup

// Column statistics of the strictly upper factor L (d x d) over rows 256 y .. 256 y + 255,
// for the 64 columns of block x:
//   mx[y][c] = max |L[k][c]| 2^-re_k over the far-field rows k < 64 (x - 3)   (re: none = 0)
//   sb[y][c] = sum |L[k][c]| rb_k over k < c                               (when rb is given)
__global__ __launch_bounds__(kThreads) void k_lstats(const float* __restrict__ L, int64_t ld, int64_t d,
                                                     const int* __restrict__ re, const float* __restrict__ rb,
                                                     int64_t dp, float* __restrict__ mx, float* __restrict__ sb) {
    __shared__ float rm[4][kB], rs[4][kB];
    const int t = threadIdx.x, c = t & 63, rq = t >> 6;
    const int64_t x = blockIdx.x, col = x * kB + c;
    const int64_t k0 = (int64_t)blockIdx.y * kPrepRows;
    const int64_t kf = max<int64_t>(0, (x - 3) * kB);
    const int64_t k1 = min<int64_t>(k0 + kPrepRows, min<int64_t>(d, col));
    float m = 0.0f, sum = 0.0f;
    if (col < d) {
        // rows k0 + rq, + 4, ... in that order, a batch of them (and of their
        // exponents and bounds) loaded at once
        constexpr int kIn = 16;
        for (int64_t kb = k0 + rq; kb < k1; kb += 4 * kIn) {
            float v[kIn], f[kIn];
            int e[kIn];
#pragma unroll
            for (int u = 0; u < kIn; ++u) {
                const int64_t k = kb + 4 * u;
                const bool in = k < k1;
                v[u] = in ? fabsf(L[k * ld + col]) : 0.0f;
                e[u] = (in && re && k < kf) ? re[k] : 0;
                f[u] = (in && rb) ? rb[k] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kIn; ++u) {
                const int64_t k = kb + 4 * u;
                if (k < k1) {
                    if (k < kf) m = nan_max(m, re ? ldexpf(v[u], -e[u]) : v[u]);
                    if (rb) sum += v[u] * f[u];
                }
            }
        }
    }
    rm[rq][c] = m;
    rs[rq][c] = sum;
    __syncthreads();
    if (rq == 0) {
        const size_t o = (size_t)blockIdx.y * dp + col;
        mx[o] = nan_max(nan_max(rm[0][c], rm[1][c]), nan_max(rm[2][c], rm[3][c]));
        if (sb) sb[o] = (rs[0][c] + rs[1][c]) + (rs[2][c] + rs[3][c]);
    }
}

// Per column c < dp: fex[c] from the maxima (mx given), and cex[c] = the exponent of
// the bound rb_c + sum_y sb[y][c] (cex given; rows c >= d have bound 0).
__global__ __launch_bounds__(kThreads) void k_lexp(const float* __restrict__ mx, const float* __restrict__ sb,
                                                   int nchunk, int64_t dp, int64_t d,
                                                   const float* __restrict__ rb, int* __restrict__ fex,
                                                   int* __restrict__ cex) {
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c >= dp) return;
    float m = 0.0f, sum = 0.0f;
    for (int y = 0; y < nchunk; ++y) {
        if (mx) m = nan_max(m, mx[(size_t)y * dp + c]);
        if (sb) sum += sb[(size_t)y * dp + c];
    }
    if (fex) fex[c] = max_exp(m);
    if (cex) cex[c] = c < d ? bound_exp(rb[c] + sum) : 0;
}

// The far-field rows of column block x (groups g < 8 (x - 3)) of L, 32 groups per
// workgroup (y), into the planes P[piece][g][c]: element (k, c) scaled by
// 2^(fex_c - re_k). Thread (c, q) writes the units of column c for groups q, q + 4, ..
// (a wave stores 1 KB of consecutive units per plane).
__global__ __launch_bounds__(kThreads) void k_lsplit(const float* __restrict__ L, int64_t ld, int64_t d,
                                                     const int* __restrict__ re, const int* __restrict__ fex,
                                                     int64_t dp, int64_t ng, f16x8* __restrict__ P) {
    const int t = threadIdx.x, c = t & 63, gq = t >> 6;
    const int64_t x = blockIdx.x, col = x * kB + c;
    const int64_t gf = max<int64_t>(0, 8 * (x - 3));
    const int64_t gb = (int64_t)blockIdx.y * (kPrepRows / 8);
    const int64_t ge = min<int64_t>(gb + kPrepRows / 8, gf);
    const int fc = fex[col];
    for (int64_t g = gb + gq; g < ge; g += 4) {
        uint32_t pk[2][4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int64_t k = 8 * g + e;  // < 64 (x - 3) <= d - 64
            const float v0 = col < d ? L[k * ld + col] : 0.0f;
            const float v1 = col < d ? L[(k + 1) * ld + col] : 0.0f;
            uint32_t h0, l0, h1, l1;
            split2_value(v0, fc - (re ? re[k] : 0), h0, l0);
            split2_value(v1, fc - (re ? re[k + 1] : 0), h1, l1);
            pk[0][e >> 1] = h0 | (h1 << 16);
            pk[1][e >> 1] = l0 | (l1 << 16);
        }
#pragma unroll
        for (int pc = 0; pc < 2; ++pc)
            *reinterpret_cast<uint4*>(&P[((int64_t)pc * ng + g) * dp + col]) =
                uint4{pk[pc][0], pk[pc][1], pk[pc][2], pk[pc][3]};
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
        p.pdone[e] = 0;
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
// far field of diagonal d: chunk c (of nch) of a pair of p (kind 0) or o^T
// (kind 1) tiles, over the blocks four or more above (p) or to the left (o) of
// the pair's leaves. The products run on fp16 MFMAs over two-piece operands
// (hi = fp16(x'), lo = fp16(x' - hi) of a power-of-two-scaled x'): three piece
// products per fp32 product, accumulated in fp32. The operands are piece
// planes, P[piece][k / 8][column] with the 8 fp16 values of k = 8g .. 8g + 7 in
// one 16-byte unit, laid out so that a 16-byte unit is an MFMA operand:
//   A of p:   L_O, row k scaled by 2^-eD_k and column i by 2^fO_i (pre-pass)
//   B of p:   D,   row k scaled by 2^eD_k                  (written by leaf (k/64, j/64))
//   A of o^T: L_I, column j scaled by 2^fI_j              (pre-pass)
//   B of o^T: C,   row i scaled by 2^eC_i (contracted over its columns l)
// so that p_ij = 2^-fO_i (A^T B)_ij and o^T_ji = 2^-(fI_j + eC_i) (A^T B)_ji. eD_k
// and eC_i come from bounds known before the sweep: |D_kl| <= max_l |W*_kl| +
// s_k Lq / 2 =: b_k (the code is clamped to [0, Lq]) and |C_il| <= b_i + sum_{k<i}
// |L_O[k,i]| b_k, each scaled to below 2^14; fO and fI from the column maxima
// (scaled to [2^14, 2^15)). A task starts once the last leaves of its K range
// have written their pieces (each leaf marks its pieces written only after the
// leaves above and to its left did, so those finished earlier). Each chunk
// writes its own fp32 64x64 partial per leaf; the leaf adds them in chunk order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void chunk_range(int kblk, int nch, int c, int& b0, int& b1) {
    const int len = (kblk + nch - 1) / nch;
    b0 = min(c * len, kblk);
    b1 = min(b0 + len, kblk);
}

// Wait until at most N of this wave's vector-memory operations are outstanding, then
// meet the other waves. Direct-to-LDS loads complete in issue order, so with N = the
// loads issued after stage s, stage s is in LDS once every wave has passed; the later
// loads stay in flight across the barrier.
// N counts only the ring's own loads, so this holds only while the kernel keeps every
// value in registers: a spill would add scratch loads and stores to the count (the
// build rejects any kernel with scratch for that reason).
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One ring stage: 32 k (four 8-k groups) of both pieces of A and B, 128 columns each
// (the quad's two rows and two columns of leaves).
#ifndef BK_PIECE_NS
#define BK_PIECE_NS 4
#endif
constexpr int kPieceNS = BK_PIECE_NS;  // stages in the ring: loads run kPieceNS - 1 stages ahead
struct PieceStage {
    f16x8 a[2][4][2 * kB];
    f16x8 b[2][4][2 * kB];
};
struct PieceRing {
    PieceStage s[kPieceNS];
    int fr[2 * kB];  // exponent of each output row (A column)
    int fc[2 * kB];  // exponent of each output column (B column)
};

__device__ __forceinline__ uint32_t lds_addr(const void* q) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)q);
}

// The MFMA operands of one stage, read in one block that also waits for them. Left
// to the compiler, these reads of the ring, whose other slots direct-to-LDS loads
// are still filling, were preceded by a wait for every load in flight (vmcnt(0)),
// which undid the prefetch; the waits for the stage's own loads are the barrier's.
// a: the lane's A unit of group kh in the wave's first 32 columns; b: likewise for B.
// fa[s][pc][h]: group 2 s + kh, piece pc, columns +32 h; fb likewise.
__device__ __forceinline__ void stage_reads(uint32_t a, uint32_t b, f16x8 (&fa)[2][2][2], f16x8 (&fb)[2][2][2]) {
    // offsets: x[pc][g][c] at 8192 pc + 2048 g + 16 c, for both operands
    asm volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %1, %16 offset:512\n\t"
        "ds_read_b128 %2, %16 offset:8192\n\t"
        "ds_read_b128 %3, %16 offset:8704\n\t"
        "ds_read_b128 %4, %16 offset:4096\n\t"
        "ds_read_b128 %5, %16 offset:4608\n\t"
        "ds_read_b128 %6, %16 offset:12288\n\t"
        "ds_read_b128 %7, %16 offset:12800\n\t"
        "ds_read_b128 %8, %17\n\t"
        "ds_read_b128 %9, %17 offset:512\n\t"
        "ds_read_b128 %10, %17 offset:8192\n\t"
        "ds_read_b128 %11, %17 offset:8704\n\t"
        "ds_read_b128 %12, %17 offset:4096\n\t"
        "ds_read_b128 %13, %17 offset:4608\n\t"
        "ds_read_b128 %14, %17 offset:12288\n\t"
        "ds_read_b128 %15, %17 offset:12800\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(fa[0][0][0]), "=&v"(fa[0][0][1]), "=&v"(fa[0][1][0]), "=&v"(fa[0][1][1]), "=&v"(fa[1][0][0]),
          "=&v"(fa[1][0][1]), "=&v"(fa[1][1][0]), "=&v"(fa[1][1][1]), "=&v"(fb[0][0][0]), "=&v"(fb[0][0][1]),
          "=&v"(fb[0][1][0]), "=&v"(fb[0][1][1]), "=&v"(fb[1][0][0]), "=&v"(fb[1][0][1]), "=&v"(fb[1][1][0]),
          "=&v"(fb[1][1][1])
        : "v"(a), "v"(b)
        : "memory");
}

// acc[h][t] += A^T B over groups [g0, g1) (whole stages) for a 128 x 128 tile: A columns
// ca .. ca + 127 of plane A (ngA groups, ncA columns), B columns cb .. cb + 127 of plane
// B. Waves 0-3 load and compute: wave w owns output rows 64 (w >> 1) .. (the quad's
// row of leaves w >> 1) and columns 64 (w & 1) .. (its column w & 1), as 2 x 2 blocks
// of 32 x 32 (h: rows +32 h, t: columns +32 t); the others only join the barriers.
// Every thread of the workgroup calls it.
__device__ __forceinline__ void far_quad(const f16x8* __restrict__ A, int64_t ngA, int64_t ncA, int64_t ca,
                                         const f16x8* __restrict__ B, int64_t ngB, int64_t ncB, int64_t cb,
                                         int64_t g0, int64_t g1, f32x16 (&acc)[2][2], PieceRing& sm, int tid) {
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool active = w < 4;
    const int kh = lane >> 5, l31 = lane & 31;
    const int ar = (w >> 1) * kB + l31;
    const int bc = (w & 1) * kB + l31;
    constexpr int kLoads = 8;  // direct loads per active wave per stage: 16 rows of 2 KB per operand
    const int64_t ns = (g1 - g0) / 4;
    auto issue = [&](int64_t s) {
        PieceStage& st = sm.s[s % kPieceNS];
        const int64_t gs = g0 + 4 * s;
#pragma unroll
        for (int h = 0; h < kLoads; ++h) {
            const int q = w + 4 * h;  // 0..31: operand q >> 4, piece, group, half row
            const int o = q & 15;
            const int pc = o >> 3, gl = (o >> 1) & 3, hf = o & 1;
            if (q < 16)
                __builtin_amdgcn_global_load_lds(A + (pc * ngA + gs + gl) * ncA + ca + kB * hf + lane,
                                                 &st.a[pc][gl][kB * hf], 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds(B + (pc * ngB + gs + gl) * ncB + cb + kB * hf + lane,
                                                 &st.b[pc][gl][kB * hf], 16, 0, 0);
        }
    };
    if (active)
        for (int s = 0; s < kPieceNS - 1; ++s)
            if (s < ns) issue(s);
    // the three piece products (lo hi', hi lo', hi hi'), smallest first
    constexpr int kPa[3] = {1, 0, 0};
    constexpr int kPb[3] = {0, 1, 0};
    for (int64_t it = 0; it < ns; ++it) {
        if (it + kPieceNS - 2 < ns) vm_wait_barrier<(kPieceNS - 2) * kLoads>();
        else vm_wait_barrier<0>();
        if (!active) continue;
        if (it + kPieceNS - 1 < ns) issue(it + kPieceNS - 1);
        const PieceStage& st = sm.s[it % kPieceNS];
        f16x8 fa[2][2][2], fb[2][2][2];  // [16-k step][piece][32-column half]
        stage_reads(lds_addr(&st.a[0][kh][ar]), lds_addr(&st.b[0][kh][bc]), fa, fb);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)  // two 16-k steps
#pragma unroll
            for (int u = 0; u < 3; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        acc[h][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[s2][kPa[u]][h], fb[s2][kPb[u]][t],
                                                                           acc[h][t], 0, 0, 0);
    }
}

union FarSmem {
    PieceRing pc;
};

// waits until the leaf that last used ring slot `slot` of diagonal dt (kRing diagonals
// back) has taken its partials
__device__ __forceinline__ void wait_ring(const SolveParams& p, int dt, int slot) {
    if (dt < kRing) return;
    const int dp = dt - kRing;
    if (slot < diag_leaves(p.M, p.N, dp)) {
        const int Ip = leaf_lo(p, dp) + slot;
        wait_flag(p, &p.setup[(int64_t)Ip * p.N + (dp - Ip)], 1);
    }
}

// Task `task` of diagonal d: a quad (chunk c of its K range) or, with fringe, the fringe
// of quad `task` (the one block after the quad's K range, for the second row or column).
__device__ __forceinline__ void far_task(const SolveParams& p, int d, int task, bool fringe, FarSmem& sm,
                                         int tid) {
    const int nch = p.nchd[d];
    const int c = fringe ? kFringe : task % nch, kind = d & 1;
    const int I = quad_lo(p.N, d) + 2 * (fringe ? task : task / nch);  // the quad's first leaf (I may be -1)
    const int J = d - I;
    const int kfirst = (kind == 0 ? I : J) - 3;  // the quad: blocks 0 .. kfirst - 1; the fringe: block kfirst
    const bool fac = kind == 0 ? p.LO != nullptr : p.LI != nullptr;
    int kb0 = 0, kb1 = 0;
    if (fringe) {
        kb0 = kfirst;
        kb1 = kfirst + 1;
    } else if (kfirst > 0) {
        chunk_range(kfirst, nch, c, kb0, kb1);
    }
    // a quad's empty chunk still writes its (zero) partial: the leaf adds every chunk
    const bool has = fac && (fringe ? kfirst >= 0 : kfirst > 0);
    // target (h, t): the leaf of A half h and B half t; a fringe has only h = 1
    auto tgt_i = [&](int h, int t) { return kind == 0 ? I + h : I + t; };
    auto tgt_j = [&](int h, int t) { return kind == 0 ? J + t : J + h; };
    auto exists = [&](int h, int t) {
        return (!fringe || h == 1) && tgt_i(h, t) >= 0 && tgt_i(h, t) < p.M && tgt_j(h, t) < p.N;
    };
    if (has) {
        const int64_t i0 = (int64_t)I * kB, j0 = (int64_t)J * kB;
        if (tid == 0) {
            // the last leaf of the K range next to the quad's farthest column (row): its
            // pieces, and so those of every leaf above and to the left of it
            if (kb1 > kb0) {
                if (kind == 0) wait_flag(p, &p.pdone[(int64_t)(kb1 - 1) * p.N + min(J + 1, p.N - 1)], 1);
                else wait_flag(p, &p.pdone[(int64_t)min(I + 1, p.M - 1) * p.N + kb1 - 1], 1);
            }
            // the leaves that last used these ring slots have read them
            for (int h = 0; h < 2; ++h)
                for (int t = 0; t < 2; ++t)
                    if (exists(h, t)) {
                        const int it = tgt_i(h, t), dt = it + tgt_j(h, t);
                        wait_ring(p, dt, it - leaf_lo(p, dt));
                    }
            acquire_agent();
            vm_wait_all();
        }
        // output exponents: rows (A columns) and, for o^T, columns (rows of C)
        const int64_t ca = kind == 0 ? i0 : j0, cb = kind == 0 ? j0 : i0;
        if (tid < 2 * kB) {
            sm.pc.fr[tid] = (kind == 0 ? p.fexo : p.fexi)[ca + tid];
        } else if (tid < 4 * kB) {
            const int64_t r = cb + tid - 2 * kB;
            sm.pc.fc[tid - 2 * kB] = (kind == 0 || r < 0 || r >= p.Mp) ? 0 : p.exc[r];
        }
        __syncthreads();
        f32x16 acc[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[h][t][v] = 0.0f;
        const f16x8* A = kind == 0 ? p.lop : p.lip;
        const f16x8* Bp = kind == 0 ? p.dpl : p.cpl;
        const int64_t ngA = (kind == 0 ? p.Mp : p.Np) / 8, ncA = kind == 0 ? p.Mp : p.Np;
        const int64_t ngB = ngA, ncB = kind == 0 ? p.Np : p.Mc;
        // the C plane's columns start one leaf early (row -64 .. -1: the first row quad)
        far_quad(A, ngA, ncA, ca, Bp, ngB, ncB, kind == 0 ? cb : cb + kB, 8 * kb0, 8 * kb1, acc, sm.pc, tid);
        if (tid < kThreads) {
            const int w = tid >> 6, lane = tid & 63;
            const int h = w >> 1, t = w & 1;
            if (exists(h, t)) {
                const int it = tgt_i(h, t), dt = it + tgt_j(h, t);
                float* part = part_ptr(p, dt, it - leaf_lo(p, dt), kind, c);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        const int col = 32 * tt + (lane & 31);
                        const int ec = sm.pc.fc[kB * t + col];
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int row = 32 * hh + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                            st_coherent(&part[row * kB + col], ldexpf(acc[hh][tt][v], -(sm.pc.fr[kB * h + row] + ec)));
                        }
                    }
            }
        }
        vm_wait_all();  // every wave's device-coherent partial stores have completed
        __syncthreads();
    }
    if (tid == 0) {
        for (int h = 0; h < 2; ++h)
            for (int t = 0; t < 2; ++t)
                if (exists(h, t))
                    __hip_atomic_fetch_add(&p.fardone[(int64_t)tgt_i(h, t) * p.N + tgt_j(h, t)], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// leaf solve: the 64x64 leaf (I, J) of diagonal d.
//
// Entry (i, j) is finalised at step i + j. Its in-leaf sums
//   pn = sum_{k<i} L_O[k][i] D[k][j],   rn = sum_{l<j} g[i][l] L_I[l][j]
// (g = C, the column feedback plus error of the row) are split into a bulk,
// which only uses entries finalised four or more steps earlier, and the three
// newest terms of each (k = i-1, i-2, i-3 and l = j-1, j-2, j-3). Three bulk
// waves compute the bulk of step st + 2 while the finaliser wave finalises step
// st. Every entry the bulk of step st + 2 reads was final by step st - 2, so
// its reads go out in the step before and stay in flight across the barrier:
// no step of a bulk wave starts with an LDS read. The dependent chain of the
// finaliser holds no LDS read either: it takes D[i-1][j], D[i-2][j] and
// D[i-3][j] from the lanes above by DPP, g[i][j-1], g[i][j-2] and g[i][j-3]
// from its own previous steps, and the bulk sums and static inputs were read
// one step ahead.
//
// Bulk work comes in units (a, quarter q): quarter q owns the k / l range
// [16q, 16q + 16), and unit (a, q) exists only where that range meets the
// bulk's range k, l <= a - 4 (144 units: one quarter for a = 4..19, up to four
// for a >= 52). The units are packed onto the lanes of three waves, one per
// SIMD, in order of a, so a lane with only zero factors does no work on a
// wave that has any. Unit (a, q) sums P along row a of L_O^T and R along
// column a of L_I, both held in registers, against 16-float chunks of D and g
// read as four adjacent 16-byte words (68-float rows spread a row group over
// the banks), and stores its two partials; the finaliser adds the four
// quarters of its entry.
//
// Waves 4 and 5 do the hand-overs, column-wise (4: D to the leaf below, and
// L_O[above, this]^T D[above, strip] into p) and row-wise (5: C to the leaf on
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
constexpr int kLeafWaves = 6;
constexpr int kLeafThreads = kLeafWaves * 64;
// Roles in the sweep by wave index. Waves are spread over the four SIMDs by
// index (SIMD w mod 4): the finaliser, whose chain sets the pace, has SIMD 3 to
// itself (sharing it with a bulk wave cost a fifth of the sweep's speed); bulk
// waves 0, 1 and 2 have one SIMD each, and hand-over waves 4 and 5 share SIMDs
// 0 and 1 with them (putting both hand-over waves on one SIMD measured slower).
constexpr int kFinWave = 3;
constexpr int kColWave = 4;  // hand-over of columns of D (to the leaf below)
constexpr int kRowWave = 5;  // hand-over of rows of C (to the leaf on the right)
constexpr int kNew = 5;          // newest terms of each in-leaf sum that the finaliser adds
constexpr int kBulkUnits = 136;  // (a, q) with 16 q <= a - 1 - kNew
constexpr int bulk_units() {
    int n = 0;
    for (int a = kNew + 1; a < kB; ++a) n += (a - 1 - kNew) / 16 + 1;
    return n;
}
static_assert(bulk_units() == kBulkUnits && kBulkUnits <= 3 * 64, "the bulk units fill three waves");
constexpr int kSuper = kB;       // super-steps of the sweep: two steps (anti-diagonals) each
constexpr int kTs = 68;  // row stride of the 64x64 tiles: 16-byte aligned rows, 4 banks apart
constexpr int kPs = 66;  // row stride of the per-entry inputs: anti-diagonal walks hit distinct banks

struct LeafSmem {
    float DT[kB][kTs];     // D transposed: DT[j][k] = D[k][j] (0 until known)
    float Gs[kB][kTs];     // g = C of the leaf, row-major (0 until known)
    float bt[kB][kTs];     // W* + o, transposed: bt[j][i] for entry (i, j)
    float pt[kB][kTs];     // p, transposed: pt[j][i]
    float wst[kB][kPs];    // W*, overwritten by eta = t - q once the entry is final
    float pnb[4][kB][4];   // bulk partials by diagonal modulo 4, entry and quarter
    float rnb[4][kB][4];
    float li[kNew][kB];    // li[e][j] = L_I[j-1-e][j]: the finaliser's terms
    float un[4][kB];       // stochastic rounding: the draws by diagonal modulo 4, one per row
    uint8_t code[kB][kB + 4];
    float DI[kB];
    int exr[kB];  // eD of the leaf's rows
    int exq[kB];  // eC of the leaf's rows
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

// wave_shr:1 with bound_ctrl: lane i receives lane i-1's value, lane 0 receives 0
__device__ __forceinline__ float lane_above0(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x138, 0xF, 0xF, true));
}

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
    // this leaf's far fields come from two quads, on this diagonal or up to two before:
    // the column quad whose first leaf is (I, J) rounded down to even indices, and the
    // row quad that starts at the odd row at or above I and the even column at or left
    // of J. They cover the blocks below fI - 3 (p) and fJ - 3 (o); in an odd row
    // (column) the quad's fringe adds block fI - 3 (fJ - 3). The set-up multiplies the
    // two blocks from there to two back.
    const int fI = I & ~1, fJ = J & ~1;
    const int dsrc_p = fI + fJ, dsrc_o = ((I & 1) ? I : I - 1) + fJ;
    const int nch_p = dsrc_p >= kFarMin ? p.nchd[dsrc_p] : 0;
    const int nch_o = dsrc_o >= kFarMin ? p.nchd[dsrc_o] : 0;
    // far-field tasks that report to this leaf: the chunks of its quads, and their
    // fringes in an odd row (column)
    const int nfar = nch_p + nch_o + ((I & 1) && dsrc_p >= kFarMin) + ((J & 1) && dsrc_o >= kFarMin);
    const bool far_p = p.LO && fI > 3, far_o = p.LI && fJ > 3;  // quad partials
    const bool fr_p = p.LO && (I & 1) && I >= 5, fr_o = p.LI && (J & 1) && J >= 5;  // fringe partials
    const int s0_p = max(0, I - 3), s0_o = max(0, J - 3);       // first block of the set-up
    const bool adj_p = p.LO && I > 0, adj_o = p.LI && J > 0;    // the adjacent blocks (handed over)
    for (int e = t; e < kNew * kB; e += kLeafThreads) sm.li[e / kB][e % kB] = 0.0f;  // no L_I[j-1-e][j] for j <= e
    __syncthreads();
    constexpr int kPer = (kB * kB + kLeafThreads - 1) / kLeafThreads;
    // ---- A: static inputs, every load of the thread in flight at once
    //   wst <- W*[i0+k][j0+c]       li <- the first kNew superdiagonals of L_I
    {
        float v5[kPer], v6[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            const int k = e >> 6, c = e & 63;
            const bool in = e < kB * kB;
            v5[u] = (in && k < R && c < Cc) ? p.W[(i0 + k) * p.ldw + j0 + c] : 0.0f;
            v6[u] = (in && p.LI && c - k >= 1 && c - k <= kNew && c < Cc) ? p.LI[(j0 + k) * p.ldli + j0 + c] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            if (e < kB * kB) {
                const int k = e >> 6, c = e & 63;
                sm.wst[k][c] = v5[u];
                if (c - k >= 1 && c - k <= kNew) sm.li[c - k - 1][c] = v6[u];
            }
        }
    }
    // ---- B: far fields from four or more blocks back: once their tasks are done,
    // the K-chunk partials are summed in chunk order into registers (every load
    // issued first; absent chunks read a valid address and are replaced by zero)
    if (t == 0) {
        if (nfar > 0) wait_flag(p, &p.fardone[leaf], nfar);
        acquire_agent();
        vm_wait_all();
    }
    __syncthreads();
    constexpr int kG = (kB * kB / 4 + kLeafThreads - 1) / kLeafThreads;
    const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 pvs[kG], ovs[kG];  // p and o^T, four consecutive entries per group
    {
        const bool any = far_p || far_o || fr_p || fr_o;
        // slots read: the quad chunks and the fringe's (slot kFringe); the others read
        // slot 0 (a valid address) and are replaced by zero
        auto sp = [&](int c) { return c < nch_p ? c : (c == kFringe && fr_p ? kFringe : 0); };
        auto so = [&](int c) { return c < nch_o ? c : (c == kFringe && fr_o ? kFringe : 0); };
        f32x4 xp[kG][kNch], xo[kG][kNch];
        if (any) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int g = min(t + u * kLeafThreads, kB * kB / 4 - 1);
#pragma unroll
                for (int c = 0; c < kNch; ++c) {
                    xp[u][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, d, slot, 0, sp(c)) + 4 * g);
                    xo[u][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, d, slot, 1, so(c)) + 4 * g);
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
                        xp[uu][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, d, slot, 0, sp(c)) + 4 * gg);
                        xo[uu][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, d, slot, 1, so(c)) + 4 * gg);
                    }
                }
            }
            f32x4 pv = z4, ov = z4;
            if (any) {
#pragma unroll
                for (int c = 0; c < kNch; ++c) {
                    const bool up = (far_p && c < nch_p) || (fr_p && c == kFringe);
                    const bool uo = (far_o && c < nch_o) || (fr_o && c == kFringe);
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
    // ---- the leaves two to four blocks up and to the left, down to the set-up's first
    // block: once the ones two back are done (those further back finished before them),
    // their blocks are multiplied (K = 64 each): p += L_O[back, this]^T D[back, J],
    // o^T += L_I[back, this]^T C^T[back, I]
    if (t == 0) {
        if (p.LO && I - 2 >= s0_p) wait_flag(p, &p.prog_d[leaf - 2 * (int64_t)p.N], kStrips);
        if (p.LI && J - 2 >= s0_o) wait_flag(p, &p.prog_c[leaf - 2], kStrips);
        acquire_agent();
        vm_wait_all();
    }
    __syncthreads();
    f32x16 ap, ao;
#pragma unroll
    for (int v = 0; v < 16; ++v) ap[v] = ao[v] = 0.0f;
#pragma unroll 1
    for (int back = 2; back <= 4; ++back) {
        const bool bp = p.LO && I - back >= s0_p, bo = p.LI && J - back >= s0_o;
        if (!bp && !bo) break;  // uniform: the blocks further back are in the far field
        //   DT <- L_O[i0-64b+k][i0+c]   Gs <- D[i0-64b+k][j0+c]
        //   pt <- L_I[j0-64b+k][j0+c]   bt <- C^T[j0-64b+k][i0+c]     (staging)
        float v1[kPer], v2[kPer], v3[kPer], v4[kPer];
        const int64_t ib = i0 - back * kB, jb = j0 - back * kB;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            const int k = e >> 6, c = e & 63;
            const bool in = e < kB * kB;
            v1[u] = (in && bp && c < R) ? p.LO[(ib + k) * p.ldlo + i0 + c] : 0.0f;
            v2[u] = (in && bp && c < Cc) ? p.delta[(ib + k) * p.ldd + j0 + c] : 0.0f;
            v3[u] = (in && bo && c < Cc) ? p.LI[(jb + k) * p.ldli + j0 + c] : 0.0f;
            v4[u] = (in && bo && c < R) ? p.ct[(jb + k) * p.m + i0 + c] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            if (e < kB * kB) {
                const int k = e >> 6, c = e & 63;
                sm.DT[k][c] = v1[u];
                sm.Gs[k][c] = v2[u];
                sm.pt[k][c] = v3[u];
                sm.bt[k][c] = v4[u];
            }
        }
        __syncthreads();
        if (w < 4) {
            if (bp) adj_gemm(&sm.DT[0][0], kTs, &sm.Gs[0][0], kTs, ap, t);
            if (bo) adj_gemm(&sm.pt[0][0], kTs, &sm.bt[0][0], kTs, ao, t);
        }
        __syncthreads();
    }
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
    if (t < kB) sm.DI[t] = (p.want_loss && t < Cc) ? p.DI[j0 + t] : 0.0f;
    // the partials of units that do not exist stay zero
    for (int e = t; e < 4 * kB * 4; e += kLeafThreads) {
        (&sm.pnb[0][0][0])[e] = 0.0f;
        (&sm.rnb[0][0][0])[e] = 0.0f;
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
        // Unit (a, quarter q) sums the k / l range [16q, 16q + 16) of two bulk sums of
        // the entries of diagonal d (x = d - a):
        //   P of entry (a, x): sum_k L_O[k][a] D[k][x],  k <= a - 1 - kNew (row a)
        //   R of entry (x, a): sum_l g[x][l] L_I[l][a],  l <= a - 1 - kNew (column a)
        // so both triangular factors stay in registers (row a of L_O^T, column a of
        // L_I) and a diagonal takes two 16-float chunks per lane: column x of D and
        // row x of g. Super-step S forms diagonals 2S + 2 and 2S + 3. Every entry they
        // read with a nonzero factor was final by step 2S - 3, i.e. before the barrier
        // that opened super-step S - 1, so the chunks are read at the end of
        // super-step S - 1 and stay in flight across its barrier; an entry written
        // while they are read meets a zero factor.
        // Units are packed in order of a: bulk thread bt < kBulkUnits takes unit
        // (a, q) with bt = sum_{a' < a} n(a') + q, n(a) = (a - 1 - kNew) / 16 + 1.
        const int bt = w * 64 + lane;  // bulk thread 0..191 (waves 0, 1, 2)
        int a = 0, q = 0;
        bool unit = false;
        {
            int first = 0;
#pragma unroll 1
            for (int aa = kNew + 1; aa < kB; ++aa) {
                const int nq = ((aa - 1 - kNew) >> 4) + 1;
                if (bt >= first && bt < first + nq) {
                    a = aa;
                    q = bt - first;
                    unit = true;
                }
                first += nq;
            }
        }
        const int k0 = 16 * q;
        float lo[16];  // L_O[i0 + k][i0 + a] for k <= a - 1 - kNew, else 0
        float li[16];  // L_I[j0 + l][j0 + a] for l <= a - 1 - kNew, else 0
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const bool nz = unit && k0 + e <= a - 1 - kNew;
            lo[e] = (nz && p.LO && a < R) ? p.LO[(i0 + k0 + e) * p.ldlo + i0 + a] : 0.0f;
            li[e] = (nz && p.LI && a < Cc) ? p.LI[(j0 + k0 + e) * p.ldli + j0 + a] : 0.0f;
        }
        // lanes with no live unit on a diagonal read nothing (their results are not stored)
        auto fetch = [&](int S, f32x4 (&c)[2][8]) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int x = 2 * S + 2 + e - a;
                if (unit && x >= 0 && x < kB) {
                    const float* dp = &sm.DT[x][k0];
                    const float* gp = &sm.Gs[x][k0];
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        c[e][h] = lds4(dp + 4 * h);
                        c[e][4 + h] = lds4(gp + 4 * h);
                    }
                }
            }
        };
        auto super = [&](int S, const f32x4 (&c)[2][8], f32x4 (&cn)[2][8]) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int dg = 2 * S + 2 + e;
                const int x = dg - a;
                float p0 = 0.0f, p1 = 0.0f, r0 = 0.0f, r1 = 0.0f;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    p0 = fmaf(lo[v], c[e][0][v], p0);
                    p1 = fmaf(lo[4 + v], c[e][1][v], p1);
                    r0 = fmaf(li[v], c[e][4][v], r0);
                    r1 = fmaf(li[4 + v], c[e][5][v], r1);
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    p0 = fmaf(lo[8 + v], c[e][2][v], p0);
                    p1 = fmaf(lo[12 + v], c[e][3][v], p1);
                    r0 = fmaf(li[8 + v], c[e][6][v], r0);
                    r1 = fmaf(li[12 + v], c[e][7][v], r1);
                }
                if (unit && x >= 0 && x < kB) {
                    sm.pnb[dg & 3][a][q] = p0 + p1;  // entry (a, x)
                    sm.rnb[dg & 3][x][q] = r0 + r1;  // entry (x, a)
                }
            }
            lds_wait_all();
            __builtin_amdgcn_sched_barrier(0);
            fetch(S + 1, cn);  // the next super-step's chunks, in flight across the barrier
            __builtin_amdgcn_sched_barrier(0);
            barrier_no_wait();
        };
        f32x4 ca[2][8], cb[2][8];
        __syncthreads();
        fetch(0, ca);  // diagonals 2 and 3: nothing final is needed yet (a nonzero factor needs a >= 6)
#pragma nounroll
        for (int S = 0; S < kSuper; S += 2) {
            super(S, ca, cb);
            super(S + 1, cb, ca);
        }
    } else if (w == kFinWave) {
        // ---------------- finaliser wave: lane i owns row i ----------------
        // Super-step S finalises steps 2S and 2S + 1 with no barrier between them.
        // Each entry adds the bulk's four quarters and the kNew newest terms of each
        // sum: D[i-1][j] .. D[i-kNew][j] (from the lanes above, by DPP: the lane
        // above's value of the previous step, passed down one lane per step) and
        // g[i][j-1] .. g[i][j-kNew] (its own previous results); eta = t - q goes into
        // W*'s slot (consumed by then) for the loss. The arithmetic runs on every
        // lane; only the stores and the carried values depend on whether the entry
        // exists.
        const int i = t & 63;
        float lon[kNew];  // L_O[i-1-e][i]
#pragma unroll
        for (int e = 0; e < kNew; ++e)
            lon[e] = (p.LO && i >= e + 1 && i < R) ? p.LO[(i0 + i - 1 - e) * p.ldlo + i0 + i] : 0.0f;
        const int Lq = (1 << p.bits) - 1;
        const float half = 0.5f * (float)Lq;
        const float fLq = (float)Lq;
        const float s = (i < R) ? p.scales[i0 + i] : 1.0f;
        const float rs = 1.0f / s;
        const bool row = i < R;
        float dcar[kNew];  // dcar[e]: D[i-e][j-1] of the previous step (e = 0: this row's own)
        float gcar[kNew];  // gcar[e]: g[i][j-1-e]
#pragma unroll
        for (int e = 0; e < kNew; ++e) dcar[e] = gcar[e] = 0.0f;
        // the per-entry inputs of a step: the far-field offsets (pt, bt), W* and the
        // kNew superdiagonals of L_I at column j
        struct In {
            float pin, base, w, l[kNew];
        };
        auto load_in = [&](int st, In& v) {
            const int jc = min(max(st - i, 0), kB - 1);
            v.pin = sm.pt[jc][i];
            v.base = sm.bt[jc][i];
            v.w = sm.wst[i][jc];
#pragma unroll
            for (int e = 0; e < kNew; ++e) v.l[e] = sm.li[e][jc];
        };
        auto entry = [&](int st, const In& v, const f32x4& pq, const f32x4& rq, float ud) {
            const int j = st - i;
            const bool live = row && j >= 0 && j < Cc;
            float dn[kNew];  // D[i-1-e][j], from the lane above's carried values
#pragma unroll
            for (int e = 0; e < kNew; ++e) dn[e] = lane_above0(dcar[e]);
            const float u = p.stochastic ? ud : 0.5f;
            float pb = (pq[0] + pq[1]) + (pq[2] + pq[3]);
            float rb = (rq[0] + rq[1]) + (rq[2] + rq[3]);
#pragma unroll
            for (int e = kNew - 1; e >= 0; --e) {
                pb = fmaf(lon[e], dn[e], pb);
                rb = fmaf(gcar[e], v.l[e], rb);
            }
            const float P = v.pin + pb;
            const float tv = v.base + P + rb;
            const float y = fmaf(tv, rs, half);
            const float cu = floorf(y + u);
            const float cf = fminf(fmaxf(cu, 0.0f), fLq);
            const float dl = fmaf(-s, cf - half, v.w);  // D = W* - s (c - Lq/2)
            const float g = P + dl;
            if (live) {
                nclamp += (cu < 0.0f || cu > fLq) ? 1 : 0;
                sm.DT[j][i] = dl;
                sm.Gs[i][j] = g;
                sm.code[i][j] = (uint8_t)cf;
                sm.wst[i][j] = fmaf(-s, cf - half, tv);  // eta
            }
            // carried values: a row's own D and g only where the entry exists
#pragma unroll
            for (int e = kNew - 1; e >= 1; --e) {
                dcar[e] = dn[e - 1];
                gcar[e] = live ? gcar[e - 1] : gcar[e];
            }
            dcar[0] = live ? dl : dcar[0];
            gcar[0] = live ? g : gcar[0];
        };
        auto super = [&](int S, const In& c0, const In& c1, In& n0, In& n1) {
            // the bulk partials of diagonals 2S and 2S + 1 (written in super-step S - 1)
            const f32x4 pq0 = lds4(&sm.pnb[(2 * S) & 3][i][0]);
            const f32x4 rq0 = lds4(&sm.rnb[(2 * S) & 3][i][0]);
            const f32x4 pq1 = lds4(&sm.pnb[(2 * S + 1) & 3][i][0]);
            const f32x4 rq1 = lds4(&sm.rnb[(2 * S + 1) & 3][i][0]);
            // the draws of diagonals 2S and 2S + 1 (written by the hand-over waves in
            // super-step S - 1)
            const float ud0 = p.stochastic ? sm.un[(2 * S) & 3][i] : 0.5f;
            const float ud1 = p.stochastic ? sm.un[(2 * S + 1) & 3][i] : 0.5f;
            // the inputs of the next super-step: the strip hand-overs that feed them
            // were added by super-step S - 1, and nothing writes them in this one
            load_in(2 * S + 2, n0);
            load_in(2 * S + 3, n1);
            entry(2 * S, c0, pq0, rq0, ud0);
            entry(2 * S + 1, c1, pq1, rq1, ud1);
            lds_wait_all();
            barrier_no_wait();
        };
        __syncthreads();
        In a0, a1, b0, b1;
        load_in(0, a0);
        load_in(1, a1);
#pragma nounroll
        for (int S = 0; S < kSuper; S += 2) {
            super(S, a0, a1, b0, b1);
            super(S + 1, b0, b1, a0, a1);
        }
    } else {
        // ---------------- hand-over waves (column-wise, row-wise) ----------------
        // Super-steps 0-23 are the three windows of the neighbour's strips 1-3 (strip
        // c: super-steps 8c - 8 .. 8c - 1), written out super-step by super-step, so
        // that each window is straight-line code: the counter read at 8c - 8 is waited
        // for only where it is checked, a super-step later, and the strip loads of
        // 8c - 7 only at the first multiply, two super-steps later. The product is
        // added at 8c - 2, before the finaliser reads the inputs of step 16c (at the
        // start of super-step 8c - 1). Super-steps 24-63 publish this leaf's strips 0-2.
        // With stochastic rounding they also draw the finaliser's uniforms off its
        // dependent chain: in super-step S, those of super-step S + 1, the column wave
        // for diagonal 2S + 2 and the row wave for 2S + 3 (row = lane), into the ring
        // slot that the finaliser read two super-steps before.
        auto put_draws = [&](int S) {
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int dg = 2 * S + (hcol ? 0 : 1);
            sm.un[dg & 3][ln] =
                uniform24(p.seed, (uint64_t)(i0 + ln) * (uint64_t)p.n + (uint64_t)(j0 + (dg - ln)));
        };
        int sst = 0;  // the super-step that the next sync_step ends
        auto sync_step = [&]() {
            if (p.stochastic) put_draws(sst + 1);
            lds_wait_all();
            barrier_no_wait();
            ++sst;
        };
        if (p.stochastic) put_draws(0);
        __syncthreads();
#pragma nounroll
        for (int cw = 1; cw < kStrips; ++cw) {
            int seen = 0;
            if (hown) seen = ld_flag(hflag);  // super-step 8c - 8
            sync_step();
            if (hown) {  // 8c - 7
                // keeps the check (and the wait for the counter's load) from moving up
                // to the super-step of the load
                asm volatile("" : "+v"(seen));
                if (seen < cw + 1) wait_flag(p, hflag, cw + 1);
                compiler_fence();
                handover_load(p, hcol, cw, i0, j0, R, Cc, h, lane);
            }
            sync_step();
            sync_step();                            // 8c - 6
            if (hown) handover_mma<0, 5>(hcol, h);  // 8c - 5 .. 8c - 3
            sync_step();
            if (hown) handover_mma<5, 10>(hcol, h);
            sync_step();
            if (hown) handover_mma<10, 16>(hcol, h);
            sync_step();
            if (hown) handover_add(sm, hcol, cw, h, lane);  // 8c - 2
            sync_step();
            sync_step();                                    // 8c - 1
        }
        // this leaf's strip c <= 2 (final after step 78 + 16c, in super-step 39 + 8c):
        // stored in super-step 40 + 8c, counter raised two super-steps later
#pragma nounroll
        for (int S = 8 * (kStrips - 1); S < kSuper; ++S) {
            // the lane index, opaque per super-step, so that the address arithmetic of the
            // stores below is not hoisted out of the sweep and held across it
            int ln = lane;
            asm volatile("" : "+v"(ln));
            if (S >= 40) {
                const int cp = (S - 40) >> 3, pp = (S - 40) & 7;
                if (cp < kStrips - 1) {
                    if (pp == 0) handover_publish(p, sm, hcol, cp, i0, j0, R, Cc, ln);
                    else if (pp == 2) handover_flag(p, hcol, leaf, cp + 1, ln);
                }
            }
            sync_step();
        }
    }
    // the last strips
    if (hwave) {
        handover_publish(p, sm, hcol, kStrips - 1, i0, j0, R, Cc, lane);
        handover_flag(p, hcol, leaf, kStrips, lane);
    }
    // ---- the pieces of D (for the column far fields of the leaves four or more below)
    // and of C (for the row far fields of the leaves four or more to the right); the
    // entries outside the matrix are zero
    {
        const bool wd = p.LO && I + 4 < p.M, wc = p.LI && J + 4 < p.N;
        if (wd || wc) {
            if (t < kB) {
                sm.exr[t] = i0 + t < p.m ? p.exd[i0 + t] : 0;
                sm.exq[t] = p.exc[i0 + t];
            }
            __syncthreads();
            for (int e = t; e < 8 * kB; e += kLeafThreads) {
                const int gl = e >> 6, x = e & 63;  // 8-entry group gl along the contraction, column x
                if (wd) {  // D[i0 + 8 gl + q][j0 + x] = DT[x][8 gl + q], row q scaled by 2^eD
                    const f32x4 v0 = lds4(&sm.DT[x][8 * gl]), v1 = lds4(&sm.DT[x][8 * gl + 4]);
                    uint32_t pk[2][4];
#pragma unroll
                    for (int q = 0; q < 8; q += 2) {
                        uint32_t h0, l0, h1, l1;
                        split2_value(q < 4 ? v0[q] : v1[q - 4], sm.exr[8 * gl + q], h0, l0);
                        split2_value(q < 4 ? v0[q + 1] : v1[q - 3], sm.exr[8 * gl + q + 1], h1, l1);
                        pk[0][q >> 1] = h0 | (h1 << 16);
                        pk[1][q >> 1] = l0 | (l1 << 16);
                    }
#pragma unroll
                    for (int pc = 0; pc < 2; ++pc)
                        st_coherent16(&p.dpl[((int64_t)pc * (p.Mp / 8) + 8 * I + gl) * p.Np + j0 + x], pk[pc]);
                }
                if (wc) {  // C[i0 + x][j0 + 8 gl + q] = Gs[x][8 gl + q], scaled by 2^eC of row x
                    const f32x4 v0 = lds4(&sm.Gs[x][8 * gl]), v1 = lds4(&sm.Gs[x][8 * gl + 4]);
                    const int ex = sm.exq[x];
                    uint32_t pk[2][4];
#pragma unroll
                    for (int q = 0; q < 8; q += 2) {
                        uint32_t h0, l0, h1, l1;
                        split2_value(q < 4 ? v0[q] : v1[q - 4], ex, h0, l0);
                        split2_value(q < 4 ? v0[q + 1] : v1[q - 3], ex, h1, l1);
                        pk[0][q >> 1] = h0 | (h1 << 16);
                        pk[1][q >> 1] = l0 | (l1 << 16);
                    }
#pragma unroll
                    for (int pc = 0; pc < 2; ++pc)
                        st_coherent16(&p.cpl[((int64_t)pc * (p.Np / 8) + 8 * J + gl) * p.Mc + kB + i0 + x], pk[pc]);
                }
            }
            vm_wait_all();  // this wave's piece stores have completed
        }
        __syncthreads();
        if (t == 0) {
            if (I > 0) wait_flag(p, &p.pdone[leaf - p.N], 1);
            if (J > 0) wait_flag(p, &p.pdone[leaf - 1], 1);
            st_flag(&p.pdone[leaf], 1);
        }
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
        if (r < nl) {
            leaf_task(p, lo, r, sm.leaf, tid);
        } else {
            const int df = group_far(p.ND, lo);
            const int nf = df >= 0 ? far_tasks(p.M, p.N, df, p.nchd[df]) : 0;
            if (r < nl + nf) far_task(p, df, r - nl, false, sm.far, tid);
            else far_task(p, lo, r - nl - nf, true, sm.far, tid);
        }
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
    int64_t Mp, Np;
    int nkcO, nkcI;  // pre-pass row chunks of L_O, L_I
    size_t ct, delta, parts, leaf_loss, leaf_clamp, info, sched, flags, seg, nchd;
    int64_t Mc;
    size_t lop, lip, dpl, cpl, bd, exd, exc, fexo, fexi, mxO, sbO, mxI, total;
};

Layout layout(int64_t m, int64_t n) {
    Layout L;
    L.M = (int)((m + kB - 1) / kB);
    L.N = (int)((n + kB - 1) / kB);
    L.maxleaf = std::min(L.M, L.N);
    L.ND = L.M + L.N - 1;
    // the planes hold whole quads: rows and columns padded to an even number of leaves
    L.Mp = (int64_t)((L.M + 1) & ~1) * kB;
    L.Np = (int64_t)((L.N + 1) & ~1) * kB;
    L.Mc = (int64_t)((L.M + 2) & ~1) * kB;
    L.nkcO = (int)((m + kPrepRows - 1) / kPrepRows);
    L.nkcI = (int)((n + kPrepRows - 1) / kPrepRows);
    const size_t nl = (size_t)L.M * L.N;
    const size_t Mp = (size_t)L.Mp, Np = (size_t)L.Np;
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
    L.flags = o;  // prog_d, prog_c, setup, fardone, pdone
    o += align256(sizeof(int) * 5 * nl);
    L.seg = o;
    o += align256(sizeof(int) * ((size_t)L.ND + 1));
    L.nchd = o;
    o += align256(sizeof(int) * (size_t)L.ND);
    // piece planes: two fp16 values (4 bytes) per element
    L.lop = o;
    o += align256(4 * Mp * Mp);
    L.lip = o;
    o += align256(4 * Np * Np);
    L.dpl = o;
    o += align256(4 * Mp * Np);
    L.cpl = o;
    o += align256(4 * (size_t)L.Mc * Np);
    L.bd = o;
    o += align256(sizeof(float) * Mp);
    L.exd = o;
    o += align256(sizeof(int) * Mp);
    L.exc = o;
    o += align256(sizeof(int) * Mp);
    L.fexo = o;
    o += align256(sizeof(int) * Mp);
    L.fexi = o;
    o += align256(sizeof(int) * Np);
    L.mxO = o;
    o += align256(sizeof(float) * (size_t)L.nkcO * Mp);
    L.sbO = o;
    o += align256(sizeof(float) * (size_t)L.nkcO * Mp);
    L.mxI = o;
    o += align256(sizeof(float) * (size_t)L.nkcI * Np);
    L.total = o;
    return L;
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
    p.pdone = p.fardone + nl;
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
    p.Mp = L.Mp;
    p.Np = L.Np;
    p.Mc = L.Mc;
    p.lop = (const f16x8*)(base + L.lop);
    p.lip = (const f16x8*)(base + L.lip);
    p.dpl = (f16x8*)(base + L.dpl);
    p.cpl = (f16x8*)(base + L.cpl);
    float* bd = (float*)(base + L.bd);
    int* exd = (int*)(base + L.exd);
    int* exc = (int*)(base + L.exc);
    int* fexo = (int*)(base + L.fexo);
    int* fexi = (int*)(base + L.fexi);
    p.exd = exd;
    p.exc = exc;
    p.fexo = fexo;
    p.fexi = fexi;

    const int init_blocks = (int)std::min<size_t>(1024, std::max<size_t>(1, (nl + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(k_solve_init, dim3((unsigned)init_blocks), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(k_scales, dim3((unsigned)a.m), dim3(kThreads), 0, stream, a.W, a.n, a.ldw,
                       a.bits, a.row_scale, a.scales, bd, exd, p.info);
    // the piece planes of the factors and the exponents of C's rows
    float* mxO = (float*)(base + L.mxO);
    float* sbO = (float*)(base + L.sbO);
    float* mxI = (float*)(base + L.mxI);
    const unsigned eg_o = (unsigned)((L.Mp + kThreads - 1) / kThreads), eg_i = (unsigned)((L.Np + kThreads - 1) / kThreads);
    if (a.LO) {
        hipLaunchKernelGGL(k_lstats, dim3((unsigned)(L.Mp / kB), (unsigned)L.nkcO), dim3(kThreads), 0, stream, a.LO,
                           a.ldlo, a.m, exd, bd, L.Mp, mxO, sbO);
        hipLaunchKernelGGL(k_lexp, dim3(eg_o), dim3(kThreads), 0, stream, mxO, sbO, L.nkcO, L.Mp, a.m, bd, fexo,
                           exc);
        hipLaunchKernelGGL(k_lsplit, dim3((unsigned)(L.Mp / kB), (unsigned)L.nkcO), dim3(kThreads), 0, stream, a.LO,
                           a.ldlo, a.m, exd, fexo, L.Mp, L.Mp / 8, (f16x8*)(base + L.lop));
    } else {  // C = D
        hipLaunchKernelGGL(k_lexp, dim3(eg_o), dim3(kThreads), 0, stream, nullptr, nullptr, 0, L.Mp, a.m, bd,
                           nullptr, exc);
    }
    if (a.LI) {
        hipLaunchKernelGGL(k_lstats, dim3((unsigned)(L.Np / kB), (unsigned)L.nkcI), dim3(kThreads), 0, stream, a.LI,
                           a.ldli, a.n, nullptr, nullptr, L.Np, mxI, nullptr);
        hipLaunchKernelGGL(k_lexp, dim3(eg_i), dim3(kThreads), 0, stream, mxI, nullptr, L.nkcI, L.Np, a.n, nullptr,
                           fexi, nullptr);
        hipLaunchKernelGGL(k_lsplit, dim3((unsigned)(L.Np / kB), (unsigned)L.nkcI), dim3(kThreads), 0, stream, a.LI,
                           a.ldli, a.n, nullptr, fexi, L.Np, L.Np / 8, (f16x8*)(base + L.lip));
    }
    const int grid = (int)std::min<int64_t>(di.cus, ntask);
    hipLaunchKernelGGL(k_solve_run, dim3((unsigned)grid), dim3(kLeafThreads), 0, stream, p);
    hipLaunchKernelGGL(k_solve_finish, dim3(1), dim3(kThreads), 0, stream, p.leaf_loss,
                       p.leaf_clamp, (int64_t)nl, a.loss, a.clamped, p.info, p.abort, a.info);
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

}  // namespace bk
