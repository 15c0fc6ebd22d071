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
// parallelism). The schedule here is a wavefront over 64x64 leaves: the leaves
// of leaf-diagonal d = I + J are solved together, one workgroup each. For
// leaf (I, J) with row block R_I and column block S_J the feedback splits into
//   p  = sum_{I'<I} L_O[R_I', R_I]^T D[R_I', S_J]   (column far field)
//   o  = sum_{J'<J} C[R_I, S_J'] L_I[S_J', S_J]      (row far field)
// plus the in-leaf sums, which the leaf workgroup runs as a 127-step
// anti-diagonal wavefront. The far fields are MFMA GEMMs. Their contributions
// from blocks on leaf-diagonals d-2 and earlier (split over K into partials)
// need only the leaves of d-2, so they are formed by extra workgroups of the
// launch that solves the leaves of d-1, on the CUs those leaves leave free.
// The two blocks adjacent to the leaf (on diagonal d-1, K = 64) are
// multiplied by the leaf workgroup itself. The leaf adds the partials in chunk order and then the adjacent
// products, so the result does not depend on scheduling. Total far-field work
// is mn(m+n) flops, the O(mn(m+n)) of the BaKron Abstract; the wavefront takes
// 2(m+n)/64 - 1 leaf launches, O(m+n).
#include <limits.h>

#include <algorithm>

#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

constexpr int kB = kTile;  // leaf edge
constexpr int kNch = 4;    // maximum K-chunks per far-field product
constexpr int kTargetWg = 1024;  // far-field workgroups aimed for per launch
constexpr int kFarKT = 64;       // k-slice depth of the far-field GEMMs

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
};

__device__ __forceinline__ int leaf_lo(const SolveParams& p, int d) { return max(0, d - (p.N - 1)); }
__device__ __forceinline__ int leaf_hi(const SolveParams& p, int d) { return min(d, p.M - 1); }

// far-field partials: parity of the diagonal, leaf slot on it, kind (0: p, 1: o^T), K-chunk
__device__ __forceinline__ float* part_ptr(const SolveParams& p, int par, int slot, int kind, int c) {
    return p.parts + ((((size_t)par * p.maxleaf + slot) * 2 + kind) * kNch + c) * (kB * kB);
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

__global__ void k_solve_init(int* info) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *info = INT_MAX;
}

// ---------------------------------------------------------------------------
// far field of diagonal d: chunk c (of nch) of p (kind 0) or o^T (kind 1) of
// one leaf, over the blocks above (p) or to the left (o) of the leaf except
// the adjacent one, i.e. blocks on diagonals d-2 and earlier. Each chunk
// writes its own 64x64 partial; the leaf adds the partials in chunk order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void chunk_range(int kblk, int nch, int c, int& b0, int& b1) {
    const int len = (kblk + nch - 1) / nch;
    b0 = min(c * len, kblk);
    b1 = min(b0 + len, kblk);
}

__device__ __forceinline__ void far_body(const SolveParams& p, int d, int nch, int task, GemmSmemF32<kFarKT>& sm) {
    if (*p.info != INT_MAX) return;  // a row scale was invalid
    const int slot = task / (2 * nch);
    const int kind = (task / nch) & 1;
    const int c = task % nch;
    const int I = leaf_lo(p, d) + slot;
    const int J = d - I;
    if ((kind == 0 && !p.LO) || (kind == 1 && !p.LI)) return;
    const int kblk = (kind == 0 ? I : J) - 1;
    if (kblk <= 0) return;
    int kb0, kb1;
    chunk_range(kblk, nch, c, kb0, kb1);  // an empty chunk writes a zero partial
    const int64_t i0 = (int64_t)I * kB, j0 = (int64_t)J * kB;
    const int R = (int)min<int64_t>(kB, p.m - i0), Cc = (int)min<int64_t>(kB, p.n - j0);
    const int64_t k0 = (int64_t)kb0 * kB, K = (int64_t)(kb1 - kb0) * kB;
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    const bool active = threadIdx.x < kThreads;  // the fifth wave only joins the barriers
    if (kind == 0)  // p[ii][jj] = sum_k L_O[k][i0+ii] D[k][j0+jj]
        tile_gemm_f32<kFarKT>(p.LO + k0 * p.ldlo + i0, p.ldlo, R, p.delta + k0 * p.ldd + j0, p.ldd, Cc,
                        K, acc, sm, active);
    else  // o^T[jj][ii] = sum_l L_I[l][j0+jj] C^T[l][i0+ii]
        tile_gemm_f32<kFarKT>(p.LI + k0 * p.ldli + j0, p.ldli, Cc, p.ct + k0 * p.m + i0, p.m, R, K, acc,
                        sm, active);
    if (!active) return;
    float* part = part_ptr(p, d & 1, slot, kind, c);
    const int cc = acc32_col();
#pragma unroll
    for (int v = 0; v < 16; ++v) part[acc32_row(v) * kB + cc] = acc[v];
}

// ---------------------------------------------------------------------------
// leaf solve: the 64x64 leaf (I, J) of diagonal d, given its far fields.
//
// Entry (i, j) is finalised at step i + j. Its in-leaf sums
//   pn = sum_{k<i} L_O[k][i] D[k][j],   rn = sum_{l<j} g[i][l] L_I[l][j]
// (g = C, the column feedback plus error of the row) are split into a bulk,
// which only uses entries finalised three or more steps earlier, and the two
// newest terms of each (k = i-1, i-2 and l = j-1, j-2). Waves 0-3 compute the
// bulk of step st + 2 while wave 4 finalises step st, so the dependent chain
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
// ---------------------------------------------------------------------------
constexpr int kLeafThreads = 5 * 64;
constexpr int kTs = 68;  // row stride of the k/l-indexed tiles
constexpr int kPs = 66;  // row stride of the per-entry inputs: anti-diagonal walks hit distinct banks

struct LeafSmem {
    float DT[kB][kTs];     // D transposed: DT[j][k] = D[k][j] (0 until known)
    float Gs[kB][kTs];     // g = C of the leaf, row-major (0 until known)
    float base[kB][kPs];   // W* + o
    float pin[kB][kPs];    // p
    float wst[kB][kPs];    // W*, overwritten by eta = t - q once the entry is final
    float pnb[3][kB];      // bulk sums, by step modulo 3 (written two steps ahead)
    float rnb[3][kB];
    float li1[kB];         // L_I[j-1][j], L_I[j-2][j]: the finaliser's terms
    float li2[kB];
    uint8_t code[kB][kB + 4];
    float DI[kB];
    double red[kLeafThreads / 64];
    int red_i[kLeafThreads / 64];
};

// acc += X^T Y over k = 0..63 for the 64x64 tile, X[k][r] at x[k * sx + r] and
// Y[k][c] at y[k * sy + c] in LDS; waves 0-3 each own a 32x32 quadrant
// (32x32x2 f32 MFMA operand and output layout of bk_common.hpp).
__device__ __forceinline__ void adj_gemm(const float* x, int sx, const float* y, int sy, f32x16& acc) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
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

__device__ __forceinline__ void leaf_body(const SolveParams& p, int d, int nch, int slot, LeafSmem& sm) {
    if (*p.info != INT_MAX) return;
    const int I = leaf_lo(p, d) + slot;
    const int J = d - I;
    const int64_t i0 = (int64_t)I * kB, j0 = (int64_t)J * kB;
    const int R = (int)min<int64_t>(kB, p.m - i0), Cc = (int)min<int64_t>(kB, p.n - j0);
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int par = d & 1;
    const bool far_p = p.LO && I > 1, far_o = p.LI && J > 1;  // all nch partials were written
    const bool adj_p = p.LO && I > 0, adj_o = p.LI && J > 0;

    if (t < 2) {  // no L_I[j-d][j] for j < d
        sm.li2[t] = 0.0f;
        if (t < 1) sm.li1[t] = 0.0f;
    }
    // ---- A: every tile load of the thread in flight at once, then LDS
    //   DT  <- L_O[i0-64+k][i0+c]   Gs   <- D[i0-64+k][j0+c]      (block above: staging)
    //   pin <- L_I[j0-64+k][j0+c]   base <- C^T[j0-64+k][i0+c]    (block to the left: staging)
    //   wst <- W*[i0+k][j0+c]       li1, li2 <- the first two superdiagonals of L_I
    {
        constexpr int kPer = (kB * kB + kLeafThreads - 1) / kLeafThreads;
        float v1[kPer], v2[kPer], v3[kPer], v4[kPer], v5[kPer], v6[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            const int k = e >> 6, c = e & 63;
            const bool in = e < kB * kB;
            const int64_t ik = i0 - kB + k, jk = j0 - kB + k;
            v1[u] = (in && adj_p && c < R) ? p.LO[ik * p.ldlo + i0 + c] : 0.0f;
            v2[u] = (in && adj_p && c < Cc) ? p.delta[ik * p.ldd + j0 + c] : 0.0f;
            v3[u] = (in && adj_o && c < Cc) ? p.LI[jk * p.ldli + j0 + c] : 0.0f;
            v4[u] = (in && adj_o && c < R) ? p.ct[jk * p.m + i0 + c] : 0.0f;
            v5[u] = (in && k < R && c < Cc) ? p.W[(i0 + k) * p.ldw + j0 + c] : 0.0f;
            v6[u] = (in && p.LI && (c - k == 1 || c - k == 2) && c < Cc) ? p.LI[(j0 + k) * p.ldli + j0 + c] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            if (e < kB * kB) {
                const int k = e >> 6, c = e & 63;
                sm.DT[k][c] = v1[u];
                sm.Gs[k][c] = v2[u];
                sm.pin[k][c] = v3[u];
                sm.base[k][c] = v4[u];
                sm.wst[k][c] = v5[u];
                if (c - k == 1) sm.li1[c] = v6[u];
                if (c - k == 2) sm.li2[c] = v6[u];
            }
        }
    }
    __syncthreads();
    f32x16 ap, ao;  // adjacent products (K = 64): p += L_O^T D, o^T += L_I^T C^T
#pragma unroll
    for (int v = 0; v < 16; ++v) ap[v] = ao[v] = 0.0f;
    if (w < 4) {
        if (adj_p) adj_gemm(&sm.DT[0][0], kTs, &sm.Gs[0][0], kTs, ap);
        if (adj_o) adj_gemm(&sm.pin[0][0], kPs, &sm.base[0][0], kPs, ao);
    }
    __syncthreads();

    // ---- B: far fields from diagonals d-2 and earlier: the K-chunk partials
    // summed in chunk order (every load issued first; absent chunks read a valid
    // address and are replaced by zero). D, g and the codes are cleared while the
    // loads are in flight (the staging in DT and Gs is consumed).
    {
        constexpr int kG = (kB * kB / 4 + kLeafThreads - 1) / kLeafThreads;
        const bool any = far_p || far_o;
        f32x4 xp[kG][kNch], xo[kG][kNch];
        if (any) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int g = min(t + u * kLeafThreads, kB * kB / 4 - 1);
#pragma unroll
                for (int c = 0; c < kNch; ++c) {
                    const int cc = min(c, nch - 1);
                    xp[u][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, par, slot, 0, cc) + 4 * g);
                    xo[u][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, par, slot, 1, cc) + 4 * g);
                }
            }
        }
        const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
        if (any) {
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            const int g = t + u * kLeafThreads;
            if (g < kB * kB / 4) {
                const int k = g >> 4, c4 = (g & 15) << 2;
                *reinterpret_cast<f32x4*>(&sm.DT[k][c4]) = z4;
                *reinterpret_cast<f32x4*>(&sm.Gs[k][c4]) = z4;
                *reinterpret_cast<uint32_t*>(&sm.code[k][c4]) = 0u;
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
                        xp[uu][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, par, slot, 0, cc) + 4 * gg);
                        xo[uu][c] = *reinterpret_cast<const f32x4*>(part_ptr(p, par, slot, 1, cc) + 4 * gg);
                    }
                }
            }
            const int g = t + u * kLeafThreads;
            if (g >= kB * kB / 4) continue;
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
            const int e = 4 * g;
            const int r = e / kB, c0 = e % kB;  // p: row r, cols c0..c0+3; o^T: row (= leaf col) r, leaf rows c0..
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sm.pin[r][c0 + k] = pv[k];
                sm.base[c0 + k][r] = ov[k];
            }
        }
    }
    __syncthreads();
    // ---- C: then the adjacent products, then W*
    if (w < 4) {
        const int cc = acc32_col();
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            sm.pin[acc32_row(v)][cc] += ap[v];
            sm.base[cc][acc32_row(v)] += ao[v];
        }
    }
    __syncthreads();
    for (int e = t; e < kB * kB; e += kLeafThreads) {
        const int i = e / kB, j = e % kB;
        sm.base[i][j] += sm.wst[i][j];
    }
    if (t < kB) {
        sm.DI[t] = (p.want_loss && t < Cc) ? p.DI[j0 + t] : 0.0f;
        sm.pnb[0][t] = sm.pnb[1][t] = sm.pnb[2][t] = 0.0f;
        sm.rnb[0][t] = sm.rnb[1][t] = sm.rnb[2][t] = 0.0f;
    }

    double loss = 0.0;
    int nclamp = 0;
    if (w < 4) {
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
        const int a = t >> 2;
        const int q = t & 3;
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
    } else {
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
            n_pin = sm.pin[0][0];
            n_base = sm.base[0][0];
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
            n_pin = sm.pin[i][jn];
            n_base = sm.base[i][jn];
            n_w = sm.wst[i][jn];
            n_l1 = sm.li1[jn];
            n_l2 = sm.li2[jn];
            slot3n = slot3n == 2 ? 0 : slot3n + 1;
            __builtin_amdgcn_sched_barrier(0);
            barrier_no_wait();
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

    // ---- outputs: codes and D along the leaf's rows, C^T along its columns; every LDS
    // read of the thread first, then the stores (four columns per store where aligned)
    {
        constexpr int kG = (kB * kB / 4 + kLeafThreads - 1) / kLeafThreads;
        const bool ovec = ((reinterpret_cast<uintptr_t>(p.delta) | reinterpret_cast<uintptr_t>(p.ct)) & 15) == 0 &&
                          (reinterpret_cast<uintptr_t>(p.codes) & 3) == 0 && ((p.ldd | p.m | p.ldc) & 3) == 0;
        uint32_t cv[kG];
        f32x4 dv[kG], gv[kG];
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            const int g = min(t + u * kLeafThreads, kB * kB / 4 - 1);
            const int r = g >> 4, c4 = (g & 15) << 2;
            cv[u] = *reinterpret_cast<const uint32_t*>(&sm.code[r][c4]);  // code[r][c4..]
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dv[u][e] = sm.DT[c4 + e][r];  // D[r][c4 + e]
                gv[u][e] = sm.Gs[c4 + e][r];  // C[c4 + e][r], row r of C^T
            }
        }
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            const int g = t + u * kLeafThreads;
            if (g >= kB * kB / 4) continue;
            const int r = g >> 4, c4 = (g & 15) << 2;
            if (r < R) {  // row i0 + r of the codes and of D, columns j0 + c4..
                uint8_t* cp = p.codes + (i0 + r) * p.ldc + j0 + c4;
                float* dp = p.delta + (i0 + r) * p.ldd + j0 + c4;
                if (ovec && c4 + 3 < Cc) {
                    *reinterpret_cast<uint32_t*>(cp) = cv[u];
                    *reinterpret_cast<f32x4*>(dp) = dv[u];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c4 + e < Cc) {
                            cp[e] = (uint8_t)(cv[u] >> (8 * e));
                            dp[e] = dv[u][e];
                        }
                }
            }
            if (r < Cc) {  // row j0 + r of C^T, columns i0 + c4..
                float* gp = p.ct + (j0 + r) * p.m + i0 + c4;
                if (ovec && c4 + 3 < R) {
                    *reinterpret_cast<f32x4*>(gp) = gv[u];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c4 + e < R) gp[e] = gv[u][e];
                }
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
        for (int k = 0; k < kLeafThreads / 64; ++k) {
            lsum += sm.red[k];
            csum += sm.red_i[k];
        }
        p.leaf_loss[(size_t)I * p.N + J] = lsum;
        p.leaf_clamp[(size_t)I * p.N + J] = csum;
    }
}

// One launch per leaf-diagonal d: workgroups 0..nleaf-1 solve the leaves of
// d (dispatched first), the others form the far fields of d + 1 (their inputs
// are the leaves of d - 1 and earlier, finished by the previous launch) on
// the CUs the leaves leave free.
union StepSmem {
    LeafSmem leaf;
    GemmSmemF32<kFarKT> far;
};

__global__ __launch_bounds__(kLeafThreads, 1) void k_step(SolveParams p, int d, int nch, int nleaf,
                                                       int nch_next) {
    __shared__ StepSmem sm;
    if ((int)blockIdx.x < nleaf) leaf_body(p, d, nch, blockIdx.x, sm.leaf);
    else far_body(p, d + 1, nch_next, blockIdx.x - nleaf, sm.far);
}

// loss = sum of leaf partials in a fixed order; clamped count; info.
__global__ __launch_bounds__(kThreads) void k_solve_finish(const double* leaf_loss,
                                                           const int* leaf_clamp, int nleaves,
                                                           double* loss, int64_t* clamped,
                                                           const int* info_ws, int32_t* info) {
    __shared__ double rl[kThreads];
    __shared__ long long rc[kThreads];
    double s = 0.0;
    long long c = 0;
    for (int e = threadIdx.x; e < nleaves; e += kThreads) {
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
        if (info) *info = (*info_ws == INT_MAX) ? 0 : *info_ws;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {
struct Layout {
    int M, N, maxleaf;
    size_t ct, delta, parts, leaf_loss, leaf_clamp, info, total;
};

Layout layout(int64_t m, int64_t n) {
    Layout L;
    L.M = (int)((m + kB - 1) / kB);
    L.N = (int)((n + kB - 1) / kB);
    L.maxleaf = std::min(L.M, L.N);
    size_t o = 0;
    L.ct = o;
    o += align256(sizeof(float) * (size_t)m * (size_t)n);
    L.delta = o;
    o += align256(sizeof(float) * (size_t)m * (size_t)n);
    L.parts = o;  // two diagonals in flight (parity)
    o += align256(sizeof(float) * 2 * (size_t)L.maxleaf * 2 * kNch * kB * kB);
    L.leaf_loss = o;
    o += align256(sizeof(double) * (size_t)L.M * L.N);
    L.leaf_clamp = o;
    o += align256(sizeof(int) * (size_t)L.M * L.N);
    L.info = o;
    o += 256;
    L.total = o;
    return L;
}
}  // namespace

size_t solve_workspace_bytes(int64_t m, int64_t n) { return layout(m, n).total; }

int run_solve(const SolveArgs& a, void* ws, hipStream_t stream) {
    const Layout L = layout(a.m, a.n);
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

    hipLaunchKernelGGL(k_solve_init, dim3(1), dim3(64), 0, stream, p.info);
    hipLaunchKernelGGL(k_scales, dim3((unsigned)a.m), dim3(kThreads), 0, stream, a.W, a.n, a.ldw,
                       a.bits, a.row_scale, a.scales, p.info);
    const int ndiag = L.M + L.N - 1;
    // per diagonal: leaf count and K-chunks per far-field product (enough
    // workgroups to fill the chip, chunks of at least 4 blocks)
    auto diag_shape = [&](int d, int& nleaf, int& nch, int& nfar) {
        const int lo = std::max(0, d - (L.N - 1)), hi = std::min(d, L.M - 1);
        nleaf = hi - lo + 1;
        const int kmax = std::max(hi, d - lo) - 1;  // blocks before the adjacent one
        nch = std::max(1, (kTargetWg + 2 * nleaf - 1) / (2 * nleaf));
        nch = std::min(nch, std::max(1, kmax / 4));
        nch = std::min(nch, kNch);
        nfar = kmax > 0 ? nleaf * 2 * nch : 0;
    };
    for (int d = 0; d < ndiag; ++d) {
        int nleaf, nch, nfar, nl1 = 0, nch1 = 1, nfar1 = 0;  // this diagonal, the next one
        diag_shape(d, nleaf, nch, nfar);
        if (d + 1 < ndiag) diag_shape(d + 1, nl1, nch1, nfar1);
        hipLaunchKernelGGL(k_step, dim3((unsigned)(nleaf + nfar1)), dim3(kLeafThreads), 0, stream, p,
                           d, nch, nleaf, nch1);
    }
    hipLaunchKernelGGL(k_solve_finish, dim3(1), dim3(kThreads), 0, stream, p.leaf_loss,
                       p.leaf_clamp, L.M * L.N, a.loss, a.clamped, p.info, a.info);
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

}  // namespace bk
