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
constexpr int kNch = 8;    // maximum K-chunks per far-field product
constexpr int kTargetWg = 1024;  // far-field workgroups aimed for per launch

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

__device__ __forceinline__ void far_body(const SolveParams& p, int d, int nch, int task, GemmSmemT& sm) {
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
    chunk_range(kblk, nch, c, kb0, kb1);
    if (kb1 <= kb0) return;
    const int64_t i0 = (int64_t)I * kB, j0 = (int64_t)J * kB;
    const int R = (int)min<int64_t>(kB, p.m - i0), Cc = (int)min<int64_t>(kB, p.n - j0);
    const int64_t k0 = (int64_t)kb0 * kB, K = (int64_t)(kb1 - kb0) * kB;
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    const bool active = threadIdx.x < kThreads;  // the fifth wave only joins the barriers
    if (kind == 0)  // p[ii][jj] = sum_k L_O[k][i0+ii] D[k][j0+jj]
        tile_gemm32_f32(p.LO + k0 * p.ldlo + i0, p.ldlo, R, p.delta + k0 * p.ldd + j0, p.ldd, Cc,
                        K, acc, sm, active);
    else  // o^T[jj][ii] = sum_l L_I[l][j0+jj] C^T[l][i0+ii]
        tile_gemm32_f32(p.LI + k0 * p.ldli + j0, p.ldli, Cc, p.ct + k0 * p.m + i0, p.m, R, K, acc,
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
// which only uses entries finalised two or more steps earlier, and the newest
// term (k = i-1, l = j-1). Waves 0-3 compute the bulk of step st+1 while wave
// 4 finalises step st, so the dependent chain per step is short and the bulk
// LDS traffic overlaps it. The finaliser takes D[i-1][j] from the lane above
// (it was that lane's result one step earlier) and g[i][j-1] from its own
// previous step, so only the two bulk sums cross LDS on the chain.
//
// Bulk lanes are (row i, quarter q) with lane = 4 i + q; quarter q owns the
// k / l chunks [8q, 8q+8) and [32+8q, 32+8q+8). With 68-float rows (16 bytes
// of bank offset per row) the four b128 reads of a row pair hit eight
// distinct bank groups.
// ---------------------------------------------------------------------------
constexpr int kLeafThreads = 5 * 64;
constexpr int kTs = 68;  // row stride of the k/l-indexed tiles
constexpr int kPs = 66;  // row stride of the per-entry inputs: anti-diagonal walks hit distinct banks

struct LeafSmem {
    float DT[kB][kTs];     // D transposed: DT[j][k] = D[k][j] (0 until known)
    float Gs[kB][kTs];     // g = C of the leaf, row-major (0 until known)
    float LIT[kB][kTs];    // L_I diagonal block transposed: LIT[j][l] = L_I[l][j], l < j
    float base[kB][kPs];   // W* + o
    float pin[kB][kPs];    // p
    float wst[kB][kPs];    // W*
    float pnb[2][kB];      // bulk sums, double buffered by step parity
    float rnb[2][kB];
    uint8_t code[kB][kB + 4];
    float DI[kB];
    double red[kLeafThreads];
    int red_i[kLeafThreads];
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

__device__ __forceinline__ float lane_above(float x) {
    // wave_shr:1 -- lane i receives lane i-1's value, lane 0 receives 0
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x138,
                                                                  0xF, 0xF, false));
}

__device__ __forceinline__ void leaf_body(const SolveParams& p, int d, int nch, int slot, LeafSmem& sm) {
    if (*p.info != INT_MAX) return;
    const int I = leaf_lo(p, d) + slot;
    const int J = d - I;
    const int64_t i0 = (int64_t)I * kB, j0 = (int64_t)J * kB;
    const int R = (int)min<int64_t>(kB, p.m - i0), Cc = (int)min<int64_t>(kB, p.n - j0);
    const int t = threadIdx.x;
    const int par = d & 1;
    const int np = (p.LO && I > 1) ? nch : 0;  // partials of p and o^T to add
    const int no = (p.LI && J > 1) ? nch : 0;
    const bool adj_p = p.LO && I > 0, adj_o = p.LI && J > 0;
    const int w = t >> 6;

    // ---- adjacent blocks (K = 64), staged in LDS regions that are set up later:
    //   p  += L_O[i0-64+k][i0+ii] D[i0-64+k][j0+jj]
    //   o^T += L_I[j0-64+l][j0+jj] C^T[j0-64+l][i0+ii]
    {
        // every load of the thread is issued before the first LDS store
        constexpr int kPer = (kB * kB + kLeafThreads - 1) / kLeafThreads;
        float v1[kPer], v2[kPer], v3[kPer], v4[kPer];
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
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + u * kLeafThreads;
            if (e < kB * kB) {
                const int k = e >> 6, c = e & 63;
                sm.DT[k][c] = v1[u];
                sm.Gs[k][c] = v2[u];
                sm.LIT[k][c] = v3[u];
                sm.wst[k][c] = v4[u];
            }
        }
    }
    __syncthreads();
    f32x16 ap, ao;
#pragma unroll
    for (int v = 0; v < 16; ++v) ap[v] = ao[v] = 0.0f;
    if (w < 4) {
        if (adj_p) adj_gemm(&sm.DT[0][0], kTs, &sm.Gs[0][0], kTs, ap);
        if (adj_o) adj_gemm(&sm.LIT[0][0], kTs, &sm.wst[0][0], kPs, ao);
    }

    // ---- far fields from diagonals d-2 and earlier (sum of the K-chunk partials, in chunk order) ----
    for (int g4 = t; g4 < kB * kB / 4; g4 += kLeafThreads) {
        const int e = 4 * g4;
        f32x4 pv = {0.f, 0.f, 0.f, 0.f}, ov = {0.f, 0.f, 0.f, 0.f};
        f32x4 xp[kNch], xo[kNch];
#pragma unroll
        for (int c = 0; c < kNch; ++c) {
            int b0, b1;
            chunk_range(I - 1, nch, c, b0, b1);
            xp[c] = (c < np && b1 > b0) ? *reinterpret_cast<const f32x4*>(part_ptr(p, par, slot, 0, c) + e)
                                        : f32x4{0.f, 0.f, 0.f, 0.f};
            chunk_range(J - 1, nch, c, b0, b1);
            xo[c] = (c < no && b1 > b0) ? *reinterpret_cast<const f32x4*>(part_ptr(p, par, slot, 1, c) + e)
                                        : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int c = 0; c < kNch; ++c) {
            pv += xp[c];
            ov += xo[c];
        }
        const int r = e / kB, c0 = e % kB;  // p: row r, cols c0..c0+3; o^T: row (= leaf col) r, leaf rows c0..
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            sm.pin[r][c0 + k] = pv[k];
            sm.base[c0 + k][r] = ov[k];
        }
    }
    __syncthreads();
    if (w < 4) {  // then the adjacent products
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
        const float wv = (i < R && j < Cc) ? p.W[(i0 + i) * p.ldw + j0 + j] : 0.0f;
        // L_I[l][jj] stored at LIT[jj][l] (here l = i, jj = j)
        const float lv = (p.LI && i < j && j < Cc) ? p.LI[(j0 + i) * p.ldli + j0 + j] : 0.0f;
        sm.wst[i][j] = wv;
        sm.base[i][j] += wv;
        sm.LIT[j][i] = lv;
        sm.DT[i][j] = 0.0f;
        sm.Gs[i][j] = 0.0f;
        sm.code[i][j] = 0;
    }
    if (t < kB) {
        sm.DI[t] = (p.want_loss && t < Cc) ? p.DI[j0 + t] : 0.0f;
        sm.pnb[0][t] = sm.pnb[1][t] = 0.0f;
        sm.rnb[0][t] = sm.rnb[1][t] = 0.0f;
    }

    double loss = 0.0;
    int nclamp = 0;
    if (w < 4) {
        // ---------------- bulk waves ----------------
        const int i = t >> 2;
        const int q = t & 3;
        const int ka = 8 * q, kb = 32 + 8 * q;  // the quarter's two 8-wide chunks
        float lo_a[8], lo_b[8];                 // L_O[i0 + k][i0 + i] for k <= i - 2
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo_a[e] = (p.LO && ka + e <= i - 2 && i < R) ? p.LO[(i0 + ka + e) * p.ldlo + i0 + i] : 0.0f;
            lo_b[e] = (p.LO && kb + e <= i - 2 && i < R) ? p.LO[(i0 + kb + e) * p.ldlo + i0 + i] : 0.0f;
        }
        const bool pa = p.LO && ka <= i - 2, pbl = p.LO && kb <= i - 2;
        __syncthreads();
        for (int st = 0; st < 2 * kB - 1; ++st) {
            const int jn = st + 1 - i;  // entry (i, jn) is finalised at the next step
            float pn = 0.0f, rn = 0.0f;
            if (jn >= 0 && jn < kB) {
                const float* dcol = &sm.DT[jn][0];
                if (pa) {
                    const f32x4 d0 = *reinterpret_cast<const f32x4*>(dcol + ka);
                    const f32x4 d1 = *reinterpret_cast<const f32x4*>(dcol + ka + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pn = fmaf(lo_a[e], d0[e], pn);
                        pn = fmaf(lo_a[4 + e], d1[e], pn);
                    }
                }
                if (pbl) {
                    const f32x4 d0 = *reinterpret_cast<const f32x4*>(dcol + kb);
                    const f32x4 d1 = *reinterpret_cast<const f32x4*>(dcol + kb + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pn = fmaf(lo_b[e], d0[e], pn);
                        pn = fmaf(lo_b[4 + e], d1[e], pn);
                    }
                }
                // rn bulk: l <= jn - 2 (l = jn - 1 is the newest term, masked below)
                const float* grow = &sm.Gs[i][0];
                const float* lcol = &sm.LIT[jn][0];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kc = h ? kb : ka;
                    if (kc <= jn - 2) {
                        const f32x4 g0 = *reinterpret_cast<const f32x4*>(grow + kc);
                        const f32x4 g1 = *reinterpret_cast<const f32x4*>(grow + kc + 4);
                        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lcol + kc);
                        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lcol + kc + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            rn = fmaf(g0[e], (kc + e == jn - 1) ? 0.0f : l0[e], rn);
                            rn = fmaf(g1[e], (kc + 4 + e == jn - 1) ? 0.0f : l1[e], rn);
                        }
                    }
                }
            }
            pn = quad_sum(pn);
            rn = quad_sum(rn);
            if (q == 0 && jn >= 0 && jn < kB) {
                sm.pnb[(st + 1) & 1][i] = pn;
                sm.rnb[(st + 1) & 1][i] = rn;
            }
            __syncthreads();
        }
    } else {
        // ---------------- finaliser wave: lane i owns row i ----------------
        const int i = t & 63;
        const float lo_last = (p.LO && i >= 1 && i < R) ? p.LO[(i0 + i - 1) * p.ldlo + i0 + i] : 0.0f;
        const int Lq = (1 << p.bits) - 1;
        const float half = 0.5f * (float)Lq;
        const float s = (i < R) ? p.scales[i0 + i] : 1.0f;
        const float rs = 1.0f / s;
        const float dO = (p.want_loss && i < R) ? (p.DO ? p.DO[i0 + i] : 1.0f) : 0.0f;
        float d_last = 0.0f;  // D of this row's previous entry (read by the lane below)
        float g_last = 0.0f;  // g of this row's previous entry
        __syncthreads();
        // static inputs of the first entry of the row (j = 0) are read at step i
        float x_pin = 0.f, x_base = 0.f, x_w = 0.f, x_l = 0.f, x_di = 0.f;
        for (int st = 0; st < 2 * kB - 1; ++st) {
            const int j = st - i;
            const float dprev = lane_above(d_last);
            if (j >= 0 && j < kB) {
                x_pin = sm.pin[i][j];
                x_base = sm.base[i][j];
                x_w = sm.wst[i][j];
                x_l = (j >= 1) ? sm.LIT[j][j - 1] : 0.0f;
                x_di = sm.DI[j];
            }
            if (j >= 0 && j < Cc && i < R) {
                float u = 0.5f;
                if (p.stochastic)
                    u = uniform24(p.seed, (uint64_t)(i0 + i) * (uint64_t)p.n + (uint64_t)(j0 + j));
                const float P = x_pin + (sm.pnb[st & 1][i] + lo_last * dprev);
                const float Rr = sm.rnb[st & 1][i] + g_last * x_l;
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
                d_last = dl;
                g_last = g;
                const float eta = fmaf(-s, cf - half, tv);
                loss += (double)(dO * x_di) * (double)eta * (double)eta;
            }
            __syncthreads();
        }
    }

    // ---- outputs ----
    for (int e = t; e < kB * kB; e += kLeafThreads) {
        const int ii = e / kB, jj = e % kB;
        if (ii < R && jj < Cc) {
            p.codes[(i0 + ii) * p.ldc + j0 + jj] = sm.code[ii][jj];
            p.delta[(i0 + ii) * p.ldd + j0 + jj] = sm.DT[jj][ii];
        }
        const int ci = e % kB, cj = e / kB;  // C^T written along the leaf's rows
        if (ci < R && cj < Cc) p.ct[(j0 + cj) * p.m + i0 + ci] = sm.Gs[ci][cj];
    }
    sm.red[t] = loss;
    sm.red_i[t] = nclamp;
    __syncthreads();
    if (t < 64) {
        double a = 0.0;
        int b = 0;
        for (int k = t; k < kLeafThreads; k += 64) {
            a += sm.red[k];
            b += sm.red_i[k];
        }
        sm.red[t] = a;
        sm.red_i[t] = b;
    }
    __syncthreads();
    for (int o = 32; o > 0; o >>= 1) {
        if (t < o) {
            sm.red[t] += sm.red[t + o];
            sm.red_i[t] += sm.red_i[t + o];
        }
        __syncthreads();
    }
    if (t == 0) {
        p.leaf_loss[(size_t)I * p.N + J] = sm.red[0];
        p.leaf_clamp[(size_t)I * p.N + J] = sm.red_i[0];
    }
}

// One launch per leaf-diagonal d: workgroups 0..nleaf-1 solve the leaves of
// d (dispatched first), the others form the far fields of d + 1 (their inputs
// are the leaves of d - 1 and earlier, finished by the previous launch) on
// the CUs the leaves leave free.
union StepSmem {
    LeafSmem leaf;
    GemmSmemT far;
};

__global__ __launch_bounds__(kLeafThreads) void k_step(SolveParams p, int d, int nch, int nleaf,
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
