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
// anti-diagonal wavefront. The far fields are MFMA GEMMs; all of them except
// the contribution of the two adjacent leaves of diagonal d-1 are formed one
// launch early by extra workgroups of the previous launch (split over K, with
// a deterministic last-block reduction), so they overlap the leaf solves; the
// adjacent contributions (K = 64) are added by the leaf workgroup itself.
// Total far-field work is mn(m+n) flops, the O(mn(m+n)) of the BaKron
// Abstract; the wavefront takes 2(m+n)/64 - 1 leaf launches, O(m+n).
#include <limits.h>

#include <algorithm>

#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

constexpr int kB = kTile;  // leaf edge
constexpr int kNch = 16;   // maximum K-chunks per far-field product
constexpr int kDs = 72;    // LDS row stride of the D tile (8 mod 32: conflict-free column walks)
constexpr int kGs = 68;    // LDS row stride of the C tile (4 mod 32)
constexpr int kLs = 72;    // LDS row stride of the L_I diagonal block

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
    float* offs;
    float* parts;
    unsigned* counters;
    double* leaf_loss;
    int* leaf_clamp;
    const float* DO;
    const float* DI;
    int want_loss;
    int* info;
    int maxleaf;
    int cbk;  // K-chunk length in 64-blocks
};

__device__ __forceinline__ int leaf_lo(const SolveParams& p, int d) { return max(0, d - (p.N - 1)); }
__device__ __forceinline__ int leaf_hi(const SolveParams& p, int d) { return min(d, p.M - 1); }

// offs / parts / counters indexing: parity of the diagonal, leaf slot, kind (0: p, 1: o)
__device__ __forceinline__ float* offs_ptr(const SolveParams& p, int par, int slot, int kind) {
    return p.offs + ((size_t)(par * p.maxleaf + slot) * 2 + kind) * (kB * kB);
}
__device__ __forceinline__ float* part_ptr(const SolveParams& p, int par, int slot, int kind,
                                           int c) {
    return p.parts + (((size_t)(par * p.maxleaf + slot) * 2 + kind) * kNch + c) * (kB * kB);
}
__device__ __forceinline__ int nchunks(int kblk, int cbk) { return kblk <= 0 ? 0 : (kblk + cbk - 1) / cbk; }

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

__global__ void k_solve_init(unsigned* counters, int ncounters, int* info) {
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < ncounters; e += gridDim.x * blockDim.x)
        counters[e] = 0u;
    if (blockIdx.x == 0 && threadIdx.x == 0) *info = INT_MAX;
}

// ---------------------------------------------------------------------------
// far-field GEMM role: one K-chunk of p (kind 0) or o^T (kind 1) of one leaf
// of diagonal d1, from blocks at least two leaves away
// ---------------------------------------------------------------------------
struct FarSmem {
    GemmSmem<float> g;
    int last;
};

__device__ void far_chunk(const SolveParams& p, int d1, int task, FarSmem& sm) {
    const int slot = task / (2 * kNch);
    const int kind = (task / kNch) & 1;
    const int c = task % kNch;
    const int I = leaf_lo(p, d1) + slot;
    const int J = d1 - I;
    if (I > leaf_hi(p, d1)) return;
    const int kblk = (kind == 0) ? I - 1 : J - 1;
    if ((kind == 0 && !p.LO) || (kind == 1 && !p.LI)) return;
    const int nv = nchunks(kblk, p.cbk);
    if (c >= nv) return;
    const int kb0 = c * p.cbk, kb1 = min(kb0 + p.cbk, kblk);
    const int64_t i0 = (int64_t)I * kB, j0 = (int64_t)J * kB;
    const int R = (int)min<int64_t>(kB, p.m - i0), Cc = (int)min<int64_t>(kB, p.n - j0);
    const int64_t k0 = (int64_t)kb0 * kB, K = (int64_t)(kb1 - kb0) * kB;
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    int rows, cols;
    if (kind == 0) {  // p[ii][jj] = sum_k L_O[k][i0+ii] D[k][j0+jj]
        tile_gemm_f32(p.LO + k0 * p.ldlo + i0, p.ldlo, R, p.delta + k0 * p.ldd + j0, p.ldd, Cc, K,
                      acc, sm.g);
        rows = R;
        cols = Cc;
    } else {  // o^T[jj][ii] = sum_l L_I[l][j0+jj] C^T[l][i0+ii]
        tile_gemm_f32(p.LI + k0 * p.ldli + j0, p.ldli, Cc, p.ct + k0 * p.m + i0, p.m, R, K, acc,
                      sm.g);
        rows = Cc;
        cols = R;
    }
    (void)rows;
    (void)cols;
    const int par = d1 & 1;
    float* part = part_ptr(p, par, slot, kind, c);
    const int cc = acc32_col();
#pragma unroll
    for (int v = 0; v < 16; ++v) part[acc32_row(v) * kB + cc] = acc[v];
    // deterministic reduction by the last chunk to finish
    __threadfence();
    __syncthreads();
    unsigned* ctr = p.counters + ((size_t)(par * p.maxleaf + slot) * 2 + kind);
    if (threadIdx.x == 0) sm.last = (atomicAdd(ctr, 1u) == (unsigned)(nv - 1));
    __syncthreads();
    if (!sm.last) return;
    __threadfence();
    float* out = offs_ptr(p, par, slot, kind);
    for (int e = threadIdx.x; e < kB * kB; e += kThreads) {
        float s = 0.0f;
        for (int q = 0; q < nv; ++q) s += part_ptr(p, par, slot, kind, q)[e];
        out[e] = s;
    }
    if (threadIdx.x == 0) *ctr = 0u;
}

// ---------------------------------------------------------------------------
// leaf role: solve the 64x64 leaf (I, J) of diagonal d
// ---------------------------------------------------------------------------
struct LeafSmem {
    union {
        GemmSmem<float> g;  // prologue GEMMs
        struct {
            float Ds[kB][kDs];  // D of the leaf (0 where not yet known)
            float Gs[kB][kGs];  // C of the leaf
        } w;
    } u;
    float LIs[kB][kLs];      // L_I diagonal block, strictly upper (0 elsewhere)
    float base[kB][kB + 1];  // W* + o
    float pin[kB][kB + 1];   // p
    float wst[kB][kB + 1];   // W*
    uint8_t code[kB][kB];
    float DI[kB];
    double red[kThreads];
    int red_i[kThreads];
};

__device__ void leaf_solve(const SolveParams& p, int d, int slot, LeafSmem& sm) {
    const int I = leaf_lo(p, d) + slot;
    const int J = d - I;
    const int64_t i0 = (int64_t)I * kB, j0 = (int64_t)J * kB;
    const int R = (int)min<int64_t>(kB, p.m - i0), Cc = (int)min<int64_t>(kB, p.n - j0);
    const int t = threadIdx.x;
    const int par = d & 1;
    const int cc = acc32_col();

    // ---- p: far part (precomputed) + adjacent block I-1 ----
    {
        f32x16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
        if (p.LO && I >= 1) {
            const int64_t k0 = i0 - kB;
            tile_gemm_f32(p.LO + k0 * p.ldlo + i0, p.ldlo, R, p.delta + k0 * p.ldd + j0, p.ldd, Cc,
                          kB, acc, sm.u.g);
        }
        const bool far = p.LO && nchunks(I - 1, p.cbk) > 0;
        const float* off = offs_ptr(p, par, slot, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = acc32_row(v);
            float x = acc[v];
            if (far) x += off[r * kB + cc];
            sm.pin[r][cc] = x;
        }
    }
    __syncthreads();
    // ---- o^T: far part + adjacent block J-1; base = W* + o ----
    {
        f32x16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
        if (p.LI && J >= 1) {
            const int64_t l0 = j0 - kB;
            tile_gemm_f32(p.LI + l0 * p.ldli + j0, p.ldli, Cc, p.ct + l0 * p.m + i0, p.m, R, kB,
                          acc, sm.u.g);
        }
        const bool far = p.LI && nchunks(J - 1, p.cbk) > 0;
        const float* off = offs_ptr(p, par, slot, 1);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int jj = acc32_row(v);  // o^T row = column of the leaf
            float x = acc[v];
            if (far) x += off[jj * kB + cc];
            sm.base[cc][jj] = x;  // cc = leaf row
        }
    }
    __syncthreads();
    // ---- LDS set-up for the wavefront ----
    for (int e = t; e < kB * kB; e += kThreads) {
        const int i = e / kB, j = e % kB;
        float wv = 0.0f;
        if (i < R && j < Cc) wv = p.W[(i0 + i) * p.ldw + j0 + j];
        sm.base[i][j] += wv;
        sm.wst[i][j] = wv;
        sm.u.w.Ds[i][j] = 0.0f;
        sm.u.w.Gs[i][j] = 0.0f;
        float l = 0.0f;
        if (p.LI && i < j && j < Cc) l = p.LI[(j0 + i) * p.ldli + j0 + j];
        sm.LIs[i][j] = l;
        sm.code[i][j] = 0;
    }
    if (t < kB) sm.DI[t] = (p.want_loss && t < Cc) ? p.DI[j0 + t] : 0.0f;

    const int i = t >> 2;  // leaf row of this thread
    const int q = t & 3;   // quarter of the in-leaf sums
    float lo_reg[16];      // L_O[i0 + 4r + q][i0 + i], strictly above the diagonal
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int k = 4 * r + q;
        lo_reg[r] = (p.LO && k < i && i < R) ? p.LO[(i0 + k) * p.ldlo + i0 + i] : 0.0f;
    }
    const int Lq = (1 << p.bits) - 1;
    const float half = 0.5f * (float)Lq;
    const float s = (i < R) ? p.scales[i0 + i] : 1.0f;
    const float dO = (p.want_loss && i < R) ? (p.DO ? p.DO[i0 + i] : 1.0f) : 0.0f;
    double loss = 0.0;
    int nclamp = 0;
    __syncthreads();

    // ---- in-leaf anti-diagonal wavefront: 2*64-1 dependent steps ----
    for (int st = 0; st < 2 * kB - 1; ++st) {
        const int j = st - i;
        const bool act = (j >= 0) && (j < kB);
        float pn = 0.0f, rn = 0.0f;
        if (act) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int k = 4 * r + q;
                pn = fmaf(lo_reg[r], sm.u.w.Ds[k][j], pn);
                rn = fmaf(sm.u.w.Gs[i][k], sm.LIs[k][j], rn);
            }
        }
        pn = quad_sum(pn);
        rn = quad_sum(rn);
        if (act && i < R && j < Cc) {
            const float P = sm.pin[i][j] + pn;
            const float tv = sm.base[i][j] + P + rn;
            const float y = tv / s + half;
            float cf;
            if (p.stochastic) {
                const float u = uniform24(p.seed, (uint64_t)(i0 + i) * (uint64_t)p.n + (uint64_t)(j0 + j));
                cf = floorf(y + u);
            } else {
                cf = floorf(y + 0.5f);
            }
            const bool clamp = (cf < 0.0f) || (cf > (float)Lq);
            cf = fminf(fmaxf(cf, 0.0f), (float)Lq);
            const float wv = sm.wst[i][j];
            const float dl = fmaf(-s, cf - half, wv);  // D = W* - s (c - Lq/2), one rounding
            if (q == 0) {
                sm.u.w.Ds[i][j] = dl;
                sm.u.w.Gs[i][j] = P + dl;
                sm.code[i][j] = (uint8_t)cf;
                const float eta = tv - s * (cf - half);
                loss += (double)dO * (double)sm.DI[j] * (double)eta * (double)eta;
                nclamp += clamp ? 1 : 0;
            }
        }
        __syncthreads();
    }

    // ---- outputs ----
    for (int e = t; e < kB * kB; e += kThreads) {
        const int ii = e / kB, jj = e % kB;
        if (ii < R && jj < Cc) {
            p.codes[(i0 + ii) * p.ldc + j0 + jj] = sm.code[ii][jj];
            p.delta[(i0 + ii) * p.ldd + j0 + jj] = sm.u.w.Ds[ii][jj];
        }
        const int ci = e % kB, cj = e / kB;  // C^T written along the leaf's rows
        if (ci < R && cj < Cc) p.ct[(j0 + cj) * p.m + i0 + ci] = sm.u.w.Gs[ci][cj];
    }
    if (p.want_loss) {
        sm.red[t] = loss;
        sm.red_i[t] = nclamp;
        __syncthreads();
        for (int o = kThreads / 2; o > 0; o >>= 1) {
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
    } else {
        sm.red_i[t] = nclamp;
        __syncthreads();
        for (int o = kThreads / 2; o > 0; o >>= 1) {
            if (t < o) sm.red_i[t] += sm.red_i[t + o];
            __syncthreads();
        }
        if (t == 0) {
            p.leaf_loss[(size_t)I * p.N + J] = 0.0;
            p.leaf_clamp[(size_t)I * p.N + J] = sm.red_i[0];
        }
    }
}

// One launch per leaf-diagonal d: workgroups [0, nleaf(d)) solve the leaves of
// d; the rest form the far-field chunks of diagonal d + 1.
__global__ __launch_bounds__(kThreads) void k_diag(SolveParams p, int d, int nleaf) {
    if (*p.info != INT_MAX) return;  // a row scale was invalid
    __shared__ union {
        LeafSmem leaf;
        FarSmem far;
    } sm;
    if ((int)blockIdx.x < nleaf) {
        leaf_solve(p, d, blockIdx.x, sm.leaf);
    } else {
        far_chunk(p, d + 1, blockIdx.x - nleaf, sm.far);
    }
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
    int M, N, maxleaf, cbk;
    size_t ct, delta, offs, parts, counters, leaf_loss, leaf_clamp, info, total;
};

Layout layout(int64_t m, int64_t n) {
    Layout L;
    L.M = (int)((m + kB - 1) / kB);
    L.N = (int)((n + kB - 1) / kB);
    L.maxleaf = std::min(L.M, L.N);
    const int kmax = std::max(L.M, L.N) - 2;
    L.cbk = std::max(1, (kmax + kNch - 1) / kNch);
    size_t o = 0;
    L.ct = o;
    o += align256(sizeof(float) * (size_t)m * (size_t)n);
    L.delta = o;
    o += align256(sizeof(float) * (size_t)m * (size_t)n);
    L.offs = o;
    o += align256(sizeof(float) * 2 * (size_t)L.maxleaf * 2 * kB * kB);
    L.parts = o;
    o += align256(sizeof(float) * 2 * (size_t)L.maxleaf * 2 * kNch * kB * kB);
    L.counters = o;
    o += align256(sizeof(unsigned) * 2 * (size_t)L.maxleaf * 2);
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
    p.offs = (float*)(base + L.offs);
    p.parts = (float*)(base + L.parts);
    p.counters = (unsigned*)(base + L.counters);
    p.leaf_loss = (double*)(base + L.leaf_loss);
    p.leaf_clamp = (int*)(base + L.leaf_clamp);
    p.DO = a.DO;
    p.DI = a.DI;
    p.want_loss = a.loss != nullptr;
    p.info = (int*)(base + L.info);
    p.maxleaf = L.maxleaf;
    p.cbk = L.cbk;

    const int ncnt = 2 * L.maxleaf * 2;
    hipLaunchKernelGGL(k_solve_init, dim3((ncnt + 255) / 256), dim3(256), 0, stream, p.counters,
                       ncnt, p.info);
    hipLaunchKernelGGL(k_scales, dim3((unsigned)a.m), dim3(kThreads), 0, stream, a.W, a.n, a.ldw,
                       a.bits, a.row_scale, a.scales, p.info);
    const int ndiag = L.M + L.N - 1;
    for (int d = 0; d < ndiag; ++d) {
        const int lo = std::max(0, d - (L.N - 1)), hi = std::min(d, L.M - 1);
        const int nleaf = hi - lo + 1;
        int nfar = 0;
        if (d + 1 < ndiag) {
            const int lo1 = std::max(0, d + 1 - (L.N - 1)), hi1 = std::min(d + 1, L.M - 1);
            nfar = (hi1 - lo1 + 1) * 2 * kNch;
        }
        hipLaunchKernelGGL(k_diag, dim3((unsigned)(nleaf + nfar)), dim3(kThreads), 0, stream, p, d,
                           nleaf);
    }
    hipLaunchKernelGGL(k_solve_finish, dim3(1), dim3(kThreads), 0, stream, p.leaf_loss,
                       p.leaf_clamp, L.M * L.N, a.loss, a.clamped, p.info, a.info);
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

}  // namespace bk
