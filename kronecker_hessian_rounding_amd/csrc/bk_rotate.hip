// bk_rotate.hip -- two-sided incoherence processing: randomised Hadamard rotations.
//
// The YAQA article (section 4) bounds the rounding error through the
// incoherence of H_O and H_I and asks, as for LDLQ, for both Hessians to be made
// incoherent before rounding; the KronQ page (method, bidirectional incoherence
// processing) extends the input-side random rotation to the output side,
// W' = R_O W R_I^T. The pages give no construction; the one used here is the
// randomised Hadamard transform. For a dimension n = 2^k r with r odd,
//   U_n = (I_r (x) H_{2^k} / sqrt(2^k)) diag(s),
// H the Sylvester Hadamard matrix (entry (i, j) = (-1)^popcount(i & j)), and
// s_i = -1 where the top bit of SplitMix64 output i of the seed is set, else +1.
// U_n is orthogonal and U_n^T = diag(s) (I_r (x) H_{2^k}) / sqrt(2^k).
//
// Both kernels work in place and are bound by HBM: every pass reads and writes
// the matrix once.
//  * Along each row (the transform index is the column): one workgroup per run
//    of whole 2^k-blocks of a row, up to 16384 floats, staged in LDS; all k
//    butterfly stages run there.
//  * Along each column (the index is the row): passes over up to 6 index bits.
//    Each lane of a wave owns one column and holds the 2^bits values of its
//    group in registers, so every load and store of a wave is 64 consecutive
//    floats of one row; the group's signs are drawn one per lane and shared by
//    a ballot.
#include <cmath>

#include "bk_common.hpp"
#include "bk_internal.hpp"

namespace bk {

constexpr int kRowMaxFloats = 16384;  // LDS staging of the row kernel (64 KB)
constexpr int kColPassBits = 6;

__device__ __forceinline__ float rht_sign(uint64_t seed, int64_t i) {
    return (splitmix64_out(seed, (uint64_t)i) >> 63) ? -1.0f : 1.0f;
}

// Workgroup (row, chunk): columns [chunk * cs, chunk * cs + len) of one row, a
// whole number of 2^kbits-blocks. U: signs, butterflies, scale; U^T: butterflies,
// scale, signs.
// kRowThreads grows with the chunk (one thread per 16 floats, 256 to 1024), so
// each butterfly stage between two barriers stays short.
template <int kRowThreads>
__global__ __launch_bounds__(kRowThreads) void k_rht_rows(float* __restrict__ A, int64_t cols, int64_t lda,
                                                          int64_t nchunk, int64_t cs, int kbits, uint64_t seed,
                                                          float scale, int transpose) {
    extern __shared__ float buf[];
    const int64_t row = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    const int64_t c0 = chunk * cs;
    const int len = (int)min<int64_t>(cs, cols - c0);
    float* p = A + row * lda + c0;
    for (int i = threadIdx.x; i < len; i += kRowThreads) {
        float v = p[i];
        if (!transpose) v *= rht_sign(seed, c0 + i);
        buf[i] = v;
    }
    __syncthreads();
    for (int s = 0; s < kbits; ++s) {
        const int h = 1 << s;
        for (int q = threadIdx.x; q < len / 2; q += kRowThreads) {
            const int lo = ((q >> s) << (s + 1)) | (q & (h - 1));
            const float a = buf[lo], b = buf[lo + h];
            buf[lo] = a + b;
            buf[lo + h] = a - b;
        }
        __syncthreads();
    }
    for (int i = threadIdx.x; i < len; i += kRowThreads) {
        float v = buf[i] * scale;
        if (transpose) v *= rht_sign(seed, c0 + i);
        p[i] = v;
    }
}

// One pass over index bits [b0, b0 + NB) of the row index, for every column.
// A group is the 2^NB rows of a 2^kbits-block that differ only in those bits;
// group g = (block, bits above, bits below). The last pass applies the scale.
// kSgn: 0, no signs in this pass; 1, signs on the loaded values (the first pass
// of U); 2, signs on the stored values (the last pass of U^T).
template <int NB, int kSgn>
__global__ __launch_bounds__(kThreads) void k_rht_cols(float* __restrict__ A, int64_t rows, int64_t cols,
                                                       int64_t lda, int kbits, int b0, uint64_t seed,
                                                       float scale, int last) {
    constexpr int kN = 1 << NB;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t c = ((int64_t)blockIdx.x * (kThreads / 64) + w) * 64 + lane;
    const bool in = c < cols;
    const int64_t G = rows >> NB;
    const int hib = kbits - b0 - NB;  // index bits above the pass
    for (int64_t g = blockIdx.y; g < G; g += gridDim.y) {
        const int64_t lo = g & (((int64_t)1 << b0) - 1);
        const int64_t rest = g >> b0;
        const int64_t hi = rest & (((int64_t)1 << hib) - 1);
        const int64_t blk = rest >> hib;
        const int64_t r0 = (blk << kbits) + (hi << (b0 + NB)) + lo;
        // the group's signs: lane j draws the sign of row j of the group, and the
        // ballot hands all of them to every lane
        uint64_t neg = 0;
        if (kSgn != 0)
            neg = __ballot((splitmix64_out(seed, (uint64_t)(r0 + ((int64_t)(lane & (kN - 1)) << b0))) >> 63) != 0);
        auto flip = [&](float x, int j) {
            return __uint_as_float(__float_as_uint(x) ^ ((uint32_t)(neg >> j) << 31));
        };
        float v[kN];
#pragma unroll
        for (int j = 0; j < kN; ++j) {
            const int64_t r = r0 + ((int64_t)j << b0);
            v[j] = in ? A[r * lda + c] : 0.0f;
        }
        if (kSgn == 1) {
            __builtin_amdgcn_sched_barrier(0);  // every load is in flight before the first sign waits on one
#pragma unroll
            for (int j = 0; j < kN; ++j) v[j] = flip(v[j], j);
        }
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
            for (int j = 0; j < kN; ++j)
                if ((j & (1 << s)) == 0) {
                    const float a = v[j], b = v[j | (1 << s)];
                    v[j] = a + b;
                    v[j | (1 << s)] = a - b;
                }
#pragma unroll
        for (int j = 0; j < kN; ++j) {
            const int64_t r = r0 + ((int64_t)j << b0);
            float x = last ? v[j] * scale : v[j];
            if (kSgn == 2) x = flip(x, j);
            if (in) A[r * lda + c] = x;
        }
    }
}

namespace {
template <int NB>
void col_pass(float* A, int64_t rows, int64_t cols, int64_t lda, int kbits, int b0, uint64_t seed, float scale,
              int first, int last, int transpose, hipStream_t stream) {
    const int64_t G = rows >> NB;
    const dim3 grid((unsigned)((cols + kThreads - 1) / kThreads), (unsigned)std::min<int64_t>(G, 65535));
    const int sgn = (first && !transpose) ? 1 : (last && transpose) ? 2 : 0;
    if (sgn == 1)
        hipLaunchKernelGGL((k_rht_cols<NB, 1>), grid, dim3(kThreads), 0, stream, A, rows, cols, lda, kbits, b0,
                           seed, scale, last);
    else if (sgn == 2)
        hipLaunchKernelGGL((k_rht_cols<NB, 2>), grid, dim3(kThreads), 0, stream, A, rows, cols, lda, kbits, b0,
                           seed, scale, last);
    else
        hipLaunchKernelGGL((k_rht_cols<NB, 0>), grid, dim3(kThreads), 0, stream, A, rows, cols, lda, kbits, b0,
                           seed, scale, last);
}
}  // namespace

int launch_rht(float* A, int64_t rows, int64_t cols, int64_t lda, int axis, uint64_t seed, int transpose,
               hipStream_t stream) {
    const int64_t n = axis == 0 ? rows : cols;
    int kbits = 0;
    while (((n >> kbits) & 1) == 0) ++kbits;  // n > 0
    const int64_t b = (int64_t)1 << kbits;
    const float scale = (float)(1.0 / std::sqrt((double)b));
    if (axis == 1) {
        if (b > kRowMaxFloats) return BAKRON_E_INVALID_ARG;
        const int64_t cs = b * (kRowMaxFloats / b < cols / b ? kRowMaxFloats / b : cols / b);
        const int64_t nchunk = (cols + cs - 1) / cs;
        if (rows * nchunk > 0x7fffffff) return BAKRON_E_INVALID_ARG;
        const dim3 grid((unsigned)(rows * nchunk));
        const size_t lds = sizeof(float) * cs;
        if (cs > 8192)
            hipLaunchKernelGGL(k_rht_rows<1024>, grid, dim3(1024), lds, stream, A, cols, lda, nchunk, cs, kbits,
                               seed, scale, transpose);
        else if (cs > 4096)
            hipLaunchKernelGGL(k_rht_rows<512>, grid, dim3(512), lds, stream, A, cols, lda, nchunk, cs, kbits,
                               seed, scale, transpose);
        else
            hipLaunchKernelGGL(k_rht_rows<256>, grid, dim3(256), lds, stream, A, cols, lda, nchunk, cs, kbits,
                               seed, scale, transpose);
    } else {
        // passes of at most 6 bits, as even as possible
        const int npass = kbits == 0 ? 1 : (kbits + kColPassBits - 1) / kColPassBits;
        int b0 = 0;
        for (int ps = 0; ps < npass; ++ps) {
            const int nb = kbits / npass + (ps < kbits % npass ? 1 : 0);
            const int first = ps == 0, last = ps == npass - 1;
            switch (nb) {
                case 0: col_pass<0>(A, rows, cols, lda, kbits, b0, seed, scale, first, last, transpose, stream); break;
                case 1: col_pass<1>(A, rows, cols, lda, kbits, b0, seed, scale, first, last, transpose, stream); break;
                case 2: col_pass<2>(A, rows, cols, lda, kbits, b0, seed, scale, first, last, transpose, stream); break;
                case 3: col_pass<3>(A, rows, cols, lda, kbits, b0, seed, scale, first, last, transpose, stream); break;
                case 4: col_pass<4>(A, rows, cols, lda, kbits, b0, seed, scale, first, last, transpose, stream); break;
                case 5: col_pass<5>(A, rows, cols, lda, kbits, b0, seed, scale, first, last, transpose, stream); break;
                default: col_pass<6>(A, rows, cols, lda, kbits, b0, seed, scale, first, last, transpose, stream); break;
            }
            b0 += nb;
        }
    }
    return hipGetLastError() == hipSuccess ? BAKRON_OK : BAKRON_E_DEVICE;
}

}  // namespace bk
