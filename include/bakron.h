/*
 * bakron.h -- C ABI of libbakron, a gfx950 (MI355X) implementation of BaKron:
 * two-sided adaptive rounding of a weight matrix under a Kronecker-factored
 * Hessian H_O (x) H_I.
 *
 * Sources (web pages, cited by title and section):
 *   "BaKron: Efficient Quantization with Kronecker-Factored Hessians"
 *       (insight.aitobox.com), Abstract: the solver schedules the two-sided
 *       rounding rule with anti-diagonal parallelism and a recursive
 *       divide-and-conquer so that it takes O(m+n) sequential steps and
 *       O(mn(m+n)) work, and is modular in the base quantiser and in the
 *       Hessian estimator.
 *   YAQA article (news.43b.com.cn/a/479517), section 4: the rounding rule
 *       W_ij = Q(W*_ij + a_i^T D[:i,:j] b_j + a_i^T D[:i,j] + D[i,:j] b_j)
 *       with a_i, b_j columns of the strictly upper L_O, L_I and D = W* - W;
 *       the factorisation H = (L + I) D (L + I)^T; the error bound.
 *   YAQA article, section 3, and the K-FAC tutorial (www.mlqm.cn), section 5:
 *       the factor estimates H_I = E[x^T x], H_O = E[g^T g] and damping; the
 *       YAQA article's Sketch A and Sketch B estimators (section 3).
 *   "KronQ: Kronecker-factored Hessian LLM quantization" (ai-feeds.com),
 *       method: bidirectional incoherence processing, W' = R_O W R_I^T, and
 *       the layer sensitivity tr(A) tr(G).
 *
 * Conventions for every entry point:
 *   - All matrix and vector pointers are DEVICE pointers (memory of the
 *     current HIP device) unless a parameter says "host". Matrices are
 *     row-major with a leading dimension (ld, in elements) >= the number of
 *     columns. No alignment is required.
 *   - The caller owns every buffer, including the workspace; the library
 *     never allocates, frees or retains memory and keeps no state between
 *     calls. Calls on different streams may run concurrently. The one
 *     exception is bakron_solve_noalloc, which works in a fixed scratch array
 *     that the library holds on each device (see there).
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream). Only bakron_ldl waits for its work to finish (bakron_ldl_async
 *     does not).
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid argument returns BAKRON_E_INVALID_ARG and enqueues nothing.
 *     A failed launch returns BAKRON_E_DEVICE. No C++ exception crosses the
 *     ABI.
 */
#ifndef BAKRON_H
#define BAKRON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BAKRON_ABI_VERSION 1

enum {
    BAKRON_OK = 0,
    BAKRON_E_INVALID_ARG = 1, /* bad pointer, size, leading dimension or option */
    BAKRON_E_NOT_SPD = 2,     /* bakron_ldl: a pivot was not positive (or not finite) */
    BAKRON_E_WORKSPACE = 3,   /* workspace pointer NULL or smaller than required */
    BAKRON_E_DEVICE = 4       /* a HIP call or kernel launch failed */
};

enum { BAKRON_ROUND_NEAREST = 0, BAKRON_ROUND_STOCHASTIC = 1 };

/*
 * Base quantiser Q (the solver is modular in it: BaKron Abstract; YAQA
 * section 4 names nearest and stochastic rounding).
 *   Grid of row i: s_i * (c - Lq/2), c in {0, ..., Lq}, Lq = 2^bits - 1.
 *   y = t / s_i + Lq/2 is the pre-rounding value t in grid steps.
 *   NEAREST:    c = clamp(floor(y + 1/2), 0, Lq)
 *   STOCHASTIC: c = clamp(floor(y + u_ij), 0, Lq), u_ij = (z >> 40) * 2^-24 with
 *               z = SplitMix64 output number i*n + j + 1 of a stream seeded
 *               with `seed` (independent of the order entries are visited).
 *   row_scale:  device [m] fp32 scales, all finite and > 0; NULL means
 *               s_i = fp32(2 * max_j |W*_ij|) / fp32(Lq), computed in fp32.
 */
typedef struct {
    int32_t bits;          /* 1..8 */
    int32_t rounding;      /* BAKRON_ROUND_NEAREST or BAKRON_ROUND_STOCHASTIC */
    uint64_t seed;         /* stochastic rounding only */
    const float* row_scale;/* device, [m], or NULL */
} bakron_quantizer;

/* Returns BAKRON_ABI_VERSION of the built library. */
int bakron_abi_version(void);

/* Static string describing a status code (never NULL). */
const char* bakron_status_str(int status);

/*
 * Hessian factor accumulation (YAQA section 3: H_I = E[x^T x]; the same form
 * gives H_O from output gradients):  H <- beta * H + alpha * X^T X.
 *   X: T x d fp32, leading dimension ldx >= d (rows are tokens).
 *   H: d x d fp32, ldh >= d. The full symmetric matrix is written (both
 *      triangles, bit-identical mirror). With beta == 0, H is not read.
 *   For H = X^T X / T pass alpha = 1/T, beta = 0; to accumulate over token
 *   chunks call again with beta = 1 and alpha = 1/T_total.
 *   T == 0 scales H by beta.
 *   ws: optional device workspace; its size picks the arithmetic.
 *      - At least bakron_hessian_accum_workspace_bytes(T, d) bytes: the
 *        product runs on the fp16 matrix cores. Each column c of X is scaled
 *        by a power of two 2^e_c that puts its largest magnitude in
 *        [2^14, 2^15), and each scaled element is cut into two fp16 pieces
 *        (x' = h + l to within 2^-22 |x'| for |x'| >= 2^-3, i.e. within 2^17
 *        of the column's largest magnitude; an absolute 2^-25 below that),
 *        stored in ws: 4 bytes per element of X, with T padded to a multiple
 *        of 32 and d to a multiple of 128, then the exponents and the
 *        column-maximum partials. Each product is the sum of three piece
 *        products (hh, hl, lh), exact in fp32 and accumulated in fp32, then
 *        scaled back by 2^-(e_i + e_j). The term left out is below
 *        2^-22 |x y|, so the error is of the order of an fp32 product's.
 *        The remainder of ws (after the pieces, 256-byte aligned) holds the
 *        split-K partials of a short last round of output tiles.
 *      - NULL or smaller: the product runs on the fp32 matrix cores (2.3x
 *        slower at T = 32768, d = 4096, 3.2x with no workspace at all). A
 *        workspace too small for the pieces is still used for those split-K
 *        partials if it is large enough.
 *      Both paths are within fp32 rounding of X^T X, but their results are
 *      not bit-identical. For a given device, T, d and path the result is
 *      deterministic.
 * Errors: INVALID_ARG for NULL X (T > 0) or H, d <= 0, T < 0, bad ld.
 */
size_t bakron_hessian_accum_workspace_bytes(int64_t T, int64_t d);
int bakron_hessian_accum(const float* X, int64_t T, int64_t d, int64_t ldx, float alpha,
                         float beta, float* H, int64_t ldh, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * The same accumulation with X stored d x T (one row per output index, the
 * contraction along the rows): H <- beta * H + alpha * X X^T. With X the m x n
 * weight gradient G_s of one sequence this gives the output-side term of
 * Sketch B (YAQA article, section 3: H_O = E_s[G_s G_s^T] / n, alpha = 1/(S n));
 * the input-side term E_s[G_s^T G_s] / m is bakron_hessian_accum with T = m.
 *   X: d x T fp32, ldx >= T. H: d x d fp32, ldh >= d, both triangles written.
 *   ws: at least bakron_hessian_accum_workspace_bytes(T, d) bytes (this form
 *       runs on the fp16 piece path only).
 * Errors: INVALID_ARG as for bakron_hessian_accum (with ldx >= T);
 * WORKSPACE if ws is NULL or too small.
 */
int bakron_hessian_accum_t(const float* X, int64_t T, int64_t d, int64_t ldx, float alpha,
                           float beta, float* H, int64_t ldh, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Sketch A (YAQA article, section 3) alternates the two factors, each token
 * weighted by the other factor's quadratic form:
 *   (H_I)_i = E_t[x_t^T x_t w_t], w_t = g_t (H_O)_{i-1} g_t^T / ||(H_O)_{i-1}||_F^2,
 * and likewise (H_O)_i with v_t = x_t (H_I)_{i-1} x_t^T / ||(H_I)_{i-1}||_F^2.
 *
 * bakron_token_weights: w[t] = y_t H y_t^T / ||H||_F^2 for the rows y_t of Y
 *   (T x d, ldy >= d), H d x d symmetric (ldh >= d); H == NULL means H = I,
 *   w[t] = ||y_t||^2 / d. The quadratic forms read H's lower triangle and
 *   diagonal only (y H y^T = sum of the diagonal blocks' forms plus twice those
 *   of the blocks below them), as fp32 MFMA tile GEMMs summed in a fixed order;
 *   ||H||_F^2 reads all of H, in fp64. ws: with H given, at least
 *   bakron_token_weights_workspace_bytes(T, d) (Y transposed, d T floats).
 * bakron_hessian_accum_w: H <- beta H + alpha sum_t w[t] x_t^T x_t for w >= 0
 *   (negative weights count as 0), X as in bakron_hessian_accum, on the
 *   fp16 piece path (ws at least bakron_hessian_accum_workspace_bytes(T, d)).
 * Errors: INVALID_ARG for NULL pointers, d <= 0, T < 0, bad ld; WORKSPACE for a
 * missing or short workspace.
 */
/*
 * The transposed form over a batch: H <- beta H + alpha sum_s X_s X_s^T for S
 * matrices X_s (d x tin, ldx >= tin) at X + s * bs (bs >= d * ldx when S > 1),
 * accumulated as one call with T = S tin tokens. With X_s the gradients G_s of
 * S sequences (an S x m x n tensor: d = m, tin = n, bs = m n) this is the whole
 * output-side term of Sketch B. ws: bakron_hessian_accum_workspace_bytes(S tin, d).
 * Errors: INVALID_ARG for NULL pointers, d <= 0, S or tin < 0, bad ld or
 * overlapping batch stride; WORKSPACE for a missing or short workspace.
 */
int bakron_hessian_accum_tb(const float* X, int64_t S, int64_t d, int64_t tin, int64_t ldx, int64_t bs,
                            float alpha, float beta, float* H, int64_t ldh, void* ws, size_t ws_bytes,
                            void* stream);

size_t bakron_token_weights_workspace_bytes(int64_t T, int64_t d);
int bakron_token_weights(const float* Y, int64_t T, int64_t d, int64_t ldy, const float* H, int64_t ldh,
                         float* w, void* ws, size_t ws_bytes, void* stream);
int bakron_hessian_accum_w(const float* X, int64_t T, int64_t d, int64_t ldx, const float* w, float alpha,
                           float beta, float* H, int64_t ldh, void* ws, size_t ws_bytes, void* stream);

/*
 * Damped LDL factorisation (YAQA section 4): with lambda = damp_rel * mean(diag H)
 * (the mean of the undamped diagonal, in fp64), factor
 *     H + lambda I = (L + I) diag(D) (L + I)^T,  L strictly UPPER triangular,
 * i.e. a Cholesky factorisation taken from the last index to the first. The
 * work is done in fp64 on the device; results are rounded to fp32.
 *   H: d x d fp32, ldh >= d; only the upper triangle (with the diagonal) is
 *      read. On return H holds L in its strict upper triangle, D on its
 *      diagonal and zeros in its strict lower triangle.
 *   D: device [d] fp32 copy of D, or NULL.
 *   damp_rel: finite, >= 0 (fp64).
 *   bad_pivot: HOST pointer or NULL; receives -1, or on BAKRON_E_NOT_SPD the
 *      index j of the first pivot (taken from the last index down) that was
 *      not positive and finite. H is then unspecified.
 *   ws: device workspace of at least bakron_ldl_workspace_bytes(d) bytes.
 * This call waits for the stream so that NOT_SPD can be reported.
 * Orders up to 8192 are factored by one persistent launch whose workgroups wait
 * on each other's progress, each wait bounded (10 s of wall clock; the
 * environment variable BAKRON_LDL_WAIT_LIMIT_US, read at each call, lowers it so
 * that tests can reach this path): a wait that runs past it stops the launch,
 * and the call returns BAKRON_E_DEVICE with *bad_pivot = -2. BAKRON_LDL_PATH =
 * "launch", read at each call, makes such orders take the chain of launches that
 * larger orders take (for tests).
 */
size_t bakron_ldl_workspace_bytes(int64_t d);
int bakron_ldl(float* H, int64_t d, int64_t ldh, double damp_rel, float* D, int64_t* bad_pivot,
               void* ws, size_t ws_bytes, void* stream);

/*
 * The same factorisation, enqueued on `stream` without waiting (the damped LDL
 * of YAQA section 4, as above). Independent factorisations, such as H_I and H_O
 * of one layer, can then run side by side on two streams: each is a chain of
 * small launches that leaves most of the GPU idle.
 *   bad_pivot_dev: DEVICE int64 (required); when the stream reaches it, it holds
 *      -1, or the index of the first pivot that was not positive and finite (H is
 *      then unspecified), or -2 if a wait between workgroups ran past its limit
 *      (see bakron_ldl). The return value reports only argument, workspace and
 *      launch errors.
 *   ws: as for bakron_ldl; it and H, D stay in use until the stream has passed
 *      the call.
 */
int bakron_ldl_async(float* H, int64_t d, int64_t ldh, double damp_rel, float* D,
                     int64_t* bad_pivot_dev, void* ws, size_t ws_bytes, void* stream);

/*
 * Two independent damped LDL factorisations (YAQA section 4, as above: H_I and
 * H_O of one layer) enqueued without waiting. When both orders are at most 8192
 * (and BAKRON_LDL_PATH is not "launch") they share one persistent launch on
 * stream_a, whose workgroups serve both chains of diagonal blocks alike, and
 * nothing is enqueued on stream_b. Otherwise A is factored on stream_a and B on
 * stream_b, side by side, both by the chain of launches (a persistent launch for
 * the smaller one would hold a slot on every compute unit that the larger one's
 * updates need). The caller orders stream_b after earlier work and stream_a after
 * stream_b as it needs; stream_b may equal stream_a. Each other argument is as
 * for bakron_ldl_async, per matrix; damp_rel applies to both. A failure of one
 * (bad pivot, or -2) leaves the other's result intact.
 */
int bakron_ldl_pair_async(float* HA, int64_t dA, int64_t ldha, float* DA, int64_t* bad_pivot_dev_A,
                          void* wsA, size_t wsA_bytes, float* HB, int64_t dB, int64_t ldhb, float* DB,
                          int64_t* bad_pivot_dev_B, void* wsB, size_t wsB_bytes, double damp_rel,
                          void* stream_a, void* stream_b);

/*
 * BaKron solve: round W* (m x n) under H_O (x) H_I given the strict upper LDL
 * factors, entry (i, j) receiving the feedback
 *     a_i^T D[:i,:j] b_j + a_i^T D[:i,j] + D[i,:j] b_j
 * from the error D = W* - W already committed (YAQA section 4), scheduled as
 * a wavefront over 64x64 leaves (anti-diagonal parallelism, BaKron Abstract)
 * whose far-field feedback is formed by MFMA GEMMs.
 *   W:     m x n fp32, ldw >= n.
 *   L_O:   m x m fp32 (ldlo >= m); only the strict upper triangle is read.
 *          NULL means H_O = I up to scale (one-sided LDLQ / GPTQ).
 *   L_I:   n x n fp32 (ldli >= n); strict upper triangle read; NULL means a
 *          diagonal H_I.
 *   q:     quantiser descriptor (host pointer), see above.
 *   codes: m x n uint8 codes c_ij, ldc >= n.
 *   scales_out: [m] fp32, receives the scales used.
 *   delta_out:  optional m x n fp32 (ldd >= n), receives D = W* - s (c - Lq/2).
 *   D_O, D_I, loss_out: if loss_out (device, 1 double) is not NULL it receives
 *          the proxy loss sum_ij D_O,i D_I,j eta_ij^2 with eta = t - q, which
 *          equals tr(D H_I D^T H_O) for the damped factors; D_I [n] is then
 *          required and D_O [m] may be NULL only if L_O is NULL (D_O = 1).
 *   clamped_out: optional device int64 count of entries whose code was clamped.
 *   info:  optional device int32; 0, or i+1 for the first row i whose scale is
 *          not finite and positive, or -1 if one of the solve's internal waits
 *          between workgroups ran past its limit (10 s of wall clock; the
 *          environment variable BAKRON_SOLVE_WAIT_LIMIT_US, read at each call,
 *          lowers it so that tests can reach this path); in both cases the
 *          outputs are unspecified.
 *   ws:    device workspace of at least bakron_solve_workspace_bytes(m, n).
 */
size_t bakron_solve_workspace_bytes(int64_t m, int64_t n);
int bakron_solve(const float* W, int64_t m, int64_t n, int64_t ldw, const float* L_O, int64_t ldlo,
                 const float* L_I, int64_t ldli, const bakron_quantizer* q, uint8_t* codes,
                 int64_t ldc, float* scales_out, float* delta_out, int64_t ldd, const float* D_O,
                 const float* D_I, double* loss_out, int64_t* clamped_out, int32_t* info,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * solve as bakron_solve, with the same arguments, outputs and errors, but its
 * workspace is a scratch array of BAKRON_NOALLOC_SCRATCH_BYTES that the
 * library holds in device memory (one per device, from the moment the library
 * is loaded on it until the process ends) instead of a caller's buffer. The
 * call allocates nothing: no hipMalloc, no hipFree, no allocating library
 * routine.
 *   Sizes: bakron_solve_workspace_bytes(m, n) must not exceed
 *      BAKRON_NOALLOC_SCRATCH_BYTES, 128 MiB (for example m = n = 2048, or
 *      m = 1024 with n up to 3072); larger shapes return BAKRON_E_WORKSPACE
 *      before anything is enqueued.
 *   Sharing: every call on a device uses that device's one array, which keeps
 *      the last call's contents (the solve clears what must start at zero).
 *      Calls that overlap on one device -- on two streams, or from two host
 *      threads -- race on it; calls in one stream are ordered and safe.
 *   Errors: those of bakron_solve (INVALID_ARG, WORKSPACE as above), and
 *      BAKRON_E_DEVICE if the scratch array's address cannot be obtained on
 *      the current device.
 */
#define BAKRON_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int bakron_solve_noalloc(const float* W, int64_t m, int64_t n, int64_t ldw, const float* L_O, int64_t ldlo,
                         const float* L_I, int64_t ldli, const bakron_quantizer* q, uint8_t* codes,
                         int64_t ldc, float* scales_out, float* delta_out, int64_t ldd, const float* D_O,
                         const float* D_I, double* loss_out, int64_t* clamped_out, int32_t* info,
                         void* stream);

/*
 * Randomised Hadamard rotation, for two-sided incoherence processing before
 * the LDL and the solve (YAQA article, section 4: both Hessians are made
 * incoherent before rounding, as for LDLQ; KronQ page, method, bidirectional
 * incoherence processing: W' = R_O W R_I^T). In place on a rows x cols fp32
 * matrix A (device, row-major, lda >= cols):
 *   axis 0: A <- U_rows A      (every column is rotated; U of order rows)
 *   axis 1: A <- A U_cols^T    (every row is rotated; U of order cols)
 *   transpose != 0 applies U^T instead of U (the inverse rotation).
 * U_n = (I_r (x) H_b / sqrt(b)) diag(s): b is the largest power of two dividing
 * n, r = n / b, H_b the Sylvester Hadamard matrix (entry (i, j) =
 * (-1)^popcount(i & j)), and s_i = -1 where bit 63 of SplitMix64 output i of
 * `seed` (the generator of the stochastic rounding) is set, else +1.
 * A layer is rotated as W' = U_O W U_I^T (axis 0 with seed_O, then axis 1 with
 * seed_I), H_I' = U_I H_I U_I^T and H_O' = U_O H_O U_O^T (both axes, one seed);
 * the proxy loss of any rounding is unchanged, and the rounded W' maps back as
 * U_O^T W' U_I. Computed in fp32: every pass reads and writes A once.
 * Errors: INVALID_ARG for NULL A, rows or cols <= 0, lda < cols, axis other
 * than 0 or 1, or (axis 1) b > 16384.
 */
int bakron_rht(float* A, int64_t rows, int64_t cols, int64_t lda, int axis, uint64_t seed, int transpose,
               void* stream);

/*
 * Per-layer bound and sensitivity report, written to out (device, 7 doubles)
 * by one workgroup summing in fp64:
 *   out[0] = tr(D_O), out[1] = tr(D_I)   (the LDL pivots; D_O NULL means H_O = I: m)
 *   out[2] = sum_i D_O,i s_i^2 / 4 * tr(D_I)
 *            (YAQA article, section 4: the loss bound with |eta_ij| <= s_i / 2,
 *            which holds for nearest rounding when no code was clamped)
 *   out[3] = tr(D_I) tr(D_O) max_i s_i^2 / 4   (the bound in the page's form)
 *   out[4] = tr(H_I), out[5] = tr(H_O)   (NaN where H_I / H_O is NULL). Pass the
 *            factors before bakron_ldl, which writes D over their diagonal.
 *   out[6] = out[4] * out[5], the KronQ page's layer sensitivity tr(A) tr(G).
 *   scales: [m] the row scales the solve used (scales_out).
 * Errors: INVALID_ARG for m or n <= 0, NULL D_I, scales or out, bad ld.
 */
int bakron_layer_report(int64_t m, int64_t n, const float* D_O, const float* D_I, const float* scales,
                        const float* H_I, int64_t ldhi, const float* H_O, int64_t ldho, double* out,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BAKRON_H */
