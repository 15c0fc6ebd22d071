// bk_api.hip -- the extern "C" entry points of libbakron: argument validation on
// the host, workspace checks, then dispatch to the kernel drivers. Every check
// happens before anything is enqueued, so an invalid call enqueues no work.
#include <mutex>

#include "bk_internal.hpp"

namespace {

bool bad_ld(int64_t ld, int64_t cols) { return ld < cols || ld <= 0; }

// The solve's workspace for callers that cannot allocate (bakron_solve_noalloc):
// one array per device, held from the moment the library is loaded on it. In
// host code `scratch` is only a stand-in for the symbol; its device address is
// taken once per device with hipGetSymbolAddress and used from then on.
__device__ __align__(256) unsigned char scratch[BAKRON_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device, or nullptr.
void* scratch_address() {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

// Host-side checks of the solve's arguments (shared by both solve entry points).
int check_solve_args(const float* W, int64_t m, int64_t n, int64_t ldw, const float* L_O, int64_t ldlo,
                     const float* L_I, int64_t ldli, const bakron_quantizer* q, const uint8_t* codes,
                     int64_t ldc, const float* scales_out, const float* delta_out, int64_t ldd,
                     const float* D_O, const float* D_I, const double* loss_out) {
    if (!W || !q || !codes || !scales_out) return BAKRON_E_INVALID_ARG;
    if (m <= 0 || n <= 0 || bad_ld(ldw, n) || bad_ld(ldc, n)) return BAKRON_E_INVALID_ARG;
    if (m > (int64_t)1 << 30 || n > (int64_t)1 << 30) return BAKRON_E_INVALID_ARG;
    if (L_O && bad_ld(ldlo, m)) return BAKRON_E_INVALID_ARG;
    if (L_I && bad_ld(ldli, n)) return BAKRON_E_INVALID_ARG;
    if (delta_out && bad_ld(ldd, n)) return BAKRON_E_INVALID_ARG;
    if (q->bits < 1 || q->bits > 8) return BAKRON_E_INVALID_ARG;
    if (q->rounding != BAKRON_ROUND_NEAREST && q->rounding != BAKRON_ROUND_STOCHASTIC)
        return BAKRON_E_INVALID_ARG;
    if (loss_out && (!D_I || (!D_O && L_O))) return BAKRON_E_INVALID_ARG;
    return BAKRON_OK;
}

bk::SolveArgs solve_args(const float* W, int64_t m, int64_t n, int64_t ldw, const float* L_O, int64_t ldlo,
                         const float* L_I, int64_t ldli, const bakron_quantizer* q, uint8_t* codes,
                         int64_t ldc, float* scales_out, float* delta_out, int64_t ldd, const float* D_O,
                         const float* D_I, double* loss_out, int64_t* clamped_out, int32_t* info) {
    bk::SolveArgs a;
    a.W = W;
    a.m = m;
    a.n = n;
    a.ldw = ldw;
    a.LO = L_O;
    a.ldlo = ldlo;
    a.LI = L_I;
    a.ldli = ldli;
    a.bits = q->bits;
    a.stochastic = q->rounding == BAKRON_ROUND_STOCHASTIC;
    a.seed = q->seed;
    a.row_scale = q->row_scale;
    a.codes = codes;
    a.ldc = ldc;
    a.scales = scales_out;
    a.delta = delta_out;
    a.ldd = ldd;
    a.DO = D_O;
    a.DI = D_I;
    a.loss = loss_out;
    a.clamped = clamped_out;
    a.info = info;
    return a;
}

}  // namespace

extern "C" {

int bakron_abi_version(void) { return BAKRON_ABI_VERSION; }

const char* bakron_status_str(int status) {
    switch (status) {
        case BAKRON_OK: return "ok";
        case BAKRON_E_INVALID_ARG: return "invalid argument";
        case BAKRON_E_NOT_SPD: return "matrix is not positive definite";
        case BAKRON_E_WORKSPACE: return "workspace missing or too small";
        case BAKRON_E_DEVICE: return "HIP runtime or kernel launch failure";
        default: return "unknown status";
    }
}

size_t bakron_hessian_accum_workspace_bytes(int64_t T, int64_t d) {
    if (d <= 0 || T < 0) return 0;
    return bk::hessian_workspace_bytes(T, d);
}

int bakron_hessian_accum(const float* X, int64_t T, int64_t d, int64_t ldx, float alpha,
                         float beta, float* H, int64_t ldh, void* ws, size_t ws_bytes,
                         void* stream) {
    if (!H || d <= 0 || T < 0 || bad_ld(ldh, d)) return BAKRON_E_INVALID_ARG;
    if (T > 0 && (!X || bad_ld(ldx, d))) return BAKRON_E_INVALID_ARG;
    return bk::launch_hessian_accum(X, T, d, ldx, alpha, beta, H, ldh, ws, ws_bytes,
                                    (hipStream_t)stream);
}

int bakron_hessian_accum_t(const float* X, int64_t T, int64_t d, int64_t ldx, float alpha,
                           float beta, float* H, int64_t ldh, void* ws, size_t ws_bytes,
                           void* stream) {
    if (!H || d <= 0 || T < 0 || bad_ld(ldh, d)) return BAKRON_E_INVALID_ARG;
    if (T > 0 && (!X || bad_ld(ldx, T))) return BAKRON_E_INVALID_ARG;
    if (!ws || ws_bytes < bk::hessian_workspace_bytes(T, d)) return BAKRON_E_WORKSPACE;
    return bk::launch_hessian_accum(X, T, d, ldx, alpha, beta, H, ldh, ws, ws_bytes,
                                    (hipStream_t)stream, true);
}

int bakron_hessian_accum_tb(const float* X, int64_t S, int64_t d, int64_t tin, int64_t ldx, int64_t bs,
                            float alpha, float beta, float* H, int64_t ldh, void* ws, size_t ws_bytes,
                            void* stream) {
    if (!H || d <= 0 || S < 0 || tin < 0 || bad_ld(ldh, d)) return BAKRON_E_INVALID_ARG;
    const int64_t T = S * tin;
    if (T > 0 && (!X || bad_ld(ldx, tin) || (S > 1 && bs < d * ldx))) return BAKRON_E_INVALID_ARG;
    if (!ws || ws_bytes < bk::hessian_workspace_bytes(T, d)) return BAKRON_E_WORKSPACE;
    return bk::launch_hessian_accum(X, T, d, ldx, alpha, beta, H, ldh, ws, ws_bytes, (hipStream_t)stream,
                                    true, nullptr, tin, bs);
}

int bakron_hessian_accum_w(const float* X, int64_t T, int64_t d, int64_t ldx, const float* w, float alpha,
                           float beta, float* H, int64_t ldh, void* ws, size_t ws_bytes, void* stream) {
    if (!H || d <= 0 || T < 0 || bad_ld(ldh, d)) return BAKRON_E_INVALID_ARG;
    if (T > 0 && (!X || !w || bad_ld(ldx, d))) return BAKRON_E_INVALID_ARG;
    if (!ws || ws_bytes < bk::hessian_workspace_bytes(T, d)) return BAKRON_E_WORKSPACE;
    return bk::launch_hessian_accum(X, T, d, ldx, alpha, beta, H, ldh, ws, ws_bytes, (hipStream_t)stream,
                                    false, w);
}

size_t bakron_token_weights_workspace_bytes(int64_t T, int64_t d) {
    if (d <= 0 || T < 0) return 0;
    return bk::token_weights_workspace_bytes(T, d);
}

int bakron_token_weights(const float* Y, int64_t T, int64_t d, int64_t ldy, const float* H, int64_t ldh,
                         float* w, void* ws, size_t ws_bytes, void* stream) {
    if (d <= 0 || T < 0 || (T > 0 && (!Y || !w || bad_ld(ldy, d))) || (H && bad_ld(ldh, d)))
        return BAKRON_E_INVALID_ARG;
    return bk::launch_token_weights(Y, T, d, ldy, H, ldh, w, ws, ws_bytes, (hipStream_t)stream);
}

size_t bakron_ldl_workspace_bytes(int64_t d) {
    if (d <= 0) return 0;
    return bk::ldl_workspace_bytes(d);
}

int bakron_ldl(float* H, int64_t d, int64_t ldh, double damp_rel, float* D, int64_t* bad_pivot,
               void* ws, size_t ws_bytes, void* stream) {
    if (bad_pivot) *bad_pivot = -1;
    if (!H || d <= 0 || bad_ld(ldh, d)) return BAKRON_E_INVALID_ARG;
    if (!(damp_rel >= 0.0) || !(damp_rel < INFINITY)) return BAKRON_E_INVALID_ARG;
    if (!ws || ws_bytes < bk::ldl_workspace_bytes(d)) return BAKRON_E_WORKSPACE;
    return bk::run_ldl(H, d, ldh, damp_rel, D, bad_pivot, ws, (hipStream_t)stream);
}

int bakron_ldl_async(float* H, int64_t d, int64_t ldh, double damp_rel, float* D,
                     int64_t* bad_pivot_dev, void* ws, size_t ws_bytes, void* stream) {
    if (!H || !bad_pivot_dev || d <= 0 || bad_ld(ldh, d)) return BAKRON_E_INVALID_ARG;
    if (!(damp_rel >= 0.0) || !(damp_rel < INFINITY)) return BAKRON_E_INVALID_ARG;
    if (!ws || ws_bytes < bk::ldl_workspace_bytes(d)) return BAKRON_E_WORKSPACE;
    return bk::enqueue_ldl(H, d, ldh, damp_rel, D, ws, (hipStream_t)stream, bad_pivot_dev);
}

int bakron_ldl_pair_async(float* HA, int64_t dA, int64_t ldha, float* DA, int64_t* bad_pivot_dev_A,
                          void* wsA, size_t wsA_bytes, float* HB, int64_t dB, int64_t ldhb, float* DB,
                          int64_t* bad_pivot_dev_B, void* wsB, size_t wsB_bytes, double damp_rel,
                          void* stream_a, void* stream_b) {
    if (!HA || !bad_pivot_dev_A || dA <= 0 || bad_ld(ldha, dA)) return BAKRON_E_INVALID_ARG;
    if (!HB || !bad_pivot_dev_B || dB <= 0 || bad_ld(ldhb, dB)) return BAKRON_E_INVALID_ARG;
    if (!(damp_rel >= 0.0) || !(damp_rel < INFINITY)) return BAKRON_E_INVALID_ARG;
    if (!wsA || wsA_bytes < bk::ldl_workspace_bytes(dA)) return BAKRON_E_WORKSPACE;
    if (!wsB || wsB_bytes < bk::ldl_workspace_bytes(dB)) return BAKRON_E_WORKSPACE;
    return bk::enqueue_ldl_pair(HA, dA, ldha, DA, wsA, bad_pivot_dev_A, HB, dB, ldhb, DB, wsB, bad_pivot_dev_B,
                                damp_rel, (hipStream_t)stream_a, (hipStream_t)stream_b);
}

size_t bakron_solve_workspace_bytes(int64_t m, int64_t n) {
    if (m <= 0 || n <= 0) return 0;
    return bk::solve_workspace_bytes(m, n);
}

int bakron_solve(const float* W, int64_t m, int64_t n, int64_t ldw, const float* L_O, int64_t ldlo,
                 const float* L_I, int64_t ldli, const bakron_quantizer* q, uint8_t* codes,
                 int64_t ldc, float* scales_out, float* delta_out, int64_t ldd, const float* D_O,
                 const float* D_I, double* loss_out, int64_t* clamped_out, int32_t* info,
                 void* ws, size_t ws_bytes, void* stream) {
    const int st = check_solve_args(W, m, n, ldw, L_O, ldlo, L_I, ldli, q, codes, ldc, scales_out, delta_out,
                                    ldd, D_O, D_I, loss_out);
    if (st != BAKRON_OK) return st;
    if (!ws || ws_bytes < bk::solve_workspace_bytes(m, n)) return BAKRON_E_WORKSPACE;
    return bk::run_solve(solve_args(W, m, n, ldw, L_O, ldlo, L_I, ldli, q, codes, ldc, scales_out, delta_out, ldd,
                                    D_O, D_I, loss_out, clamped_out, info),
                         ws, (hipStream_t)stream);
}

int bakron_solve_noalloc(const float* W, int64_t m, int64_t n, int64_t ldw, const float* L_O, int64_t ldlo,
                         const float* L_I, int64_t ldli, const bakron_quantizer* q, uint8_t* codes,
                         int64_t ldc, float* scales_out, float* delta_out, int64_t ldd, const float* D_O,
                         const float* D_I, double* loss_out, int64_t* clamped_out, int32_t* info,
                         void* stream) {
    const int st = check_solve_args(W, m, n, ldw, L_O, ldlo, L_I, ldli, q, codes, ldc, scales_out, delta_out,
                                    ldd, D_O, D_I, loss_out);
    if (st != BAKRON_OK) return st;
    if (bk::solve_workspace_bytes(m, n) > BAKRON_NOALLOC_SCRATCH_BYTES) return BAKRON_E_WORKSPACE;
    void* ws = scratch_address();
    if (ws == nullptr) return BAKRON_E_DEVICE;
    return bk::run_solve(solve_args(W, m, n, ldw, L_O, ldlo, L_I, ldli, q, codes, ldc, scales_out, delta_out, ldd,
                                    D_O, D_I, loss_out, clamped_out, info),
                         ws, (hipStream_t)stream);
}

int bakron_layer_report(int64_t m, int64_t n, const float* D_O, const float* D_I, const float* scales,
                        const float* H_I, int64_t ldhi, const float* H_O, int64_t ldho, double* out,
                        void* stream) {
    if (m <= 0 || n <= 0 || !D_I || !scales || !out) return BAKRON_E_INVALID_ARG;
    if ((H_I && bad_ld(ldhi, n)) || (H_O && bad_ld(ldho, m))) return BAKRON_E_INVALID_ARG;
    return bk::launch_layer_report(m, n, D_O, D_I, scales, H_I, ldhi, H_O, ldho, out, (hipStream_t)stream);
}

int bakron_rht(float* A, int64_t rows, int64_t cols, int64_t lda, int axis, uint64_t seed, int transpose,
               void* stream) {
    if (!A || rows <= 0 || cols <= 0 || bad_ld(lda, cols) || (axis != 0 && axis != 1))
        return BAKRON_E_INVALID_ARG;
    if (axis == 1 && (cols & -cols) > 16384) return BAKRON_E_INVALID_ARG;
    return bk::launch_rht(A, rows, cols, lda, axis, seed, transpose, (hipStream_t)stream);
}

}  // extern "C"
