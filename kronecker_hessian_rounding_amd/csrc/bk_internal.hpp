// bk_internal.hpp -- host-side interfaces between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bakron.h"

namespace bk {

// Round a byte count up to a 256-byte boundary (workspace carving).
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Compute units and the wall clock of s_memrealtime of the current device, read once per device.
struct DeviceInfo {
    int cus = 0;
    int clock_khz = 0;
};
inline DeviceInfo device_info() {
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

// --- Hessian factor accumulation (bk_accum.hip) ---
size_t hessian_workspace_bytes(int64_t T, int64_t d);
// trans: X is stored d x T (H = X X^T); wt: per-token weights (H = sum_k wt_k
// x_k^T x_k); both need the workspace of the piece path
int launch_hessian_accum(const float* X, int64_t T, int64_t d, int64_t ldx, float alpha,
                         float beta, float* H, int64_t ldh, void* ws, size_t ws_bytes,
                         hipStream_t stream, bool trans = false, const float* wt = nullptr,
                         int64_t tin = 0, int64_t bs = 0);

// --- Sketch A token weights (bk_sketch.hip) ---
size_t token_weights_workspace_bytes(int64_t T, int64_t d);
int launch_token_weights(const float* Y, int64_t T, int64_t d, int64_t ldy, const float* H, int64_t ldh,
                         float* w, void* ws, size_t ws_bytes, hipStream_t stream);

// --- LDL factorisation (bk_ldl.hip) ---
size_t ldl_workspace_bytes(int64_t d);
// Enqueues the whole factorisation on `stream` without waiting; with info_dev
// (device int64) non-null, the status (-1, the first failing pivot, or -2 for a
// wait that timed out) lands there. allow_sched false keeps it to the launch chain.
int enqueue_ldl(float* H, int64_t d, int64_t ldh, double damp_rel, float* D, void* ws,
                hipStream_t stream, int64_t* info_dev, bool allow_sched = true);
int run_ldl(float* H, int64_t d, int64_t ldh, double damp_rel, float* D, int64_t* bad_pivot,
            void* ws, hipStream_t stream);
// Two factorisations: in one launch on `stream` when both take the scheduled
// path, else A on `stream` and B on `stream_b`, both by the launch chain.
// info* are device int64, required.
int enqueue_ldl_pair(float* HA, int64_t dA, int64_t ldha, float* DA, void* wsA, int64_t* infoA,
                     float* HB, int64_t dB, int64_t ldhb, float* DB, void* wsB, int64_t* infoB,
                     double damp_rel, hipStream_t stream, hipStream_t stream_b);

// --- incoherence rotation (bk_rotate.hip) ---
int launch_rht(float* A, int64_t rows, int64_t cols, int64_t lda, int axis, uint64_t seed, int transpose,
               hipStream_t stream);

// --- bound and sensitivity report (bk_report.hip) ---
int launch_layer_report(int64_t m, int64_t n, const float* DO, const float* DI, const float* scales,
                        const float* HI, int64_t ldhi, const float* HO, int64_t ldho, double* out,
                        hipStream_t stream);

// --- rounding solve (bk_solve.hip) ---
struct SolveArgs {
    const float* W;
    int64_t m, n, ldw;
    const float* LO;
    int64_t ldlo;
    const float* LI;
    int64_t ldli;
    int bits;
    int stochastic;
    uint64_t seed;
    const float* row_scale;
    uint8_t* codes;
    int64_t ldc;
    float* scales;
    float* delta;
    int64_t ldd;
    const float* DO;
    const float* DI;
    double* loss;
    int64_t* clamped;
    int32_t* info;
};
size_t solve_workspace_bytes(int64_t m, int64_t n);
int run_solve(const SolveArgs& a, void* ws, hipStream_t stream);

}  // namespace bk
