"""MI355X-native BaKron: two-sided adaptive rounding under a Kronecker-factored Hessian.

The computation runs in libbakron (HIP kernels for gfx950, C ABI in
include/bakron.h); this package is a thin ctypes binding that takes PyTorch
tensors for device memory and uses the current stream.

  hessian_accum(X)            H <- beta H + alpha X^T X            (fp16 pieces, fp32 accuracy)
  sketch_b(grads)             H_I = E[G^T G]/m, H_O = E[G G^T]/n from per-sequence gradients
  sketch_a(X, G, iters)       alternating factor estimate with per-token weights
  ldl(H, damp_rel)            H + lambda I = (L + I) D (L + I)^T   (fp64, L strictly upper)
  ldl_pair(HA, HB, damp_rel)  two independent factorisations side by side on two streams
  check_ldl_pair(status)      raise for the statuses a non-waiting ldl_pair(..., status=) left
  solve(W, L_O, L_I, bits)    BaKron rounding: codes, scales, error, proxy loss
  solve_noalloc(W, L_O, L_I, bits, out)  the same, allocating nothing (library-held scratch)
  rotate_layer(W, HI, HO, sO, sI) two-sided randomised Hadamard rotation (incoherence processing)
  quantize_layer(W, X, G, b)  the whole per-layer path
"""
from ._binding import (  # noqa: F401
    BAKRON_E_DEVICE, BAKRON_E_INVALID_ARG, BAKRON_E_NOT_SPD, BAKRON_E_WORKSPACE, BAKRON_OK,
    EXPORTS, LIB, LIB_PATH, NOALLOC_SCRATCH_BYTES, BakronError, SolveResult, abi_version, check_ldl_pair,
    hessian_accum, ldl, ldl_pair, layer_report, quantize_layer, release_workspace, rht, rotate_layer, sketch_a, sketch_b,
    solve, solve_noalloc, token_weights,
)
