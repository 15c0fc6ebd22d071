"""ctypes binding of libbakron (include/bakron.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libbakron. Tensors must be CUDA (ROCm) tensors on the current
device, row-major with unit column stride; PyTorch supplies device memory and
the current stream. If the built library is missing this module raises
ImportError: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch  # loads the HIP runtime first; libbakron binds to the same one

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libbakron.so")

BAKRON_OK = 0
BAKRON_E_INVALID_ARG = 1
BAKRON_E_NOT_SPD = 2
BAKRON_E_WORKSPACE = 3
BAKRON_E_DEVICE = 4
ROUNDING = {"nearest": 0, "stochastic": 1}


class BakronError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


class _Quantizer(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("row_scale", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libbakron.so is not built (%s); run "
                          "`python -m kronecker_hessian_rounding_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    f32 = ctypes.c_float
    lib.bakron_abi_version.restype = ctypes.c_int
    lib.bakron_abi_version.argtypes = []
    lib.bakron_status_str.restype = ctypes.c_char_p
    lib.bakron_status_str.argtypes = [ctypes.c_int]
    lib.bakron_hessian_accum_workspace_bytes.restype = sz
    lib.bakron_hessian_accum_workspace_bytes.argtypes = [i64, i64]
    lib.bakron_hessian_accum.restype = ctypes.c_int
    lib.bakron_hessian_accum.argtypes = [vp, i64, i64, i64, f32, f32, vp, i64, vp, sz, vp]
    lib.bakron_hessian_accum_t.restype = ctypes.c_int
    lib.bakron_hessian_accum_t.argtypes = [vp, i64, i64, i64, f32, f32, vp, i64, vp, sz, vp]
    lib.bakron_hessian_accum_tb.restype = ctypes.c_int
    lib.bakron_hessian_accum_tb.argtypes = [vp, i64, i64, i64, i64, i64, f32, f32, vp, i64, vp, sz, vp]
    lib.bakron_hessian_accum_w.restype = ctypes.c_int
    lib.bakron_hessian_accum_w.argtypes = [vp, i64, i64, i64, vp, f32, f32, vp, i64, vp, sz, vp]
    lib.bakron_token_weights_workspace_bytes.restype = sz
    lib.bakron_token_weights_workspace_bytes.argtypes = [i64, i64]
    lib.bakron_token_weights.restype = ctypes.c_int
    lib.bakron_token_weights.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp, sz, vp]
    lib.bakron_ldl_workspace_bytes.restype = sz
    lib.bakron_ldl_workspace_bytes.argtypes = [i64]
    lib.bakron_ldl.restype = ctypes.c_int
    lib.bakron_ldl.argtypes = [vp, i64, i64, ctypes.c_double, vp, ctypes.POINTER(i64), vp, sz, vp]
    lib.bakron_ldl_async.restype = ctypes.c_int
    lib.bakron_ldl_async.argtypes = [vp, i64, i64, ctypes.c_double, vp, vp, vp, sz, vp]
    lib.bakron_ldl_pair_async.restype = ctypes.c_int
    lib.bakron_ldl_pair_async.argtypes = [vp, i64, i64, vp, vp, vp, sz, vp, i64, i64, vp, vp, vp, sz,
                                          ctypes.c_double, vp, vp]
    lib.bakron_layer_report.restype = ctypes.c_int
    lib.bakron_layer_report.argtypes = [i64, i64, vp, vp, vp, vp, i64, vp, i64, vp, vp]
    lib.bakron_rht.restype = ctypes.c_int
    lib.bakron_rht.argtypes = [vp, i64, i64, i64, ctypes.c_int, ctypes.c_uint64, ctypes.c_int, vp]
    lib.bakron_solve_workspace_bytes.restype = sz
    lib.bakron_solve_workspace_bytes.argtypes = [i64, i64]
    lib.bakron_solve.restype = ctypes.c_int
    lib.bakron_solve.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, ctypes.POINTER(_Quantizer),
                                 vp, i64, vp, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.bakron_solve_noalloc.restype = ctypes.c_int
    lib.bakron_solve_noalloc.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, ctypes.POINTER(_Quantizer),
                                         vp, i64, vp, vp, i64, vp, vp, vp, vp, vp, vp]
    return lib


LIB = _load()

# bytes of the device scratch array that bakron_solve_noalloc works in
NOALLOC_SCRATCH_BYTES = 128 << 20

EXPORTS = ("bakron_abi_version", "bakron_status_str", "bakron_hessian_accum_workspace_bytes",
           "bakron_hessian_accum", "bakron_hessian_accum_t", "bakron_hessian_accum_tb",
           "bakron_hessian_accum_w",
           "bakron_token_weights_workspace_bytes", "bakron_token_weights", "bakron_ldl_workspace_bytes", "bakron_ldl", "bakron_ldl_async",
           "bakron_ldl_pair_async",
           "bakron_solve_workspace_bytes", "bakron_solve", "bakron_solve_noalloc", "bakron_rht",
           "bakron_layer_report")


def abi_version() -> int:
    return int(LIB.bakron_abi_version())


def _check(fn: str, status: int):
    if status != BAKRON_OK:
        raise BakronError(fn, status, LIB.bakron_status_str(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _mat(t: torch.Tensor, name: str, dtype=torch.float32) -> int:
    """Validate a row-major device matrix; returns its leading dimension."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a CUDA/ROCm tensor" % name)
    if t.dtype != dtype or t.dim() != 2:
        raise ValueError("%s must be a 2-D %s tensor" % (name, dtype))
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must have unit column stride" % name)
    return max(int(t.stride(0)), int(t.shape[1]))


def _vec(t: Optional[torch.Tensor], name: str, n: int, dtype=torch.float32):
    if t is None:
        return None
    if not t.is_cuda or t.dtype != dtype or t.numel() != n or not t.is_contiguous():
        raise ValueError("%s must be a contiguous CUDA %s vector of length %d" % (name, dtype, n))
    return t


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


_ws_cache: dict = {}


def _workspace(nbytes: int, device, slot: int = 0) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    key = (str(device), "ws", slot)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def release_workspace():
    _ws_cache.clear()


_aux_streams: dict = {}


def _aux_stream(device) -> torch.cuda.Stream:
    """A second stream per device (default priority) for work beside the current stream."""
    key = str(device)
    s = _aux_streams.get(key)
    if s is None:
        s = torch.cuda.Stream(device=device)
        _aux_streams[key] = s
    return s


# --------------------------------------------------------------------------
def hessian_accum(X: torch.Tensor, H: Optional[torch.Tensor] = None, alpha: Optional[float] = None,
                  beta: float = 0.0, pieces: bool = True, transposed: bool = False,
                  weights: Optional[torch.Tensor] = None) -> torch.Tensor:
    """H <- beta H + alpha X^T X (default alpha = 1/T) on the device.

    pieces=True passes the full workspace: each fp32 product is formed from two
    fp16 pieces per operand (of power-of-two-scaled columns) on the fp16 matrix
    cores. pieces=False passes none,
    which selects the fp32 matrix-core path. transposed=True takes X as d x T and
    forms alpha X X^T (piece path only). weights (T,) forms
    alpha sum_t w_t x_t^T x_t (piece path only).
    """
    ldx = _mat(X, "X")
    if transposed:
        if not pieces:
            raise ValueError("the transposed form runs on the fp16 piece path only")
        d, T = X.shape
    else:
        T, d = X.shape
    if H is None:
        H = torch.empty((d, d), dtype=torch.float32, device=X.device)
    ldh = _mat(H, "H")
    if tuple(H.shape) != (d, d):
        raise ValueError("H must be %d x %d" % (d, d))
    if alpha is None:
        alpha = 1.0 / max(T, 1)
    nb = LIB.bakron_hessian_accum_workspace_bytes(T, d) if pieces else 0
    ws = _workspace(nb, X.device)
    if weights is not None:
        if transposed or not pieces:
            raise ValueError("token weights take the untransposed fp16 piece path")
        wv = _vec(weights, "weights", T)
        _check("bakron_hessian_accum_w",
               LIB.bakron_hessian_accum_w(_ptr(X), T, d, ldx, _ptr(wv), alpha, beta, _ptr(H), ldh, _ptr(ws),
                                          nb, _stream()))
        return H
    fn = LIB.bakron_hessian_accum_t if transposed else LIB.bakron_hessian_accum
    _check("bakron_hessian_accum_t" if transposed else "bakron_hessian_accum",
           fn(_ptr(X), T, d, ldx, alpha, beta, _ptr(H), ldh, _ptr(ws), nb, _stream()))
    return H


def token_weights(Y: torch.Tensor, H: Optional[torch.Tensor] = None,
                  w: Optional[torch.Tensor] = None) -> torch.Tensor:
    """w_t = y_t H y_t^T / ||H||_F^2 for the rows of Y (T x d); H None means the identity."""
    ldy = _mat(Y, "Y")
    T, d = Y.shape
    ldh = 0
    if H is not None:
        ldh = _mat(H, "H")
        if tuple(H.shape) != (d, d):
            raise ValueError("H must be %d x %d" % (d, d))
    if w is None:
        w = torch.empty(T, dtype=torch.float32, device=Y.device)
    nb = LIB.bakron_token_weights_workspace_bytes(T, d) if H is not None else 0
    ws = _workspace(nb, Y.device, slot=1)
    _check("bakron_token_weights", LIB.bakron_token_weights(_ptr(Y), T, d, ldy, _ptr(H), ldh, _ptr(w),
                                                            _ptr(ws), nb, _stream()))
    return w


def sketch_a(X: torch.Tensor, G: torch.Tensor, iters: int = 3):
    """Sketch A factors (YAQA article, section 3) from token inputs X (T x n) and output
    gradients G (T x m): `iters` alternating updates from E[x^T x] and I. Returns (H_I, H_O)."""
    T = X.shape[0]
    HI = hessian_accum(X)
    HO = None
    for _ in range(iters):
        w = token_weights(G, HO)
        v = token_weights(X, HI)
        HI_new = hessian_accum(X, alpha=1.0 / T, weights=w)
        HO = hessian_accum(G, HO, alpha=1.0 / T, weights=v)
        HI = HI_new
    return HI, HO


def sketch_b(grads, HI: Optional[torch.Tensor] = None, HO: Optional[torch.Tensor] = None):
    """Sketch B factors from per-sequence weight gradients (S x m x n, or a sequence of m x n):
    H_I = E_s[G_s^T G_s] / m and H_O = E_s[G_s G_s^T] / n. Returns (H_I, H_O)."""
    S = len(grads)
    if S == 0:
        raise ValueError("sketch_b needs at least one gradient")
    m, n = grads[0].shape
    # every argument is checked before the first launch
    dev = grads[0].device
    for g in grads:
        if not isinstance(g, torch.Tensor) or not g.is_cuda or g.dtype != torch.float32:
            raise ValueError("grads must be CUDA float32 tensors")
        if tuple(g.shape) != (m, n) or g.device != dev:
            raise ValueError("every gradient must be %d x %d on %s" % (m, n, dev))
    for H, d, name in ((HI, n, "H_I"), (HO, m, "H_O")):
        if H is not None:
            _mat(H, name)
            if tuple(H.shape) != (d, d) or H.device != dev:
                raise ValueError("%s must be %d x %d on %s" % (name, d, d, dev))
    # sum_s G_s^T G_s is X^T X of the gradients stacked vertically: for one contiguous
    # S x m x n tensor H_I is a single accumulation over S m tokens
    # and sum_s G_s G_s^T is one transposed accumulation over the batch (S n tokens)
    stacked = isinstance(grads, torch.Tensor) and grads.dim() == 3 and grads.is_contiguous()
    if stacked:
        if HO is None:
            HO = torch.empty((m, m), dtype=torch.float32, device=dev)
        ldho = _mat(HO, "H_O")
        HI = hessian_accum(grads.reshape(S * m, n), HI, alpha=1.0 / (S * m), beta=0.0)
        nb = LIB.bakron_hessian_accum_workspace_bytes(S * n, m)
        ws = _workspace(nb, grads.device)
        _check("bakron_hessian_accum_tb",
               LIB.bakron_hessian_accum_tb(_ptr(grads), S, m, n, n, m * n, 1.0 / (S * n), 0.0, _ptr(HO), ldho,
                                           _ptr(ws), nb, _stream()))
        return HI, HO
    for s in range(S):
        beta = 0.0 if s == 0 else 1.0
        HI = hessian_accum(grads[s], HI, alpha=1.0 / (S * m), beta=beta)
        HO = hessian_accum(grads[s], HO, alpha=1.0 / (S * n), beta=beta, transposed=True)
    return HI, HO


def ldl(H: torch.Tensor, damp_rel: float = 0.01, D: Optional[torch.Tensor] = None):
    """In place: H + damp_rel*mean(diag H)*I = (L + I) diag(D) (L + I)^T, L strictly upper.

    Returns (H, D): H holds L above its diagonal, D on it and zeros below.
    Raises BakronError(status=BAKRON_E_NOT_SPD) with .bad_pivot on failure, or
    (status=BAKRON_E_DEVICE, .bad_pivot = -2) if a wait between workgroups timed out.
    """
    ldh = _mat(H, "H")
    d = H.shape[0]
    if H.shape[1] != d:
        raise ValueError("H must be square")
    if D is None:
        D = torch.empty(d, dtype=torch.float32, device=H.device)
    _vec(D, "D", d)
    nb = LIB.bakron_ldl_workspace_bytes(d)
    ws = _workspace(nb, H.device)
    bad = ctypes.c_int64(-1)
    st = LIB.bakron_ldl(_ptr(H), d, ldh, damp_rel, _ptr(D), ctypes.byref(bad), _ptr(ws), nb,
                        _stream())
    if st != BAKRON_OK:
        err = BakronError("bakron_ldl", st, LIB.bakron_status_str(st).decode())
        err.bad_pivot = int(bad.value)
        raise err
    return H, D


def ldl_pair(HA: torch.Tensor, HB: torch.Tensor, damp_rel: float = 0.01,
             DA: Optional[torch.Tensor] = None, DB: Optional[torch.Tensor] = None,
             status: Optional[torch.Tensor] = None):
    """Two independent damped LDL factorisations at once (H_I and H_O of one layer).

    bakron_ldl_pair_async with the current stream and a second one that starts after
    the current stream's earlier work; the current stream then waits for it. Without
    `status` the call waits for both to report their pivots and raises
    BakronError(status=BAKRON_E_NOT_SPD) with .bad_pivot and .which (0 for HA, 1 for
    HB), or (status=BAKRON_E_DEVICE, .bad_pivot = -2) if a wait between workgroups
    timed out. With `status` (a device int64 tensor of 2 entries) nothing waits: the
    two statuses land there in stream order, work queued after the call runs right
    behind the factorisations, and check_ldl_pair(status) raises the same errors
    later. Returns ((HA, DA), (HB, DB)).
    """
    mats = []
    for H, D, name in ((HA, DA, "HA"), (HB, DB, "HB")):
        ldh = _mat(H, name)
        d = H.shape[0]
        if H.shape[1] != d:
            raise ValueError("%s must be square" % name)
        if D is None:
            D = torch.empty(d, dtype=torch.float32, device=H.device)
        _vec(D, "D" + name[1], d)
        mats.append((H, D, d, ldh))
    dev = HA.device
    if status is not None:
        if (status.device != dev or status.dtype != torch.int64 or status.numel() != 2
                or not status.is_contiguous()):
            raise ValueError("status must be a contiguous int64 tensor of 2 entries on %s" % dev)
        info = status
    else:
        info = torch.empty((2,), dtype=torch.int64, device=dev)  # the library writes both
    cur = torch.cuda.current_stream(dev)
    aux = _aux_stream(dev)
    ws = [_workspace(LIB.bakron_ldl_workspace_bytes(m[2]), dev, slot=k) for k, m in enumerate(mats)]
    start = torch.cuda.Event()
    start.record(cur)
    aux.wait_event(start)
    (HA_, DA_, dA, lda), (HB_, DB_, dB, ldb) = mats
    st = LIB.bakron_ldl_pair_async(_ptr(HA_), dA, lda, _ptr(DA_), ctypes.c_void_p(info.data_ptr()),
                                   _ptr(ws[0]), ws[0].numel(), _ptr(HB_), dB, ldb, _ptr(DB_),
                                   ctypes.c_void_p(info.data_ptr() + 8), _ptr(ws[1]), ws[1].numel(),
                                   damp_rel, ctypes.c_void_p(cur.cuda_stream), ctypes.c_void_p(aux.cuda_stream))
    done = torch.cuda.Event()
    done.record(aux)
    cur.wait_event(done)
    _check("bakron_ldl_pair_async", st)
    if status is None:
        check_ldl_pair(info)
    return (mats[0][0], mats[0][1]), (mats[1][0], mats[1][1])


def check_ldl_pair(status: torch.Tensor) -> None:
    """Waits for the statuses that ldl_pair(..., status=status) left and raises as ldl_pair."""
    bad = status.cpu().tolist()  # waits for both factorisations
    for k in range(2):
        if bad[k] >= 0 or bad[k] == -2:
            st = BAKRON_E_NOT_SPD if bad[k] >= 0 else BAKRON_E_DEVICE
            err = BakronError("bakron_ldl_pair_async", st, LIB.bakron_status_str(st).decode())
            err.bad_pivot = int(bad[k])
            err.which = k
            raise err


@dataclass
class SolveResult:
    codes: torch.Tensor
    scales: torch.Tensor
    delta: Optional[torch.Tensor]
    loss: Optional[torch.Tensor]      # device double [1]
    clamped: torch.Tensor             # device int64 [1]
    info: torch.Tensor                # device int32 [1]


def solve(W: torch.Tensor, L_O: Optional[torch.Tensor], L_I: Optional[torch.Tensor], bits: int,
          rounding: str = "nearest", seed: int = 0, row_scale: Optional[torch.Tensor] = None,
          D_O: Optional[torch.Tensor] = None, D_I: Optional[torch.Tensor] = None,
          want_delta: bool = False, want_loss: bool = False,
          out: Optional[SolveResult] = None) -> SolveResult:
    """BaKron two-sided rounding of W (m x n) given strict-upper LDL factors L_O, L_I."""
    ldw = _mat(W, "W")
    m, n = W.shape
    ldlo = ldli = 0
    if L_O is not None:
        ldlo = _mat(L_O, "L_O")
        if tuple(L_O.shape) != (m, m):
            raise ValueError("L_O must be %d x %d" % (m, m))
    if L_I is not None:
        ldli = _mat(L_I, "L_I")
        if tuple(L_I.shape) != (n, n):
            raise ValueError("L_I must be %d x %d" % (n, n))
    _vec(row_scale, "row_scale", m)
    _vec(D_O, "D_O", m)
    _vec(D_I, "D_I", n)
    dev = W.device
    if out is None:
        out = SolveResult(
            codes=torch.empty((m, n), dtype=torch.uint8, device=dev),
            scales=torch.empty(m, dtype=torch.float32, device=dev),
            delta=torch.empty((m, n), dtype=torch.float32, device=dev) if want_delta else None,
            loss=torch.empty(1, dtype=torch.float64, device=dev) if want_loss else None,
            clamped=torch.empty(1, dtype=torch.int64, device=dev),
            info=torch.empty(1, dtype=torch.int32, device=dev))
    q = _Quantizer(int(bits), ROUNDING[rounding], int(seed) & (2**64 - 1),
                   None if row_scale is None else row_scale.data_ptr())
    nb = LIB.bakron_solve_workspace_bytes(m, n)
    ws = _workspace(nb, dev)
    ldd = n if out.delta is None else _mat(out.delta, "delta")
    st = LIB.bakron_solve(_ptr(W), m, n, ldw, _ptr(L_O), ldlo, _ptr(L_I), ldli, ctypes.byref(q),
                          _ptr(out.codes), _mat(out.codes, "codes", torch.uint8), _ptr(out.scales),
                          _ptr(out.delta), ldd, _ptr(D_O), _ptr(D_I), _ptr(out.loss),
                          _ptr(out.clamped), _ptr(out.info), _ptr(ws), nb, _stream())
    _check("bakron_solve", st)
    return out


def solve_noalloc(W: torch.Tensor, L_O: Optional[torch.Tensor], L_I: Optional[torch.Tensor], bits: int,
                  out: SolveResult, rounding: str = "nearest", seed: int = 0,
                  row_scale: Optional[torch.Tensor] = None, D_O: Optional[torch.Tensor] = None,
                  D_I: Optional[torch.Tensor] = None) -> SolveResult:
    """solve() through bakron_solve_noalloc: the caller passes every output in `out`
    (codes, scales, info, and optionally delta, loss, clamped) and nothing is
    allocated, by this function or by the library, which works in its own device
    scratch array (shapes up to NOALLOC_SCRATCH_BYTES of workspace). For callers that
    cannot allocate, e.g. under HIP graph capture. Calls that overlap on one device
    share the array and race."""
    ldw = _mat(W, "W")
    m, n = W.shape
    ldlo = ldli = 0
    if L_O is not None:
        ldlo = _mat(L_O, "L_O")
        if tuple(L_O.shape) != (m, m):
            raise ValueError("L_O must be %d x %d" % (m, m))
    if L_I is not None:
        ldli = _mat(L_I, "L_I")
        if tuple(L_I.shape) != (n, n):
            raise ValueError("L_I must be %d x %d" % (n, n))
    _vec(row_scale, "row_scale", m)
    _vec(D_O, "D_O", m)
    _vec(D_I, "D_I", n)
    if tuple(out.codes.shape) != (m, n) or out.scales.numel() != m:
        raise ValueError("out.codes must be %d x %d and out.scales [%d]" % (m, n, m))
    if out.delta is not None and tuple(out.delta.shape) != (m, n):
        raise ValueError("out.delta must be %d x %d" % (m, n))
    q = _Quantizer(int(bits), ROUNDING[rounding], int(seed) & (2**64 - 1),
                   None if row_scale is None else row_scale.data_ptr())
    ldd = n if out.delta is None else _mat(out.delta, "delta")
    st = LIB.bakron_solve_noalloc(_ptr(W), m, n, ldw, _ptr(L_O), ldlo, _ptr(L_I), ldli, ctypes.byref(q),
                                  _ptr(out.codes), _mat(out.codes, "codes", torch.uint8), _ptr(out.scales),
                                  _ptr(out.delta), ldd, _ptr(D_O), _ptr(D_I), _ptr(out.loss),
                                  _ptr(out.clamped), _ptr(out.info), _stream())
    _check("bakron_solve_noalloc", st)
    return out


def layer_report(D_O: Optional[torch.Tensor], D_I: torch.Tensor, scales: torch.Tensor,
                 H_I: Optional[torch.Tensor] = None, H_O: Optional[torch.Tensor] = None) -> dict:
    """Bound and sensitivity terms of a rounded layer (fp64 sums on the device).

    Keys: tr_DO, tr_DI, bound_sharp, bound_page, tr_HI, tr_HO (NaN when not given;
    pass the factors before ldl, which writes D over their diagonal), sensitivity
    = tr_HI * tr_HO.
    """
    n = int(D_I.shape[0])
    m = int(scales.shape[0])
    ldhi = _mat(H_I, "H_I") if H_I is not None else 0
    ldho = _mat(H_O, "H_O") if H_O is not None else 0
    out = torch.empty(7, dtype=torch.float64, device=D_I.device)
    _check("bakron_layer_report", LIB.bakron_layer_report(m, n, _ptr(D_O), _ptr(D_I), _ptr(scales),
                                                          _ptr(H_I), ldhi, _ptr(H_O), ldho, _ptr(out),
                                                          _stream()))
    v = out.cpu().tolist()
    keys = ("tr_DO", "tr_DI", "bound_sharp", "bound_page", "tr_HI", "tr_HO", "sensitivity")
    return dict(zip(keys, v))


def rht(A: torch.Tensor, axis: int, seed: int, transpose: bool = False) -> torch.Tensor:
    """In place: axis 0: A <- U A (U of order rows); axis 1: A <- A U^T (U of order cols).

    U = (I_r (x) H_b / sqrt(b)) diag(s) with random signs from `seed`;
    transpose=True applies U^T, the inverse.
    """
    lda = _mat(A, "A")
    rows, cols = A.shape
    _check("bakron_rht", LIB.bakron_rht(_ptr(A), rows, cols, lda, int(axis), int(seed) & (2**64 - 1),
                                        1 if transpose else 0, _stream()))
    return A


def rotate_layer(W: torch.Tensor, HI: Optional[torch.Tensor], HO: Optional[torch.Tensor], seed_O: int,
                 seed_I: int, transpose: bool = False):
    """Two-sided incoherence processing, in place: W <- U_O W U_I^T, H_I <- U_I H_I U_I^T,
    H_O <- U_O H_O U_O^T (H_I and H_O may be None). transpose=True undoes it."""
    rht(W, 0, seed_O, transpose)
    rht(W, 1, seed_I, transpose)
    for H, seed in ((HI, seed_I), (HO, seed_O)):
        if H is not None:
            rht(H, 0, seed, transpose)
            rht(H, 1, seed, transpose)
    return W, HI, HO


def quantize_layer(W: torch.Tensor, X: torch.Tensor, G: Optional[torch.Tensor], bits: int,
                   rounding: str = "nearest", seed: int = 0, damp_rel: float = 0.01,
                   want_delta: bool = False, want_loss: bool = True, workspace=None):
    """The whole per-layer path on the device: H_I from X, H_O from G (or H_O = I when
    G is None, damped to (1 + damp_rel) I), damping + LDL of both, scales, and the
    BaKron solve."""
    m, n = W.shape
    if workspace is None:
        workspace = {}
    HI = hessian_accum(X, workspace.get("HI"))
    status = None
    if G is not None:
        HO = hessian_accum(G, workspace.get("HO"))
        # the two factorisations are independent: run them side by side; their
        # statuses are read once the solve is queued behind them
        status = torch.empty(2, dtype=torch.int64, device=W.device)
        (HI, DI), (HO, DO) = ldl_pair(HI, HO, damp_rel, workspace.get("DI"), workspace.get("DO"),
                                      status=status)
        LO = HO
    else:
        HI, DI = ldl(HI, damp_rel, workspace.get("DI"))
        # H_O = I is damped like any factor: (1 + damp_rel) I, so L_O = 0 (the codes of
        # H_O = I) and D_O = 1 + damp_rel, which enters the proxy loss
        LO = None
        DO = workspace.get("DO")
        if DO is None:
            DO = torch.empty(m, dtype=torch.float32, device=W.device)
        DO.fill_(1.0 + damp_rel)
    res = solve(W, LO, HI, bits, rounding, seed, D_O=DO, D_I=DI, want_delta=want_delta,
                want_loss=want_loss, out=workspace.get("out"))
    if status is not None:
        # the solve has no value-dependent control flow, so it ends normally on the
        # factors of a failed factorisation; the failure is raised here
        check_ldl_pair(status)
    return res, (LO, DO, HI, DI)
