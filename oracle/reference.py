"""Plain fp64 CPU reference ("the oracle") for the BaKron rounding pipeline.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's cpu_baseline leg. The HIP library and its Python binding never
import it, and it imports nothing from them.

Sources (cited by page title and section):
  [YAQA-2]  YAQA article (news.43b.com.cn/a/479517), section 2: the layer
            Hessian is approximated by a Kronecker product H_O (m x m) (x)
            H_I (n x n) of the vectorised weight.
  [YAQA-3]  same article, section 3: H_I = E[x^T x] over tokens (the
            initialisation H_1 of Sketch A); Sketch A, the alternating
            estimator with per-token weights <H, y^T y> / ||H||_F^2; Sketch B, one round of power
            iteration from H_I = H_O = I: H_I = E_s[G_s^T G_s] / m and
            H_O = E_s[G_s G_s^T] / n over per-sequence weight gradients G_s.
  [YAQA-4]  same article, section 4: the rounding rule
            W_ij = Q(W*_ij + a_i^T D[:i,:j] b_j + a_i^T D[:i,j] + D[i,:j] b_j),
            a_i / b_j columns of the strictly upper L_O / L_I, Q nearest or
            stochastic; the LDL form H = (L + I) D (L + I)^T; the error bound
            vec(D)^T (H_O (x) H_I) vec(D) <= tr(D_I) tr(D_O) sigma^2.
  [BaKron]  "BaKron: Efficient Quantization with Kronecker-Factored Hessians"
            (insight.aitobox.com), Abstract: BaKron is an exact, faster
            schedule of that rule (anti-diagonal parallelism plus a recursive
            divide-and-conquer), modular in the base quantiser.
  [KFAC-5]  K-FAC tutorial (www.mlqm.cn/news/1313094), section 5: the factor
            estimate A = X^T X / N plus a small multiple of the identity.
  [KronQ]   "KronQ: Kronecker-factored Hessian LLM quantization" (ai-feeds.com),
            method, "bidirectional incoherence processing": the random
            rotation of the input side is extended to the output side,
            W' = R_O W R_I^T.

Readings where the pages are silent or garbled (each is listed in the design doc):
  * L is strictly UPPER and H = (L + I) D (L + I)^T (one paragraph says unit
    lower; only the upper reading matches the prefix index sets of the rule).
  * ":i" excludes i. D = W* - W is added as feedback.
  * vec is row-major, so the proxy loss is tr(D H_I D^T H_O).
  * Q is the symmetric per-row grid s_i (c - Lq/2), c in 0..Lq, Lq = 2^b - 1,
    s_i = fp32(2 max_j |W*_ij|) / fp32(Lq) computed in fp32; nearest is
    floor(y + 1/2), stochastic floor(y + u) with u from SplitMix64; both
    clamped to [0, Lq]; y = t / s_i + Lq / 2.
  * Damping adds 0.01 * mean(diag H) * I (mean over the undamped diagonal).
  * The incoherence rotation (the pages name random rotations, not their
    construction): for n = 2^k r with r odd, U_n = (I_r (x) H_{2^k} / sqrt(2^k))
    diag(s), H the Sylvester Hadamard matrix, s_i = -1 if the top bit of
    SplitMix64 output i of the seed is set, else +1.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

__all__ = [
    "hessian", "hessian_entries", "damp", "udu", "udu_lapack", "row_scales", "sweep",
    "replay", "replay_rows", "proxy_loss", "loss_identity", "bound_terms", "splitmix64",
    "uniform_matrix", "pipeline", "rht_signs", "rht_block", "sylvester", "rht_matrix",
    "rht_apply", "rotate_layer", "sketch_b", "token_weights", "weighted_hessian", "sketch_a",
]

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    i64, u64, dp, fp, vp = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p,
                            ctypes.c_void_p, ctypes.c_void_p)
    lib.orc_splitmix64.argtypes = [u64, u64]
    lib.orc_splitmix64.restype = u64
    lib.orc_uniform.argtypes = [u64, u64]
    lib.orc_uniform.restype = ctypes.c_double
    sweep_args = [i64, i64, fp, dp, dp, fp, ctypes.c_int, ctypes.c_int, u64, dp, vp, dp, dp, dp,
                  dp, ctypes.POINTER(ctypes.c_int64)]
    for name in ("orc_sweep_naive", "orc_sweep_accum"):
        fn = getattr(lib, name)
        fn.argtypes = sweep_args
        fn.restype = ctypes.c_int
    lib.orc_udu.argtypes = [i64, dp, dp, dp, ctypes.POINTER(ctypes.c_int64)]
    lib.orc_udu.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# Random draws for stochastic rounding (SplitMix64, counter-based)
# --------------------------------------------------------------------------
def splitmix64(seed: int, idx: int) -> int:
    """Output number idx+1 of a SplitMix64 stream whose state starts at seed."""
    return int(_load().orc_splitmix64(seed & (2**64 - 1), idx))


_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _splitmix_outputs(seed: int, count: int) -> np.ndarray:
    """SplitMix64 outputs 1 .. count of the stream seeded with `seed` (uint64)."""
    with np.errstate(over="ignore"):
        idx = np.arange(1, count + 1, dtype=np.uint64)
        z = np.uint64(seed & (2**64 - 1)) + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform_matrix(seed: int, m: int, n: int) -> np.ndarray:
    """u_ij = (splitmix64(seed, i*n + j) >> 40) * 2^-24 as an fp64 m x n array."""
    z = _splitmix_outputs(seed, m * n)
    return ((z >> np.uint64(40)).astype(np.float64) * 2.0**-24).reshape(m, n)


# --------------------------------------------------------------------------
# Hessian factors [YAQA-3], [KFAC-5]
# --------------------------------------------------------------------------
def hessian(X: np.ndarray) -> np.ndarray:
    """H = X^T X / T in fp64, X a T x d matrix of per-token rows."""
    x = np.asarray(X, dtype=np.float64)
    return x.T @ x / x.shape[0]


def hessian_entries(X: np.ndarray, rows, cols) -> np.ndarray:
    """Selected entries H[rows[k], cols[k]] of X^T X / T, each an fp64 dot product."""
    out = np.empty(len(rows), dtype=np.float64)
    for k, (a, b) in enumerate(zip(rows, cols)):
        out[k] = np.dot(X[:, a].astype(np.float64), X[:, b].astype(np.float64)) / X.shape[0]
    return out


def damp(H: np.ndarray, rel: float = 0.01) -> np.ndarray:
    """H + rel * mean(diag H) * I, the mean taken over the undamped diagonal."""
    h = np.array(H, dtype=np.float64, copy=True)
    mu = float(np.mean(np.diag(h)))
    h[np.diag_indices_from(h)] += rel * mu
    return h


# --------------------------------------------------------------------------
# LDL form H = (L + I) diag(D) (L + I)^T, L strictly upper [YAQA-4]
# --------------------------------------------------------------------------
def udu(H: np.ndarray):
    """Column recurrence from the last index to the first (plain O(d^3) loops).

    Returns (L, D). Raises ValueError naming the first non-positive pivot.
    """
    h = np.ascontiguousarray(H, dtype=np.float64)
    d = h.shape[0]
    L = np.zeros((d, d), dtype=np.float64)
    D = np.zeros(d, dtype=np.float64)
    bad = ctypes.c_int64(-1)
    rc = _load().orc_udu(d, _ptr(h), _ptr(L), _ptr(D), ctypes.byref(bad))
    if rc != 0:
        raise ValueError("matrix is not positive definite: pivot %d" % bad.value)
    return L, D


def udu_lapack(H: np.ndarray):
    """The same factors from LAPACK's Cholesky of the index-reversed matrix.

    If J reverses the index order and J H J = C' C'^T (C' lower), then
    H = C C^T with C = J C' J upper, L + I = C diag(C)^-1 and D = diag(C)^2.
    """
    h = np.asarray(H, dtype=np.float64)
    c = np.linalg.cholesky(h[::-1, ::-1])[::-1, ::-1]
    dc = np.diag(c).copy()
    L = c / dc[None, :]
    L[np.diag_indices_from(L)] = 0.0
    return np.triu(L, 1), dc * dc


# --------------------------------------------------------------------------
# Base quantiser grid
# --------------------------------------------------------------------------
def row_scales(W: np.ndarray, bits: int) -> np.ndarray:
    """s_i = fp32(2 * max_j |W*_ij|) / fp32(2^bits - 1), all in fp32."""
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    w = np.asarray(W, dtype=np.float32)
    amax = np.max(np.abs(w), axis=1)
    if not np.all(np.isfinite(amax)) or np.any(amax == 0):
        raise ValueError("every row needs a finite, non-zero absmax")
    return (np.float32(2.0) * amax) / np.float32(2**bits - 1)


def _strict_upper(L, d):
    if L is None:
        return None
    a = np.asarray(L, dtype=np.float64)
    assert a.shape == (d, d)
    return np.ascontiguousarray(np.triu(a, 1))


# --------------------------------------------------------------------------
# The rounding sweep [YAQA-4], scheduled row-major
# --------------------------------------------------------------------------
def sweep(W, LO, LI, scales, bits, rounding="nearest", seed=0, u=None, method="accum"):
    """Round W* entry by entry in row-major order under the two-sided rule.

    LO (m x m) / LI (n x n): only the strict upper triangles are used; None
    means the factor is zero (H = D, e.g. H_O = I). method="naive" evaluates
    the rule's three sums directly (O(m^2 n^2)); "accum" re-associates them
    (O(mn(m+n))). Returns codes (uint8), delta = W* - q, t (pre-rounding),
    eta = t - q, margin (steps to the nearest code boundary), clamped.
    """
    w = np.ascontiguousarray(W, dtype=np.float32)
    m, n = w.shape
    lo = _strict_upper(LO, m)
    li = _strict_upper(LI, n)
    if li is None:
        li = np.zeros((n, n))
    s = np.ascontiguousarray(scales, dtype=np.float32)
    assert s.shape == (m,)
    stoch = {"nearest": 0, "stochastic": 1}[rounding]
    uu = None if u is None else np.ascontiguousarray(u, dtype=np.float64)
    codes = np.zeros((m, n), dtype=np.uint8)
    delta, tpre, eta, margin = (np.zeros((m, n)) for _ in range(4))
    clamped = ctypes.c_int64(0)
    fn = {"naive": _load().orc_sweep_naive, "accum": _load().orc_sweep_accum}[method]
    rc = fn(m, n, _ptr(w), _ptr(lo), _ptr(li), _ptr(s), bits, stoch, seed & (2**64 - 1), _ptr(uu),
            _ptr(codes), _ptr(delta), _ptr(tpre), _ptr(eta), _ptr(margin), ctypes.byref(clamped))
    if rc != 0:
        raise MemoryError("oracle sweep failed")
    return dict(codes=codes, delta=delta, t=tpre, eta=eta, margin=margin, clamped=clamped.value)


def _quantise(y, Lq, u):
    """Codes and boundary margins for values y in grid steps (vectorised)."""
    if u is None:
        c = np.floor(y + 0.5)
        b = np.clip(np.floor(y), 0, Lq - 1) + 0.5
        mg = np.abs(y - b)
    else:
        v = y + u
        c = np.floor(v)
        mg = np.abs(v - np.clip(np.floor(v + 0.5), 1, Lq))
    return np.clip(c, 0, Lq).astype(np.int64), mg


def replay(W, LO, LI, scales, bits, codes, rounding="nearest", seed=0, u=None, band=1e-4,
           DO=None, DI=None):
    """Check candidate codes against the rule, feeding back the candidate's own error.

    With D^ = W* - s (c^ - Lq/2) rebuilt from the candidate's codes, the rule's
    pre-rounding value for every entry is t^ = W* + (A_O^T D^ A_I - D^) with
    A = L + I unit upper, because (A_O^T D^ A_I)_ij sums exactly the entries
    (k <= i, l <= j) the rule feeds back, plus D^_ij itself. An entry passes
    if its code equals Q(t^); a mismatch is a counted flip if the two codes
    are adjacent and y (or y + u) lies within `band` grid steps of the
    boundary between them; anything else is a failure.
    """
    w = np.asarray(W, dtype=np.float64)
    m, n = w.shape
    Lq = 2**bits - 1
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None]
    c_hat = np.asarray(codes).astype(np.int64)
    q = s * (c_hat - Lq / 2.0)
    dh = w - q
    ao = np.eye(m) if LO is None else np.triu(np.asarray(LO, np.float64), 1) + np.eye(m)
    ai = np.eye(n) if LI is None else np.triu(np.asarray(LI, np.float64), 1) + np.eye(n)
    e = ao.T @ dh @ ai
    t = w + (e - dh)
    y = t / s + Lq / 2.0
    if rounding == "stochastic":
        uu = uniform_matrix(seed, m, n) if u is None else np.asarray(u, np.float64)
    else:
        uu = None
    return _classify(y, Lq, uu, c_hat, band, t, q, s, DO, DI)


def replay_rows(W, LO, LI, scales, bits, codes, rows, rounding="nearest", seed=0, band=1e-4,
                batch=256):
    """replay() restricted to selected full rows (cheap at very large sizes).

    For row i: t^_i = W*_i + (a_i^T D^[:i+1]) A_I - D^_i with a_i column i of A_O
    restricted to rows 0..i, evaluated with the candidate's committed error D^.
    Rows are taken `batch` at a time: the a_i of a batch form one matrix, so the two
    products are matrix products (the same sums as the definition).
    """
    w = np.asarray(W, dtype=np.float32)
    m, n = w.shape
    Lq = 2**bits - 1
    rows = np.asarray(rows, dtype=np.int64)
    top = int(rows.max()) + 1
    s_all = np.asarray(scales, dtype=np.float32).astype(np.float64)
    # D^ = W* - s (c^ - Lq/2) for every row up to the last sampled one, formed once
    dh = np.empty((top, n), dtype=np.float64)
    for r0 in range(0, top, 1024):
        r1 = min(top, r0 + 1024)
        dh[r0:r1] = w[r0:r1].astype(np.float64) - s_all[r0:r1, None] * (
            np.asarray(codes[r0:r1]).astype(np.float64) - Lq / 2.0)
    li = None if LI is None else np.asarray(LI)
    E = np.empty((len(rows), n), dtype=np.float64)
    for b0 in range(0, len(rows), batch):
        rb = rows[b0:b0 + batch]
        # A[r, k] = L_O[k, i_r] for k < i_r, 1 at k = i_r, 0 beyond
        A = np.zeros((len(rb), top), dtype=np.float64)
        for r, i in enumerate(rb):
            if LO is not None and i > 0:
                A[r, :i] = np.asarray(LO[:i, i], dtype=np.float64)
            A[r, i] = 1.0
        V = A @ dh                                    # rows of A_O^T D^
        if li is not None:
            # V A_I = V + V L_I, with L_I taken 2048 columns at a time in fp64
            VL = np.empty_like(V)
            for j0 in range(0, n, 2048):
                blk = np.triu(np.asarray(li[:, j0:j0 + 2048], dtype=np.float64), 1 - j0)
                VL[:, j0:j0 + 2048] = V @ blk
            V += VL
        E[b0:b0 + len(rb)] = V
    dr = dh[rows]
    q = w[rows].astype(np.float64) - dr
    t = w[rows].astype(np.float64) + (E - dr)
    y = t / s_all[rows][:, None] + Lq / 2.0
    uu = None
    if rounding == "stochastic":
        uu = np.stack([_uniform_row(seed, i, n) for i in rows])
    return _classify(y, Lq, uu, np.asarray(codes)[rows].astype(np.int64), band,
                     t, q, s_all[rows][:, None], None, None)


def _uniform_row(seed, i, n):
    with np.errstate(over="ignore"):
        idx = np.arange(i * n + 1, i * n + n + 1, dtype=np.uint64)
        z = np.uint64(seed & (2**64 - 1)) + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return (z >> np.uint64(40)).astype(np.float64) * 2.0**-24


def _classify(y, Lq, u, c_hat, band, t, q, s, DO, DI):
    c_or, _ = _quantise(y, Lq, u)
    mism = c_or != c_hat
    v = y if u is None else y + u
    lo = np.minimum(c_or, c_hat)
    # boundary between codes k and k+1: y = k + 1/2 (nearest) or y + u = k + 1 (stochastic)
    bnd = lo + (0.5 if u is None else 1.0)
    dist = np.abs(v - bnd)
    flip = mism & (np.abs(c_or - c_hat) == 1) & (dist < band)
    bad = mism & ~flip
    eta = t - q
    out = dict(oracle_codes=c_or.astype(np.uint8), mismatches=int(mism.sum()),
               flips=int(flip.sum()), bad=int(bad.sum()),
               max_flip_margin=float(dist[flip].max()) if flip.any() else 0.0,
               bad_index=np.argwhere(bad)[:10], t=t, eta=eta, y=y)
    if DO is not None and DI is not None:
        out["loss"] = loss_identity(eta, DO, DI)
    return out


# --------------------------------------------------------------------------
# Proxy loss and bound [YAQA-4]
# --------------------------------------------------------------------------
def proxy_loss(delta, HO, HI) -> float:
    """vec(D)^T (H_O (x) H_I) vec(D) = tr(D H_I D^T H_O) for row-major vec."""
    d = np.asarray(delta, dtype=np.float64)
    ho = np.eye(d.shape[0]) if HO is None else np.asarray(HO, np.float64)
    return float(np.sum((d @ np.asarray(HI, np.float64)) * (ho @ d)))


def loss_identity(eta, DO, DI) -> float:
    """sum_ij D_O,i D_I,j eta_ij^2 (equals the proxy loss for the rule's codes)."""
    e = np.asarray(eta, dtype=np.float64)
    return float(np.asarray(DO, np.float64) @ (e * e) @ np.asarray(DI, np.float64))


def bound_terms(scales, DO, DI):
    """(sharp, page) bounds for unclamped nearest rounding, where |eta_ij| <= s_i / 2.

    sharp = sum_i D_O,i s_i^2 / 4 * tr(D_I); page = tr(D_I) tr(D_O) max_i s_i^2 / 4.
    """
    s = np.asarray(scales, dtype=np.float64)
    do = np.asarray(DO, np.float64)
    di = np.asarray(DI, np.float64)
    sharp = float(np.sum(do * s * s / 4.0) * np.sum(di))
    page = float(np.sum(di) * np.sum(do) * np.max(s) ** 2 / 4.0)
    return sharp, page


# --------------------------------------------------------------------------
# Whole chain on the CPU
# --------------------------------------------------------------------------
def pipeline(W, X, G, bits, rounding="nearest", seed=0, damp_rel=0.01, method="accum",
             one_sided=False):
    """Factors from X / G, damping, LDL, fp32 scales and the free-run sweep.

    one_sided=True takes H_O = I. Damping applies to both factors, so that
    factor is (1 + damp_rel) I: L_O = 0 and D_O = 1 + damp_rel (the codes are
    those of H_O = I; the proxy loss carries the factor 1 + damp_rel).
    """
    HI = damp(hessian(X), damp_rel)
    LI, DI = udu(HI) if HI.shape[0] <= 2048 else udu_lapack(HI)
    if one_sided:
        m = W.shape[0]
        HO = damp(np.eye(m), damp_rel)
        LO, DO = None, np.diag(HO).copy()
    else:
        HO = damp(hessian(G), damp_rel)
        LO, DO = udu(HO) if HO.shape[0] <= 2048 else udu_lapack(HO)
    s = row_scales(W, bits)
    res = sweep(W, LO, LI, s, bits, rounding, seed, method=method)
    res.update(HI=HI, HO=HO, LI=LI, LO=LO, DI=DI, DO=DO, scales=s)
    return res


# --------------------------------------------------------------------------
# Two-sided incoherence processing. [YAQA-4]: the error bound tightens as H_O
# and H_I become more incoherent, so, as for LDLQ, both Hessians are to be made
# incoherent before rounding. [KronQ] (bidirectional incoherence processing):
# the input-side random rotation is extended to the output side,
# W' = R_O W R_I^T. The construction of the rotation is a reading (see the
# module docstring): a randomised Hadamard transform, block-diagonal where n is
# not a power of two.
# --------------------------------------------------------------------------
def rht_signs(n: int, seed: int) -> np.ndarray:
    """s_i = -1 where the top bit of SplitMix64 output i of `seed` is set, else +1 (fp64)."""
    z = _splitmix_outputs(seed, n)
    return np.where((z >> np.uint64(63)) == np.uint64(1), -1.0, 1.0)


def rht_block(n: int) -> int:
    """2^k, the largest power of two dividing n."""
    return n & -n


def sylvester(b: int) -> np.ndarray:
    """The Sylvester Hadamard matrix of order b (a power of two), by doubling."""
    H = np.ones((1, 1))
    while H.shape[0] < b:
        H = np.block([[H, H], [H, -H]])
    return H


def rht_matrix(n: int, seed: int) -> np.ndarray:
    """U_n = (I_r (x) H_b / sqrt(b)) diag(s), b = rht_block(n), r = n / b, as a dense fp64 matrix."""
    b = rht_block(n)
    Hb = sylvester(b) / np.sqrt(b)
    B = np.kron(np.eye(n // b), Hb)
    return B * rht_signs(n, seed)[None, :]


def rht_apply(A, axis: int, seed: int, transpose: bool = False) -> np.ndarray:
    """axis 0: U A (U of order rows); axis 1: A U^T (U of order cols); U^T for transpose.

    The same U_n as rht_matrix, applied block by block (H_b is symmetric, so
    U^T = diag(s) (I_r (x) H_b / sqrt(b))); for orders too large for a dense U.
    """
    A = np.asarray(A, np.float64)
    X = A if axis == 0 else A.T  # the vectors to rotate are the columns of X
    n = X.shape[0]
    b = rht_block(n)
    Hb = sylvester(b) / np.sqrt(b)
    s = rht_signs(n, seed)[:, None]
    if not transpose:
        X = s * X
    Y = np.matmul(Hb, X.reshape(n // b, b, -1)).reshape(n, -1)
    if transpose:
        Y = s * Y
    return Y if axis == 0 else Y.T


def rotate_layer(W, HI, HO, seed_O: int, seed_I: int):
    """(U_O W U_I^T, U_I H_I U_I^T, U_O H_O U_O^T) in fp64; HO may be None (H_O = I stays I)."""
    m, n = W.shape
    UO = rht_matrix(m, seed_O)
    UI = rht_matrix(n, seed_I)
    W2 = UO @ np.asarray(W, np.float64) @ UI.T
    HI2 = UI @ np.asarray(HI, np.float64) @ UI.T
    HO2 = None if HO is None else UO @ np.asarray(HO, np.float64) @ UO.T
    return W2, HI2, HO2


# --------------------------------------------------------------------------
# Sketch B [YAQA-3]: one round of power iteration on the Hessian from the
# identity. With (H_I)_0 = (H_O)_0 = I the update
#   (H_I)_1 = E_s[G_s^T (H_O)_0 G_s] / ||(H_O)_0||_F^2,
#   (H_O)_1 = E_s[G_s (H_I)_0 G_s^T] / ||(H_I)_0||_F^2
# reduces to E_s[G_s^T G_s] / m and E_s[G_s G_s^T] / n, G_s the m x n weight
# gradient of sequence s.
# --------------------------------------------------------------------------
def sketch_b(grads):
    """(H_I, H_O) in fp64 from per-sequence gradients grads[s] (m x n each)."""
    G = [np.asarray(g, np.float64) for g in grads]
    S = len(G)
    m, n = G[0].shape
    HI = np.zeros((n, n))
    HO = np.zeros((m, m))
    for g in G:
        HI += g.T @ g
        HO += g @ g.T
    return HI / (S * m), HO / (S * n)


# --------------------------------------------------------------------------
# Sketch A [YAQA-3]: tokens are taken as independent, and the factors are
# updated in turn, each token weighted by the other factor's quadratic form:
#   (H_I)_i = E_t[x_t^T x_t <(H_O)_{i-1}, g_t^T g_t>] / ||(H_O)_{i-1}||_F^2
#   (H_O)_i = E_t[g_t^T g_t <(H_I)_{i-1}, x_t^T x_t>] / ||(H_I)_{i-1}||_F^2
# from (H_I)_0 = E[x^T x] and (H_O)_0 = I; <H, y^T y> = y H y^T. Both updates of
# an iteration use the previous iterates.
# --------------------------------------------------------------------------
def token_weights(Y, H=None) -> np.ndarray:
    """w_t = y_t H y_t^T / ||H||_F^2 for the rows y_t of Y (fp64); H None means the identity."""
    Y = np.asarray(Y, np.float64)
    if H is None:
        return np.sum(Y * Y, axis=1) / Y.shape[1]
    H = np.asarray(H, np.float64)
    return np.einsum("tk,kc,tc->t", Y, H, Y, optimize=True) / np.sum(H * H)


def weighted_hessian(X, w) -> np.ndarray:
    """sum_t w_t x_t^T x_t / T in fp64: one Sketch A update of a factor, the token
    weights w (T,) taken as given."""
    X = np.asarray(X, np.float64)
    w = np.asarray(w, np.float64)
    return (X * w[:, None]).T @ X / X.shape[0]


def sketch_a(X, G, iters: int = 3):
    """(H_I, H_O) after `iters` Sketch A iterations (fp64)."""
    X = np.asarray(X, np.float64)
    G = np.asarray(G, np.float64)
    T = X.shape[0]
    HI = X.T @ X / T
    HO = None
    for _ in range(iters):
        w = token_weights(G, HO)
        v = token_weights(X, HI)
        HI, HO = weighted_hessian(X, w), weighted_hessian(G, v)
    return HI, HO
