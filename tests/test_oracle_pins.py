"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each test here compares the oracle with something that is not the oracle: a
library routine, a textbook algorithm written out independently in this file,
a closed form, an invariant, or brute force. Sources, cited by page title and
section:
  YAQA article (news.43b.com.cn/a/479517), section 4: rounding rule, LDL form,
      error bound; section 2: Kronecker-factored Hessian H_O (x) H_I; the
      one-sided objective of LDLQ/GPTQ (section 1).
  "BaKron: Efficient Quantization with Kronecker-Factored Hessians", Abstract:
      the solver is GPTQ applied in the vectorised weight domain, scheduled with
      anti-diagonal parallelism and divide-and-conquer; modular in the quantiser.
  K-FAC tutorial (www.mlqm.cn/news/1313094), sections 2 and 5: Kronecker-product
      identities and the X^T X / N factor estimate.
  KronQ page (ai-feeds.com), method, bidirectional incoherence processing: the
      weight is rotated on both sides, W' = R_O W R_I^T, before quantisation.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers written independently of the oracle (test-local textbook versions)
# ----------------------------------------------------------------------------
def spd(d, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    k = 2 * d + 4
    z = rng.standard_normal((k, d)) * rng.lognormal(0.0, spread, size=d)[None, :]
    return z.T @ z / k + 0.05 * np.eye(d)


def q_nearest(y, Lq):
    return np.clip(np.floor(y + 0.5), 0, Lq)


def tiny_problem(m=12, n=10, seed=7, bits=2):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((m, n)) * 0.02).astype(np.float32)
    HO = spd(m, seed + 1)
    HI = spd(n, seed + 2)
    LO, DO = oracle.udu(HO)
    LI, DI = oracle.udu(HI)
    s = oracle.row_scales(w, bits)
    return w, HO, HI, LO, DO, LI, DI, s


def tiny_config():
    w, x, g = workloads.make_inputs("tiny")
    HI = oracle.damp(oracle.hessian(x))
    HO = oracle.damp(oracle.hessian(g))
    LI, DI = oracle.udu(HI)
    LO, DO = oracle.udu(HO)
    return w, HO, HI, LO, DO, LI, DI


def codes_equal_or_tie(a, b, margin, tol=1e-9):
    diff = a != b
    assert np.all(margin[diff] < tol), (int(diff.sum()), margin[diff][:5])


# ----------------------------------------------------------------------------
# random draws
# ----------------------------------------------------------------------------
def test_splitmix64_published_seed0_outputs():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "splitmix64_seed0.txt"))
            if ln.strip() and not ln.startswith("#")]
    for idx, val in rows:
        assert oracle.splitmix64(0, int(idx)) == int(val, 16)


def test_uniform_matrix_matches_c_and_is_uniform():
    u = oracle.uniform_matrix(1234, 64, 96)
    for (i, j) in [(0, 0), (3, 7), (63, 95), (10, 50)]:
        z = oracle.splitmix64(1234, i * 96 + j)
        assert u[i, j] == (z >> 40) * 2.0**-24
    big = oracle.uniform_matrix(99, 512, 512).ravel()
    assert big.min() >= 0.0 and big.max() < 1.0
    hist = np.histogram(big, bins=16, range=(0, 1))[0]
    exp = big.size / 16
    chi2 = float(np.sum((hist - exp) ** 2 / exp))
    assert chi2 < 60.0  # 15 dof; p ~ 1e-7


# ----------------------------------------------------------------------------
# P1: LDL form H = (L + I) D (L + I)^T, L strictly upper
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("d,seed", [(1, 0), (2, 1), (17, 2), (64, 3), (200, 4)])
def test_udu_reconstructs_and_matches_lapack(d, seed):
    H = spd(d, seed, spread=1.5)
    L, D = oracle.udu(H)
    assert np.all(np.tril(L) == 0.0)
    assert np.all(D > 0)
    A = L + np.eye(d)
    rec = A @ np.diag(D) @ A.T
    assert np.linalg.norm(rec - H) / np.linalg.norm(H) < 1e-13
    # LAPACK route: Cholesky of the index-reversed matrix, mapped back
    c = np.linalg.cholesky(H[::-1, ::-1])[::-1, ::-1]
    dc = np.diag(c)
    assert np.allclose(D, dc * dc, rtol=1e-11, atol=0)
    assert np.allclose(L, np.triu(c / dc[None, :], 1), rtol=1e-9, atol=1e-11)
    L2, D2 = oracle.udu_lapack(H)
    assert np.allclose(L2, L, rtol=1e-9, atol=1e-11) and np.allclose(D2, D, rtol=1e-11)


def test_udu_reports_first_bad_pivot():
    H = spd(8, 5)
    H[5, 5] = -1.0
    with pytest.raises(ValueError, match="pivot 5"):
        oracle.udu(H)


def test_udu_only_reads_upper_triangle():
    H = spd(9, 11)
    Hb = np.triu(H) + np.tril(np.full_like(H, 123.0), -1)
    L1, D1 = oracle.udu(H)
    L2, D2 = oracle.udu(Hb)
    assert np.array_equal(L1, L2) and np.array_equal(D1, D2)


# ----------------------------------------------------------------------------
# P12: Hessian accumulation H = X^T X / T
# ----------------------------------------------------------------------------
def test_hessian_is_mean_outer_product():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((37, 9)).astype(np.float32)
    H = oracle.hessian(X)
    outer = sum(np.outer(r.astype(np.float64), r.astype(np.float64)) for r in X) / 37
    assert np.allclose(H, outer, rtol=1e-14, atol=1e-15)
    assert np.array_equal(H, H.T)
    assert np.linalg.eigvalsh(H).min() > -1e-12
    rows, cols = [0, 3, 8], [5, 3, 1]
    assert np.allclose(oracle.hessian_entries(X, rows, cols), H[rows, cols], rtol=1e-14)


def test_damping_uses_undamped_mean_diagonal():
    H = np.diag([1.0, 2.0, 3.0, 6.0])
    Hd = oracle.damp(H, 0.01)
    assert np.allclose(np.diag(Hd), [1.03, 2.03, 3.03, 6.03])


# ----------------------------------------------------------------------------
# naive (rule written out) vs accumulator form
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("shape,bits,rounding", [((64, 64), 2, "nearest"), ((40, 72), 3, "nearest"),
                                                 ((33, 17), 2, "stochastic"), ((1, 5), 4, "nearest"),
                                                 ((6, 1), 1, "nearest")])
def test_naive_and_accumulator_sweeps_agree(shape, bits, rounding):
    m, n = shape
    w, HO, HI, LO, DO, LI, DI, s = tiny_problem(m, n, seed=m * n, bits=bits)
    a = oracle.sweep(w, LO, LI, s, bits, rounding, seed=5, method="naive")
    b = oracle.sweep(w, LO, LI, s, bits, rounding, seed=5, method="accum")
    assert np.array_equal(a["codes"], b["codes"])
    assert np.allclose(a["t"], b["t"], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# P2: loss identity tr(D H_I D^T H_O) = sum D_O,i D_I,j eta_ij^2
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_loss_identity_on_tiny_config(rounding):
    w, HO, HI, LO, DO, LI, DI = tiny_config()
    s = oracle.row_scales(w, 2)
    r = oracle.sweep(w, LO, LI, s, 2, rounding, seed=4000)
    lhs = oracle.proxy_loss(r["delta"], HO, HI)
    rhs = oracle.loss_identity(r["eta"], DO, DI)
    assert abs(lhs - rhs) <= 1e-10 * abs(lhs)


def test_loss_identity_fails_for_codes_not_from_the_rule():
    # the identity is a property of the rule's codes, not of arbitrary codes
    w, HO, HI, LO, DO, LI, DI, s = tiny_problem(10, 8, seed=21)
    r = oracle.sweep(w, LO, LI, s, 2)
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 4, size=w.shape)
    q = s[:, None].astype(np.float64) * (codes - 1.5)
    delta = w - q
    # eta of these codes under the rule's own pre-rounding values
    rp = oracle.replay(w, LO, LI, s, 2, codes)
    lhs = oracle.proxy_loss(delta, HO, HI)
    assert abs(lhs - oracle.loss_identity(rp["eta"], DO, DI)) < 1e-10 * lhs  # replay's t is exact
    assert abs(lhs - oracle.loss_identity(r["eta"], DO, DI)) > 1e-3 * lhs


def test_kron_vec_equals_trace_form():
    # K-FAC tutorial section 2: (A (x) B) vec(V) = vec(B V A^T) for column-major vec;
    # with row-major vec the same product is H_O V H_I, so the quadratic form is a trace.
    rng = np.random.default_rng(1)
    HO, HI = spd(5, 1), spd(4, 2)
    V = rng.standard_normal((5, 4))
    vr = V.ravel()  # row-major vec
    assert np.isclose(vr @ np.kron(HO, HI) @ vr, oracle.proxy_loss(V, HO, HI), rtol=1e-13)
    vc = V.ravel(order="F")  # column-major vec
    assert np.allclose(np.kron(HI, HO) @ vc, (HO @ V @ HI.T).ravel(order="F"))


# ----------------------------------------------------------------------------
# P3: error bound (nearest, no clamping): L <= sum_i D_O,i s_i^2/4 tr(D_I) <= page form
# ----------------------------------------------------------------------------
def headroom_scales(w, bits, factor=1.5):
    # scales with room beyond the absmax, so that feedback never pushes a value
    # off the grid (the bound assumes |eta| <= s/2, i.e. no clamping)
    return (np.float32(2.0 * factor) * np.max(np.abs(w), axis=1)) / np.float32(2**bits - 1)


@pytest.mark.parametrize("bits", [2, 3, 4, 6])
def test_error_bound_without_clamping(bits):
    w, HO, HI, LO, DO, LI, DI = tiny_config()
    s = headroom_scales(w, bits)
    r = oracle.sweep(w, LO, LI, s, bits)
    assert r["clamped"] == 0
    assert np.all(np.abs(r["eta"]) <= s[:, None] / 2 * (1 + 1e-12))
    loss = oracle.proxy_loss(r["delta"], HO, HI)
    sharp, page = oracle.bound_terms(s, DO, DI)
    assert loss <= sharp <= page


def test_error_bound_on_random_factors():
    w, HO, HI, LO, DO, LI, DI, _ = tiny_problem(12, 10, seed=3, bits=4)
    s = headroom_scales(w, 4, 2.0)
    r = oracle.sweep(w, LO, LI, s, 4)
    assert r["clamped"] == 0
    loss = oracle.proxy_loss(r["delta"], HO, HI)
    sharp, page = oracle.bound_terms(s, DO, DI)
    assert loss <= sharp <= page


# ----------------------------------------------------------------------------
# P4: GPTQ/LDLQ in the vectorised weight domain on H_O (x) H_I gives the same codes
# ----------------------------------------------------------------------------
def ldlq_vectorised(w, HO, HI, s, bits):
    m, n = w.shape
    Lq = 2**bits - 1
    H = np.kron(HO, HI)  # row-major vec: p = i * n + j
    c = np.linalg.cholesky(H[::-1, ::-1])[::-1, ::-1]
    U = np.triu(c / np.diag(c)[None, :], 1)  # strictly upper factor of H
    wv = w.astype(np.float64).ravel()
    sv = np.repeat(s.astype(np.float64), n)
    err = np.zeros(m * n)
    codes = np.zeros(m * n, dtype=np.int64)
    for p in range(m * n):
        t = wv[p] + U[:p, p] @ err[:p]
        cp = q_nearest(t / sv[p] + Lq / 2, Lq)
        codes[p] = cp
        err[p] = wv[p] - sv[p] * (cp - Lq / 2)
    return codes.reshape(m, n)


@pytest.mark.parametrize("case", ["random", "tiny_config"])
def test_matches_ldlq_in_vectorised_domain(case):
    if case == "random":
        w, HO, HI, LO, DO, LI, DI, s = tiny_problem(14, 11, seed=42, bits=2)
        bits = 2
    else:
        w, HO, HI, LO, DO, LI, DI = tiny_config()
        bits = 2
        s = oracle.row_scales(w, bits)
    ref = ldlq_vectorised(w, HO, HI, s, bits)
    r = oracle.sweep(w, LO, LI, s, bits)
    codes_equal_or_tie(r["codes"], ref, r["margin"])


# ----------------------------------------------------------------------------
# P5: H_O = I reduces to one-sided LDLQ = GPTQ (Frantar et al. 2022)
# ----------------------------------------------------------------------------
def gptq(w, HI, s, bits):
    """GPTQ column loop with the upper Cholesky factor of H^-1."""
    Lq = 2**bits - 1
    m, n = w.shape
    U = np.linalg.cholesky(np.linalg.inv(HI)).T  # H^-1 = U^T U
    W = w.astype(np.float64).copy()
    sc = s.astype(np.float64)
    codes = np.zeros((m, n), dtype=np.int64)
    for j in range(n):
        c = q_nearest(W[:, j] / sc + Lq / 2, Lq)
        codes[:, j] = c
        err = (W[:, j] - sc * (c - Lq / 2)) / U[j, j]
        W[:, j + 1:] -= err[:, None] * U[j, j + 1:][None, :]
    return codes


@pytest.mark.parametrize("shape,bits", [((64, 64), 2), ((30, 48), 3)])
def test_one_sided_reduces_to_gptq(shape, bits):
    m, n = shape
    w, x, g = workloads.make_inputs("tiny", m=m, n=n)
    HI = oracle.damp(oracle.hessian(x))
    LI, DI = oracle.udu(HI)
    HO = oracle.damp(np.eye(m))  # H_O = I, damped: 1.01 I has L_O = 0
    LO, DO = oracle.udu(HO)
    assert np.all(LO == 0)
    s = oracle.row_scales(w, bits)
    r = oracle.sweep(w, LO, LI, s, bits)
    r0 = oracle.sweep(w, None, LI, s, bits)
    assert np.array_equal(r["codes"], r0["codes"])
    codes_equal_or_tie(r["codes"], gptq(w, HI, s, bits), r["margin"], tol=1e-8)


# ----------------------------------------------------------------------------
# P6: diagonal Hessians (L = 0) reduce to round-to-nearest
# ----------------------------------------------------------------------------
def test_diagonal_hessians_give_round_to_nearest():
    w, *_ = tiny_problem(20, 30, seed=9)
    s = oracle.row_scales(w, 3)
    r = oracle.sweep(w, np.zeros((20, 20)), np.zeros((30, 30)), s, 3)
    rtn = q_nearest(w.astype(np.float64) / s[:, None].astype(np.float64) + 3.5, 7)
    assert np.array_equal(r["codes"], rtn)
    # the absmax entries of each row land on the outer codes
    for i in range(20):
        jmax = np.argmax(np.abs(w[i]))
        assert r["codes"][i, jmax] == (7 if w[i, jmax] > 0 else 0)


# ----------------------------------------------------------------------------
# P7: independence of the visiting order (anti-diagonal / quadrant schedules)
# ----------------------------------------------------------------------------
def sweep_in_order(w, LO, LI, s, bits, order):
    """Evaluate the rule entry by entry in the given order; unknown entries are NaN,
    so a non-topological order poisons the result."""
    m, n = w.shape
    Lq = 2**bits - 1
    D = np.full((m, n), np.nan)
    codes = np.zeros((m, n), dtype=np.int64)
    AO, AI = np.triu(LO, 1), np.triu(LI, 1)
    for (i, j) in order:
        a, b = AO[:i, i], AI[:j, j]
        f = a @ D[:i, :j] @ b + a @ D[:i, j] + D[i, :j] @ b
        t = float(w[i, j]) + f
        c = q_nearest(t / float(s[i]) + Lq / 2, Lq)
        codes[i, j] = c
        D[i, j] = float(w[i, j]) - float(s[i]) * (c - Lq / 2)
    assert not np.isnan(D).any()
    return codes


def sweep_column_major_accumulator(w, LO, LI, s, bits):
    """Column-major order with the transposed accumulator:
    R_ij = sum_{l<j} D_il L_I[l,j], G'_ij = R_ij + D_ij, t_ij = W_ij + R_ij + sum_{k<i} L_O[k,i] G'_kj."""
    m, n = w.shape
    Lq = 2**bits - 1
    D = np.zeros((m, n))
    Gp = np.zeros((m, n))
    codes = np.zeros((m, n), dtype=np.int64)
    AO, AI = np.triu(LO, 1), np.triu(LI, 1)
    for j in range(n):
        R = D[:, :j] @ AI[:j, j]
        for i in range(m):
            t = float(w[i, j]) + R[i] + AO[:i, i] @ Gp[:i, j]
            c = q_nearest(t / float(s[i]) + Lq / 2, Lq)
            codes[i, j] = c
            D[i, j] = float(w[i, j]) - float(s[i]) * (c - Lq / 2)
            Gp[i, j] = R[i] + D[i, j]
    return codes


def sweep_quadrants(w, LO, LI, s, bits):
    """Recursive 2x2 quadrant construction: solve Q11, then Q12 and Q21 with the
    offsets Q11 induces, then Q22 with the offsets of Q11, Q12 and Q21."""
    m, n = w.shape
    Lq = 2**bits - 1
    AO = np.triu(LO, 1) + np.eye(m)
    AI = np.triu(LI, 1) + np.eye(n)
    D = np.zeros((m, n))
    codes = np.zeros((m, n), dtype=np.int64)

    def solve(r0, r1, c0, c1, off):
        if r1 - r0 == 1 and c1 - c0 == 1:
            t = float(w[r0, c0]) + off[0, 0]
            c = q_nearest(t / float(s[r0]) + Lq / 2, Lq)
            codes[r0, c0] = c
            D[r0, c0] = float(w[r0, c0]) - float(s[r0]) * (c - Lq / 2)
            return
        rm = r0 + max(1, (r1 - r0) // 2) if r1 - r0 > 1 else r1
        cm = c0 + max(1, (c1 - c0) // 2) if c1 - c0 > 1 else c1
        R1, R2 = slice(r0, rm), slice(rm, r1)
        C1, C2 = slice(c0, cm), slice(cm, c1)
        o = off
        a, b = rm - r0, cm - c0
        solve(r0, rm, c0, cm, o[:a, :b])
        if cm < c1:
            o12 = o[:a, b:] + AO[R1, R1].T @ D[R1, C1] @ AI[C1, C2]
            solve(r0, rm, cm, c1, o12)
        if rm < r1:
            o21 = o[a:, :b] + AO[R1, R2].T @ D[R1, C1] @ AI[C1, C1]
            solve(rm, r1, c0, cm, o21)
        if rm < r1 and cm < c1:
            o22 = (o[a:, b:] + AO[R1, R2].T @ (D[R1, C1] @ AI[C1, C2] + D[R1, C2] @ AI[C2, C2])
                   + AO[R2, R2].T @ D[R2, C1] @ AI[C1, C2])
            solve(rm, r1, cm, c1, o22)

    solve(0, m, 0, n, np.zeros((m, n)))
    return codes


@pytest.mark.parametrize("shape", [(16, 16), (13, 9), (7, 20)])
def test_order_independence(shape):
    m, n = shape
    w, HO, HI, LO, DO, LI, DI, s = tiny_problem(m, n, seed=100 + m, bits=2)
    ref = oracle.sweep(w, LO, LI, s, 2)
    mg = ref["margin"]
    anti = [(i, d - i) for d in range(m + n - 1) for i in range(m) if 0 <= d - i < n]
    colmajor = [(i, j) for j in range(n) for i in range(m)]
    # a random topological order: repeatedly pick a random ready entry
    rng = np.random.default_rng(m * n)
    done = np.zeros((m, n), bool)
    ready = {(0, 0)}
    rand = []
    while ready:
        e = sorted(ready)[rng.integers(len(ready))]
        ready.remove(e)
        rand.append(e)
        i, j = e
        done[i, j] = True
        for (a, b) in ((i + 1, j), (i, j + 1)):
            if a < m and b < n and (a == 0 or done[a - 1, b]) and (b == 0 or done[a, b - 1]):
                ready.add((a, b))
    for order in (anti, colmajor, rand):
        codes_equal_or_tie(ref["codes"], sweep_in_order(w, LO, LI, s, 2, order), mg)
    codes_equal_or_tie(ref["codes"], sweep_column_major_accumulator(w, LO, LI, s, 2), mg)
    codes_equal_or_tie(ref["codes"], sweep_quadrants(w, LO, LI, s, 2), mg)


def test_order_check_detects_non_topological_order():
    w, HO, HI, LO, DO, LI, DI, s = tiny_problem(4, 4, seed=1)
    bad = [(1, 1)] + [(i, j) for i in range(4) for j in range(4) if (i, j) != (1, 1)]
    with pytest.raises((AssertionError, ValueError)):
        sweep_in_order(w, LO, LI, s, 2, bad)


# ----------------------------------------------------------------------------
# P8: brute force over all 4^9 code matrices at m = n = 3, 2 bits
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_bruteforce_3x3(seed):
    w, HO, HI, LO, DO, LI, DI, _ = tiny_problem(3, 3, seed=seed, bits=2)
    s = headroom_scales(w, 2, 2.0)
    r = oracle.sweep(w, LO, LI, s, 2)
    K = np.kron(HO, HI)
    allc = np.array(list(itertools.product(range(4), repeat=9)), dtype=np.float64)
    sv = np.repeat(s.astype(np.float64), 3)
    dv = w.astype(np.float64).ravel()[None, :] - sv[None, :] * (allc - 1.5)
    losses = np.einsum("ap,pq,aq->a", dv, K, dv)
    best = losses.min()
    mine = oracle.proxy_loss(r["delta"], HO, HI)
    assert best <= mine * (1 + 1e-12)
    # the loss of the rule's codes appears in the enumeration
    idx = int(np.dot(r["codes"].ravel().astype(np.int64), 4 ** np.arange(8, -1, -1)))
    assert np.isclose(losses[idx], mine, rtol=1e-12)
    assert r["clamped"] == 0
    sharp, page = oracle.bound_terms(s, DO, DI)
    assert mine <= sharp <= page


# ----------------------------------------------------------------------------
# P9: transposition swaps the roles of H_O and H_I (one common scale)
# ----------------------------------------------------------------------------
def test_transpose_symmetry():
    w, HO, HI, LO, DO, LI, DI, _ = tiny_problem(15, 11, seed=77)
    sc = np.float32(2.0 * np.abs(w).max() / 3.0)
    r = oracle.sweep(w, LO, LI, np.full(15, sc, np.float32), 2)
    rt = oracle.sweep(np.ascontiguousarray(w.T), LI, LO, np.full(11, sc, np.float32), 2)
    codes_equal_or_tie(r["codes"], rt["codes"].T, r["margin"])


# ----------------------------------------------------------------------------
# P10: scaling H_O and H_I leaves L, hence the codes, unchanged
# ----------------------------------------------------------------------------
def test_hessian_scale_invariance():
    w, HO, HI, LO, DO, LI, DI, s = tiny_problem(12, 9, seed=5)
    LO2, DO2 = oracle.udu(7.5 * HO)
    LI2, DI2 = oracle.udu(0.01 * HI)
    assert np.allclose(LO2, LO, atol=1e-12) and np.allclose(DO2, 7.5 * DO, rtol=1e-12)
    r1 = oracle.sweep(w, LO, LI, s, 2)
    r2 = oracle.sweep(w, LO2, LI2, s, 2)
    codes_equal_or_tie(r1["codes"], r2["codes"], r1["margin"])


# ----------------------------------------------------------------------------
# P11: stochastic rounding
# ----------------------------------------------------------------------------
def test_stochastic_with_half_is_nearest():
    w, HO, HI, LO, DO, LI, DI, s = tiny_problem(10, 12, seed=8)
    a = oracle.sweep(w, LO, LI, s, 2, "nearest")
    b = oracle.sweep(w, LO, LI, s, 2, "stochastic", u=np.full((10, 12), 0.5))
    assert np.array_equal(a["codes"], b["codes"])


def test_stochastic_rounding_is_unbiased():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((4, 8)) * 0.02).astype(np.float32)
    s = oracle.row_scales(w, 2)
    qs = []
    for seed in range(400):
        r = oracle.sweep(w, np.zeros((4, 4)), np.zeros((8, 8)), s, 2, "stochastic", seed=seed)
        assert r["clamped"] == 0
        qs.append(s[:, None].astype(np.float64) * (r["codes"] - 1.5))
    qs = np.array(qs)
    sigma = s[:, None].astype(np.float64) / 2 / np.sqrt(400)
    assert np.all(np.abs(qs.mean(0) - w) < 5 * sigma)


# ----------------------------------------------------------------------------
# replay checker
# ----------------------------------------------------------------------------
def test_replay_accepts_own_codes_and_flags_planted_errors():
    w, HO, HI, LO, DO, LI, DI = tiny_config()
    s = oracle.row_scales(w, 2)
    r = oracle.sweep(w, LO, LI, s, 2)
    rp = oracle.replay(w, LO, LI, s, 2, r["codes"], DO=DO, DI=DI)
    assert rp["mismatches"] == 0 and rp["bad"] == 0
    assert abs(rp["loss"] - oracle.proxy_loss(r["delta"], HO, HI)) < 1e-10 * rp["loss"]
    # a planted wrong code is caught even though later entries follow it consistently
    bad = r["codes"].copy()
    i, j = 20, 30
    bad[i, j] = (bad[i, j] + 1) % 4
    rp2 = oracle.replay(w, LO, LI, s, 2, bad)
    assert rp2["bad"] >= 1 and [i, j] in rp2["bad_index"].tolist()
    # replay restricted to rows agrees with the full replay
    rows = [0, 20, 63]
    rr = oracle.replay_rows(w, LO, LI, s, 2, bad, rows)
    assert np.allclose(rr["t"], rp2["t"][rows], rtol=1e-12, atol=1e-14)


def test_replay_counts_boundary_flips():
    # W = [-1, 1.5] at 2 bits has s = 1 exactly and y(-1) = 0.5, the boundary between
    # codes 0 and 1: either code is acceptable there, and the other one is a counted flip
    w = np.array([[-1.0, 1.5]], dtype=np.float32)
    s = oracle.row_scales(w, 2)
    assert s[0] == np.float32(1.0)
    r = oracle.sweep(w, None, None, s, 2)
    assert r["codes"].tolist() == [[1, 3]] and r["margin"][0, 0] == 0.0
    rp = oracle.replay(w, None, None, s, 2, np.array([[0, 3]]))
    assert rp["flips"] == 1 and rp["bad"] == 0 and rp["max_flip_margin"] == 0.0
    rp = oracle.replay(w, None, None, s, 2, np.array([[2, 3]]))
    assert rp["flips"] == 0 and rp["bad"] == 1


# ----------------------------------------------------------------------------
# sensitivity: plausible mistakes in the rule are caught by the pins above
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("mutation", ["drop_cross", "drop_column", "sign", "row_of_LO",
                                      "swap_factors", "lower_ldl_reading"])
def test_pins_catch_mutated_rules(mutation):
    # each mutation is a plausible slip in writing the rule; the vectorised-domain
    # LDLQ reference (P4) must disagree with every one of them
    w, HO, HI, LO, DO, LI, DI, s = tiny_problem(12, 12, seed=42, bits=2)
    m, n = w.shape
    AO, AI = np.triu(LO, 1), np.triu(LI, 1)
    if mutation == "row_of_LO":
        AO = AO.T            # a_i taken as a row of L_O instead of a column
    if mutation == "swap_factors":
        AO, AI = AI, AO      # H_O and H_I exchanged
    if mutation == "lower_ldl_reading":
        # the other reading of the factorisation paragraph: H = (L + I) D (L + I)^T with
        # L strictly LOWER (top-down LDL^T), its transpose used as the upper factor
        def lower_ldl_t(H):
            c = np.linalg.cholesky(H)
            return np.tril(c / np.diag(c)[None, :], -1).T
        AO, AI = lower_ldl_t(HO), lower_ldl_t(HI)
    D = np.zeros((m, n))
    codes = np.zeros((m, n), dtype=np.int64)
    for i in range(m):
        for j in range(n):
            a, b = AO[:i, i], AI[:j, j]
            cross = a @ D[:len(a), :len(b)] @ b
            col = a @ D[:len(a), j]
            row = D[i, :len(b)] @ b
            if mutation == "drop_cross":
                cross = 0.0
            if mutation == "drop_column":
                col = 0.0
            f = cross + col + row
            if mutation == "sign":
                f = -f
            t = float(w[i, j]) + f
            c = q_nearest(t / float(s[i]) + 1.5, 3)
            codes[i, j] = c
            D[i, j] = float(w[i, j]) - float(s[i]) * (c - 1.5)
    ref = ldlq_vectorised(w, HO, HI, s, 2)
    assert not np.array_equal(codes, ref)


# ----------------------------------------------------------------------------
# incoherence rotation (KronQ, bidirectional incoherence processing; YAQA
# article, section 4: incoherence processing of both Hessians before rounding)
# ----------------------------------------------------------------------------
def test_rht_signs_follow_the_published_splitmix64_outputs():
    # the top bits of the golden seed-0 outputs e220..., 6e78..., 06c4...
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "splitmix64_seed0.txt"))
            if ln.strip() and not ln.startswith("#")]
    want = [-1.0 if int(val, 16) >> 63 else 1.0 for _, val in rows]
    assert list(oracle.rht_signs(len(want), 0)) == want


@pytest.mark.parametrize("b", [1, 2, 4, 64, 512])
def test_sylvester_matches_scipy_hadamard(b):
    import scipy.linalg
    assert np.array_equal(oracle.sylvester(b), scipy.linalg.hadamard(b).astype(np.float64))


@pytest.mark.parametrize("n,seed", [(1, 3), (2, 3), (12, 7), (64, 0), (100, 11), (448, 5), (3, 9)])
def test_rht_matrix_is_orthogonal_and_block_hadamard(n, seed):
    import scipy.linalg
    U = oracle.rht_matrix(n, seed)
    assert np.abs(U.T @ U - np.eye(n)).max() < 1e-12
    # block structure: the largest power of two dividing n, written out here
    b = 1
    while n % (2 * b) == 0:
        b *= 2
    assert oracle.rht_block(n) == b
    s = oracle.rht_signs(n, seed)
    Hb = scipy.linalg.hadamard(b) / np.sqrt(b)
    for r in range(n // b):
        blk = slice(r * b, (r + 1) * b)
        assert np.allclose(U[blk, blk], Hb * s[None, blk], atol=1e-15)
        off = np.ones(n, bool)
        off[blk] = False
        assert np.all(U[blk][:, off] == 0.0)


def test_rotation_keeps_the_proxy_loss_and_the_spectrum():
    # tr(D H_I D^T H_O) is unchanged when D, H_I and H_O are rotated together, and
    # each Hessian keeps its eigenvalues
    rng = np.random.default_rng(4)
    m, n = 24, 40
    D = rng.standard_normal((m, n))
    HI, HO = spd(n, 1), spd(m, 2)
    D2, HI2, HO2 = oracle.rotate_layer(D, HI, HO, 31, 32)
    l1 = np.trace(D @ HI @ D.T @ HO)
    l2 = np.trace(D2 @ HI2 @ D2.T @ HO2)
    assert abs(l1 - l2) <= 1e-10 * abs(l1)
    assert np.allclose(np.linalg.eigvalsh(HI2), np.linalg.eigvalsh(HI), rtol=1e-10)
    assert np.allclose(np.linalg.eigvalsh(HO2), np.linalg.eigvalsh(HO), rtol=1e-10)
    # the weight is rotated on the left by U_O and on the right by U_I^T, not transposed
    UO, UI = oracle.rht_matrix(m, 31), oracle.rht_matrix(n, 32)
    assert np.allclose(UO.T @ D2 @ UI, D, atol=1e-12)


def test_rotated_rounding_keeps_the_loss_identity():
    # rounding the rotated problem is ordinary BaKron rounding: the loss identity
    # (sum D_O D_I eta^2 = tr(Delta H_I Delta^T H_O)) holds on the rotated factors
    w = workloads.make_w(32, 48, 3)
    HI = oracle.damp(spd(48, 5))
    HO = oracle.damp(spd(32, 6))
    W2, HI2, HO2 = oracle.rotate_layer(w, HI, HO, 1, 2)
    LI, DI = oracle.udu(HI2)
    LO, DO = oracle.udu(HO2)
    s = oracle.row_scales(W2.astype(np.float32), 3)
    res = oracle.sweep(W2.astype(np.float32), LO, LI, s, 3)
    lhs = oracle.loss_identity(res["eta"], DO, DI)
    rhs = oracle.proxy_loss(res["delta"], HO2, HI2)
    assert abs(lhs - rhs) <= 1e-9 * abs(rhs)


@pytest.mark.parametrize("shape", [(12, 20), (7, 64), (96, 5)])
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("transpose", [False, True])
def test_rht_apply_is_the_dense_rotation(shape, axis, transpose):
    rng = np.random.default_rng(8)
    A = rng.standard_normal(shape)
    U = oracle.rht_matrix(shape[axis], 77)
    if transpose:
        U = U.T
    want = U @ A if axis == 0 else A @ U.T
    assert np.allclose(oracle.rht_apply(A, axis, 77, transpose), want, atol=1e-12)


# ----------------------------------------------------------------------------
# Sketch B (YAQA article, section 3): H_I = E_s[G_s^T G_s] / m, H_O = E_s[G_s G_s^T] / n
# ----------------------------------------------------------------------------
def test_sketch_b_traces_are_the_mean_squared_gradient_norm():
    rng = np.random.default_rng(12)
    grads = [rng.standard_normal((6, 9)) * rng.lognormal(0, 1, size=9) for _ in range(5)]
    HI, HO = oracle.sketch_b(grads)
    fro2 = np.mean([np.sum(g * g) for g in grads])
    assert abs(6 * np.trace(HI) - fro2) <= 1e-12 * fro2
    assert abs(9 * np.trace(HO) - fro2) <= 1e-12 * fro2
    for H in (HI, HO):
        assert np.array_equal(H, H.T) or np.abs(H - H.T).max() <= 1e-14 * np.abs(H).max()
        assert np.linalg.eigvalsh(H).min() >= -1e-12 * np.abs(H).max()


def test_sketch_b_rank_one_gradients():
    # G_s = u_s v_s^T: G^T G = |u|^2 v v^T and G G^T = |v|^2 u u^T
    rng = np.random.default_rng(13)
    us = [rng.standard_normal(7) for _ in range(3)]
    vs = [rng.standard_normal(4) for _ in range(3)]
    HI, HO = oracle.sketch_b([np.outer(u, v) for u, v in zip(us, vs)])
    HI_want = sum(np.dot(u, u) * np.outer(v, v) for u, v in zip(us, vs)) / (3 * 7)
    HO_want = sum(np.dot(v, v) * np.outer(u, u) for u, v in zip(us, vs)) / (3 * 4)
    assert np.allclose(HI, HI_want, rtol=1e-13, atol=1e-15)
    assert np.allclose(HO, HO_want, rtol=1e-13, atol=1e-15)


def test_sketch_b_brute_force():
    rng = np.random.default_rng(14)
    grads = [rng.standard_normal((3, 4)) for _ in range(2)]
    HI, HO = oracle.sketch_b(grads)
    for i in range(4):
        for j in range(4):
            want = sum(g[a][i] * g[a][j] for g in grads for a in range(3)) / (2 * 3)
            assert abs(HI[i, j] - want) <= 1e-13
    for i in range(3):
        for j in range(3):
            want = sum(g[i][b] * g[j][b] for g in grads for b in range(4)) / (2 * 4)
            assert abs(HO[i, j] - want) <= 1e-13


# ----------------------------------------------------------------------------
# Sketch A (YAQA article, section 3): alternating factor estimates with
# per-token weights <H, y^T y> / ||H||_F^2, from H_I = E[x^T x] and H_O = I
# ----------------------------------------------------------------------------
def test_sketch_a_first_step_with_equal_gradient_norms():
    # with ||g_t|| the same for every token the first H_I is E[x^T x] scaled by ||g||^2 / m
    rng = np.random.default_rng(21)
    T, n, m = 200, 6, 5
    X = rng.standard_normal((T, n))
    G = rng.standard_normal((T, m))
    G *= 3.0 / np.linalg.norm(G, axis=1, keepdims=True)
    HI, _ = oracle.sketch_a(X, G, 1)
    assert np.allclose(HI, (9.0 / m) * (X.T @ X / T), rtol=1e-12)


def test_sketch_a_brute_force_two_iterations():
    rng = np.random.default_rng(22)
    T, n, m = 7, 3, 4
    X = rng.standard_normal((T, n))
    G = rng.standard_normal((T, m))

    def quad(y, H):
        return sum(y[a] * H[a][b] * y[b] for a in range(len(y)) for b in range(len(y)))

    def fro2(H):
        return sum(H[a][b] ** 2 for a in range(len(H)) for b in range(len(H)))

    HI = [[sum(X[t][a] * X[t][b] for t in range(T)) / T for b in range(n)] for a in range(n)]
    HO = [[1.0 if a == b else 0.0 for b in range(m)] for a in range(m)]
    for _ in range(2):
        w = [quad(G[t], HO) / fro2(HO) for t in range(T)]
        v = [quad(X[t], HI) / fro2(HI) for t in range(T)]
        HI, HO = ([[sum(w[t] * X[t][a] * X[t][b] for t in range(T)) / T for b in range(n)] for a in range(n)],
                  [[sum(v[t] * G[t][a] * G[t][b] for t in range(T)) / T for b in range(m)] for a in range(m)])
    hi, ho = oracle.sketch_a(X, G, 2)
    assert np.allclose(hi, np.array(HI), rtol=1e-12, atol=1e-15)
    assert np.allclose(ho, np.array(HO), rtol=1e-12, atol=1e-15)


def test_token_weights_identity_and_scale():
    rng = np.random.default_rng(23)
    Y = rng.standard_normal((9, 5))
    assert np.allclose(oracle.token_weights(Y), np.sum(Y * Y, axis=1) / 5, rtol=1e-14)
    H = spd(5, 3)
    # <aH, y^T y> / ||aH||_F^2 = (1/a) <H, y^T y> / ||H||_F^2
    assert np.allclose(oracle.token_weights(Y, 7.0 * H), oracle.token_weights(Y, H) / 7.0, rtol=1e-13)
    # and against the quadratic form written out
    want = np.array([sum(y[a] * H[a, b] * y[b] for a in range(5) for b in range(5)) for y in Y]) / np.sum(H * H)
    assert np.allclose(oracle.token_weights(Y, H), want, rtol=1e-12)


# ----------------------------------------------------------------------------
# bound terms (YAQA article, section 4, error bound): closed forms
# ----------------------------------------------------------------------------
def test_bound_terms_closed_form():
    # written out by hand: D_O = (1, 2, 3), D_I = (4, 5), s = (1/2, 1, 2)
    #   sharp = (1 * 1/16 + 2 * 1/4 + 3 * 1) * (4 + 5) = 3.5625 * 9 = 32.0625
    #   page  = (4 + 5) * (1 + 2 + 3) * 2^2 / 4     = 54
    sharp, page = oracle.bound_terms(np.array([0.5, 1.0, 2.0], np.float32), [1.0, 2.0, 3.0], [4.0, 5.0])
    assert sharp == 32.0625 and page == 54.0
    # equal scales: both forms are tr(D_O) tr(D_I) s^2 / 4
    sharp, page = oracle.bound_terms(np.full(3, 0.5, np.float32), [1.0, 2.0, 3.0], [4.0, 5.0])
    assert sharp == page == 6.0 * 9.0 * 0.25 / 4.0


def test_bound_is_attained_with_every_residual_at_half_a_step():
    # Diagonal factors (L = 0: round to nearest, no feedback) and every W*_ij a whole
    # multiple of s_i, so that y = W*/s + 3/2 (2 bits) sits exactly halfway between
    # two codes: |eta_ij| = s_i / 2 for every entry and nothing clamps. The loss
    # sum_ij D_O,i D_I,j eta_ij^2 then equals the sharp bound exactly.
    rng = np.random.default_rng(31)
    m, n = 5, 7
    s = np.float32(2.0) ** rng.integers(-8, -3, size=m).astype(np.float32)
    w = (s[:, None] * rng.integers(-1, 2, size=(m, n))).astype(np.float32)
    DO = rng.lognormal(0.0, 1.0, m)
    DI = rng.lognormal(0.0, 1.0, n)
    r = oracle.sweep(w, np.zeros((m, m)), np.zeros((n, n)), s, 2)
    assert r["clamped"] == 0
    assert np.all(np.abs(r["eta"]) == s[:, None].astype(np.float64) / 2)
    loss = oracle.proxy_loss(r["delta"], np.diag(DO), np.diag(DI))
    sharp, page = oracle.bound_terms(s, DO, DI)
    assert abs(loss - sharp) <= 1e-13 * sharp
    assert page >= sharp


@pytest.mark.parametrize("mutation", ["no_quarter", "page_for_sharp", "sum_not_max", "swapped"])
def test_bound_pins_catch_mutated_terms(mutation):
    # plausible slips in writing the bound; the closed-form and attained-bound pins
    # above must reject every one of them
    def mutated(scales, DO, DI):
        s = np.asarray(scales, np.float64)
        do, di = np.asarray(DO, np.float64), np.asarray(DI, np.float64)
        if mutation == "no_quarter":
            return float(np.sum(do * s * s) * np.sum(di)), float(np.sum(di) * np.sum(do) * np.max(s) ** 2)
        if mutation == "page_for_sharp":
            v = float(np.sum(di) * np.sum(do) * np.max(s) ** 2 / 4.0)
            return v, v
        if mutation == "sum_not_max":
            return (float(np.sum(do * s * s / 4.0) * np.sum(di)),
                    float(np.sum(di) * np.sum(do) * np.sum(s * s) / 4.0))
        return float(np.sum(di * s[: len(di)] ** 2 / 4.0) * np.sum(do)), float(
            np.sum(di) * np.sum(do) * np.max(s) ** 2 / 4.0)

    sharp, page = mutated(np.array([0.5, 1.0, 2.0]), [1.0, 2.0, 3.0], [4.0, 5.0])
    assert (sharp, page) != (32.0625, 54.0)


# ----------------------------------------------------------------------------
# the whole CPU chain: pipeline() against an independent chain written here
# (numpy X^T X / T, damping, vectorised LDLQ on H_O (x) H_I; GPTQ when H_O = I)
# ----------------------------------------------------------------------------
def test_pipeline_matches_an_independent_chain():
    w, x, g = workloads.make_inputs("tiny", m=14, n=12, T=96)
    r = oracle.pipeline(w, x, g, 2)
    x64, g64 = x.astype(np.float64), g.astype(np.float64)
    HI = x64.T @ x64 / 96
    HI += 0.01 * np.trace(HI) / 12 * np.eye(12)
    HO = g64.T @ g64 / 96
    HO += 0.01 * np.trace(HO) / 14 * np.eye(14)
    assert np.allclose(r["HI"], HI, rtol=1e-13) and np.allclose(r["HO"], HO, rtol=1e-13)
    s = (np.float32(2.0) * np.max(np.abs(w), axis=1)) / np.float32(3.0)
    assert np.array_equal(r["scales"], s)
    codes_equal_or_tie(r["codes"], ldlq_vectorised(w, HO, HI, s, 2), r["margin"], tol=1e-8)
    A_O, A_I = np.triu(r["LO"], 1) + np.eye(14), np.triu(r["LI"], 1) + np.eye(12)
    assert np.allclose(A_O @ np.diag(r["DO"]) @ A_O.T, HO, rtol=1e-12, atol=1e-14 * np.abs(HO).max())
    assert np.allclose(A_I @ np.diag(r["DI"]) @ A_I.T, HI, rtol=1e-12, atol=1e-14 * np.abs(HI).max())


def test_pipeline_one_sided_damps_the_identity():
    # H_O = I, damped like every factor: (1 + 0.01) I, so L_O = 0 and D_O = 1.01;
    # the codes are GPTQ's on H_I and the loss is 1.01 tr(D H_I D^T)
    w, x, _ = workloads.make_inputs("tiny", m=20, n=24, T=128)
    r = oracle.pipeline(w, x, None, 3, one_sided=True)
    assert r["LO"] is None and np.all(r["DO"] == 1.01)
    x64 = x.astype(np.float64)
    HI = x64.T @ x64 / 128
    HI += 0.01 * np.trace(HI) / 24 * np.eye(24)
    codes_equal_or_tie(r["codes"], gptq(w, HI, r["scales"], 3), r["margin"], tol=1e-8)
    loss = oracle.loss_identity(r["eta"], r["DO"], r["DI"])
    want = 1.01 * np.sum((r["delta"] @ HI) * r["delta"])
    assert abs(loss - want) <= 1e-10 * want


# ----------------------------------------------------------------------------
# weighted accumulation (one Sketch A update with the weights given)
# ----------------------------------------------------------------------------
def test_weighted_hessian_brute_force():
    rng = np.random.default_rng(24)
    T, d = 9, 4
    X = rng.standard_normal((T, d))
    w = rng.lognormal(0.0, 1.0, T)
    w[3] = 0.0
    H = oracle.weighted_hessian(X, w)
    for a in range(d):
        for b in range(d):
            want = sum(w[t] * X[t][a] * X[t][b] for t in range(T)) / T
            assert abs(H[a, b] - want) <= 1e-13 * max(1.0, abs(want))
    # unit weights give X^T X / T
    assert np.allclose(oracle.weighted_hessian(X, np.ones(T)), X.T @ X / T, rtol=1e-14)
