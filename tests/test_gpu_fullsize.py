"""Parity at the full workload sizes, through the same calls bench.py times.

At these sizes the oracle cannot run the whole chain, so each stage is checked
on outputs the oracle can compute one by one, or by properties that hold at
any size:
  * Hessian factor: sampled entries (diagonal, outlier columns, random pairs)
    against fp64 dot products over all tokens;
  * LDL: sampled entries of (L+I) D (L+I)^T against the damped fp32 factor the
    device was given (backward error), with D > 0 and L strictly upper;
  * solve: one FULL row from every 64-row block of leaves (plus the first and
    last rows) replayed by the oracle with the device's factors and the device's
    own committed error (every code exact or a counted flip inside the 1e-4
    band); the device's proxy loss against the oracle's tr(D H_I D^T H_O) with
    the damped factors, evaluated in fp64 row block by row block.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import record_parity

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def note(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def bk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kronecker_hessian_rounding_amd as m
    return m


def sample_pairs(d, special, rng, k=96):
    idx = list(special) + list(rng.integers(0, d, size=k))
    rows = list(idx) + list(rng.integers(0, d, size=k))
    cols = list(idx[::-1]) + list(rng.integers(0, d, size=k))
    rows += list(special)
    cols += list(special)  # diagonal entries of the special columns
    return np.array(rows), np.array(cols)


def check_hessian(Hg, x, special, rng, label):
    """Sampled entries of the device's X^T X / T against fp64 dot products."""
    d = x.shape[1]
    T = x.shape[0]
    r, c = sample_pairs(d, special, rng)
    got = Hg[torch.from_numpy(r).cuda(), torch.from_numpy(c).cuda()].cpu().numpy().astype(np.float64)
    ref = oracle.hessian_entries(x, r, c)
    # |X|^T |X| / T of the sampled pairs bounds the fp32 accumulation error
    mag = np.array([np.dot(np.abs(x[:, a]).astype(np.float64), np.abs(x[:, b]).astype(np.float64)) / T
                    for a, b in zip(r, c)])
    err = np.abs(got - ref) / (4 * U32 * np.sqrt(T) * mag + 1e-300)
    note("  %s: %d sampled entries, max err / bound = %.3g" % (label, len(r), err.max()))
    assert np.all(err <= 1.0)


def check_ldl(Hbefore_rows, Hbefore_diag, Hf, Df, rows, lam, label):
    """(L+I) D (L+I)^T at sampled (i, j) against the damped factor the device saw."""
    d = Hf.shape[0]
    Dv = Df.cpu().numpy().astype(np.float64)
    assert np.all(Dv > 0)
    sel = torch.from_numpy(np.array(rows)).cuda()
    Lrows = Hf[sel].cpu().numpy().astype(np.float64)  # rows of the output: L above the diagonal
    for a, i in enumerate(rows):
        assert np.all(Lrows[a, :i] == 0.0)  # zeros below the diagonal
    U = np.triu(Lrows, 1)
    for a, i in enumerate(rows):
        U[a, i] = 1.0
    worst = 0.0
    for a, i in enumerate(rows):
        for b, j in enumerate(rows):
            if j < i:
                continue
            rec = float(np.sum(U[a] * Dv * U[b]))
            h = float(Hbefore_rows[a][j]) + (lam if i == j else 0.0)
            scale = np.sqrt((Hbefore_diag[i] + lam) * (Hbefore_diag[j] + lam))
            worst = max(worst, abs(rec - h) / (8 * U32 * scale))
    note("  %s: backward error / bound = %.3g over %d pairs" % (label, worst, len(rows) * (len(rows) + 1) // 2))
    assert worst <= 1.0


def run_chain(bk, name, rng):
    wl = workloads.get(name)
    note("%s: generating inputs (m=%d n=%d T=%d)" % (name, wl.m, wl.n, wl.T))
    w, x, g = workloads.make_inputs(name)
    dev = torch.device("cuda:0")
    W, X, G = (torch.from_numpy(a).to(dev) for a in (w, x, g))
    note("%s: Hessian factors" % name)
    HI = bk.hessian_accum(X)
    HO = bk.hessian_accum(G)
    torch.cuda.synchronize()
    special_x = list(np.argsort(-np.abs(x[:64]).mean(0))[:8])  # heavy (outlier) columns
    check_hessian(HI, x, special_x, rng, "H_I")
    check_hessian(HO, g, [0, wl.m - 1], rng, "H_O")
    # keep what the LDL will see, for the backward-error check
    rows_i = sorted(set([0, 1, wl.n // 2, wl.n - 2, wl.n - 1] + list(rng.integers(0, wl.n, 4))))
    rows_o = sorted(set([0, 1, wl.m // 2, wl.m - 2, wl.m - 1] + list(rng.integers(0, wl.m, 4))))
    HIr = HI[torch.tensor(rows_i).cuda()].cpu().numpy()
    HOr = HO[torch.tensor(rows_o).cuda()].cpu().numpy()
    HId = torch.diagonal(HI).cpu().numpy().astype(np.float64)
    HOd = torch.diagonal(HO).cpu().numpy().astype(np.float64)
    lam_i, lam_o = 0.01 * HId.mean(), 0.01 * HOd.mean()
    # the undamped factors, for the proxy-loss check (up70b: 3.3 GB for H_O)
    HIc = HI.cpu().numpy()
    HOc = HO.cpu().numpy()
    note("%s: LDL" % name)
    HI, DI = bk.ldl(HI, 0.01)
    HO, DO = bk.ldl(HO, 0.01)
    check_ldl(HIr, HId, HI, DI, rows_i, lam_i, "L_I")
    check_ldl(HOr, HOd, HO, DO, rows_o, lam_o, "L_O")
    return w, W, HI, DI, HO, DO, HIc, HOc, lam_i, lam_o


def loss_blockwise(dl, HIc, lam_i, HOc, lam_o, rows=2048):
    """tr(D H_I D^T H_O) in fp64 with the damped factors, H_O taken a row block at a time."""
    hi = HIc.astype(np.float64)
    hi[np.diag_indices_from(hi)] += lam_i
    DH = dl @ hi                                    # D H_I
    del hi
    total = 0.0
    for r0 in range(0, dl.shape[0], rows):
        r1 = min(dl.shape[0], r0 + rows)
        ho = HOc[r0:r1].astype(np.float64)
        ho[:, r0:r1][np.diag_indices(r1 - r0)] += lam_o
        total += float(np.sum((ho @ dl) * DH[r0:r1]))  # rows r0..r1 of H_O D, against D H_I
    return total


def check_solve(bk, name, w, W, HI, DI, HO, DO, bits, rounding, seed, rng, HIc, HOc, lam_i, lam_o):
    m, n = w.shape
    note("%s: solve %d-bit %s" % (name, bits, rounding))
    res = bk.solve(W, HO, HI, bits, rounding, seed, D_O=DO, D_I=DI, want_loss=True)
    torch.cuda.synchronize()
    assert int(res.info.item()) == 0
    codes = res.codes.cpu().numpy()
    scales = res.scales.cpu().numpy()
    assert np.array_equal(scales, oracle.row_scales(w, bits))
    LO = HO.cpu().numpy()  # L_O above the diagonal (replay reads only the strict upper triangle)
    LI = HI.cpu().numpy()
    # one row from every 64-row block of leaves, plus the first and the last row
    blocks = (m + 63) // 64
    rows = sorted(set([0, m - 1] + [min(m - 1, 64 * b + int(rng.integers(0, 64))) for b in range(blocks)]))
    note("  replaying %d rows" % len(rows))
    rp = oracle.replay_rows(w, LO, LI, scales, bits, codes, rows, rounding, seed)
    note("  replayed %d rows: mismatches %d, flips %d, bad %d, max flip margin %.2e" % (
        len(rows), rp["mismatches"], rp["flips"], rp["bad"], rp["max_flip_margin"]))
    loss = float(res.loss.item())
    Lq = 2**bits - 1
    note("  proxy loss in fp64 (row blocks)")
    dl = w.astype(np.float64) - scales[:, None].astype(np.float64) * (codes - Lq / 2.0)
    del codes
    ref = loss_blockwise(dl, HIc, lam_i, HOc, lam_o)
    del dl
    rel = abs(loss - ref) / ref
    note("  proxy loss device %.10g  oracle %.10g  rel %.2e  clamped %d" % (loss, ref, rel, int(res.clamped.item())))
    record_parity("full-" + name, m=m, n=n, bits=bits, rounding=rounding, one_sided=False, entries=m * n,
                  replayed=len(rows) * n, rows_replayed=len(rows), flips=rp["flips"],
                  max_flip_margin=rp["max_flip_margin"], replay_mismatches=rp["mismatches"], bad=rp["bad"],
                  clamped=int(res.clamped.item()), loss=loss, loss_ref=ref, loss_rel=rel)
    assert rp["bad"] == 0
    assert rp["max_flip_margin"] < 1e-4
    assert rel <= 1e-4
    return res


@pytest.mark.timeout(600)
def test_attn_full_size(bk):
    rng = np.random.default_rng(11)
    w, W, HI, DI, HO, DO, HIc, HOc, li, lo = run_chain(bk, "attn", rng)
    for bits in (2, 4):
        for rounding in ("nearest", "stochastic"):
            check_solve(bk, "attn", w, W, HI, DI, HO, DO, bits, rounding, 4002, rng, HIc, HOc, li, lo)


@pytest.mark.timeout(900)
def test_mlp_down_full_size(bk):
    rng = np.random.default_rng(12)
    w, W, HI, DI, HO, DO, HIc, HOc, li, lo = run_chain(bk, "mlp_down", rng)
    check_solve(bk, "mlp_down", w, W, HI, DI, HO, DO, 2, "nearest", 4003, rng, HIc, HOc, li, lo)


@pytest.mark.timeout(1100)
def test_up70b_full_size(bk):
    rng = np.random.default_rng(13)
    w, W, HI, DI, HO, DO, HIc, HOc, li, lo = run_chain(bk, "up70b", rng)
    check_solve(bk, "up70b", w, W, HI, DI, HO, DO, 2, "nearest", 4004, rng, HIc, HOc, li, lo)
