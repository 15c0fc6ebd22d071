"""GPU parity of the HIP path against the CPU oracle (element by element).

Acceptance (from the method's definition; see the oracle's replay()):
  * codes: identical to the oracle's rounding of the pre-rounding value that the
    rule gives with the device's own committed error, except counted flips whose
    value lies within 1e-4 grid steps of the boundary between the two codes;
  * scales: bit-identical (both sides compute them in fp32);
  * proxy loss: within 1e-4 relative of the oracle's;
  * Hessian accumulation: |H^ - H| <= 4 u sqrt(max(T, 64)) (|X|^T |X| / T)
    entrywise (fp32 accumulation over T terms, u = 2^-24);
  * LDL: fp64 on the device, so L^ and D^ agree with the fp64 oracle to a
    couple of fp32 ulps; backward error ||H - (L^+I)D^(L^+I)^T|| / ||H|| <= 1e-6.
"""
import ctypes
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


def dev():
    return torch.device("cuda:0")


def factors(m, n, T=None, name="tiny", one_sided=False):
    """Damped fp64 oracle factors for scaled workloads; returned as fp32 (shared inputs)."""
    T = T or max(4 * max(m, n), 256)
    w, x, g = workloads.make_inputs(name, m=m, n=n, T=T)
    HI = oracle.damp(oracle.hessian(x))
    LI, DI = oracle.udu(HI)
    if one_sided:
        # H_O = I damped like every factor: 1.01 I, so L_O = 0 and D_O = 1.01
        LO, DO = None, np.full(m, 1.01)
    else:
        HO = oracle.damp(oracle.hessian(g))
        LO, DO = oracle.udu(HO)
    f32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    return w, f32(LO), f32(LI), f32(DO), f32(DI)


def check_solve(bk, w, LO, LI, DO, DI, bits, rounding="nearest", seed=0, row_scale=None,
                free_run=True, label=""):
    m, n = w.shape
    note("solve %s m=%d n=%d bits=%d %s seed=%d" % (label, m, n, bits, rounding, seed))
    d = dev()
    T = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(d)
    res = bk.solve(T(w), T(LO), T(LI), bits, rounding, seed,
                   row_scale=T(row_scale), D_O=T(DO), D_I=T(DI),
                   want_delta=True, want_loss=True)
    torch.cuda.synchronize()
    assert int(res.info.item()) == 0
    codes = res.codes.cpu().numpy()
    scales = res.scales.cpu().numpy()
    if row_scale is None:
        assert np.array_equal(scales, oracle.row_scales(w, bits))
    else:
        assert np.array_equal(scales, row_scale)
    lo64 = None if LO is None else LO.astype(np.float64)
    li64 = None if LI is None else LI.astype(np.float64)
    rp = oracle.replay(w, lo64, li64, scales, bits, codes, rounding, seed,
                       DO=DO.astype(np.float64), DI=DI.astype(np.float64))
    assert rp["bad"] == 0, ("mismatches outside the 1e-4 band", rp["bad"], rp["bad_index"])
    assert rp["max_flip_margin"] < 1e-4
    # the device's committed error is W* - s (c - Lq/2)
    Lq = 2**bits - 1
    dl = res.delta.cpu().numpy().astype(np.float64)
    exact = w.astype(np.float64) - scales[:, None].astype(np.float64) * (codes - Lq / 2.0)
    assert np.max(np.abs(dl - exact)) <= 2 * U32 * np.max(np.abs(exact)) + 1e-30
    loss = float(res.loss.item())
    # 1e-4 relative, with a floor for degenerate near-zero losses (every value on the grid):
    # 1e-7 of the size of the loss bound sum_i D_O,i s_i^2/4 tr(D_I)
    floor = 1e-7 * oracle.bound_terms(scales, DO, DI)[0]
    tol = lambda ref: 1e-4 * abs(ref) + floor
    assert abs(loss - rp["loss"]) <= tol(rp["loss"]), (loss, rp["loss"])
    assert int(res.clamped.item()) >= 0
    out = dict(flips=rp["flips"], loss=loss, codes=codes)
    rec = dict(m=m, n=n, bits=bits, rounding=rounding, one_sided=LO is None, entries=m * n,
               replayed=m * n, flips=rp["flips"], max_flip_margin=rp["max_flip_margin"],
               replay_mismatches=rp["mismatches"], bad=rp["bad"], clamped=int(res.clamped.item()),
               loss=loss, loss_ref=rp["loss"], loss_rel=abs(loss - rp["loss"]) / max(abs(rp["loss"]), 1e-300))
    if free_run:
        fr = oracle.sweep(w, lo64, li64, scales, bits, rounding, seed)
        mism = int((fr["codes"] != codes).sum())
        fl = oracle.loss_identity(fr["eta"], DO.astype(np.float64), DI.astype(np.float64))
        out.update(free_mismatch=mism, free_loss=fl)
        rec.update(free_mismatch=mism, free_loss=fl, free_clamped=fr["clamped"],
                   free_loss_rel=abs(loss - fl) / max(abs(fl), 1e-300))
        note("  flips=%d free-run mismatches=%d loss=%.8g free=%.8g clamped=%d/%d" % (
            rp["flips"], mism, loss, fl, int(res.clamped.item()), fr["clamped"]))
        record_parity(label or "solve", **rec)
        if mism == 0:
            assert int(res.clamped.item()) == fr["clamped"]
        assert abs(loss - fl) <= tol(fl)
    else:
        record_parity(label or "solve", **rec)
    return out


# ----------------------------------------------------------------------------
# Hessian factor accumulation
# ----------------------------------------------------------------------------
# pieces=True: two fp16 pieces per element of power-of-two-scaled columns on the fp16
# matrix cores (the default);
# pieces=False: the fp32 matrix-core path. Both are held to the same fp32 bound.
@pytest.mark.parametrize("pieces", [True, False])
@pytest.mark.parametrize("T,d", [(1024, 64), (333, 100), (8192, 512), (1, 5), (2000, 129), (0, 7),
                                 (4000, 2907)])
def test_hessian_accum_matches_oracle(bk, T, d, pieces):
    # (4000, 2907): 276 output tiles of 128, so the last short round is split over
    # the tokens into partials; ragged in both T and d
    note("hessian T=%d d=%d pieces=%s" % (T, d, pieces))
    x = workloads.make_x(max(T, 1), d, 99 + d, "gauss", 2 if d > 2 else 0)[:T]
    X = torch.from_numpy(np.ascontiguousarray(x)).to(dev())
    if T == 0:
        H = torch.full((d, d), 3.0, device=dev())
        bk.hessian_accum(X, H, alpha=1.0, beta=0.5, pieces=pieces)
        assert torch.all(H.cpu() == 1.5)
        return
    H = bk.hessian_accum(X, pieces=pieces).cpu().numpy()
    assert np.array_equal(H, H.T)
    ref = oracle.hessian(x)
    ax = np.abs(x.astype(np.float64))
    bound = 4 * U32 * np.sqrt(max(T, 64)) * (ax.T @ ax) / T + 1e-30
    assert np.all(np.abs(H - ref) <= bound), np.max(np.abs(H - ref) / bound)


@pytest.mark.parametrize("pieces", [True, False])
def test_hessian_accum_chunks_and_strides(bk, pieces):
    note("hessian chunked + strided pieces=%s" % pieces)
    x = workloads.make_x(3000, 96, 5, "gauss", 2)
    big = np.zeros((3000, 128), dtype=np.float32)
    big[:, :96] = x
    Xb = torch.from_numpy(big).to(dev())
    Xv = Xb[:, :96]  # leading dimension 128
    H = torch.empty((96, 96), device=dev())
    bk.hessian_accum(Xv[:1000], H, alpha=1.0 / 3000, beta=0.0, pieces=pieces)
    bk.hessian_accum(Xv[1000:], H, alpha=1.0 / 3000, beta=1.0, pieces=pieces)
    ref = oracle.hessian(x)
    ax = np.abs(x.astype(np.float64))
    bound = 8 * U32 * np.sqrt(3000) * (ax.T @ ax) / 3000
    assert np.all(np.abs(H.cpu().numpy() - ref) <= bound)


@pytest.mark.parametrize("pieces", [True, False])
@pytest.mark.parametrize("off", [4, 1])
def test_hessian_accum_strided_whole_tiles(bk, off, pieces):
    # a 256-column view of a wider buffer. On the fp32 path, at a 16-byte offset the
    # whole 128x128 tiles stream their k-slices straight into LDS; at a 4-byte offset
    # they take the register path. T is odd, so the last k-slice is partial either way.
    note("hessian strided whole tiles, column offset %d pieces=%s" % (off, pieces))
    T, d = 4133, 256
    x = workloads.make_x(T, d, 17 + off, "gauss", 2)
    big = np.zeros((T, d + 8), dtype=np.float32)
    big[:, off:off + d] = x
    Xb = torch.from_numpy(big).to(dev())
    H = bk.hessian_accum(Xb[:, off:off + d], pieces=pieces).cpu().numpy()
    assert np.array_equal(H, H.T)
    ref = oracle.hessian(x)
    ax = np.abs(x.astype(np.float64))
    bound = 4 * U32 * np.sqrt(T) * (ax.T @ ax) / T
    assert np.all(np.abs(H - ref) <= bound), np.max(np.abs(H - ref) / bound)


@pytest.mark.parametrize("pieces", [True, False])
def test_hessian_accum_nonfinite_inputs_stay_in_their_rows(bk, pieces):
    # An Inf and a NaN in X make every entry of their columns' rows and columns of H
    # non-finite (NaN or Inf: the piece split of an Inf is Inf, NaN, and its column keeps
    # the exponent 0); every
    # other entry keeps the usual fp32 bound.
    note("hessian non-finite inputs pieces=%s" % pieces)
    T, d = 700, 150
    x = workloads.make_x(T, d, 31, "gauss", 2)
    bad = [17, 140]
    xb = x.copy()
    xb[5, bad[0]] = np.inf
    xb[600, bad[1]] = np.nan
    H = bk.hessian_accum(torch.from_numpy(xb).to(dev()), pieces=pieces).cpu().numpy()
    for c in bad:
        assert not np.any(np.isfinite(H[c, :])) and not np.any(np.isfinite(H[:, c]))
    keep = np.setdiff1d(np.arange(d), bad)
    Hk = H[np.ix_(keep, keep)]
    ref = oracle.hessian(x)[np.ix_(keep, keep)]
    ax = np.abs(x[:, keep].astype(np.float64))
    bound = 4 * U32 * np.sqrt(T) * (ax.T @ ax) / T
    assert np.all(np.abs(Hk - ref) <= bound)


# ----------------------------------------------------------------------------
# damped LDL
# ----------------------------------------------------------------------------
LDL_PATHS = ["scheduled", "launch"]


@pytest.mark.parametrize("path", LDL_PATHS)
@pytest.mark.parametrize("d", [1, 5, 64, 100, 257, 512, 1000, 1500, 2100])
def test_ldl_matches_oracle(bk, d, path, monkeypatch):
    # orders up to 128 blocks take the scheduled (persistent) path by default; the
    # launch chain is forced here for the same sizes
    monkeypatch.setenv("BAKRON_LDL_PATH", path)
    note("ldl d=%d %s" % (d, path))
    x = workloads.make_x(max(2 * d, 64), d, 7 + d, "gauss", min(2, d))
    H32 = oracle.hessian(x).astype(np.float32)
    ref_H = oracle.damp(H32.astype(np.float64), 0.01)
    L, D = oracle.udu(ref_H)
    Ht = torch.from_numpy(H32.copy()).to(dev())
    Hg, Dg = bk.ldl(Ht, 0.01)
    Hc = Hg.cpu().numpy()
    Lg = np.triu(Hc, 1).astype(np.float64)
    Dv = Dg.cpu().numpy().astype(np.float64)
    assert np.all(np.tril(Hc, -1) == 0)
    assert np.array_equal(np.diag(Hc), Dg.cpu().numpy())
    assert np.all(np.abs(Lg - L) <= 4 * U32 * np.abs(L) + 1e-6 * U32 * max(1.0, np.abs(L).max()))
    assert np.all(np.abs(Dv - D) <= 4 * U32 * D)
    A = Lg + np.eye(d)
    rec = A @ np.diag(Dv) @ A.T
    assert np.linalg.norm(rec - ref_H) / np.linalg.norm(ref_H) < 1e-6


@pytest.mark.parametrize("path", LDL_PATHS)
@pytest.mark.parametrize("d,extra", [(256, 4), (1024, 3), (777, 4), (1100, 12)])
def test_ldl_strided_view(bk, d, extra, path, monkeypatch):
    # H as a view of a wider buffer (leading dimension d + extra): 16-byte aligned rows
    # with whole tiles take the wide loads and stores, others the element-wise ones;
    # the result equals the contiguous call bit for bit and the rest of the buffer
    # is untouched
    monkeypatch.setenv("BAKRON_LDL_PATH", path)
    note("ldl strided view d=%d ld=%d %s" % (d, d + extra, path))
    H = oracle.hessian(workloads.make_x(d + 64, d, 60 + d, "gauss", 2)).astype(np.float32)
    ref, refD = bk.ldl(torch.from_numpy(H).to(dev()), 0.01)
    big = torch.full((d, d + extra), 7.0, device=dev())
    big[:, :d] = torch.from_numpy(H).to(dev())
    got, gotD = bk.ldl(big[:, :d], 0.01)
    assert torch.equal(got, ref) and torch.equal(gotD, refD)
    assert bool((big[:, d:] == 7.0).all())


@pytest.mark.parametrize("path", LDL_PATHS)
def test_ldl_reports_first_bad_pivot(bk, path, monkeypatch):
    monkeypatch.setenv("BAKRON_LDL_PATH", path)
    note("ldl not-SPD %s" % path)
    x = workloads.make_x(256, 130, 3, "gauss", 2)
    H = oracle.hessian(x).astype(np.float32)
    H[77, 77] = -5.0
    H[120, 120] = -5.0
    with pytest.raises(ValueError, match="pivot 120"):
        oracle.udu(oracle.damp(H.astype(np.float64)))
    with pytest.raises(bk.BakronError) as ei:
        bk.ldl(torch.from_numpy(H).to(dev()), 0.01)
    assert ei.value.status == bk.BAKRON_E_NOT_SPD
    assert ei.value.bad_pivot == 120


@pytest.mark.parametrize("d", [777, 2048, 3000])
def test_ldl_scheduled_matches_launch_chain(bk, d, monkeypatch):
    # the same blocked factorisation by the two schedules: they sum the updates of a
    # tile in different groupings, so the fp64 factors differ by rounding only and
    # the fp32 results by at most a few units in the last place
    note("ldl scheduled vs launch d=%d" % d)
    H = oracle.hessian(workloads.make_x(d + 64, d, 40 + d, "gauss", 2)).astype(np.float32)
    g = torch.from_numpy(H).to(dev())
    monkeypatch.setenv("BAKRON_LDL_PATH", "launch")
    Hl, Dl = bk.ldl(g.clone(), 0.01)
    monkeypatch.setenv("BAKRON_LDL_PATH", "scheduled")
    Hs, Ds = bk.ldl(g.clone(), 0.01)
    Hl, Hs = Hl.cpu().numpy().astype(np.float64), Hs.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Hs - Hl) <= 4 * U32 * np.abs(Hl) + 1e-9 * np.abs(Hl).max())
    assert np.all(np.abs(Ds.cpu().numpy() - Dl.cpu().numpy()) <= 4 * U32 * np.abs(Dl.cpu().numpy()))
    # and again, bit for bit: the scheduled path applies each tile's updates in a fixed order
    Hs2, Ds2 = bk.ldl(g.clone(), 0.01)
    assert np.array_equal(Hs2.cpu().numpy().astype(np.float64), Hs) and torch.equal(Ds2, Ds)


def test_ldl_expired_wait_is_reported(bk, monkeypatch):
    # The scheduled LDL's workgroups wait on each other's tile counters, each wait
    # bounded in time. A 1 us limit, set from the host, makes them expire: the call
    # must stop (every kernel still ends) and report BAKRON_E_DEVICE with pivot -2;
    # the next call runs normally.
    note("ldl with a 1 us wait limit")
    H = oracle.hessian(workloads.make_x(1200, 1000, 9, "gauss", 2)).astype(np.float32)
    g = torch.from_numpy(H).to(dev())
    monkeypatch.setenv("BAKRON_LDL_PATH", "scheduled")
    monkeypatch.setenv("BAKRON_LDL_WAIT_LIMIT_US", "1")
    with pytest.raises(bk.BakronError) as ei:
        bk.ldl(g.clone(), 0.01)
    assert ei.value.status == bk.BAKRON_E_DEVICE and ei.value.bad_pivot == -2
    monkeypatch.delenv("BAKRON_LDL_WAIT_LIMIT_US")
    Hf, Df = bk.ldl(g.clone(), 0.01)
    assert torch.isfinite(Df).all() and bool((Df > 0).all())


def test_ldl_pair_matches_single_calls(bk):
    # the two factorisations run side by side on two streams; each must equal the
    # single-call result exactly (same kernels, same inputs)
    note("ldl pair d=300 and d=700")
    HA = oracle.hessian(workloads.make_x(700, 300, 21, "gauss", 2)).astype(np.float32)
    HB = oracle.hessian(workloads.make_x(1500, 700, 22, "gauss", 2)).astype(np.float32)
    ga, gb = torch.from_numpy(HA).to(dev()), torch.from_numpy(HB).to(dev())
    (pa, da), (pb, db) = bk.ldl_pair(ga.clone(), gb.clone(), 0.01)
    sa, ea = bk.ldl(ga.clone(), 0.01)
    sb, eb = bk.ldl(gb.clone(), 0.01)
    assert torch.equal(pa, sa) and torch.equal(da, ea)
    assert torch.equal(pb, sb) and torch.equal(db, eb)


def test_ldl_pair_past_one_launch_matches_single_calls(bk, monkeypatch):
    # an order above 8192 keeps both factorisations on the chain of launches, on two
    # streams: each equals its single call on that path bit for bit
    note("ldl pair d=8256 and d=300 (two streams, launch chain)")
    g = torch.Generator().manual_seed(31)
    X = torch.randn(8320, 8256, generator=g).to(dev())
    HA = bk.hessian_accum(X)
    HB = torch.from_numpy(oracle.hessian(workloads.make_x(700, 300, 21, "gauss", 2)).astype(np.float32)).to(dev())
    (pa, da), (pb, db) = bk.ldl_pair(HA.clone(), HB.clone(), 0.01)
    monkeypatch.setenv("BAKRON_LDL_PATH", "launch")
    sa, ea = bk.ldl(HA.clone(), 0.01)
    sb, eb = bk.ldl(HB.clone(), 0.01)
    assert torch.equal(pa, sa) and torch.equal(da, ea)
    assert torch.equal(pb, sb) and torch.equal(db, eb)


def test_ldl_pair_two_workgroups_per_cu_matches_single_calls(bk, monkeypatch):
    # a pair of order 6144 runs with two workgroups per compute unit, each single call
    # with one: the scheduled path applies every tile's updates in a fixed order, so the
    # results agree bit for bit, and with the launch chain to rounding
    note("ldl pair d=6144 and d=6144 (scheduled, two workgroups per CU)")
    g = torch.Generator().manual_seed(33)
    HA = bk.hessian_accum(torch.randn(6208, 6144, generator=g).to(dev()))
    HB = bk.hessian_accum((torch.randn(6400, 6144, generator=g) * torch.rand(6144, generator=g)).to(dev()))
    (pa, da), (pb, db) = bk.ldl_pair(HA.clone(), HB.clone(), 0.01)
    sa, ea = bk.ldl(HA.clone(), 0.01)
    sb, eb = bk.ldl(HB.clone(), 0.01)
    assert torch.equal(pa, sa) and torch.equal(da, ea)
    assert torch.equal(pb, sb) and torch.equal(db, eb)
    monkeypatch.setenv("BAKRON_LDL_PATH", "launch")
    la, fa = bk.ldl(HA.clone(), 0.01)
    la, pa = la.double(), pa.double()
    assert bool((torch.abs(pa - la) <= 4 * U32 * torch.abs(la) + 1e-9 * torch.abs(la).max()).all())
    assert bool((torch.abs(da - fa) <= 4 * U32 * torch.abs(fa)).all())


def test_ldl_single_8192_two_workgroups_per_cu(bk, monkeypatch):
    # a single factor of order 8192 (the largest the persistent launch takes) runs with
    # two workgroups per compute unit: it agrees with the launch chain to rounding and
    # repeats bit for bit
    note("ldl d=8192 scheduled (two workgroups per CU) vs launch chain")
    g = torch.Generator().manual_seed(35)
    H = bk.hessian_accum((torch.randn(8256, 8192, generator=g) * torch.rand(8192, generator=g)).to(dev()))
    s1, e1 = bk.ldl(H.clone(), 0.01)
    s2, e2 = bk.ldl(H.clone(), 0.01)
    assert torch.equal(s1, s2) and torch.equal(e1, e2)
    monkeypatch.setenv("BAKRON_LDL_PATH", "launch")
    la, fa = bk.ldl(H.clone(), 0.01)
    la, s1 = la.double(), s1.double()
    assert bool((torch.abs(s1 - la) <= 4 * U32 * torch.abs(la) + 1e-9 * torch.abs(la).max()).all())
    assert bool((torch.abs(e1 - fa) <= 4 * U32 * torch.abs(fa)).all())


@pytest.mark.parametrize("which", [0, 1])
def test_ldl_pair_failure_leaves_the_other_intact(bk, which):
    # one launch factors both matrices; a bad pivot in one stops only that one
    note("ldl pair, one launch, matrix %d not SPD" % which)
    good = oracle.hessian(workloads.make_x(900, 700, 5, "gauss", 2)).astype(np.float32)
    bad = oracle.hessian(workloads.make_x(400, 330, 3, "gauss", 2)).astype(np.float32)
    bad[200, 200] = -5.0
    ref, _ = bk.ldl(torch.from_numpy(good).to(dev()), 0.01)
    mats = [torch.from_numpy(good).to(dev()), torch.from_numpy(bad).to(dev())]
    if which == 0:
        mats.reverse()
    Ds = [torch.empty(m.shape[0], device=dev()) for m in mats]
    info = torch.full((2,), -1, dtype=torch.int64, device=dev())
    ws = [torch.empty(bk.LIB.bakron_ldl_workspace_bytes(m.shape[0]), dtype=torch.uint8, device=dev())
          for m in mats]
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = bk.LIB.bakron_ldl_pair_async(
        P(mats[0]), mats[0].shape[0], mats[0].shape[0], P(Ds[0]), P(info), P(ws[0]), ws[0].numel(),
        P(mats[1]), mats[1].shape[0], mats[1].shape[0], P(Ds[1]), ctypes.c_void_p(info.data_ptr() + 8),
        P(ws[1]), ws[1].numel(), 0.01, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == bk.BAKRON_OK
    got = info.cpu().tolist()
    assert got[which] == 200 and got[1 - which] == -1
    assert torch.equal(mats[1 - which], ref)


@pytest.mark.parametrize("which", [0, 1])
def test_ldl_pair_reports_which_failed(bk, which):
    note("ldl pair not-SPD in matrix %d" % which)
    good = oracle.hessian(workloads.make_x(300, 90, 5, "gauss", 2)).astype(np.float32)
    bad = oracle.hessian(workloads.make_x(400, 130, 3, "gauss", 2)).astype(np.float32)
    bad[120, 120] = -5.0
    mats = [torch.from_numpy(good).to(dev()), torch.from_numpy(bad).to(dev())]
    if which == 0:
        mats.reverse()
    with pytest.raises(bk.BakronError) as ei:
        bk.ldl_pair(mats[0], mats[1], 0.01)
    assert ei.value.status == bk.BAKRON_E_NOT_SPD
    assert ei.value.which == which
    assert ei.value.bad_pivot == 120


@pytest.mark.parametrize("which", [None, 0, 1])
def test_ldl_pair_deferred_status(bk, which):
    # with a status tensor the call does not wait: work queued after it runs behind
    # both factorisations, and check_ldl_pair raises what the waiting call raises
    note("ldl pair, deferred status, not-SPD matrix %s" % which)
    good = oracle.hessian(workloads.make_x(300, 90, 5, "gauss", 2)).astype(np.float32)
    other = oracle.hessian(workloads.make_x(400, 130, 3, "gauss", 2)).astype(np.float32)
    if which is not None:
        other[120, 120] = -5.0
    mats = [torch.from_numpy(good).to(dev()), torch.from_numpy(other).to(dev())]
    if which == 0:
        mats.reverse()
    with pytest.raises(ValueError):
        bk.ldl_pair(mats[0].clone(), mats[1].clone(), 0.01,
                    status=torch.empty(2, dtype=torch.int32, device=dev()))
    refs = [bk.ldl(m.clone(), 0.01) for m in mats] if which is None else None
    status = torch.full((2,), 7, dtype=torch.int64, device=dev())
    (pa, da), (pb, db) = bk.ldl_pair(mats[0], mats[1], 0.01, status=status)
    after = (pa.sum(dim=0, dtype=torch.float64), pb.sum(dim=0, dtype=torch.float64))
    if which is None:
        bk.check_ldl_pair(status)
        assert status.cpu().tolist() == [-1, -1]
        assert torch.equal(pa, refs[0][0]) and torch.equal(da, refs[0][1])
        assert torch.equal(pb, refs[1][0]) and torch.equal(db, refs[1][1])
        assert torch.equal(after[0], refs[0][0].sum(dim=0, dtype=torch.float64))
        assert torch.equal(after[1], refs[1][0].sum(dim=0, dtype=torch.float64))
    else:
        with pytest.raises(bk.BakronError) as ei:
            bk.check_ldl_pair(status)
        assert ei.value.status == bk.BAKRON_E_NOT_SPD
        assert ei.value.which == which
        assert ei.value.bad_pivot == 120


# ----------------------------------------------------------------------------
# the BaKron solve
# ----------------------------------------------------------------------------
def test_solve_tiny_config_nearest(bk):
    w, x, g = workloads.make_inputs("tiny")
    HI, HO = oracle.damp(oracle.hessian(x)), oracle.damp(oracle.hessian(g))
    (LI, DI), (LO, DO) = oracle.udu(HI), oracle.udu(HO)
    f = lambda a: a.astype(np.float32)
    out = check_solve(bk, w, f(LO), f(LI), f(DO), f(DI), 2, label="tiny")
    assert out["free_mismatch"] == 0


def test_solve_tiny_config_stochastic(bk):
    w, LO, LI, DO, DI = factors(64, 64, 1024)
    check_solve(bk, w, LO, LI, DO, DI, 2, "stochastic", seed=4000, label="tiny-stoch")


@pytest.mark.parametrize("m,n", [(1, 1), (1, 64), (64, 1), (3, 200), (65, 129), (100, 70),
                                 (130, 66), (128, 128), (200, 333)])
def test_solve_ragged_shapes(bk, m, n):
    w, LO, LI, DO, DI = factors(m, n)
    check_solve(bk, w, LO, LI, DO, DI, 2, label="ragged")


@pytest.mark.parametrize("m,n,bits,rounding,recipe", [
    (700, 1500, 2, "nearest", "tiny"),
    (1500, 700, 3, "stochastic", "tiny"),
    (1000, 1000, 4, "nearest", "mlp_down"),
])
def test_solve_many_leaf_diagonals(bk, m, n, bits, rounding, recipe):
    # dozens of leaf-diagonals: split-K far fields, the adjacent-block products of
    # the leaf, ragged last leaves, every entry replayed against the oracle
    w, LO, LI, DO, DI = factors(m, n, name=recipe)
    check_solve(bk, w, LO, LI, DO, DI, bits, rounding, seed=4002, label="many-diagonals")


@pytest.mark.parametrize("bits", [1, 3, 4, 8])
def test_solve_bit_widths(bk, bits):
    w, LO, LI, DO, DI = factors(96, 160)
    check_solve(bk, w, LO, LI, DO, DI, bits, label="bits")


def test_solve_one_sided_is_ldlq(bk):
    w, LO, LI, DO, DI = factors(150, 200, one_sided=True)
    out = check_solve(bk, w, None, LI, DO, DI, 3, label="one-sided")
    # H_O = I: the rows are independent one-sided LDLQ problems
    assert out["free_mismatch"] == 0


def test_solve_row_factor_only(bk):
    # L_I absent (H_I diagonal): only the column feedback through L_O remains, so the
    # column of leaves below a leaf hands over D while nothing passes along a row
    w, LO, LI, DO, DI = factors(260, 150)
    check_solve(bk, w, LO, None, DO, DI, 2, label="L_I absent")


def test_solve_strided_operands(bk):
    # every matrix a view with an odd leading dimension: the far-field GEMMs take the
    # register-staged path, the strip hand-overs and the outputs use the strides
    m, n, bits = 200, 330, 2
    w, LO, LI, DO, DI = factors(m, n)
    note("solve strided m=%d n=%d" % (m, n))
    d = dev()

    def strided(a, extra, dtype=torch.float32):
        buf = torch.full((a.shape[0], a.shape[1] + extra), float("nan"), dtype=dtype, device=d)
        v = buf[:, : a.shape[1]]
        v.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(d))
        return v

    Wv, LOv, LIv = strided(w, 3), strided(LO, 5), strided(LI, 1)
    codes_buf = torch.zeros((m, n + 7), dtype=torch.uint8, device=d)
    delta_buf = torch.full((m, n + 2), float("nan"), dtype=torch.float32, device=d)
    out = bk.SolveResult(codes=codes_buf[:, :n], scales=torch.empty(m, dtype=torch.float32, device=d),
                         delta=delta_buf[:, :n], loss=torch.empty(1, dtype=torch.float64, device=d),
                         clamped=torch.empty(1, dtype=torch.int64, device=d),
                         info=torch.empty(1, dtype=torch.int32, device=d))
    res = bk.solve(Wv, LOv, LIv, bits, D_O=torch.from_numpy(DO).to(d), D_I=torch.from_numpy(DI).to(d),
                   want_loss=True, out=out)
    torch.cuda.synchronize()
    assert int(res.info.item()) == 0
    codes = res.codes.cpu().numpy()
    scales = res.scales.cpu().numpy()
    assert np.array_equal(scales, oracle.row_scales(w, bits))
    rp = oracle.replay(w, LO.astype(np.float64), LI.astype(np.float64), scales, bits, codes,
                       DO=DO.astype(np.float64), DI=DI.astype(np.float64))
    assert rp["bad"] == 0 and rp["max_flip_margin"] < 1e-4
    Lq = 2**bits - 1
    exact = w.astype(np.float64) - scales[:, None].astype(np.float64) * (codes - Lq / 2.0)
    assert np.max(np.abs(res.delta.cpu().numpy() - exact)) <= 2 * U32 * np.max(np.abs(exact))
    floor = 1e-7 * oracle.bound_terms(scales, DO, DI)[0]
    assert abs(float(res.loss.item()) - rp["loss"]) <= 1e-4 * abs(rp["loss"]) + floor
    # nothing outside the views was written
    assert torch.all(codes_buf[:, n:] == 0) and torch.all(torch.isnan(delta_buf[:, n:]))


def test_solve_diagonal_factors_is_rtn(bk):
    w, _, _, _, _ = factors(70, 90)
    d = dev()
    res = bk.solve(torch.from_numpy(w).to(d), None, None, 3)
    s = oracle.row_scales(w, 3)
    rtn = np.clip(np.floor(w.astype(np.float64) / s[:, None].astype(np.float64) + 3.5 + 0.5), 0, 7)
    got = res.codes.cpu().numpy()
    y = w.astype(np.float64) / s[:, None].astype(np.float64) + 3.5
    tie = np.abs((y - np.floor(y)) - 0.5) < 1e-5
    assert np.all((got == rtn) | tie)


def test_solve_user_scales(bk):
    w, LO, LI, DO, DI = factors(80, 100)
    rs = (1.7 * np.max(np.abs(w), axis=1) / 7.0).astype(np.float32)
    check_solve(bk, w, LO, LI, DO, DI, 3, row_scale=rs, label="user-scales")


def test_solve_reports_zero_row(bk):
    w, LO, LI, DO, DI = factors(70, 40)
    w[33] = 0.0
    d = dev()
    res = bk.solve(torch.from_numpy(w).to(d), torch.from_numpy(LO).to(d),
                   torch.from_numpy(LI).to(d), 2)
    assert int(res.info.item()) == 34


def test_solve_expired_wait_is_reported(bk, monkeypatch):
    # The solve's workgroups wait on each other's progress counters, each wait bounded
    # in time. A 1 us limit, set from the host, makes them expire: the solve must stop
    # (every kernel still ends) and report info = -1; the next call runs normally.
    note("solve with a 1 us wait limit")
    w, LO, LI, DO, DI = factors(300, 260)
    d = dev()
    T = lambda a: torch.from_numpy(a).to(d)
    monkeypatch.setenv("BAKRON_SOLVE_WAIT_LIMIT_US", "1")
    res = bk.solve(T(w), T(LO), T(LI), 2)
    assert int(res.info.item()) == -1
    monkeypatch.delenv("BAKRON_SOLVE_WAIT_LIMIT_US")
    res = bk.solve(T(w), T(LO), T(LI), 2)
    assert int(res.info.item()) == 0


def test_solve_small_config(bk):
    w, x, g = workloads.make_inputs("small")
    HI, HO = oracle.damp(oracle.hessian(x)), oracle.damp(oracle.hessian(g))
    (LI, DI), (LO, DO) = oracle.udu(HI), oracle.udu(HO)
    f = lambda a: a.astype(np.float32)
    check_solve(bk, w, f(LO), f(LI), f(DO), f(DI), 3, label="small")
    check_solve(bk, w, None, f(LI), np.full(512, 1.01, np.float32), f(DI), 3, label="small-H_O=I")


def test_solve_is_deterministic(bk):
    w, LO, LI, DO, DI = factors(300, 260)
    d = dev()
    T = lambda a: torch.from_numpy(a).to(d)
    a = bk.solve(T(w), T(LO), T(LI), 2, D_O=T(DO), D_I=T(DI), want_loss=True, want_delta=True)
    a_codes, a_delta, a_loss = a.codes.clone(), a.delta.clone(), a.loss.clone()
    b = bk.solve(T(w), T(LO), T(LI), 2, D_O=T(DO), D_I=T(DI), want_loss=True, want_delta=True)
    assert torch.equal(a_codes, b.codes) and torch.equal(a_delta, b.delta)
    assert torch.equal(a_loss, b.loss)


# ----------------------------------------------------------------------------
# two-sided incoherence processing: randomised Hadamard rotation
# ----------------------------------------------------------------------------
def rht_tol(a, axis):
    """4 (k + 2) u_fp32 ||x||_2 for every rotated vector x (the columns for axis 0,
    the rows for axis 1): k butterfly stages, the scale and the signs, each one
    fp32 rounding of quantities bounded by ||x||_2."""
    n = a.shape[axis]
    k = (n & -n).bit_length() - 1
    return 4 * (k + 2) * U32 * np.linalg.norm(a.astype(np.float64), axis=axis, keepdims=True)


@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("rows,cols,axis", [
    (64, 64, 0), (64, 64, 1), (100, 48, 0), (100, 48, 1), (512, 300, 0), (300, 512, 1),
    (4096, 96, 0),   # 12 index bits: two column passes of 6
    (8192, 40, 0),   # 13 bits: passes of 5, 4 and 4
    (7, 5, 0), (7, 5, 1),  # odd orders: signs only
    (40, 20480, 1),  # 4096-blocks, 16384-float chunks: one of four blocks, one of one
    (3, 28672, 1),   # 7 blocks of 4096: chunks of 4 and 3 blocks
])
def test_rht_matches_oracle(bk, rows, cols, axis, transpose):
    note("rht %dx%d axis %d transpose %d" % (rows, cols, axis, transpose))
    rng = np.random.default_rng(rows * 7 + cols)
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    seed = 1000 + rows + cols
    A = torch.from_numpy(a).to(dev())
    bk.rht(A, axis, seed, transpose)
    got = A.cpu().numpy().astype(np.float64)
    ref = oracle.rht_apply(a, axis, seed, transpose)
    assert np.all(np.abs(got - ref) <= rht_tol(a, axis)), np.max(np.abs(got - ref) / rht_tol(a, axis))


@pytest.mark.parametrize("axis", [0, 1])
def test_rht_strided_view_leaves_the_rest(bk, axis):
    note("rht strided view axis %d" % axis)
    rng = np.random.default_rng(3)
    big = rng.standard_normal((96, 133)).astype(np.float32)
    B = torch.from_numpy(big).to(dev())
    view = B[:, 5:5 + 64]  # leading dimension 133, 64 columns
    a = big[:, 5:5 + 64].copy()
    bk.rht(view, axis, 21)
    got = B.cpu().numpy()
    ref = oracle.rht_apply(a, axis, 21)
    assert np.all(np.abs(got[:, 5:69] - ref) <= rht_tol(a, axis))
    assert np.array_equal(got[:, :5], big[:, :5]) and np.array_equal(got[:, 69:], big[:, 69:])


@pytest.mark.parametrize("rows,cols", [(4096, 4096), (16, 16384)])
def test_rht_round_trip_keeps_norms(bk, rows, cols):
    # at the attention shape both axes, against the oracle; at a 16384-long row block
    # (too large for a dense oracle H_b) the properties that hold at any size:
    # U^T U = I and ||U x|| = ||x||
    note("rht round trip %dx%d" % (rows, cols))
    rng = np.random.default_rng(rows + cols)
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    A = torch.from_numpy(a).to(dev())
    bk.rht(A, 0, 5)
    bk.rht(A, 1, 6)
    once = A.cpu().numpy().astype(np.float64)
    kb = (rows & -rows).bit_length() + (cols & -cols).bit_length()
    fro = np.linalg.norm(a.astype(np.float64))
    assert abs(np.linalg.norm(once) - fro) <= 4 * (kb + 4) * U32 * fro
    if rows * cols <= 4096 * 4096 and max(rows & -rows, cols & -cols) <= 4096:
        ref = oracle.rht_apply(oracle.rht_apply(a, 0, 5), 1, 6)
        assert np.linalg.norm(once - ref) <= 4 * (kb + 4) * U32 * fro
    bk.rht(A, 1, 6, transpose=True)
    bk.rht(A, 0, 5, transpose=True)
    back = A.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(back - a) <= 8 * (kb + 4) * U32 * fro


def test_rotated_layer_through_ldl_and_solve(bk):
    # two-sided incoherence processing between the Hessians and the LDL, all on the
    # device; the rotation against the oracle's, then the solve on the rotated layer
    # against the oracle's replay with the device's own factors
    m, n, T = 96, 128, 1024
    w, x, g = workloads.make_inputs("tiny", m=m, n=n, T=T)
    note("rotated layer m=%d n=%d" % (m, n))
    d = dev()
    W = torch.from_numpy(np.ascontiguousarray(w)).to(d)
    HI = bk.hessian_accum(torch.from_numpy(x).to(d))
    HO = bk.hessian_accum(torch.from_numpy(g).to(d))
    hi0, ho0 = HI.cpu().numpy(), HO.cpu().numpy()
    bk.rotate_layer(W, HI, HO, 11, 12)
    rw, rhi, rho = oracle.rotate_layer(w, hi0, ho0, 11, 12)
    km, kn = (m & -m).bit_length(), (n & -n).bit_length()
    for got, ref, src in ((W, rw, w), (HI, rhi, hi0), (HO, rho, ho0)):
        err = np.linalg.norm(got.cpu().numpy().astype(np.float64) - ref)
        assert err <= 4 * (km + kn + 4) * U32 * np.linalg.norm(src.astype(np.float64))
    w2 = W.cpu().numpy()
    Hi, Di = bk.ldl(HI, 0.01)
    Ho, Do = bk.ldl(HO, 0.01)
    LI = np.triu(Hi.cpu().numpy(), 1)
    LO = np.triu(Ho.cpu().numpy(), 1)
    check_solve(bk, w2, LO, LI, Do.cpu().numpy(), Di.cpu().numpy(), 3, label="rotated")


# ----------------------------------------------------------------------------
# Sketch B: H_I = E_s[G_s^T G_s] / m, H_O = E_s[G_s G_s^T] / n (YAQA article, section 3)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("d,T", [(64, 1024), (100, 333), (129, 2000), (5, 1), (300, 77)])
def test_hessian_accum_transposed_matches_oracle(bk, d, T):
    # X stored d x T: H = X X^T / T
    note("hessian transposed d=%d T=%d" % (d, T))
    x = workloads.make_x(T, d, 41 + d, "gauss", 2 if d > 2 else 0)  # T x d
    xt = np.ascontiguousarray(x.T)
    H = bk.hessian_accum(torch.from_numpy(xt).to(dev()), transposed=True).cpu().numpy()
    assert np.array_equal(H, H.T)
    ref = oracle.hessian(x)
    ax = np.abs(x.astype(np.float64))
    bound = 4 * U32 * np.sqrt(max(T, 64)) * (ax.T @ ax) / T + 1e-30
    assert np.all(np.abs(H - ref) <= bound), np.max(np.abs(H - ref) / bound)


def test_hessian_accum_transposed_strided_view(bk):
    note("hessian transposed strided view")
    T, d = 333, 70
    x = workloads.make_x(T, d, 44, "gauss", 2)
    big = np.zeros((d, T + 11), dtype=np.float32)
    big[:, 3:3 + T] = x.T
    view = torch.from_numpy(big).to(dev())[:, 3:3 + T]  # leading dimension T + 11, 4-byte offset
    H = bk.hessian_accum(view, transposed=True).cpu().numpy()
    ref = oracle.hessian(x)
    ax = np.abs(x.astype(np.float64))
    assert np.all(np.abs(H - ref) <= 4 * U32 * np.sqrt(T) * (ax.T @ ax) / T)


def test_hessian_accum_transposed_needs_the_piece_workspace(bk):
    note("hessian transposed without workspace")
    X = torch.zeros((8, 16), device=dev())
    with pytest.raises(ValueError):
        bk.hessian_accum(X, transposed=True, pieces=False)
    H = torch.empty((8, 8), device=dev())
    st = bk.LIB.bakron_hessian_accum_t(ctypes.c_void_p(X.data_ptr()), 16, 8, 16, 1.0, 0.0,
                                       ctypes.c_void_p(H.data_ptr()), 8, None, 0, None)
    assert st == bk.BAKRON_E_WORKSPACE


@pytest.mark.parametrize("S,m,n", [(3, 96, 130), (1, 64, 64), (4, 33, 257), (2, 48, 256), (5, 40, 100)])
def test_sketch_b_matches_oracle(bk, S, m, n):
    note("sketch B S=%d m=%d n=%d" % (S, m, n))
    g = workloads.make_grads(S, m, n, 50 + m)
    Gt = torch.from_numpy(g).to(dev())
    HI, HO = bk.sketch_b(Gt)  # one stacked accumulation for H_I
    HI, HO = HI.cpu().numpy(), HO.cpu().numpy()
    HI2, HO2 = bk.sketch_b([Gt[s] for s in range(S)])  # one call per sequence
    HI2, HO2 = HI2.cpu().numpy(), HO2.cpu().numpy()
    ri, ro = oracle.sketch_b(list(g))
    ag = np.abs(g.astype(np.float64))
    # S accumulations of K-long sums, each within the fp32 bound, plus the S - 1
    # fp32 additions into H: 8 u sqrt(S K) of the mean |G|-product
    bi = 8 * U32 * np.sqrt(S * m) * sum(a.T @ a for a in ag) / (S * m) + 1e-30
    bo = 8 * U32 * np.sqrt(S * n) * sum(a @ a.T for a in ag) / (S * n) + 1e-30
    for hi in (HI, HI2):
        assert np.all(np.abs(hi - ri) <= bi), np.max(np.abs(hi - ri) / bi)
        assert np.array_equal(hi, hi.T)
    for ho in (HO, HO2):  # the batched transposed call, and one call per sequence
        assert np.all(np.abs(ho - ro) <= bo), np.max(np.abs(ho - ro) / bo)
        assert np.array_equal(ho, ho.T)


# ----------------------------------------------------------------------------
# per-layer bound and sensitivity report (YAQA article, section 4; KronQ page)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("m,n,one_sided", [(64, 48, False), (300, 257, False), (40, 3000, True)])
def test_layer_report_matches_oracle(bk, m, n, one_sided):
    note("layer report m=%d n=%d one_sided=%d" % (m, n, one_sided))
    rng = np.random.default_rng(m + n)
    DO = None if one_sided else rng.lognormal(0.0, 1.0, m).astype(np.float32)
    DI = rng.lognormal(0.0, 1.0, n).astype(np.float32)
    s = rng.lognormal(-4.0, 0.5, m).astype(np.float32)
    HO = rng.standard_normal((m, m)).astype(np.float32)
    T = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    HIt = torch.from_numpy(rng.standard_normal((n, n + 3)).astype(np.float32)).to(dev())
    HIv = HIt[:, :n]  # a view with leading dimension n + 3
    hi = HIv.cpu().numpy()
    r = bk.layer_report(T(DO), T(DI), T(s), H_I=HIv, H_O=T(HO))
    do = np.ones(m) if DO is None else DO
    sharp, page = oracle.bound_terms(s, do, DI)
    want = dict(tr_DO=float(np.sum(do, dtype=np.float64)), tr_DI=float(np.sum(DI, dtype=np.float64)),
                bound_sharp=sharp, bound_page=page, tr_HI=float(np.trace(hi.astype(np.float64))),
                tr_HO=float(np.trace(HO.astype(np.float64))))
    want["sensitivity"] = want["tr_HI"] * want["tr_HO"]
    for k, v in want.items():
        assert abs(r[k] - v) <= 1e-12 * max(1.0, abs(v)), (k, r[k], v)
    r2 = bk.layer_report(T(DO), T(DI), T(s))
    assert np.isnan(r2["tr_HI"]) and np.isnan(r2["tr_HO"]) and np.isnan(r2["sensitivity"])
    assert r2["bound_sharp"] == r["bound_sharp"]


# ----------------------------------------------------------------------------
# Sketch A: token weights and the weighted accumulation (YAQA article, section 3)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T,d,identity", [(100, 64, False), (333, 129, False), (64, 5, False),
                                          (1000, 300, False), (77, 40, True)])
def test_token_weights_match_oracle(bk, T, d, identity):
    note("token weights T=%d d=%d identity=%d" % (T, d, identity))
    y = workloads.make_x(T, d, 60 + d, "gauss", 2 if d > 2 else 0)
    H = None if identity else oracle.hessian(workloads.make_x(4 * d, d, 61 + d, "gauss", 0)).astype(np.float32)
    Ht = None if H is None else torch.from_numpy(H).to(dev())
    w = bk.token_weights(torch.from_numpy(y).to(dev()), Ht).cpu().numpy().astype(np.float64)
    ref = oracle.token_weights(y, None if H is None else H.astype(np.float64))
    if identity:
        assert np.all(np.abs(w - ref) <= 2 * U32 * ref)
    else:
        ay = np.abs(y.astype(np.float64))
        h64 = H.astype(np.float64)
        mag = np.einsum("tk,kc,tc->t", ay, np.abs(h64), ay) / np.sum(h64 * h64)
        assert np.all(np.abs(w - ref) <= 4 * U32 * np.sqrt(d) * mag + 2 * U32 * np.abs(ref))


@pytest.mark.parametrize("T,d", [(1024, 64), (2000, 129), (333, 100)])
def test_hessian_accum_weighted_matches_oracle(bk, T, d):
    note("hessian weighted T=%d d=%d" % (T, d))
    x = workloads.make_x(T, d, 70 + d, "gauss", 2)
    wt = np.random.default_rng(d).lognormal(0.0, 1.0, T).astype(np.float32)
    wt[::7] = 0.0
    H = bk.hessian_accum(torch.from_numpy(x).to(dev()), alpha=1.0 / T,
                         weights=torch.from_numpy(wt).to(dev())).cpu().numpy()
    x64, w64 = x.astype(np.float64), wt.astype(np.float64)
    ref = oracle.weighted_hessian(x64, w64)
    ax = np.abs(x64)
    # the fp32 sqrt(w) scaling (2 u relative on each product) on top of the fp32 SYRK bound
    bound = (4 * np.sqrt(T) + 4) * U32 * (ax * w64[:, None]).T @ ax / T + 1e-30
    assert np.all(np.abs(H - ref) <= bound), np.max(np.abs(H - ref) / bound)
    assert np.array_equal(H, H.T)


def test_sketch_a_matches_oracle(bk):
    # each device iteration against the oracle's step from the device's previous
    # iterates (so that errors do not compound), then three iterations end to end
    T, n, m = 2048, 96, 80
    w_, x, g = workloads.make_inputs("tiny", m=m, n=n, T=T)
    note("sketch A T=%d n=%d m=%d" % (T, n, m))
    X, G = torch.from_numpy(x).to(dev()), torch.from_numpy(g).to(dev())
    HI, HO = bk.hessian_accum(X), None
    x64, g64 = x.astype(np.float64), g.astype(np.float64)
    for it in range(3):
        hi_prev = HI.cpu().numpy().astype(np.float64)
        ho_prev = None if HO is None else HO.cpu().numpy().astype(np.float64)
        w = bk.token_weights(G, HO)
        v = bk.token_weights(X, HI)
        HI_new = bk.hessian_accum(X, alpha=1.0 / T, weights=w)
        HO = bk.hessian_accum(G, HO, alpha=1.0 / T, weights=v)
        HI = HI_new
        wr = oracle.token_weights(g64, ho_prev)
        vr = oracle.token_weights(x64, hi_prev)
        hi_ref = oracle.weighted_hessian(x64, wr)
        ho_ref = oracle.weighted_hessian(g64, vr)
        # entry by entry: the weights' own fp32 bound (as in the token-weight test:
        # 4 u sqrt(d) |y|^T |H| |y| / ||H||_F^2 + 2 u |w|, or 2 u |w| for the identity)
        # carried through the accumulation, plus the weighted accumulation's bound
        for got, ref, y, yo, wref, hprev in ((HI, hi_ref, x64, g64, wr, ho_prev),
                                             (HO, ho_ref, g64, x64, vr, hi_prev)):
            if hprev is None:
                dw = 2 * U32 * np.abs(wref)
            else:
                ayo = np.abs(yo)
                mag = np.einsum("tk,kc,tc->t", ayo, np.abs(hprev), ayo) / np.sum(hprev * hprev)
                dw = 4 * U32 * np.sqrt(yo.shape[1]) * mag + 2 * U32 * np.abs(wref)
            ay = np.abs(y)
            bound = (ay * dw[:, None]).T @ ay / T + (4 * np.sqrt(T) + 4) * U32 * (ay * np.abs(wref)[:, None]).T @ ay / T
            err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
            assert np.all(err <= bound + 1e-30), (it, float(np.max(err / (bound + 1e-30))))
    hi3, ho3 = bk.sketch_a(X, G, 3)
    ri, ro = oracle.sketch_a(x64, g64, 3)
    assert np.linalg.norm(hi3.cpu().numpy() - ri) / np.linalg.norm(ri) < 1e-5
    assert np.linalg.norm(ho3.cpu().numpy() - ro) / np.linalg.norm(ro) < 1e-5


# ----------------------------------------------------------------------------
# end to end: the device chain (quantize_layer) against the oracle chain (pipeline)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name,bits,one_sided", [("tiny", 2, False), ("small", 3, False), ("small", 3, True)])
def test_chain_matches_oracle_chain(bk, name, bits, one_sided):
    # The device forms its factors in fp32 (Hessian) and fp64 (LDL, rounded to fp32);
    # the oracle forms them in fp64 throughout. The device's codes must replay cleanly
    # against the device's own factors, and the two chains' proxy losses must agree
    # to 1e-4 (each chain's loss under its own damped factors; H_O = I is damped to
    # 1.01 I on both sides). Free-run code differences between the chains are counted
    # and recorded.
    w, x, g = workloads.make_inputs(name)
    note("chain %s bits=%d one_sided=%d" % (name, bits, one_sided))
    d = dev()
    W, X, G = (torch.from_numpy(a).to(d) for a in (w, x, g))
    res, (LO, DO, LI, DI) = bk.quantize_layer(W, X, None if one_sided else G, bits, want_delta=True)
    torch.cuda.synchronize()
    assert int(res.info.item()) == 0
    ref = oracle.pipeline(w, x, g, bits, one_sided=one_sided)
    codes = res.codes.cpu().numpy()
    scales = res.scales.cpu().numpy()
    assert np.array_equal(scales, ref["scales"])
    do = DO.cpu().numpy().astype(np.float64)
    di = DI.cpu().numpy().astype(np.float64)
    if one_sided:
        assert np.all(do == np.float32(1.01))
    lo = None if one_sided else np.triu(LO.cpu().numpy(), 1).astype(np.float64)
    li = np.triu(LI.cpu().numpy(), 1).astype(np.float64)
    rp = oracle.replay(w, lo, li, scales, bits, codes, DO=do, DI=di)
    assert rp["bad"] == 0 and rp["max_flip_margin"] < 1e-4
    loss = float(res.loss.item())
    assert abs(loss - rp["loss"]) <= 1e-4 * abs(rp["loss"])
    ref_loss = oracle.loss_identity(ref["eta"], ref["DO"], ref["DI"])
    mism = int((codes != ref["codes"]).sum())
    rel = abs(loss - ref_loss) / ref_loss
    # the device's codes under the oracle chain's own fp64 factors
    cross = oracle.proxy_loss(res.delta.cpu().numpy().astype(np.float64),
                              None if one_sided else ref["HO"], ref["HI"]) * (1.01 if one_sided else 1.0)
    note("  chain: free-run mismatches %d, loss device %.10g oracle chain %.10g rel %.2e, "
         "device codes under oracle factors rel %.2e" % (mism, loss, ref_loss, rel, abs(cross - ref_loss) / ref_loss))
    record_parity("chain-" + name + ("-H_O=I" if one_sided else ""), m=w.shape[0], n=w.shape[1], bits=bits,
                  rounding="nearest", one_sided=one_sided, entries=w.size, replayed=w.size,
                  flips=rp["flips"], max_flip_margin=rp["max_flip_margin"], bad=rp["bad"],
                  replay_mismatches=rp["mismatches"], clamped=int(res.clamped.item()),
                  free_mismatch=mism, free_clamped=ref["clamped"], loss=loss, loss_ref=rp["loss"],
                  loss_rel=abs(loss - rp["loss"]) / rp["loss"], free_loss=ref_loss, free_loss_rel=rel,
                  cross_loss_rel=abs(cross - ref_loss) / ref_loss)
    assert rel <= 1e-4


def test_sketch_b_checks_the_output_factors(bk):
    # a wrong-shape H_O (k x m with k < m would pass a leading-dimension check) and a
    # factor on the wrong dtype are rejected before anything is launched; a
    # preallocated strided H_O is filled in place
    note("sketch B output checks")
    S, m, n = 2, 40, 72
    g = workloads.make_grads(S, m, n, 77)
    Gt = torch.from_numpy(g).to(dev())
    with pytest.raises(ValueError):
        bk.sketch_b(Gt, HO=torch.empty((m // 2, m), device=dev()))
    with pytest.raises(ValueError):
        bk.sketch_b(Gt, HI=torch.empty((n, n), dtype=torch.float64, device=dev()))
    big = torch.full((m, m + 5), float("nan"), device=dev())
    HOv = big[:, 2:2 + m]
    HI, HO = bk.sketch_b(Gt, HO=HOv)
    assert HO.data_ptr() == HOv.data_ptr()
    ri, ro = oracle.sketch_b(list(g))
    ag = np.abs(g.astype(np.float64))
    bo = 8 * U32 * np.sqrt(S * n) * sum(a @ a.T for a in ag) / (S * n) + 1e-30
    assert np.all(np.abs(HOv.cpu().numpy() - ro) <= bo)
    rest = big.cpu().numpy()
    assert np.all(np.isnan(rest[:, :2])) and np.all(np.isnan(rest[:, 2 + m:]))
