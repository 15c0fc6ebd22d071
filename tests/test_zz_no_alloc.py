"""bakron_solve_noalloc (the solve for callers that cannot allocate) against
bakron_solve, through the C ABI: the two entry points run the same kernels, so
every output must be identical, and the codes must replay cleanly against the
oracle. Two calls in a row, the second on a smaller layer, so the second runs in
the scratch array the first one left behind."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def note(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def bk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kronecker_hessian_rounding_amd as m
    return m


def layer(m, n, seed):
    w, x, g = workloads.make_inputs("tiny", m=m, n=n, T=max(4 * max(m, n), 256))
    HI = oracle.damp(oracle.hessian(x))
    HO = oracle.damp(oracle.hessian(g))
    (LI, DI), (LO, DO) = oracle.udu(HI), oracle.udu(HO)
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return w, f(LO), f(LI), f(DO), f(DI)


def outputs(m, n, d):
    return dict(codes=torch.full((m, n), 255, dtype=torch.uint8, device=d),
                scales=torch.full((m,), float("nan"), device=d),
                delta=torch.full((m, n), float("nan"), device=d),
                loss=torch.full((1,), float("nan"), dtype=torch.float64, device=d),
                clamped=torch.full((1,), -1, dtype=torch.int64, device=d),
                info=torch.full((1,), 99, dtype=torch.int32, device=d))


def call(bk, fn, tensors, o, bits, rounding, seed):
    W, LO, LI, DO, DI = tensors
    m, n = W.shape
    q = bk._binding._Quantizer(bits, bk._binding.ROUNDING[rounding], seed, None)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [p(W), m, n, n, p(LO), m, p(LI), n, ctypes.byref(q), p(o["codes"]), n, p(o["scales"]),
            p(o["delta"]), n, p(DO), p(DI), p(o["loss"]), p(o["clamped"]), p(o["info"])]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if fn == "noalloc":
        st = bk.LIB.bakron_solve_noalloc(*args, stream)
    else:
        nb = bk.LIB.bakron_solve_workspace_bytes(m, n)
        ws = torch.empty(nb, dtype=torch.uint8, device=W.device)
        st = bk.LIB.bakron_solve(*args, p(ws), nb, stream)
        torch.cuda.synchronize()
        del ws
    assert st == bk.BAKRON_OK
    torch.cuda.synchronize()


@pytest.mark.parametrize("shapes", [((700, 600, 2, "nearest"), (130, 66, 3, "stochastic")),
                                    ((1024, 2000, 2, "nearest"), (300, 260, 4, "nearest"))])
def test_noalloc_matches_solve(bk, shapes):
    d = torch.device("cuda:0")
    for k, (m, n, bits, rounding) in enumerate(shapes):
        note("noalloc call %d: m=%d n=%d bits=%d %s" % (k, m, n, bits, rounding))
        w, LO, LI, DO, DI = layer(m, n, 7 + k)
        tensors = [torch.from_numpy(a).to(d) for a in (w, LO, LI, DO, DI)]
        ref, got = outputs(m, n, d), outputs(m, n, d)
        call(bk, "solve", tensors, ref, bits, rounding, 4000 + k)
        call(bk, "noalloc", tensors, got, bits, rounding, 4000 + k)
        assert int(got["info"].item()) == 0 and int(ref["info"].item()) == 0
        for key in ("codes", "scales", "delta", "loss", "clamped"):
            assert torch.equal(got[key], ref[key]), key
        codes = got["codes"].cpu().numpy()
        scales = got["scales"].cpu().numpy()
        rp = oracle.replay(w, LO.astype(np.float64), LI.astype(np.float64), scales, bits, codes, rounding,
                           4000 + k, DO=DO.astype(np.float64), DI=DI.astype(np.float64))
        assert rp["bad"] == 0 and rp["max_flip_margin"] < 1e-4
        assert abs(float(got["loss"].item()) - rp["loss"]) <= 1e-4 * rp["loss"]
        note("  identical to bakron_solve; flips %d, loss %.8g" % (rp["flips"], float(got["loss"].item())))


def test_noalloc_binding_allocates_nothing_per_call(bk):
    # the binding's solve_noalloc with preallocated outputs: the caching allocator's
    # count of device allocations does not move across the call
    d = torch.device("cuda:0")
    m, n = 200, 150
    w, LO, LI, DO, DI = layer(m, n, 3)
    W, LOt, LIt, DOt, DIt = (torch.from_numpy(a).to(d) for a in (w, LO, LI, DO, DI))
    o = outputs(m, n, d)
    out = bk.SolveResult(**o)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats(d).get("allocation.all.allocated", 0)
    bk.solve_noalloc(W, LOt, LIt, 2, out, D_O=DOt, D_I=DIt)
    torch.cuda.synchronize()
    after = torch.cuda.memory_stats(d).get("allocation.all.allocated", 0)
    assert after == before
    ref = bk.solve(W, LOt, LIt, 2, D_O=DOt, D_I=DIt, want_delta=True, want_loss=True)
    torch.cuda.synchronize()
    assert torch.equal(out.codes, ref.codes) and torch.equal(out.loss, ref.loss)
