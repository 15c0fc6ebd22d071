"""bench.py's host-side pieces: the replay of a step's codes and the counter keys (no GPU)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402


def _tiny_step(bits=2, rounding="nearest", seed=4000):
    w, x, g = workloads.make_inputs("tiny")
    LI, DI = oracle.udu(oracle.damp(oracle.hessian(x)))
    LO, DO = oracle.udu(oracle.damp(oracle.hessian(g)))
    s = oracle.row_scales(w, bits)
    r = oracle.sweep(w, LO, LI, s, bits, rounding, seed)
    dev = {"W": w, "codes": r["codes"].copy(), "scales": s, "DO": DO, "DI": DI,
           "loss": oracle.loss_identity(r["eta"], DO, DI)}
    return dev, LO, LI


def test_replay_of_exact_codes_is_clean():
    for rounding in ("nearest", "stochastic"):
        dev, LO, LI = _tiny_step(rounding=rounding)
        full = bench._replay(dev, LO, LI, 2, rounding, 4000, None)
        assert full["entries"] == 64 * 64 and full["mismatches"] == 0 and full["bad"] == 0
        assert full["loss_rel"] < 1e-12
        part = bench._replay(dev, LO, LI, 2, rounding, 4000, 16)
        assert part["entries"] == 16 * 64 and part["mismatches"] == 0 and part["bad"] == 0


def test_replay_counts_a_wrong_code_as_bad():
    dev, LO, LI = _tiny_step()
    # an entry far from any boundary, moved by one code: a bad entry, not a flip
    i, j = 5, 7
    c = int(dev["codes"][i, j])
    dev["codes"][i, j] = c + 1 if c < 3 else c - 1
    rp = bench._replay(dev, LO, LI, 2, "nearest", 4000, None)
    assert rp["bad"] >= 1 and rp["flips"] == 0
    rows = bench._replay(dev, LO, LI, 2, "nearest", 4000, i + 1)
    assert rows["bad"] >= 1


def test_no_replay_without_a_step():
    assert bench._replay(None, None, None, 2, "nearest", 0, None) is None


def test_counter_readings_follow_the_source_key(monkeypatch):
    # a reading taken on other sources is not reported
    key = ("solve", "attn", "0" * 16)
    monkeypatch.setattr(bench, "COUNTERS", {key: {"fetch_kib": 1.0, "write_kib": 1.0, "mfma_busy": 0.5,
                                                  "clock_ghz": 2.0}})
    assert bench.traffic_bytes("solve", "attn") is None
    assert bench.mfma_counters("solve", "attn") is None
    real = ("solve", "attn", bench.source_key("solve"))
    monkeypatch.setattr(bench, "COUNTERS", {real: {"fetch_kib": 1.0, "write_kib": 2.0, "mfma_busy": 0.5,
                                                   "clock_ghz": 2.0}})
    assert bench.mfma_counters("solve", "attn") == {"mfma_busy": 0.5, "clock_ghz": 2.0}
    cal = bench.CAL_BYTES / 1024.0
    want = 1024.0 * (1.0 * cal / bench.CAL_FETCH_KIB + 2.0 * cal / bench.CAL_WRITE_KIB)
    assert np.isclose(bench.traffic_bytes("solve", "attn"), want)
