"""The seeded input sets and their .npy cache (host only)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import workloads  # noqa: E402


def test_inputs_are_reproducible():
    a = workloads.make_inputs("tiny")
    b = workloads.make_inputs("tiny")
    for u, v in zip(a, b):
        assert u.dtype == np.float32 and np.array_equal(u, v)


def test_input_cache_round_trip(tmp_path, monkeypatch):
    d = str(tmp_path / "cache")
    first = workloads.make_inputs("small", m=96, n=80, T=300, cache_dir=d)
    files = sorted(os.listdir(d))
    assert len(files) == 3 and all(f.endswith(".npy") for f in files)

    def no_draw(*args, **kwargs):
        raise AssertionError("drew inputs although the cache holds them")

    monkeypatch.setattr(workloads, "make_w", no_draw)
    monkeypatch.setattr(workloads, "make_x", no_draw)
    monkeypatch.setattr(workloads, "make_g", no_draw)
    again = workloads.make_inputs("small", m=96, n=80, T=300, cache_dir=d)
    for u, v in zip(first, again):
        assert np.array_equal(u, v)
    # another shape is another key: it must draw (and here fails to)
    with pytest.raises(AssertionError, match="drew inputs"):
        workloads.make_inputs("small", m=96, n=81, T=300, cache_dir=d)


def test_input_cache_from_environment(tmp_path, monkeypatch):
    d = str(tmp_path / "env_cache")
    monkeypatch.setenv("BAKRON_INPUT_CACHE", d)
    w, x, g = workloads.make_inputs("tiny")
    assert len(os.listdir(d)) == 3
    ref = workloads.make_inputs("tiny", cache_dir="")
    for u, v in zip((w, x, g), ref):
        assert np.array_equal(u, v)
