"""Seeded synthetic inputs for the BaKron rounding pipeline.

This module only draws random numbers. It holds none of the method's
arithmetic (no Hessian, factorisation, scale or rounding), so that the CPU
oracle and the HIP path can both consume the same bytes without sharing any
computation.

The five workloads stand in for real layers whose weights and calibration
data are not available: a tiny 64x64 case, a 512x512 case, an attention
projection (4096x4096), an MLP down-projection (4096x14336) and a 70B-scale
MLP up-projection (28672x8192). The Hessian factors of the Kronecker model
are built from a synthetic input matrix X (T x n, one row per token) and a
synthetic output-gradient matrix G (T x m), following the factor definitions
H_I = E[x^T x] and H_O = E[g^T g] (YAQA article, section 3 "Kronecker-factored
Hessian estimation"; K-FAC tutorial on mlqm.cn, section 3).

Recipe (all fp32, numpy PCG64 streams):
  W*  m x n : N(0, 0.02^2) times a per-row lognormal(0, 0.3) factor.
  X   T x n : N(0, 1) times a per-column lognormal(0, 1) factor, then a few
              outlier columns multiplied by 20 (2 for tiny/small, 8 for the
              attention and up-projection shapes). For the down-projection
              (post-activation inputs) X = |N(0, 1)| times lognormal(0, 1)
              per column, with 0.5 % of the columns (72) multiplied by 30.
  G   T x m : N(0, 1) times a per-column lognormal(0, 0.5) factor.
Seeds: W 1000+k, X 2000+k, G 3000+k, stochastic rounding 4000+k for
workload k = 0..4.
Sketch B (YAQA article, section 3) takes per-sequence weight gradients instead
of X and G: make_grads draws S x m x n with the G row scales and the X column
scales and outliers (seed 5000+k in bench.py).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_w", "make_x", "make_g", "make_grads", "make_inputs"]


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    m: int            # output features (rows of W*)
    n: int            # input features (columns of W*)
    T: int            # tokens used for both factors
    bits: tuple       # bit widths exercised
    roundings: tuple  # "nearest" / "stochastic"
    x_kind: str       # "gauss" or "relu"
    x_outliers: int
    x_outlier_mult: float

    @property
    def seed_w(self) -> int:
        return 1000 + self.key

    @property
    def seed_x(self) -> int:
        return 2000 + self.key

    @property
    def seed_g(self) -> int:
        return 3000 + self.key

    @property
    def seed_round(self) -> int:
        return 4000 + self.key


WORKLOADS = {
    "tiny": Workload(0, "tiny", 64, 64, 1024, (2,), ("nearest",), "gauss", 2, 20.0),
    "small": Workload(1, "small", 512, 512, 8192, (3,), ("nearest",), "gauss", 2, 20.0),
    "attn": Workload(2, "attn", 4096, 4096, 32768, (2, 4), ("nearest", "stochastic"),
                     "gauss", 8, 20.0),
    "mlp_down": Workload(3, "mlp_down", 4096, 14336, 32768, (2,), ("nearest",), "relu", 72, 30.0),
    "up70b": Workload(4, "up70b", 28672, 8192, 16384, (2,), ("nearest",), "gauss", 8, 20.0),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def make_w(m: int, n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    row = rng.lognormal(0.0, 0.3, size=m).astype(np.float32)
    w = rng.standard_normal((m, n), dtype=np.float32)
    w *= np.float32(0.02)
    w *= row[:, None]
    return w


def make_x(T: int, n: int, seed: int, kind: str = "gauss", outliers: int = 2,
           mult: float = 20.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    col = rng.lognormal(0.0, 1.0, size=n).astype(np.float32)
    idx = rng.choice(n, size=min(outliers, n), replace=False) if outliers > 0 else np.zeros(0, int)
    col[idx] *= np.float32(mult)
    x = rng.standard_normal((T, n), dtype=np.float32)
    if kind == "relu":
        np.abs(x, out=x)
    elif kind != "gauss":
        raise ValueError(kind)
    x *= col[None, :]
    return x


def make_g(T: int, m: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    col = rng.lognormal(0.0, 0.5, size=m).astype(np.float32)
    g = rng.standard_normal((T, m), dtype=np.float32)
    g *= col[None, :]
    return g


# Bump when the recipe above changes: cached inputs drawn under another version
# are then ignored.
RECIPE_VERSION = 1


def _cache_paths(cache_dir: str, wl: Workload, m: int, n: int, T: int):
    """The three .npy files of one input set, named by workload, shape, seeds and recipe."""
    import hashlib
    import os

    key = "%r|%d|%d|%d|%d" % (wl, m, n, T, RECIPE_VERSION)
    tag = "%s-%dx%d-T%d-s%d-%s" % (wl.name, m, n, T, wl.key, hashlib.sha256(key.encode()).hexdigest()[:12])
    return [os.path.join(cache_dir, "%s-%s.npy" % (tag, part)) for part in ("w", "x", "g")]


def make_inputs(name: str, m: int | None = None, n: int | None = None, T: int | None = None,
                cache_dir: str | None = None):
    """(W*, X, G) for a named workload; m/n/T may be overridden for scaled-down variants.

    cache_dir (default: the BAKRON_INPUT_CACHE environment variable, if set): a
    directory of .npy files keyed by workload, shape, seeds and recipe version. A
    set found there is loaded instead of drawn (plain arrays, no pickles); one
    drawn here is written there. The arrays are the same either way.
    """
    import os

    wl = WORKLOADS[name]
    m = wl.m if m is None else m
    n = wl.n if n is None else n
    T = wl.T if T is None else T
    if cache_dir is None:
        cache_dir = os.environ.get("BAKRON_INPUT_CACHE") or None
    paths = _cache_paths(cache_dir, wl, m, n, T) if cache_dir else None
    if paths and all(os.path.exists(p) for p in paths):
        w, x, g = (np.load(p, allow_pickle=False) for p in paths)
        if w.shape == (m, n) and x.shape == (T, n) and g.shape == (T, m):
            return w, x, g
    w = make_w(m, n, wl.seed_w)
    x = make_x(T, n, wl.seed_x, wl.x_kind, min(wl.x_outliers, n), wl.x_outlier_mult)
    g = make_g(T, m, wl.seed_g)
    if paths:
        os.makedirs(cache_dir, exist_ok=True)
        for p, a in zip(paths, (w, x, g)):
            tmp = "%s.tmp%d.npy" % (p[:-4], os.getpid())
            np.save(tmp, a, allow_pickle=False)
            os.replace(tmp, p)
    return w, x, g



def make_grads(S: int, m: int, n: int, seed: int, outliers: int = 8, mult: float = 20.0) -> np.ndarray:
    """S per-sequence weight gradients (S x m x n fp32) for the Sketch B estimate.

    G_s = N(0, 1) scaled per output row by lognormal(0, 0.5) (the output-gradient
    recipe) and per input column by lognormal(0, 1) with `outliers` columns
    multiplied by `mult` (the input recipe): a weight gradient is a sum of
    outer products of output gradients and inputs, so it carries both scales.
    """
    rng = np.random.default_rng(seed)
    row = rng.lognormal(0.0, 0.5, size=m).astype(np.float32)
    col = rng.lognormal(0.0, 1.0, size=n).astype(np.float32)
    idx = rng.choice(n, size=min(outliers, n), replace=False) if outliers > 0 else np.zeros(0, int)
    col[idx] *= np.float32(mult)
    g = rng.standard_normal((S, m, n), dtype=np.float32)
    g *= row[None, :, None]
    g *= col[None, None, :]
    return g
