"""Seeded synthetic inputs for LayerNorm workloads.

Shared by the tests, the smoke check and the benchmark; it holds none of the
method's arithmetic.  Each tensor is drawn in float64 from its own numpy
PCG64 stream (children of ``SeedSequence(seed)``, always spawned in the same
fixed order so a tensor's values do not depend on which others are asked
for), then cast to the storage dtype.  The GPU library and the oracle both
read the identical stored values.

Default distributions (N(a, b) = mean a, standard deviation b):
x ~ N(0, 1), residual ~ N(0, 1), bias ~ N(0, 0.02), gamma ~ U(0.5, 1.5),
beta ~ N(0, 0.1), dy ~ N(0, 1).  With `outlier_frac` > 0, that fraction
of the x entries (drawn after x from x's stream) is replaced by
+-`outlier_value`: the occasional activation outliers of a few hundred that
large models carry.
"""
from __future__ import annotations

import numpy as np
import torch

NAMES = ("x", "residual", "bias", "gamma", "beta", "dy")


def _generators(seed: int):
    children = np.random.SeedSequence(int(seed)).spawn(len(NAMES))
    return {n: np.random.Generator(np.random.PCG64(c)) for n, c in zip(NAMES, children)}


def to_storage(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Cast float64 samples to the storage dtype (CPU tensor)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(dtype)


def layer_inputs(rows: int, cols: int, dtype: torch.dtype, seed: int = 0,
                 x_mean: float = 0.0, x_std: float = 1.0,
                 names=NAMES, outlier_frac: float = 0.0,
                 outlier_value: float = 300.0) -> dict:
    """Dict of CPU tensors in `dtype`: [rows, cols] x, residual, dy and
    [cols] bias, gamma, beta (only those listed in `names`)."""
    gens = _generators(seed)

    def draw_x(g):
        a = g.normal(x_mean, x_std, size=(rows, cols))
        if outlier_frac > 0.0:
            hit = g.random(size=(rows, cols)) < outlier_frac
            sign = np.where(g.random(size=(rows, cols)) < 0.5, -1.0, 1.0)
            a = np.where(hit, sign * outlier_value, a)
        return a

    draw = {
        "x": draw_x,
        "residual": lambda g: g.normal(0.0, 1.0, size=(rows, cols)),
        "bias": lambda g: g.normal(0.0, 0.02, size=(cols,)),
        "gamma": lambda g: g.uniform(0.5, 1.5, size=(cols,)),
        "beta": lambda g: g.normal(0.0, 0.1, size=(cols,)),
        "dy": lambda g: g.normal(0.0, 1.0, size=(rows, cols)),
    }
    return {n: to_storage(draw[n](gens[n]), dtype) for n in names}


def class_labels(rows: int, classes: int, seed: int = 0, ignore_frac: float = 0.0,
                 ignore_index: int = -100) -> torch.Tensor:
    """[rows] int64 class indices, uniform over [0, classes), from their own
    PCG64 stream; with `ignore_frac` > 0 that fraction of the rows (drawn
    after the labels) is set to `ignore_index`."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), 7919])))
    lab = g.integers(0, classes, size=rows, dtype=np.int64)
    if ignore_frac > 0.0:
        lab = np.where(g.random(rows) < ignore_frac, np.int64(ignore_index), lab)
    return torch.from_numpy(np.ascontiguousarray(lab))


def logits(rows: int, ld: int, dtype: torch.dtype, seed: int = 0, mean: float = 0.0,
           std: float = 2.0) -> torch.Tensor:
    """[rows, ld] logits ~ N(mean, std) in `dtype` (CPU), from their own
    PCG64 stream (columns past the classes, if any, hold values too: padding
    a kernel must not use)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), 104729])))
    return to_storage(g.normal(mean, std, size=(rows, ld)), dtype)


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 numpy copy of a (CPU or GPU) tensor."""
    return t.detach().to("cpu", torch.float64).numpy()
