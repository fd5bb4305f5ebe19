"""Helpers shared by the tests: move seeded inputs to the GPU, compare with the oracle."""
from __future__ import annotations

import numpy as np

import ttt_inputs as ti


def to_device(inp, device="cuda:0", dtype=None):
    return ti.to_device(inp, device, dtype)


def rows(t, chains=None):
    """[B, H, ...] device tensor -> [n, ...] numpy fp64 for the given flat chains."""
    a = t.float().cpu().numpy()
    a = a.reshape((-1,) + a.shape[2:])
    return a if chains is None else a[np.asarray(chains)]


def max_rel(x, ref) -> float:
    """max over chains of max|x - ref| / max|ref| (per chain slice)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    xs, rs = x.reshape(x.shape[0], -1), ref.reshape(ref.shape[0], -1)
    den = np.abs(rs).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(xs - rs).max(axis=1) / den).max())
