"""Helpers shared by the tests: move seeded inputs to the GPU, compare with the oracle."""
from __future__ import annotations

import numpy as np

import ttt_inputs as ti


def to_device(inp: ti.Inputs, device="cuda:0", dtype=None):
    """Q, K, V, W1 (and W2), eta of a full-chain Inputs as device tensors.

    Returns dict(q, k, v, w1, w2, eta) with Q/K/V shaped [B, H, T, d] in the
    config's storage dtype (the exact bits the oracle reads).
    """
    import torch

    cfg = inp.cfg
    assert len(inp.chains) == cfg.chains and np.all(inp.chains == np.arange(cfg.chains))
    shape = (cfg.B, cfg.H, cfg.T, cfg.d)
    dtype = dtype or cfg.dtype

    def qkv(x):
        if dtype == "bf16":
            bits = ti.bf16_round(x)[1]
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).reshape(shape).to(device)
        return torch.from_numpy(np.ascontiguousarray(x)).reshape(shape).to(device)

    out = dict(q=qkv(inp.q), k=qkv(inp.k), v=qkv(inp.v),
               w1=torch.from_numpy(inp.w1).to(device),
               w2=None if inp.w2 is None else torch.from_numpy(inp.w2).to(device))
    sb, sh, st = inp.eta_strides
    if (sb, sh, st) == (0, 0, 0):
        out["eta"] = torch.from_numpy(inp.eta_buf[:1].copy()).to(device)
    elif (sb, sh, st) == (0, 1, 0):
        out["eta"] = torch.from_numpy(inp.eta_buf.copy()).to(device)
    else:
        out["eta"] = torch.from_numpy(inp.eta_buf.reshape(cfg.B, cfg.H, cfg.T).copy()).to(device)
    return out


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
