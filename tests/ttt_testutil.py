"""Helpers shared by the tests: move seeded inputs to the GPU, compare with the oracle.

Parity bars (max over chains of max|x - ref| / max|ref|, per output tensor):

* CONTRACT_BF16 = 2e-3 for bf16 Q/K/V with fp32 outputs, CONTRACT_FP32 = 1e-5
  for fp32 inputs: the tolerances the workload is specified with.
* REGRESS_MFMA = 5e-5, the regression bound of the matrix-core paths.  Every
  fp32 operand enters the bf16 matrix cores as a hi + lo pair, each rounded to
  nearest (bf16 keeps 8 significant bits): |x - hi| <= 2^-8 |x| and
  |x - hi - lo| <= 2^-16 |x|.  Products of bf16 pairs are exact and sums are
  fp32, so a mini-batch adds at most about 2^-16 + 64 * 2^-24 ~ 2e-5 of relative
  error, and the recurrence does not grow it (measured 3e-6 .. 7e-6 at every
  workload).  A dropped lo pass leaves an operand with up to 2^-8 ~ 4e-3
  relative error, eighty times the bound.
* REGRESS_MFMA_LN_MLP = 5e-4 for TTT-MLP with a layer norm inside f and
  random gamma, beta: the recurrence then amplifies rounding on some chains
  (the same arithmetic in fp32 numpy is 5.9e-6 .. 5.7e-5 off the fp64 oracle
  at T = 80 .. 512 on sampled chains; with gamma = 1, beta = 0 the kernel
  holds REGRESS_MFMA at the full workload length).

Besides the max-norm error, :func:`errors` reports the elementwise relative
error with a floor of 1e-6 max|ref| per chain (pure elementwise relative error
is ill-posed near zeros) and the Frobenius relative error, max over chains.
"""
from __future__ import annotations

import numpy as np

import ttt_inputs as ti

CONTRACT_BF16 = 2e-3
CONTRACT_FP32 = 1e-5
REGRESS_MFMA = 5e-5
REGRESS_MFMA_LN_MLP = 5e-4


def to_device(inp, device="cuda:0", dtype=None):
    return ti.to_device(inp, device, dtype)


def rows(t, chains=None):
    """[B, H, ...] device tensor -> [n, ...] numpy fp64 for the given flat chains."""
    a = t.float().cpu().numpy()
    a = a.reshape((-1,) + a.shape[2:])
    return a if chains is None else a[np.asarray(chains)]


def _flat(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    return x.reshape(x.shape[0], -1), ref.reshape(ref.shape[0], -1)


def max_rel(x, ref) -> float:
    """max over chains of max|x - ref| / max|ref| (per chain slice)."""
    xs, rs = _flat(x, ref)
    den = np.abs(rs).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(xs - rs).max(axis=1) / den).max())


def errors(x, ref) -> dict:
    """max_rel, the elementwise relative error with a 1e-6 max|ref| floor, and the
    Frobenius relative error, each the max over chains."""
    xs, rs = _flat(x, ref)
    amax = np.abs(rs).max(axis=1, keepdims=True)
    amax = np.where(amax == 0, 1.0, amax)
    diff = np.abs(xs - rs)
    elem = (diff / np.maximum(np.abs(rs), 1e-6 * amax)).max(axis=1)
    fn = np.sqrt((rs * rs).sum(axis=1))
    frob = np.sqrt((diff * diff).sum(axis=1)) / np.where(fn == 0, 1.0, fn)
    return {"max": float((diff.max(axis=1) / amax[:, 0]).max()), "elem": float(elem.max()),
            "frob": float(frob.max())}


def parity(label, pairs, contract=CONTRACT_BF16, regress=None):
    """Compare each (name, x, ref) of ``pairs``; print the three errors of every
    output and assert max_rel < contract (and < regress, the path's regression
    bound, when given) and the Frobenius error < contract.  Returns the errors."""
    out = {}
    for name, x, ref in pairs:
        out[name] = errors(x, ref)
    print(f"[{label}] " + "  ".join(f"{n}: max {e['max']:.2e} elem {e['elem']:.2e} frob {e['frob']:.2e}"
                                    for n, e in out.items()), flush=True)
    for n, e in out.items():
        assert e["max"] < contract, (label, n, e, "contract", contract)
        assert e["frob"] < contract, (label, n, e, "contract", contract)
        if regress is not None:
            assert e["max"] < regress, (label, n, e, "regression bound", regress)
    return out
