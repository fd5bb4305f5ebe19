"""TEST INFRASTRUCTURE -- the fp64 CPU oracle of the TTT layer forward pass.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP library
(``test_sequence_layer_amd``) and neither imports the other; the only module
both sides use is ``ttt_inputs`` (seeded random inputs, no method arithmetic).

Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
(aharts.cn / itmax.cn).  Sections cited: 03 §1 (hidden state = weights W_t,
output with the updated W_t, update = one GD step), 03 §5 (multi-view
reconstruction loss |f(theta_K x; W) - theta_V x|^2, output f(theta_Q x; W)),
03 §6 (mini-batch GD: gradients at the state before the mini-batch), 03 §7
(dual form), 03 §8 (linear f + batch GD equals linear attention), 03 §9
(TTT-Linear f = W x, TTT-MLP with hidden width 4x and GELU).

Contents
  linear_primal / mlp_primal   fp64 primal form in C (OpenMP over chains) --
                               THE oracle the HIP path is compared with.
  linear_primal_exact          the same primal loop in pure Python over any
                               number type (fractions.Fraction for exact runs).
  linear_dual_exact            the dual form written out from 03 §7, pure
                               Python, any number type (self-check only).
  linear_ln_primal             fp64 primal form of TTT-Linear with layer norm
                               and residual inside f (03 §9), in C.
  linear_grads                 gradients of TTT-Linear: torch fp64 autograd
                               through the primal loop (linear_primal_torch).
  linear_primal_grads          the same gradients by a hand-written reverse
                               pass of the primal loop in C (fast; pinned by
                               finite differences and against linear_grads).
  mlp_grads                    gradients of TTT-MLP: torch fp64 autograd
                               through mlp_primal_torch.
  mlp_primal_grads             the same by a hand-written reverse pass of the
                               TTT-MLP primal loop in C (pinned by finite
                               differences, against mlp_grads, eta = 0).
  mlp_ln_grads                 gradients of TTT-MLP with layer norm and
                               residual inside f (dgamma, dbeta included):
                               torch fp64 autograd through mlp_ln_primal_torch
                               (pinned against the C forward oracle
                               mlp_ln_primal, by gradcheck and by eta = 0).
  linear_dual_f64, mlp_dual_f64, linear_naive_f64, mlp_primal_np,
  linear_ln_dual_f64
                               numpy fp64 forms used only to check the oracle.
  gelu, gelu_prime             exact-erf GELU and its derivative (numpy).

Parity pins: every function above is checked in tests/test_oracle_*.py
against closed forms, invariants and exact-rational arithmetic.  The absolute
values at full workload size are not printed on the pages (every formula and
plot there was an image) -- beyond the pins, parity is unpinned by the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction  # noqa: F401  (re-exported for tests)
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_LIB = os.path.join(_HERE, "libttt_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle into oracle/libttt_oracle.so (gcc, OpenMP)."""
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", _SRC, "-o", _LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_linear_primal.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, dp, i]
    lib.oracle_linear_primal.restype = None
    lib.oracle_mlp_primal.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, dp, i]
    lib.oracle_mlp_primal.restype = None
    lib.oracle_linear_ln_primal.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, ctypes.c_double, dp, dp, dp, i]
    lib.oracle_linear_ln_primal.restype = None
    lib.oracle_linear_primal_grads.argtypes = [i, i, i, i] + [dp] * 12 + [i]
    lib.oracle_mlp_ln_primal.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, ctypes.c_double, dp, dp, dp,
                                         dp, i]
    lib.oracle_linear_primal_grads.restype = None
    lib.oracle_mlp_primal_grads.argtypes = [i, i, i, i, i] + [dp] * 15 + [i]
    lib.oracle_mlp_primal_grads.restype = None
    lib.oracle_linear_ln_primal_grads.argtypes = ([i, i, i, i] + [dp] * 6 + [ctypes.c_double] + [dp] * 3 + [dp] * 7
                                                  + [i])
    lib.oracle_linear_ln_primal_grads.restype = None
    lib.oracle_max_threads.restype = i
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def linear_primal(q, k, v, w0, eta, b: int, threads: int = 0):
    """TTT-Linear, primal form, fp64, for n independent chains.

    q, k, v : [n, T, d];  w0 : [n, d, d] (z = W q);  eta : [n, T]
    returns (z [n, T, d], w_final [n, d, d]) in fp64.
    """
    q, k, v, w0, eta = map(_f64, (q, k, v, w0, eta))
    n, T, d = q.shape
    assert k.shape == v.shape == (n, T, d) and w0.shape == (n, d, d) and eta.shape == (n, T)
    assert b >= 1
    z = np.empty((n, T, d))
    wf = np.empty((n, d, d))
    if n:
        _load().oracle_linear_primal(n, T, d, b, _ptr(q), _ptr(k), _ptr(v), _ptr(w0), _ptr(eta),
                                     _ptr(z), _ptr(wf), int(threads))
    return z, wf


def linear_primal_grads(q, k, v, w0, eta, b: int, dz, dwf=None, threads: int = 0):
    """Gradients of  sum(dz * Z) + sum(dwf * W_final)  of TTT-Linear, by
    reverse-mode differentiation of the primal token loop, fp64, in C.

    Shapes as linear_primal; dz : [n, T, d], dwf : [n, d, d] or None.
    returns (dq, dk, dv, deta [n, T], dw0 [n, d, d]).
    """
    q, k, v, w0, eta, dz = map(_f64, (q, k, v, w0, eta, dz))
    n, T, d = q.shape
    assert k.shape == v.shape == dz.shape == (n, T, d) and w0.shape == (n, d, d) and eta.shape == (n, T)
    assert b >= 1
    dwf_p = None
    if dwf is not None:
        dwf = _f64(dwf)
        assert dwf.shape == (n, d, d)
        dwf_p = _ptr(dwf)
    dq, dk, dv = (np.empty((n, T, d)) for _ in range(3))
    deta = np.empty((n, T))
    dw0 = np.empty((n, d, d))
    if n:
        _load().oracle_linear_primal_grads(n, T, d, b, _ptr(q), _ptr(k), _ptr(v), _ptr(w0), _ptr(eta),
                                           _ptr(dz), dwf_p, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta), _ptr(dw0),
                                           int(threads))
    return dq, dk, dv, deta, dw0


def mlp_primal_grads(q, k, v, w1, w2, eta, b: int, dz, dw1f=None, dw2f=None, threads: int = 0):
    """Gradients of  sum(dz * Z) + sum(dw1f * W1_final) + sum(dw2f * W2_final)
    of TTT-MLP, by reverse-mode differentiation of the primal token loop
    (mlp_primal), fp64, in C.

    Shapes as mlp_primal; dz : [n, T, d], dw1f : [n, dh, d] or None,
    dw2f : [n, d, dh] or None.
    returns (dq, dk, dv, deta [n, T], dw1 [n, dh, d], dw2 [n, d, dh]).
    """
    q, k, v, w1, w2, eta, dz = map(_f64, (q, k, v, w1, w2, eta, dz))
    n, T, d = q.shape
    dh = w1.shape[1]
    assert k.shape == v.shape == dz.shape == (n, T, d) and eta.shape == (n, T)
    assert w1.shape == (n, dh, d) and w2.shape == (n, d, dh) and b >= 1
    ptrs = []
    for x, shape in ((dw1f, (n, dh, d)), (dw2f, (n, d, dh))):
        if x is None:
            ptrs.append(None)
        else:
            x = _f64(x)
            assert x.shape == shape
            ptrs.append(x)
    dq, dk, dv = (np.empty((n, T, d)) for _ in range(3))
    deta = np.empty((n, T))
    dw1 = np.empty((n, dh, d))
    dw2 = np.empty((n, d, dh))
    if n:
        _load().oracle_mlp_primal_grads(n, T, d, dh, b, _ptr(q), _ptr(k), _ptr(v), _ptr(w1), _ptr(w2), _ptr(eta),
                                        _ptr(dz), None if ptrs[0] is None else _ptr(ptrs[0]),
                                        None if ptrs[1] is None else _ptr(ptrs[1]), _ptr(dq), _ptr(dk), _ptr(dv),
                                        _ptr(deta), _ptr(dw1), _ptr(dw2), int(threads))
    return dq, dk, dv, deta, dw1, dw2


def linear_ln_primal_grads(q, k, v, w0, gamma, beta, eta, b: int, dz, dwf=None, eps: float = 1e-6,
                           threads: int = 0):
    """Gradients of  sum(dz * Z) + sum(dwf * W_final)  of TTT-Linear with LN +
    residual inside f (linear_ln_primal), by reverse-mode differentiation of the
    primal token loop, fp64, in C.  gamma, beta : [n, d] per chain.

    returns (dq, dk, dv, deta [n, T], dw0 [n, d, d], dgamma [n, d], dbeta [n, d]).
    """
    q, k, v, w0, gamma, beta, eta, dz = map(_f64, (q, k, v, w0, gamma, beta, eta, dz))
    n, T, d = q.shape
    assert k.shape == v.shape == dz.shape == (n, T, d) and w0.shape == (n, d, d) and eta.shape == (n, T)
    assert gamma.shape == beta.shape == (n, d) and b >= 1
    dwf_p = None
    if dwf is not None:
        dwf = _f64(dwf)
        assert dwf.shape == (n, d, d)
        dwf_p = _ptr(dwf)
    dq, dk, dv = (np.empty((n, T, d)) for _ in range(3))
    deta = np.empty((n, T))
    dw0 = np.empty((n, d, d))
    dgamma, dbeta = np.empty((n, d)), np.empty((n, d))
    if n:
        _load().oracle_linear_ln_primal_grads(n, T, d, b, _ptr(q), _ptr(k), _ptr(v), _ptr(w0), _ptr(gamma),
                                              _ptr(beta), float(eps), _ptr(eta), _ptr(dz), dwf_p, _ptr(dq),
                                              _ptr(dk), _ptr(dv), _ptr(deta), _ptr(dw0), _ptr(dgamma), _ptr(dbeta),
                                              int(threads))
    return dq, dk, dv, deta, dw0, dgamma, dbeta


def mlp_primal(q, k, v, w1, w2, eta, b: int, threads: int = 0):
    """TTT-MLP (f = W2 GELU(W1 x)), primal form, fp64.

    q, k, v : [n, T, d];  w1 : [n, dh, d];  w2 : [n, d, dh];  eta : [n, T]
    returns (z, w1_final, w2_final).
    """
    q, k, v, w1, w2, eta = map(_f64, (q, k, v, w1, w2, eta))
    n, T, d = q.shape
    dh = w1.shape[1]
    assert w1.shape == (n, dh, d) and w2.shape == (n, d, dh) and eta.shape == (n, T)
    z = np.empty((n, T, d))
    w1f = np.empty((n, dh, d))
    w2f = np.empty((n, d, dh))
    if n:
        _load().oracle_mlp_primal(n, T, d, dh, b, _ptr(q), _ptr(k), _ptr(v), _ptr(w1), _ptr(w2),
                                  _ptr(eta), _ptr(z), _ptr(w1f), _ptr(w2f), int(threads))
    return z, w1f, w2f


def linear_ln_primal(q, k, v, w0, gamma, beta, eta, b: int, eps: float = 1e-6, threads: int = 0):
    """TTT-Linear with LN + residual, f(x) = x + LN(W x), primal form, fp64.

    q, k, v : [n, T, d];  w0 : [n, d, d];  gamma, beta : [n, d];  eta : [n, T]
    returns (z, w_final).
    """
    q, k, v, w0, gamma, beta, eta = map(_f64, (q, k, v, w0, gamma, beta, eta))
    n, T, d = q.shape
    assert w0.shape == (n, d, d) and gamma.shape == (n, d) and beta.shape == (n, d) and eta.shape == (n, T)
    z = np.empty((n, T, d))
    wf = np.empty((n, d, d))
    if n:
        _load().oracle_linear_ln_primal(n, T, d, b, _ptr(q), _ptr(k), _ptr(v), _ptr(w0), _ptr(gamma),
                                        _ptr(beta), float(eps), _ptr(eta), _ptr(z), _ptr(wf), int(threads))
    return z, wf


def mlp_ln_primal(q, k, v, w1, w2, gamma, beta, eta, b: int, eps: float = 1e-6, threads: int = 0):
    """TTT-MLP with LN + residual, f(x) = x + LN(W2 GELU(W1 x)), primal form, fp64.

    q, k, v : [n, T, d];  w1 : [n, dh, d];  w2 : [n, d, dh];  gamma, beta : [n, d];
    eta : [n, T].  returns (z, w1_final, w2_final).
    """
    q, k, v, w1, w2, gamma, beta, eta = map(_f64, (q, k, v, w1, w2, gamma, beta, eta))
    n, T, d = q.shape
    dh = w1.shape[1]
    assert w1.shape == (n, dh, d) and w2.shape == (n, d, dh) and eta.shape == (n, T)
    assert gamma.shape == (n, d) and beta.shape == (n, d)
    z = np.empty((n, T, d))
    w1f = np.empty((n, dh, d))
    w2f = np.empty((n, d, dh))
    if n:
        _load().oracle_mlp_ln_primal(n, T, d, dh, b, _ptr(q), _ptr(k), _ptr(v), _ptr(w1), _ptr(w2), _ptr(gamma),
                                     _ptr(beta), float(eps), _ptr(eta), _ptr(z), _ptr(w1f), _ptr(w2f),
                                     int(threads))
    return z, w1f, w2f


def run_inputs(inp, threads: int = 0):
    """Run the oracle on a ``ttt_inputs.Inputs`` (its selected chains)."""
    cfg = inp.cfg
    eta = inp.eta_rows()
    if cfg.is_mlp:
        return mlp_primal(inp.q, inp.k, inp.v, inp.w_rows(1), inp.w_rows(2), eta, cfg.b, threads)
    return linear_primal(inp.q, inp.k, inp.v, inp.w_rows(1), eta, cfg.b, threads)


# ----------------------------------------------------------------------------
# Pure-Python forms over any number type (exact with fractions.Fraction).
# Vectors are lists, matrices are lists of rows; tokens are indexed 0..T-1.
# ----------------------------------------------------------------------------

def _mv(M, x):
    return [sum((m * xi for m, xi in zip(row, x)), 0) for row in M]


def _dot(x, y):
    return sum((a * c for a, c in zip(x, y)), 0)


def linear_primal_exact(q, k, v, w0, eta, b):
    """Primal TTT-Linear for one chain (03 §1, §5, §6): lists in, lists out."""
    d = len(w0)
    W = [list(r) for r in w0]
    z = []
    T = len(q)
    for t0 in range(0, T, b):
        Wb = [list(r) for r in W]           # state before the mini-batch
        for t in range(t0, min(t0 + b, T)):
            e = [a - c for a, c in zip(_mv(Wb, k[t]), v[t])]
            for i in range(d):
                for j in range(d):
                    W[i][j] -= eta[t] * 2 * e[i] * k[t][j]
            z.append(_mv(W, q[t]))          # output with the updated W_t
    return z, W


def linear_dual_exact(q, k, v, w0, eta, b):
    """Dual form of 03 §7 for one chain, pure Python, any number type.

    Per mini-batch with start state W (columns = tokens of the mini-batch):
      E = W K - V,  A[s][t] = eta_s (k_s . q_t) for s <= t (else 0),
      Z = W Q - 2 E A,  W_next = W - 2 E diag(eta) K^T.
    """
    d = len(w0)
    W = [list(r) for r in w0]
    T = len(q)
    z = []
    for t0 in range(0, T, b):
        ts = list(range(t0, min(t0 + b, T)))
        E = {s: [a - c for a, c in zip(_mv(W, k[s]), v[s])] for s in ts}
        for t in ts:
            wq = _mv(W, q[t])
            corr = [0] * d
            for s in ts:
                if s <= t:
                    a = eta[s] * _dot(k[s], q[t])
                    corr = [c + a * e for c, e in zip(corr, E[s])]
            z.append([x - 2 * c for x, c in zip(wq, corr)])
        Wn = [list(r) for r in W]
        for s in ts:
            for i in range(d):
                for j in range(d):
                    Wn[i][j] -= 2 * eta[s] * E[s][i] * k[s][j]
        W = Wn
    return z, W


# ----------------------------------------------------------------------------
# numpy fp64 forms (self-checks of the C oracle only)
# ----------------------------------------------------------------------------

def linear_dual_f64(q, k, v, w0, eta, b):
    """Dual form (03 §7) per chain in fp64, column notation.  Shapes as linear_primal."""
    q, k, v, w0, eta = map(_f64, (q, k, v, w0, eta))
    n, T, d = q.shape
    z = np.empty((n, T, d))
    wf = np.empty((n, d, d))
    for c in range(n):
        W = w0[c].copy()
        for t0 in range(0, T, b):
            sl = slice(t0, min(t0 + b, T))
            K, V, Q = k[c, sl].T, v[c, sl].T, q[c, sl].T      # d x b columns
            et = eta[c, sl]
            E = W @ K - V
            A = np.triu(K.T @ Q) * et[:, None]               # A[s,t] = eta_s k_s.q_t [s<=t]
            z[c, sl] = (W @ Q - 2.0 * E @ A).T
            W = W - 2.0 * (E * et[None, :]) @ K.T
        wf[c] = W
    return z, wf


def linear_naive_f64(q, k, v, w0, eta, b):
    """The 'naive' form of 03 §7: materialise every d x d gradient G_t."""
    q, k, v, w0, eta = map(_f64, (q, k, v, w0, eta))
    n, T, d = q.shape
    z = np.empty((n, T, d))
    wf = np.empty((n, d, d))
    for c in range(n):
        W = w0[c].copy()
        for t0 in range(0, T, b):
            ts = range(t0, min(t0 + b, T))
            G = [2.0 * np.outer(W @ k[c, t] - v[c, t], k[c, t]) for t in ts]
            for j, t in enumerate(ts):
                Wt = W - sum(eta[c, s] * G[i] for i, s in enumerate(ts) if s <= t)
                z[c, t] = Wt @ q[c, t]
            W = W - sum(eta[c, s] * G[i] for i, s in enumerate(ts))
        wf[c] = W
    return z, wf


def _ln_cols(Y, gamma, beta, eps):
    """Layer norm of every column of Y (d x b): (normalised, std) with per-row gamma, beta."""
    mu = Y.mean(axis=0, keepdims=True)
    s = np.sqrt(((Y - mu) ** 2).mean(axis=0, keepdims=True) + eps)
    Yh = (Y - mu) / s
    return gamma[:, None] * Yh + beta[:, None], Yh, s


def linear_ln_dual_f64(q, k, v, w0, gamma, beta, eta, b, eps=1e-6):
    """Dual form of TTT-Linear with LN + residual, fp64 (self-check only).

    Per mini-batch (columns = tokens, start state W): Y = W K, LN statistics per
    column, G = 2 (K + LN(Y) - V) * gamma, D = (G - mean(G) - Yh mean(G Yh)) / s
    (column means over the d rows), Z = Q + LN(W Q - D (diag(eta) triu(K^T Q))),
    W <- W - D diag(eta) K^T.
    """
    q, k, v, w0, gamma, beta, eta = map(_f64, (q, k, v, w0, gamma, beta, eta))
    n, T, d = q.shape
    z = np.empty((n, T, d))
    wf = np.empty((n, d, d))
    for c in range(n):
        W = w0[c].copy()
        for t0 in range(0, T, b):
            sl = slice(t0, min(t0 + b, T))
            K, V, Q = k[c, sl].T, v[c, sl].T, q[c, sl].T
            et = eta[c, sl]
            Y = W @ K
            L, Yh, s = _ln_cols(Y, gamma[c], beta[c], eps)
            G = 2.0 * (K + L - V) * gamma[c][:, None]
            Dl = (G - G.mean(axis=0, keepdims=True) - Yh * (G * Yh).mean(axis=0, keepdims=True)) / s
            YQ = W @ Q - Dl @ (np.triu(K.T @ Q) * et[:, None])
            z[c, sl] = (Q + _ln_cols(YQ, gamma[c], beta[c], eps)[0]).T
            W = W - (Dl * et[None, :]) @ K.T
        wf[c] = W
    return z, wf


def linear_primal_torch(q, k, v, w0, eta, b):
    """The primal TTT-Linear loop (03 §1, §5, §6) on torch CPU tensors, any dtype.

    Shapes as linear_primal; differentiable, so torch autograd of this loop is
    the reference gradient of the layer.
    """
    import torch

    n, T, d = q.shape
    W = w0.clone()
    zs = []
    for t0 in range(0, T, b):
        Wb = W
        for t in range(t0, min(t0 + b, T)):
            e = torch.einsum("nij,nj->ni", Wb, k[:, t]) - v[:, t]
            W = W - (2.0 * eta[:, t])[:, None, None] * e[:, :, None] * k[:, t][:, None, :]
            zs.append(torch.einsum("nij,nj->ni", W, q[:, t]))
    return torch.stack(zs, dim=1), W


def linear_grads(q, k, v, w0, eta, b, dz, dwf=None):
    """Gradients of  sum(dz * Z) + sum(dwf * W_final)  of TTT-Linear, fp64 autograd
    through the primal loop.  w0 : [n, d, d] (per chain), eta : [n, T].

    returns (dq, dk, dv, deta [n, T], dw0 [n, d, d]) as numpy fp64.
    """
    import torch

    def t(x):
        return torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)

    q_, k_, v_, w_, e_ = t(q), t(k), t(v), t(w0), t(eta)
    z, wf = linear_primal_torch(q_, k_, v_, w_, e_, b)
    loss = (z * torch.tensor(np.asarray(dz, np.float64))).sum()
    if dwf is not None:
        loss = loss + (wf * torch.tensor(np.asarray(dwf, np.float64))).sum()
    loss.backward()
    return tuple(x.grad.numpy() for x in (q_, k_, v_, e_, w_))


def linear_ln_primal_torch(q, k, v, w0, gamma, beta, eta, b, eps=1e-6):
    """The primal TTT-Linear loop with LN + residual inside f, f(x) = x + LN(W x)
    (03 §9), on torch CPU tensors, any dtype; differentiable.

    Token t of a mini-batch: y = Wb k_t (Wb: the state before the mini-batch),
    loss |k_t + LN(y) - v_t|^2, whose gradient with respect to W is delta k_t^T
    with delta the loss gradient pulled back through LN to y (autograd is not
    used for it: it is written out, as the forward computes it);
    W_t = W_{t-1} - eta_t delta k_t^T;  z_t = q_t + LN(W_t q_t).
    LN(y) = gamma * (y - mean(y)) / sqrt(var(y) + eps) + beta over the d entries.
    Shapes: q, k, v [n, T, d]; w0 [n, d, d]; gamma, beta [n, d]; eta [n, T].
    """
    import torch

    def ln_stats(y):
        mu = y.mean(dim=1, keepdim=True)
        dv = y - mu
        s = torch.sqrt((dv * dv).mean(dim=1, keepdim=True) + eps)
        return dv / s, s

    n, T, d = q.shape
    W = w0.clone()
    zs = []
    for t0 in range(0, T, b):
        Wb = W
        for t in range(t0, min(t0 + b, T)):
            yh, s = ln_stats(torch.einsum("nij,nj->ni", Wb, k[:, t]))
            g = 2.0 * (k[:, t] + gamma * yh + beta - v[:, t]) * gamma
            delta = (g - g.mean(dim=1, keepdim=True) - yh * (g * yh).mean(dim=1, keepdim=True)) / s
            W = W - eta[:, t][:, None, None] * delta[:, :, None] * k[:, t][:, None, :]
            uh, _ = ln_stats(torch.einsum("nij,nj->ni", W, q[:, t]))
            zs.append(q[:, t] + gamma * uh + beta)
    return torch.stack(zs, dim=1), W


def linear_ln_grads(q, k, v, w0, gamma, beta, eta, b, dz, dwf=None, eps=1e-6):
    """Gradients of  sum(dz * Z) + sum(dwf * W_final)  of TTT-Linear with LN +
    residual inside f, fp64 autograd through linear_ln_primal_torch.
    w0 : [n, d, d], gamma, beta : [n, d], eta : [n, T] (all per chain).

    returns (dq, dk, dv, deta [n, T], dw0 [n, d, d], dgamma [n, d], dbeta [n, d]).
    """
    import torch

    def t(x):
        return torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)

    q_, k_, v_, w_, g_, b_, e_ = t(q), t(k), t(v), t(w0), t(gamma), t(beta), t(eta)
    z, wf = linear_ln_primal_torch(q_, k_, v_, w_, g_, b_, e_, b, eps)
    loss = (z * torch.tensor(np.asarray(dz, np.float64))).sum()
    if dwf is not None:
        loss = loss + (wf * torch.tensor(np.asarray(dwf, np.float64))).sum()
    loss.backward()
    return tuple(x.grad.numpy() for x in (q_, k_, v_, e_, w_, g_, b_))


def gelu(x):
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def gelu_prime(x):
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + erf(x / np.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def mlp_primal_np(q, k, v, w1, w2, eta, b):
    """numpy fp64 primal TTT-MLP (same rule as mlp_primal), for cross-checks."""
    q, k, v, w1, w2, eta = map(_f64, (q, k, v, w1, w2, eta))
    n, T, d = q.shape
    z = np.empty((n, T, d))
    W1f = np.empty_like(w1)
    W2f = np.empty_like(w2)
    for c in range(n):
        W1, W2 = w1[c].copy(), w2[c].copy()
        for t0 in range(0, T, b):
            W1b, W2b = W1.copy(), W2.copy()
            for t in range(t0, min(t0 + b, T)):
                h = W1b @ k[c, t]
                a = gelu(h)
                e2 = 2.0 * (W2b @ a - v[c, t])
                g1 = (W2b.T @ e2) * gelu_prime(h)
                W2 = W2 - eta[c, t] * np.outer(e2, a)
                W1 = W1 - eta[c, t] * np.outer(g1, k[c, t])
                z[c, t] = W2 @ gelu(W1 @ q[c, t])
        W1f[c], W2f[c] = W1, W2
    return z, W1f, W2f


def mlp_primal_torch(q, k, v, w1, w2, eta, b):
    """The primal TTT-MLP loop (03 §6, §9) on torch CPU tensors, any dtype:
    per token h = W1b k, e = 2 (W2b GELU(h) - v), W2 -= eta e GELU(h)^T,
    W1 -= eta ((W2b^T e) * GELU'(h)) k^T, z = W2 GELU(W1 q).  Differentiable
    (GELU' is written out, so autograd also takes its derivative), so torch
    autograd of this loop is the reference gradient of the layer.
    """
    import torch

    def phi_cdf(x):
        return 0.5 * (1.0 + torch.erf(x / 2.0 ** 0.5))

    def gelu_t(x):
        return x * phi_cdf(x)

    def gelu_prime_t(x):
        return phi_cdf(x) + x * torch.exp(-0.5 * x * x) / (2.0 * np.pi) ** 0.5

    n, T, d = q.shape
    W1, W2 = w1.clone(), w2.clone()
    zs = []
    for t0 in range(0, T, b):
        W1b, W2b = W1, W2
        for t in range(t0, min(t0 + b, T)):
            h = torch.einsum("nij,nj->ni", W1b, k[:, t])
            a = gelu_t(h)
            e = 2.0 * (torch.einsum("nij,nj->ni", W2b, a) - v[:, t])
            g = torch.einsum("nij,ni->nj", W2b, e) * gelu_prime_t(h)
            et = eta[:, t][:, None, None]
            W2 = W2 - et * e[:, :, None] * a[:, None, :]
            W1 = W1 - et * g[:, :, None] * k[:, t][:, None, :]
            zs.append(torch.einsum("nij,nj->ni", W2, gelu_t(torch.einsum("nij,nj->ni", W1, q[:, t]))))
    return torch.stack(zs, dim=1), W1, W2


def mlp_grads(q, k, v, w1, w2, eta, b, dz, dw1f=None, dw2f=None):
    """Gradients of  sum(dz * Z) + sum(dw1f * W1_final) + sum(dw2f * W2_final)  of
    TTT-MLP, fp64 autograd through mlp_primal_torch.

    returns (dq, dk, dv, deta [n, T], dw1 [n, dh, d], dw2 [n, d, dh]) as numpy fp64.
    """
    import torch

    def t(x):
        return torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)

    q_, k_, v_, w1_, w2_, e_ = t(q), t(k), t(v), t(w1), t(w2), t(eta)
    z, f1, f2 = mlp_primal_torch(q_, k_, v_, w1_, w2_, e_, b)
    loss = (z * torch.tensor(np.asarray(dz, np.float64))).sum()
    if dw1f is not None:
        loss = loss + (f1 * torch.tensor(np.asarray(dw1f, np.float64))).sum()
    if dw2f is not None:
        loss = loss + (f2 * torch.tensor(np.asarray(dw2f, np.float64))).sum()
    loss.backward()
    return tuple(x.grad.numpy() for x in (q_, k_, v_, e_, w1_, w2_))


def mlp_ln_primal_torch(q, k, v, w1, w2, gamma, beta, eta, b, eps=1e-6):
    """The primal TTT-MLP loop with LN + residual inside f,
    f(x) = x + LN(W2 GELU(W1 x)) (03 §9; the update rule of 03 §6), on torch CPU
    tensors, any dtype; differentiable.

    Token t of a mini-batch (W1b, W2b: the state before the mini-batch):
    h = W1b k_t, a = GELU(h), y = W2b a, loss |k_t + LN(y) - v_t|^2; its gradient
    pulled back through LN to y is delta (written out, as the forward computes
    it), so the step is W2 -= eta_t delta a^T, W1 -= eta_t ((W2b^T delta) * GELU'(h)) k_t^T;
    z_t = q_t + LN(W2_t GELU(W1_t q_t)).
    LN(y) = gamma * (y - mean(y)) / sqrt(var(y) + eps) + beta over the d entries.
    Shapes: q, k, v [n, T, d]; w1 [n, dh, d]; w2 [n, d, dh]; gamma, beta [n, d]; eta [n, T].
    """
    import torch

    def phi_cdf(x):
        return 0.5 * (1.0 + torch.erf(x / 2.0 ** 0.5))

    def gelu_t(x):
        return x * phi_cdf(x)

    def gelu_prime_t(x):
        return phi_cdf(x) + x * torch.exp(-0.5 * x * x) / (2.0 * np.pi) ** 0.5

    def ln_stats(y):
        mu = y.mean(dim=1, keepdim=True)
        dv = y - mu
        s = torch.sqrt((dv * dv).mean(dim=1, keepdim=True) + eps)
        return dv / s, s

    n, T, d = q.shape
    W1, W2 = w1.clone(), w2.clone()
    zs = []
    for t0 in range(0, T, b):
        W1b, W2b = W1, W2
        for t in range(t0, min(t0 + b, T)):
            h = torch.einsum("nij,nj->ni", W1b, k[:, t])
            a = gelu_t(h)
            yh, s = ln_stats(torch.einsum("nij,nj->ni", W2b, a))
            g = 2.0 * (k[:, t] + gamma * yh + beta - v[:, t]) * gamma
            delta = (g - g.mean(dim=1, keepdim=True) - yh * (g * yh).mean(dim=1, keepdim=True)) / s
            g1 = torch.einsum("nij,ni->nj", W2b, delta) * gelu_prime_t(h)
            et = eta[:, t][:, None, None]
            W2 = W2 - et * delta[:, :, None] * a[:, None, :]
            W1 = W1 - et * g1[:, :, None] * k[:, t][:, None, :]
            uh, _ = ln_stats(torch.einsum("nij,nj->ni", W2, gelu_t(torch.einsum("nij,nj->ni", W1, q[:, t]))))
            zs.append(q[:, t] + gamma * uh + beta)
    return torch.stack(zs, dim=1), W1, W2


def mlp_ln_grads(q, k, v, w1, w2, gamma, beta, eta, b, dz, dw1f=None, dw2f=None, eps=1e-6):
    """Gradients of  sum(dz * Z) + sum(dw1f * W1_final) + sum(dw2f * W2_final)  of
    TTT-MLP with LN + residual, fp64 autograd through mlp_ln_primal_torch.

    returns (dq, dk, dv, deta [n, T], dw1 [n, dh, d], dw2 [n, d, dh], dgamma [n, d],
    dbeta [n, d]) as numpy fp64.
    """
    import torch

    def t(x):
        return torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)

    q_, k_, v_, w1_, w2_, g_, b_, e_ = t(q), t(k), t(v), t(w1), t(w2), t(gamma), t(beta), t(eta)
    z, f1, f2 = mlp_ln_primal_torch(q_, k_, v_, w1_, w2_, g_, b_, e_, b, eps)
    loss = (z * torch.tensor(np.asarray(dz, np.float64))).sum()
    if dw1f is not None:
        loss = loss + (f1 * torch.tensor(np.asarray(dw1f, np.float64))).sum()
    if dw2f is not None:
        loss = loss + (f2 * torch.tensor(np.asarray(dw2f, np.float64))).sum()
    loss.backward()
    return tuple(x.grad.numpy() for x in (q_, k_, v_, e_, w1_, w2_, g_, b_))


def mlp_dual_f64(q, k, v, w1, w2, eta, b):
    """Dual form of TTT-MLP, fp64 (the 03 §7 identity applied layer by layer).

    Column notation per mini-batch (start weights W1, W2):
      H_K = W1 K, A_K = gelu(H_K), E = 2 (W2 A_K - V),
      D1 = (W2^T E) * gelu'(H_K),
      H_Q = W1 Q - D1 (diag(eta) triu(K^T Q)),  A_Q = gelu(H_Q),
      Z = W2 A_Q - E (diag(eta) triu(A_K^T A_Q)),
      W1 -= D1 diag(eta) K^T,  W2 -= E diag(eta) A_K^T.
    """
    q, k, v, w1, w2, eta = map(_f64, (q, k, v, w1, w2, eta))
    n, T, d = q.shape
    z = np.empty((n, T, d))
    W1f = np.empty_like(w1)
    W2f = np.empty_like(w2)
    for c in range(n):
        W1, W2 = w1[c].copy(), w2[c].copy()
        for t0 in range(0, T, b):
            sl = slice(t0, min(t0 + b, T))
            K, V, Q = k[c, sl].T, v[c, sl].T, q[c, sl].T
            et = eta[c, sl]
            HK = W1 @ K
            AK = gelu(HK)
            E = 2.0 * (W2 @ AK - V)
            D1 = (W2.T @ E) * gelu_prime(HK)
            HQ = W1 @ Q - D1 @ (np.triu(K.T @ Q) * et[:, None])
            AQ = gelu(HQ)
            z[c, sl] = (W2 @ AQ - E @ (np.triu(AK.T @ AQ) * et[:, None])).T
            W1 = W1 - (D1 * et[None, :]) @ K.T
            W2 = W2 - (E * et[None, :]) @ AK.T
        W1f[c], W2f[c] = W1, W2
    return z, W1f, W2f


def mlp_ln_dual_f64(q, k, v, w1, w2, gamma, beta, eta, b, eps=1e-6):
    """Dual form of TTT-MLP with LN + residual, fp64 (self-check only).

    Per mini-batch (columns = tokens, start weights W1, W2):
      H_K = W1 K, A_K = gelu(H_K), Y = W2 A_K, LN statistics per column,
      G = 2 (K + LN(Y) - V) * gamma,  Dl = (G - mean(G) - Yh mean(G Yh)) / s,
      D1 = (W2^T Dl) * gelu'(H_K),
      H_Q = W1 Q - D1 (diag(eta) triu(K^T Q)),  A_Q = gelu(H_Q),
      Z = Q + LN(W2 A_Q - Dl (diag(eta) triu(A_K^T A_Q))),
      W1 -= D1 diag(eta) K^T,  W2 -= Dl diag(eta) A_K^T.
    """
    q, k, v, w1, w2, gamma, beta, eta = map(_f64, (q, k, v, w1, w2, gamma, beta, eta))
    n, T, d = q.shape
    z = np.empty((n, T, d))
    W1f = np.empty_like(w1)
    W2f = np.empty_like(w2)
    for c in range(n):
        W1, W2 = w1[c].copy(), w2[c].copy()
        for t0 in range(0, T, b):
            sl = slice(t0, min(t0 + b, T))
            K, V, Q = k[c, sl].T, v[c, sl].T, q[c, sl].T
            et = eta[c, sl]
            HK = W1 @ K
            AK = gelu(HK)
            L, Yh, s = _ln_cols(W2 @ AK, gamma[c], beta[c], eps)
            G = 2.0 * (K + L - V) * gamma[c][:, None]
            Dl = (G - G.mean(axis=0, keepdims=True) - Yh * (G * Yh).mean(axis=0, keepdims=True)) / s
            D1 = (W2.T @ Dl) * gelu_prime(HK)
            HQ = W1 @ Q - D1 @ (np.triu(K.T @ Q) * et[:, None])
            AQ = gelu(HQ)
            YQ = W2 @ AQ - Dl @ (np.triu(AK.T @ AQ) * et[:, None])
            z[c, sl] = (Q + _ln_cols(YQ, gamma[c], beta[c], eps)[0]).T
            W1 = W1 - (D1 * et[None, :]) @ K.T
            W2 = W2 - (Dl * et[None, :]) @ AK.T
        W1f[c], W2f[c] = W1, W2
    return z, W1f, W2f


def max_rel_err(x, ref, axis_slices: Optional[int] = None) -> float:
    """max over slices of max|x - ref| / max|ref|, slices along the leading axis."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if x.size == 0:
        return 0.0
    xs = x.reshape(x.shape[0], -1)
    rs = ref.reshape(ref.shape[0], -1)
    num = np.abs(xs - rs).max(axis=1)
    den = np.abs(rs).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())
