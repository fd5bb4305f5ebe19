"""Pins of the TTT-MLP oracle (f(x) = W2 GELU(W1 x), hidden width dh).

Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
(aharts.cn / itmax.cn), part 03 §9 (TTT-MLP: two layers, hidden width 4x the
input, GELU), with the update/output rules of 03 §1, §5, §6.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.stats import norm

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, n, T, d, dh, eta_scale=1.0 / 16, wstd=0.3):
    r = np.random.default_rng(seed)
    q = r.standard_normal((n, T, d)) / np.sqrt(d)
    k = r.standard_normal((n, T, d)) / np.sqrt(d)
    v = r.standard_normal((n, T, d)) / np.sqrt(d)
    w1 = r.standard_normal((n, dh, d)) * wstd
    w2 = r.standard_normal((n, d, dh)) * wstd
    eta = eta_scale / (1.0 + np.exp(-r.standard_normal((n, T))))
    return q, k, v, w1, w2, eta


# -- GELU is the exact-erf form x * Phi(x) ------------------------------------

def test_gelu_against_normal_cdf():
    x = np.linspace(-6, 6, 97)
    np.testing.assert_allclose(oracle.gelu(x), x * norm.cdf(x), rtol=1e-14, atol=1e-15)
    # textbook values: Phi(1) = 0.8413447460685429, Phi(0) = 1/2
    assert abs(oracle.gelu(1.0) - 0.8413447460685429) < 1e-15
    assert oracle.gelu(0.0) == 0.0
    assert abs(oracle.gelu_prime(0.0) - 0.5) < 1e-16
    # GELU(x) - GELU(-x) = x
    np.testing.assert_allclose(oracle.gelu(x) - oracle.gelu(-x), x, rtol=0, atol=1e-14)


def test_gelu_prime_is_derivative():
    x = np.linspace(-5, 5, 41)
    h = 1e-6
    fd = (oracle.gelu(x + h) - oracle.gelu(x - h)) / (2 * h)
    np.testing.assert_allclose(oracle.gelu_prime(x), fd, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(oracle.gelu_prime(x), norm.cdf(x) + x * norm.pdf(x), rtol=1e-13, atol=1e-15)


# -- hand-worked example --------------------------------------------------------

def test_handworked():
    with open(os.path.join(GOLDEN, "mlp_handworked.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        A = lambda key: np.array(c[key], float)[None]  # noqa: E731
        z, w1f, w2f = oracle.mlp_primal(A("q"), A("k"), A("v"), A("w1"), A("w2"),
                                        np.array(c["eta"])[None], c["b"])
        np.testing.assert_allclose(z[0], np.array(c["z"]), rtol=1e-15)
        np.testing.assert_allclose(w1f[0], np.array(c["w1_final"]), rtol=1e-15)
        np.testing.assert_allclose(w2f[0], np.array(c["w2_final"]), rtol=1e-15)


# -- P12a: the step is the gradient of |W2 GELU(W1 k) - v|^2 in both layers -----

def test_step_is_gradient_fd():
    r = np.random.default_rng(3)
    d, dh = 3, 5
    W1 = r.standard_normal((dh, d))
    W2 = r.standard_normal((d, dh))
    k, v, q = r.standard_normal(d), r.standard_normal(d), r.standard_normal(d)
    eta = 0.01
    _, w1f, w2f = oracle.mlp_primal(q[None, None], k[None, None], v[None, None], W1[None], W2[None],
                                    np.array([[eta]]), 1)
    g1 = (W1 - w1f[0]) / eta
    g2 = (W2 - w2f[0]) / eta

    def loss(A, B):
        hidden = A @ k
        act = hidden * norm.cdf(hidden)
        return float(np.sum((B @ act - v) ** 2))

    h = 1e-6
    fd1 = np.zeros_like(W1)
    for i in range(dh):
        for j in range(d):
            P, M = W1.copy(), W1.copy()
            P[i, j] += h
            M[i, j] -= h
            fd1[i, j] = (loss(P, W2) - loss(M, W2)) / (2 * h)
    fd2 = np.zeros_like(W2)
    for i in range(d):
        for j in range(dh):
            P, M = W2.copy(), W2.copy()
            P[i, j] += h
            M[i, j] -= h
            fd2[i, j] = (loss(W1, P) - loss(W1, M)) / (2 * h)
    np.testing.assert_allclose(g1, fd1, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(g2, fd2, rtol=1e-6, atol=1e-7)


# -- P12b: eta = 0 => Z = W2 GELU(W1 Q) ------------------------------------------

def test_eta_zero():
    q, k, v, w1, w2, eta = _rand(4, 2, 32, 8, 32)
    z, w1f, w2f = oracle.mlp_primal(q, k, v, w1, w2, np.zeros_like(eta), 16)
    np.testing.assert_array_equal(w1f, w1)
    np.testing.assert_array_equal(w2f, w2)
    for c in range(2):
        hid = q[c] @ w1[c].T
        np.testing.assert_allclose(z[c], (hid * norm.cdf(hid)) @ w2[c].T, rtol=0, atol=1e-14)


# -- W2 = 0 and batch GD: kernelised causal linear attention ---------------------

def test_zero_second_layer_is_feature_linear_attention():
    """With W2_0 = 0 and b = T, the W1 gradient vanishes for the whole (single)
    mini-batch, W1 never moves, and z_t = sum_{s<=t} 2 eta_s v_s (phi(k_s) . phi(q_t))
    with phi(x) = GELU(W1 x): causal linear attention with a GELU feature map."""
    q, k, v, w1, _, eta = _rand(5, 2, 24, 6, 16)
    z, w1f, w2f = oracle.mlp_primal(q, k, v, w1, np.zeros((2, 6, 16)), eta, 24)
    for c in range(2):
        np.testing.assert_array_equal(w1f[c], w1[c])
        hk, hq = k[c] @ w1[c].T, q[c] @ w1[c].T
        fk, fq = hk * norm.cdf(hk), hq * norm.cdf(hq)
        att = np.tril(fq @ fk.T) * (2.0 * eta[c])[None, :]      # [t, s]
        np.testing.assert_allclose(z[c], att @ v[c], rtol=0, atol=1e-13)
        np.testing.assert_allclose(w2f[c], (v[c] * 2.0 * eta[c][:, None]).T @ fk, rtol=0, atol=1e-13)


# -- P12c: b = 1 is online GD on the two-layer model ------------------------------

def test_b1_is_online_gd():
    q, k, v, w1, w2, eta = _rand(6, 1, 20, 4, 8)
    z, w1f, w2f = oracle.mlp_primal(q, k, v, w1, w2, eta, 1)
    W1, W2 = w1[0].copy(), w2[0].copy()
    for t in range(20):
        hid = W1 @ k[0, t]
        act = hid * norm.cdf(hid)
        e = 2 * (W2 @ act - v[0, t])
        g1 = np.outer((W2.T @ e) * (norm.cdf(hid) + hid * norm.pdf(hid)), k[0, t])
        g2 = np.outer(e, act)
        W1, W2 = W1 - eta[0, t] * g1, W2 - eta[0, t] * g2
        hq = W1 @ q[0, t]
        np.testing.assert_allclose(z[0, t], W2 @ (hq * norm.cdf(hq)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(w1f[0], W1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(w2f[0], W2, rtol=0, atol=1e-13)


# -- P12d: dual form (layer by layer) == primal; C == numpy primal -----------------

@pytest.mark.parametrize("n,T,d,dh,b", [(1, 32, 8, 32, 16), (2, 40, 16, 64, 8), (1, 21, 6, 24, 4)])
def test_dual_and_numpy_vs_c(n, T, d, dh, b):
    q, k, v, w1, w2, eta = _rand(n * T + d, n, T, d, dh, wstd=0.1)
    z, w1f, w2f = oracle.mlp_primal(q, k, v, w1, w2, eta, b)
    zd, w1d, w2d = oracle.mlp_dual_f64(q, k, v, w1, w2, eta, b)
    assert oracle.max_rel_err(z, zd) < 1e-12
    assert oracle.max_rel_err(w1f, w1d) < 1e-12
    assert oracle.max_rel_err(w2f, w2d) < 1e-12
    zn, w1n, w2n = oracle.mlp_primal_np(q, k, v, w1, w2, eta, b)
    assert oracle.max_rel_err(z, zn) < 1e-13
    assert oracle.max_rel_err(w1f, w1n) < 1e-13
    assert oracle.max_rel_err(w2f, w2n) < 1e-13


def test_mini_batch_boundary_matters():
    """Gradients at the mini-batch start (b=16) differ from online GD (b=1) --
    a guard that the snapshot is taken at all."""
    q, k, v, w1, w2, eta = _rand(7, 1, 32, 8, 32, eta_scale=0.5)
    z16 = oracle.mlp_primal(q, k, v, w1, w2, eta, 16)[0]
    z1 = oracle.mlp_primal(q, k, v, w1, w2, eta, 1)[0]
    assert np.abs(z16 - z1).max() > 1e-6
    # ...but the first token of every mini-batch sees the same state either way only at t=0
    np.testing.assert_allclose(z16[0, 0], z1[0, 0], rtol=0, atol=1e-15)


# -- P12f: state passing -----------------------------------------------------------

def test_state_passing_bitwise():
    q, k, v, w1, w2, eta = _rand(8, 2, 48, 8, 32)
    z, w1f, w2f = oracle.mlp_primal(q, k, v, w1, w2, eta, 16)
    za, w1a, w2a = oracle.mlp_primal(q[:, :32], k[:, :32], v[:, :32], w1, w2, eta[:, :32], 16)
    zb, w1b, w2b = oracle.mlp_primal(q[:, 32:], k[:, 32:], v[:, 32:], w1a, w2a, eta[:, 32:], 16)
    np.testing.assert_array_equal(z, np.concatenate([za, zb], axis=1))
    np.testing.assert_array_equal(w1f, w1b)
    np.testing.assert_array_equal(w2f, w2b)


def test_hidden_permutation():
    """Permuting the hidden units (rows of W1, columns of W2) changes nothing observable."""
    q, k, v, w1, w2, eta = _rand(9, 1, 32, 8, 32)
    perm = np.random.default_rng(2).permutation(32)
    z, w1f, w2f = oracle.mlp_primal(q, k, v, w1, w2, eta, 8)
    zp, w1p, w2p = oracle.mlp_primal(q, k, v, w1[:, perm], w2[:, :, perm], eta, 8)
    np.testing.assert_allclose(zp, z, rtol=0, atol=1e-14)
    np.testing.assert_allclose(w1p, w1f[:, perm], rtol=0, atol=1e-14)
    np.testing.assert_allclose(w2p, w2f[:, :, perm], rtol=0, atol=1e-14)
    assert math.isfinite(float(np.abs(z).max()))
