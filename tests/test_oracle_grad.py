"""Pins of the gradient oracle of TTT-Linear (torch fp64 autograd of the primal loop).

The backward of the layer is defined by its forward ([TTT] news article, part
03 §1, §5, §6; part 03 §4: the TTT layer has a backward like any other layer).
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(seed, n, T, d, eta_scale=0.1):
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((n, T, d)) / np.sqrt(d) for _ in range(3))
    w0 = r.standard_normal((n, d, d)) * 0.3
    eta = eta_scale * (0.5 + r.random((n, T)))
    return q, k, v, w0, eta


def test_torch_loop_matches_c_oracle():
    q, k, v, w0, eta = _rand(1, 3, 40, 8)
    zc, wc = oracle.linear_primal(q, k, v, w0, eta, 16)
    zt, wt = oracle.linear_primal_torch(*(torch.tensor(x) for x in (q, k, v, w0, eta)), 16)
    np.testing.assert_allclose(zt.numpy(), zc, rtol=0, atol=1e-14)
    np.testing.assert_allclose(wt.numpy(), wc, rtol=0, atol=1e-14)


@pytest.mark.parametrize("T,b", [(6, 2), (6, 3), (5, 2), (4, 4)])
def test_gradcheck_finite_differences(T, b):
    q, k, v, w0, eta = _rand(2 + T + b, 2, T, 3)
    ins = tuple(torch.tensor(x, requires_grad=True) for x in (q, k, v, w0, eta))
    r = np.random.default_rng(5)
    dz = torch.tensor(r.standard_normal((2, T, 3)))
    dwf = torch.tensor(r.standard_normal((2, 3, 3)))

    def f(q_, k_, v_, w_, e_):
        z, wf = oracle.linear_primal_torch(q_, k_, v_, w_, e_, b)
        return (z * dz).sum() + (wf * dwf).sum()

    assert torch.autograd.gradcheck(f, ins, eps=1e-6, atol=1e-8, rtol=1e-6)


def test_eta_zero_closed_form():
    """eta = 0: Z = W0 Q, so dQ = W0^T dZ, dW0 = sum_t dz_t q_t^T + dWf, dK = dV = 0."""
    q, k, v, w0, _ = _rand(3, 2, 12, 5)
    r = np.random.default_rng(6)
    dz, dwf = r.standard_normal((2, 12, 5)), r.standard_normal((2, 5, 5))
    dq, dk, dv, deta, dw0 = oracle.linear_grads(q, k, v, w0, np.zeros((2, 12)), 4, dz, dwf)
    np.testing.assert_allclose(dq, np.einsum("nij,nti->ntj", w0, dz), atol=1e-14)
    np.testing.assert_allclose(dw0, np.einsum("nti,ntj->nij", dz, q) + dwf, atol=1e-14)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_array_equal(dv, 0.0)
    # deta is not zero: d Z / d eta at eta = 0 is the first-order effect of one step
    assert np.abs(deta).max() > 1e-3


def test_linear_in_upstream_gradients():
    q, k, v, w0, eta = _rand(4, 1, 16, 4)
    r = np.random.default_rng(7)
    dz1, dz2 = r.standard_normal((2, 1, 16, 4))
    g1 = oracle.linear_grads(q, k, v, w0, eta, 4, dz1)
    g2 = oracle.linear_grads(q, k, v, w0, eta, 4, dz2)
    g3 = oracle.linear_grads(q, k, v, w0, eta, 4, 2.0 * dz1 - 3.0 * dz2)
    for a, bb, c in zip(g1, g2, g3):
        np.testing.assert_allclose(c, 2.0 * a - 3.0 * bb, rtol=1e-12, atol=1e-13)


def test_dv_of_final_state():
    """dWf only: W_final is affine in V with W_final = ... + 2 sum_s eta_s v_s k_s^T (P4, b = T),
    so with W0 = 0 and one mini-batch, dV_s = 2 eta_s dWf k_s."""
    q, k, v, _, eta = _rand(5, 1, 8, 4)
    dwf = np.random.default_rng(8).standard_normal((1, 4, 4))
    _, _, dv, _, _ = oracle.linear_grads(q, k, v, np.zeros((1, 4, 4)), eta, 8, np.zeros((1, 8, 4)), dwf)
    np.testing.assert_allclose(dv[0], 2.0 * eta[0][:, None] * (k[0] @ dwf[0].T), atol=1e-14)


# ---- the C reverse pass (used at full size) ----------------------------------------

@pytest.mark.parametrize("n,T,d,b", [(2, 12, 4, 4), (1, 10, 3, 4), (3, 7, 5, 1), (2, 16, 8, 16), (1, 33, 6, 8)])
def test_c_reverse_pass_matches_autograd(n, T, d, b):
    q, k, v, w0, eta = _rand(10 + T + b, n, T, d)
    r = np.random.default_rng(11)
    dz, dwf = r.standard_normal((n, T, d)), r.standard_normal((n, d, d))
    a = oracle.linear_grads(q, k, v, w0, eta, b, dz, dwf)
    c = oracle.linear_primal_grads(q, k, v, w0, eta, b, dz, dwf)
    for x, y in zip(a, c):
        np.testing.assert_allclose(y, x, rtol=1e-11, atol=1e-12)
    a0 = oracle.linear_grads(q, k, v, w0, eta, b, dz)
    c0 = oracle.linear_primal_grads(q, k, v, w0, eta, b, dz)
    for x, y in zip(a0, c0):
        np.testing.assert_allclose(y, x, rtol=1e-11, atol=1e-12)


def test_c_reverse_pass_finite_differences():
    """Central differences of the C forward (oracle_linear_primal), entry by entry."""
    n, T, d, b = 1, 6, 3, 4
    q, k, v, w0, eta = _rand(12, n, T, d)
    r = np.random.default_rng(13)
    dz, dwf = r.standard_normal((n, T, d)), r.standard_normal((n, d, d))

    def loss(q_, k_, v_, w_, e_):
        z, wf = oracle.linear_primal(q_, k_, v_, w_, e_, b)
        return float((z * dz).sum() + (wf * dwf).sum())

    grads = oracle.linear_primal_grads(q, k, v, w0, eta, b, dz, dwf)
    ins = [q, k, v, eta, w0]
    h = 1e-6
    for which, g in enumerate(grads):
        x = ins[which]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if j == which else ins[j] for j in range(5)]
            args_m = [xm if j == which else ins[j] for j in range(5)]
            fd[idx] = (loss(args_p[0], args_p[1], args_p[2], args_p[4], args_p[3]) -
                       loss(args_m[0], args_m[1], args_m[2], args_m[4], args_m[3])) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_c_reverse_pass_dual_form_single_minibatch():
    """b = T (one mini-batch), W0 = 0, dZ = 0: E = -V, so W_final = 2 V diag(eta) K^T is
    linear in V and dV_s = 2 eta_s dWf k_s whatever Q."""
    q, k, v, _, eta = _rand(14, 2, 8, 5)
    dwf = np.random.default_rng(15).standard_normal((2, 5, 5))
    _, _, dv, _, _ = oracle.linear_primal_grads(q, k, v, np.zeros((2, 5, 5)), eta, 8, np.zeros((2, 8, 5)), dwf)
    np.testing.assert_allclose(dv, 2.0 * eta[:, :, None] * np.einsum("nij,ntj->nti", dwf, k), atol=1e-14)
