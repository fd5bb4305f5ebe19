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
