"""Pins of the gradient oracle of TTT-MLP: the C reverse pass of the primal
token loop (oracle.mlp_primal_grads) against finite differences of the C
forward oracle, torch fp64 autograd of a torch version of the same loop, and
the eta = 0 closed form.

Pages: [TTT] news article, part 03 §4 (the layer is trained end to end, so it
has a backward like any other layer), §6 (mini-batch gradient steps), §9
(TTT-MLP: two layers, hidden width 4d, GELU).
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(seed, n, T, d, dh, eta_scale=0.15, wscale=0.6):
    r = np.random.default_rng(seed)
    q, k, v = (0.7 * r.standard_normal((n, T, d)) for _ in range(3))
    w1 = wscale * r.standard_normal((n, dh, d))
    w2 = wscale * r.standard_normal((n, d, dh))
    eta = eta_scale * (0.5 + r.random((n, T)))
    return q, k, v, w1, w2, eta


def _upstream(seed, n, T, d, dh):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, T, d)), r.standard_normal((n, dh, d)), r.standard_normal((n, d, dh))


NAMES = ("dq", "dk", "dv", "deta", "dw1", "dw2")


def test_torch_loop_matches_c_oracle():
    q, k, v, w1, w2, eta = _rand(1, 2, 20, 4, 7)
    zc, c1, c2 = oracle.mlp_primal(q, k, v, w1, w2, eta, 8)
    zt, t1, t2 = oracle.mlp_primal_torch(*(torch.tensor(x) for x in (q, k, v, w1, w2, eta)), 8)
    for a, b in ((zt, zc), (t1, c1), (t2, c2)):
        assert oracle.max_rel_err(a.numpy(), b) < 1e-13


def test_torch_gradcheck():
    """The autograd reference is itself checked by torch's finite differences."""
    q, k, v, w1, w2, eta = _rand(2, 1, 5, 3, 4)
    ins = tuple(torch.tensor(x, requires_grad=True) for x in (q, k, v, w1, w2, eta))
    dz, d1, d2 = (torch.tensor(x) for x in _upstream(3, 1, 5, 3, 4))

    def f(*a):
        z, f1, f2 = oracle.mlp_primal_torch(*a, 2)
        return (z * dz).sum() + (f1 * d1).sum() + (f2 * d2).sum()

    assert torch.autograd.gradcheck(f, ins, eps=1e-6, atol=1e-7, rtol=1e-6)


@pytest.mark.parametrize("T,b", [(7, 3), (8, 4), (6, 1), (5, 5), (9, 16)])
def test_c_reverse_pass_matches_autograd(T, b):
    q, k, v, w1, w2, eta = _rand(4 + T + b, 2, T, 3, 5)
    dz, d1, d2 = _upstream(5 + T, 2, T, 3, 5)
    got = oracle.mlp_primal_grads(q, k, v, w1, w2, eta, b, dz, d1, d2)
    ref = oracle.mlp_grads(q, k, v, w1, w2, eta, b, dz, d1, d2)
    for name, g, r in zip(NAMES, got, ref):
        assert oracle.max_rel_err(g, r) < 1e-11, name


@pytest.mark.parametrize("which", range(6))
def test_c_reverse_pass_matches_finite_differences(which):
    """Central differences of the C forward oracle along a random direction,
    for each input in turn (independent of torch)."""
    n, T, d, dh, b = 2, 7, 3, 5, 3
    q, k, v, w1, w2, eta = _rand(6, n, T, d, dh)
    dz, d1, d2 = _upstream(7, n, T, d, dh)
    args = [q, k, v, w1, w2, eta]
    grad_of = {0: 0, 1: 1, 2: 2, 3: 4, 4: 5, 5: 3}   # argument -> position in the returned tuple
    g = oracle.mlp_primal_grads(q, k, v, w1, w2, eta, b, dz, d1, d2)[grad_of[which]]
    direction = np.random.default_rng(8 + which).standard_normal(args[which].shape)

    def loss(x):
        a = list(args)
        a[which] = x
        z, f1, f2 = oracle.mlp_primal(*a, b)
        return (dz * z).sum() + (d1 * f1).sum() + (d2 * f2).sum()

    eps = 1e-6
    fd = (loss(args[which] + eps * direction) - loss(args[which] - eps * direction)) / (2 * eps)
    an = float((g * direction).sum())
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd))


def test_eta_zero_closed_form():
    """eta = 0: the weights never move, Z = W2 GELU(W1 Q): dK = dV = 0 exactly,
    dQ = W1^T (GELU'(W1 q) * W2^T dz), dW1 = sum (GELU'(u) * W2^T dz) q^T + dW1f,
    dW2 = sum dz GELU(u)^T + dW2f; deta is the first-order effect of one step."""
    n, T, d, dh = 2, 10, 4, 6
    q, k, v, w1, w2, _ = _rand(9, n, T, d, dh)
    dz, d1, d2 = _upstream(10, n, T, d, dh)
    dq, dk, dv, deta, dw1, dw2 = oracle.mlp_primal_grads(q, k, v, w1, w2, np.zeros((n, T)), 4, dz, d1, d2)
    u = np.einsum("nij,ntj->nti", w1, q)
    du = np.einsum("nij,nti->ntj", w2, dz) * oracle.gelu_prime(u)
    np.testing.assert_allclose(dq, np.einsum("nij,nti->ntj", w1, du), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dw1, np.einsum("nti,ntj->nij", du, q) + d1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dw2, np.einsum("nti,ntj->nij", dz, oracle.gelu(u)) + d2, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_array_equal(dv, 0.0)
    assert np.abs(deta).max() > 1e-3


def test_linear_in_upstream_gradients():
    q, k, v, w1, w2, eta = _rand(11, 1, 12, 3, 5)
    ua, ub = _upstream(12, 1, 12, 3, 5), _upstream(13, 1, 12, 3, 5)
    ga = oracle.mlp_primal_grads(q, k, v, w1, w2, eta, 4, *ua)
    gb = oracle.mlp_primal_grads(q, k, v, w1, w2, eta, 4, *ub)
    gs = oracle.mlp_primal_grads(q, k, v, w1, w2, eta, 4, *(2.0 * a - b for a, b in zip(ua, ub)))
    for name, a, b, s in zip(NAMES, ga, gb, gs):
        np.testing.assert_allclose(s, 2.0 * a - b, rtol=1e-12, atol=1e-12, err_msg=name)
