"""Pins of the gradient oracle of TTT-MLP with layer norm and residual inside f
(oracle.mlp_ln_grads: torch fp64 autograd of oracle.mlp_ln_primal_torch).

The torch loop is checked against the C forward oracle (mlp_ln_primal, itself
pinned in test_oracle_mlp_ln.py) and torch's finite differences check its
gradients; the eta = 0 case reduces to the gradient of a closed form.

Pages: [TTT] news article, part 03 §4 (the layer is trained end to end), §6
(mini-batch gradient steps), §9 (f(x) = x + LN(MLP(x)): layer norm and a
residual; TTT-MLP with hidden width 4d and GELU).
"""
import numpy as np
import pytest
import torch

import oracle

NAMES = ("dq", "dk", "dv", "deta", "dw1", "dw2", "dgamma", "dbeta")


def _rand(seed, n, T, d, dh, eta_scale=0.15, wscale=0.6):
    r = np.random.default_rng(seed)
    q, k, v = (0.7 * r.standard_normal((n, T, d)) for _ in range(3))
    w1 = wscale * r.standard_normal((n, dh, d))
    w2 = wscale * r.standard_normal((n, d, dh))
    gamma = 1.0 + 0.3 * r.standard_normal((n, d))
    beta = 0.2 * r.standard_normal((n, d))
    eta = eta_scale * (0.5 + r.random((n, T)))
    return q, k, v, w1, w2, gamma, beta, eta


def _upstream(seed, n, T, d, dh):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, T, d)), r.standard_normal((n, dh, d)), r.standard_normal((n, d, dh))


@pytest.mark.parametrize("T,b", [(8, 4), (7, 3), (5, 1), (6, 6)])
def test_torch_loop_matches_c_forward_oracle(T, b):
    q, k, v, w1, w2, gamma, beta, eta = _rand(20 + T, 2, T, 4, 6)
    zc, f1c, f2c = oracle.mlp_ln_primal(q, k, v, w1, w2, gamma, beta, eta, b)
    tt = lambda x: torch.tensor(x, dtype=torch.float64)  # noqa: E731
    zt, f1t, f2t = oracle.mlp_ln_primal_torch(*map(tt, (q, k, v, w1, w2, gamma, beta, eta)), b)
    for got, ref in ((zt, zc), (f1t, f1c), (f2t, f2c)):
        assert oracle.max_rel_err(got.numpy(), ref) < 1e-12


@pytest.mark.parametrize("T,b", [(4, 2), (3, 1), (4, 4)])
def test_gradcheck(T, b):
    """The autograd reference against torch's central differences, every input."""
    q, k, v, w1, w2, gamma, beta, eta = _rand(30 + T + b, 1, T, 3, 4)
    dz, d1, d2 = _upstream(31 + T, 1, T, 3, 4)
    ins = tuple(torch.tensor(x, dtype=torch.float64, requires_grad=True)
                for x in (q, k, v, w1, w2, gamma, beta, eta))

    def f(*xs):
        z, f1, f2 = oracle.mlp_ln_primal_torch(*xs, b)
        return (z * torch.tensor(dz)).sum() + (f1 * torch.tensor(d1)).sum() + (f2 * torch.tensor(d2)).sum()

    assert torch.autograd.gradcheck(f, ins, eps=1e-6, atol=1e-6, rtol=1e-5)


def test_eta_zero_closed_form():
    """eta = 0: the weights never move, Z = Q + LN(W2 GELU(W1 Q)): dK = dV = 0
    exactly, and every other gradient is that of the closed form."""
    q, k, v, w1, w2, gamma, beta, _ = _rand(40, 2, 6, 4, 6)
    eta = np.zeros((2, 6))
    dz, d1, d2 = _upstream(41, 2, 6, 4, 6)
    got = dict(zip(NAMES, oracle.mlp_ln_grads(q, k, v, w1, w2, gamma, beta, eta, 3, dz, d1, d2)))
    assert np.all(got["dk"] == 0) and np.all(got["dv"] == 0)
    ins = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, w1, w2, gamma, beta)]
    Q, W1, W2, G, B = ins
    h = torch.einsum("nij,ntj->nti", W1, Q)
    y = torch.einsum("nij,ntj->nti", W2, h * 0.5 * (1.0 + torch.erf(h / 2.0 ** 0.5)))
    mu = y.mean(dim=2, keepdim=True)
    yh = (y - mu) / torch.sqrt(((y - mu) ** 2).mean(dim=2, keepdim=True) + 1e-6)
    z = Q + G[:, None, :] * yh + B[:, None, :]
    loss = (z * torch.tensor(dz)).sum() + (W1 * torch.tensor(d1)).sum() + (W2 * torch.tensor(d2)).sum()
    loss.backward()
    for name, x in zip(("dq", "dw1", "dw2", "dgamma", "dbeta"), ins):
        assert oracle.max_rel_err(got[name], x.grad.numpy()) < 1e-12, name


def test_linear_in_upstream_gradients():
    q, k, v, w1, w2, gamma, beta, eta = _rand(50, 1, 8, 3, 5)
    ua, ub = _upstream(51, 1, 8, 3, 5), _upstream(52, 1, 8, 3, 5)
    ga = oracle.mlp_ln_grads(q, k, v, w1, w2, gamma, beta, eta, 4, *ua)
    gb = oracle.mlp_ln_grads(q, k, v, w1, w2, gamma, beta, eta, 4, *ub)
    gs = oracle.mlp_ln_grads(q, k, v, w1, w2, gamma, beta, eta, 4, *(2.0 * a - b for a, b in zip(ua, ub)))
    for name, a, b, s in zip(NAMES, ga, gb, gs):
        np.testing.assert_allclose(s, 2.0 * a - b, rtol=1e-11, atol=1e-11, err_msg=name)
