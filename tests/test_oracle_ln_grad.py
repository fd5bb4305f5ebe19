"""Pins of the gradient oracles of TTT-Linear with LN + residual inside f
(f(x) = x + LN(W x), [TTT] news article part 03 §9; the layer is trained end to
end, 03 §4): the fp64 autograd of the primal loop (oracle.linear_ln_grads) and
the hand-written C reverse pass (oracle.linear_ln_primal_grads)."""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

NAMES = ("dq", "dk", "dv", "deta", "dw0", "dgamma", "dbeta")


def _case(n, T, d, seed, eta_scale=0.1, w_scale=0.3):
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((n, T, d)) / np.sqrt(d) for _ in range(3))
    w0 = r.standard_normal((n, d, d)) * w_scale
    gamma = 1.0 + 0.3 * r.standard_normal((n, d))
    beta = 0.1 * r.standard_normal((n, d))
    eta = eta_scale * (0.5 + r.random((n, T)))
    dz = r.standard_normal((n, T, d))
    dwf = r.standard_normal((n, d, d))
    return q, k, v, w0, gamma, beta, eta, dz, dwf


@pytest.mark.parametrize("n,T,d,b", [(1, 6, 4, 3), (2, 7, 5, 3), (1, 8, 6, 8)])
def test_autograd_oracle_gradcheck(n, T, d, b):
    """torch.autograd.gradcheck (central differences) of the autograd oracle,
    every input including gamma and beta, a short last mini-batch included."""
    q, k, v, w0, gamma, beta, eta, _, _ = _case(n, T, d, 10 + T)
    args = [torch.tensor(x, requires_grad=True) for x in (q, k, v, w0, gamma, beta, eta)]

    def f(*xs):
        z, wf = oracle.linear_ln_primal_torch(*xs, b)
        return z, wf

    assert torch.autograd.gradcheck(f, args, eps=1e-6, atol=1e-6, rtol=1e-5)


@pytest.mark.parametrize("n,T,d,b,with_dwf", [(2, 11, 6, 4, True), (1, 9, 5, 1, True), (2, 8, 4, 8, False),
                                              (1, 13, 8, 5, True)])
def test_c_reverse_pass_matches_autograd(n, T, d, b, with_dwf):
    q, k, v, w0, gamma, beta, eta, dz, dwf = _case(n, T, d, 20 + T + b)
    dwf = dwf if with_dwf else None
    ga = oracle.linear_ln_grads(q, k, v, w0, gamma, beta, eta, b, dz, dwf)
    gc = oracle.linear_ln_primal_grads(q, k, v, w0, gamma, beta, eta, b, dz, dwf)
    for name, x, y in zip(NAMES, gc, ga):
        assert np.abs(x - y).max() <= 1e-11 * max(1.0, np.abs(y).max()), name


def test_c_reverse_pass_finite_differences():
    """Central differences of the C forward (oracle.linear_ln_primal) of the scalar
    L = sum(dz * Z) + sum(dwf * W_final), every entry of every input, against the
    C reverse pass: independent of torch."""
    n, T, d, b = 1, 6, 4, 3
    q, k, v, w0, gamma, beta, eta, dz, dwf = _case(n, T, d, 31, eta_scale=0.2)
    inputs = dict(q=q, k=k, v=v, w0=w0, gamma=gamma, beta=beta, eta=eta)

    def loss(**kw):
        z, wf = oracle.linear_ln_primal(kw["q"], kw["k"], kw["v"], kw["w0"], kw["gamma"], kw["beta"], kw["eta"], b)
        return float((z * dz).sum() + (wf * dwf).sum())

    grads = dict(zip(("q", "k", "v", "eta", "w0", "gamma", "beta"),
                     oracle.linear_ln_primal_grads(q, k, v, w0, gamma, beta, eta, b, dz, dwf)))
    h = 1e-6
    for name, x in inputs.items():
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = (loss(**{**inputs, name: xp}) - loss(**{**inputs, name: xm})) / (2 * h)
        assert np.abs(fd - grads[name]).max() <= 1e-6 * max(1.0, np.abs(fd).max()), name


def _ln(x, eps):
    mu = x.mean()
    s = np.sqrt(((x - mu) ** 2).mean() + eps)
    return (x - mu) / s, s


def _ln_back(h, xh, s):
    return (h - h.mean() - xh * (h * xh).mean()) / s


def test_eta_zero_closed_form():
    """eta = 0: the state never moves (W_t = W0), so z_t = q_t + LN(W0 q_t) and,
    written out directly: dq_t = dz_t + W0^T LNback(u_t, gamma dz_t),
    dW0 = sum_t du_t q_t^T + dW_final, dk = dv = 0, dgamma = sum_t dz_t uhat_t,
    dbeta = sum_t dz_t, and deta_t = -delta_t . (A_t k_t) with delta_t the LN
    gradient factor of token t at W0 and A_t = dW_final + sum_{t' >= t} du_t' q_t'^T."""
    n, T, d, b, eps = 1, 7, 5, 3, 1e-6
    q, k, v, w0, gamma, beta, _, dz, dwf = _case(n, T, d, 41)
    eta = np.zeros((n, T))
    got = dict(zip(NAMES, oracle.linear_ln_primal_grads(q, k, v, w0, gamma, beta, eta, b, dz, dwf)))
    W, g_, b_ = w0[0], gamma[0], beta[0]
    du, uh = [], []
    for t in range(T):
        xh, s = _ln(W @ q[0, t], eps)
        uh.append(xh)
        du.append(_ln_back(g_ * dz[0, t], xh, s))
    dq = np.stack([dz[0, t] + W.T @ du[t] for t in range(T)])
    dw0 = sum(np.outer(du[t], q[0, t]) for t in range(T)) + dwf[0]
    deta = np.empty(T)
    for t in range(T):
        yh, s = _ln(W @ k[0, t], eps)
        g = 2.0 * (k[0, t] + g_ * yh + b_ - v[0, t]) * g_
        delta = (g - g.mean() - yh * (g * yh).mean()) / s
        A = dwf[0] + sum(np.outer(du[u], q[0, u]) for u in range(t, T))
        deta[t] = -delta @ (A @ k[0, t])
    np.testing.assert_allclose(got["dq"][0], dq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["dw0"][0], dw0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["deta"][0], deta, rtol=0, atol=1e-12)
    assert np.abs(got["dk"]).max() == 0.0 and np.abs(got["dv"]).max() == 0.0
    np.testing.assert_allclose(got["dgamma"][0], sum(dz[0, t] * uh[t] for t in range(T)), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["dbeta"][0], dz[0].sum(axis=0), rtol=0, atol=1e-12)


def test_linear_in_upstream_gradients():
    n, T, d, b = 2, 9, 6, 4
    q, k, v, w0, gamma, beta, eta, dz, dwf = _case(n, T, d, 51)
    r = np.random.default_rng(52)
    dz2, dwf2 = r.standard_normal(dz.shape), r.standard_normal(dwf.shape)
    g1 = oracle.linear_ln_primal_grads(q, k, v, w0, gamma, beta, eta, b, dz, dwf)
    g2 = oracle.linear_ln_primal_grads(q, k, v, w0, gamma, beta, eta, b, dz2, dwf2)
    g3 = oracle.linear_ln_primal_grads(q, k, v, w0, gamma, beta, eta, b, 2 * dz - 3 * dz2, 2 * dwf - 3 * dwf2)
    for x1, x2, x3 in zip(g1, g2, g3):
        np.testing.assert_allclose(x3, 2 * x1 - 3 * x2, rtol=0, atol=1e-11 * max(1.0, np.abs(x3).max()))


def test_gradients_ill_conditioned_at_workload_length():
    """The reason the GPU tests bound the 1.3B-shape LN gradients at 1e-3 rather
    than 1e-4: at that length (8,192 tokens, per-token eta) the exact
    gradients themselves move by more than 1e-4 (relative, max-norm) when K is
    perturbed by 1e-6 relative, while at 256 tokens they move by far less."""
    import ttt_inputs as ti

    def worst_change(cfg):
        sub = ti.generate(cfg, chains=[0])
        dz, dwf = ti.upstream_grads(cfg, chains=[0])
        r = np.random.default_rng(3)
        gamma, beta = 1.0 + 0.3 * r.standard_normal((1, cfg.d)), 0.1 * r.standard_normal((1, cfg.d))
        q, k, v, w0 = (x.astype(np.float64) for x in (sub.q, sub.k, sub.v, sub.w_rows()))
        g0 = oracle.linear_ln_primal_grads(q, k, v, w0, gamma, beta, sub.eta_rows(), cfg.b, dz, dwf)
        k2 = k * (1 + 1e-6 * r.standard_normal(k.shape))
        g1 = oracle.linear_ln_primal_grads(q, k2, v, w0, gamma, beta, sub.eta_rows(), cfg.b, dz, dwf)
        return max(np.abs(a - b).max() / np.abs(b).max() for a, b in zip(g1, g0))

    assert worst_change(ti.CONFIGS["l1p3b"]) > 1e-4
    assert worst_change(ti.CONFIGS["l1p3b"].with_(B=1, H=1, T=256)) < 2e-5
