"""Pins of the TTT-Linear oracle against what the pages and the mathematics fix.

Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
(aharts.cn / itmax.cn), part 03.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign, index or transpose, a misplaced mini-batch boundary, the mask
diagonal) fails at least one of them.
"""
import json
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_frac(rng, lo=-4, hi=4, den=(1, 2, 3, 4)):
    return Fraction(rng.randint(lo, hi), rng.choice(den))


def _rand_case(rng, d, T, eta_per_token):
    q = [[_rand_frac(rng) for _ in range(d)] for _ in range(T)]
    k = [[_rand_frac(rng) for _ in range(d)] for _ in range(T)]
    v = [[_rand_frac(rng) for _ in range(d)] for _ in range(T)]
    w0 = [[_rand_frac(rng) for _ in range(d)] for _ in range(d)]
    if eta_per_token:
        eta = [Fraction(rng.randint(1, 5), 16) for _ in range(T)]
    else:
        eta = [Fraction(1, 8)] * T
    return q, k, v, w0, eta


def _f(x):
    return np.array([[float(a) for a in r] for r in x])


def _c_oracle(q, k, v, w0, eta, b):
    z, wf = oracle.linear_primal(_f(q)[None], _f(k)[None], _f(v)[None], _f(w0)[None],
                                 np.array([[float(e) for e in eta]]), b)
    return z[0], wf[0]


# -- hand-worked examples (tests/golden) -------------------------------------

def _golden_cases():
    with open(os.path.join(GOLDEN, "linear_handworked.json")) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_handworked_exact_and_c(case):
    eta = [Fraction(e) for e in case["eta"]]
    conv = lambda m: [[Fraction(x) for x in r] for r in m]  # noqa: E731
    q, k, v, w0 = conv(case["q"]), conv(case["k"]), conv(case["v"]), conv(case["w0"])
    z, wf = oracle.linear_primal_exact(q, k, v, w0, eta, case["b"])
    assert z == conv(case["z"])
    assert wf == conv(case["w_final"])
    zc, wc = _c_oracle(q, k, v, w0, eta, case["b"])
    np.testing.assert_array_equal(zc, np.array(case["z"], float))
    np.testing.assert_array_equal(wc, np.array(case["w_final"], float))


# -- P1a: dual form == primal form, exactly (03 §7) -----------------------------

@pytest.mark.parametrize("d,T,b", [(2, 4, 1), (2, 4, 2), (3, 6, 3), (3, 6, 6), (4, 8, 4),
                                   (4, 12, 4), (3, 7, 3), (2, 5, 2), (4, 8, 8)])
@pytest.mark.parametrize("per_token", [False, True])
def test_dual_equals_primal_exact(d, T, b, per_token):
    rng = random.Random(1000 * d + 10 * T + b + per_token)
    case = _rand_case(rng, d, T, per_token)
    zp, wp = oracle.linear_primal_exact(*case, b)
    zd, wd = oracle.linear_dual_exact(*case, b)
    assert zp == zd
    assert wp == wd


# -- the C oracle agrees with the exact primal (to fp64 rounding) -------------

@pytest.mark.parametrize("d,T,b", [(2, 4, 2), (3, 7, 3), (4, 12, 4), (4, 9, 1), (4, 8, 8)])
def test_c_oracle_matches_exact(d, T, b):
    rng = random.Random(77 + d * T * b)
    case = _rand_case(rng, d, T, True)
    ze, we = oracle.linear_primal_exact(*case, b)
    zc, wc = _c_oracle(*case, b)
    ze, we = _f(ze), _f(we)
    assert np.abs(zc - ze).max() <= 1e-12 * max(1.0, np.abs(ze).max())
    assert np.abs(wc - we).max() <= 1e-12 * max(1.0, np.abs(we).max())


# -- P1b / P11: fp64 dual and naive (materialised G_t) forms vs the C oracle --

def _rand_f64(seed, n, T, d, eta_scale=1.0 / 64):
    r = np.random.default_rng(seed)
    q = r.standard_normal((n, T, d)) / np.sqrt(d)
    k = r.standard_normal((n, T, d)) / np.sqrt(d)
    v = r.standard_normal((n, T, d)) / np.sqrt(d)
    w0 = r.standard_normal((n, d, d)) * 0.02
    eta = eta_scale / (1.0 + np.exp(-r.standard_normal((n, T))))
    return q, k, v, w0, eta


@pytest.mark.parametrize("n,T,d,b", [(1, 64, 16, 4), (3, 256, 64, 16), (2, 50, 8, 16), (2, 33, 8, 5)])
def test_c_oracle_vs_dual_and_naive_f64(n, T, d, b):
    q, k, v, w0, eta = _rand_f64(n * T + d + b, n, T, d)
    z, wf = oracle.linear_primal(q, k, v, w0, eta, b)
    zd, wd = oracle.linear_dual_f64(q, k, v, w0, eta, b)
    assert oracle.max_rel_err(z, zd) < 1e-12
    assert oracle.max_rel_err(wf, wd) < 1e-12
    if T <= 64:
        zn, wn = oracle.linear_naive_f64(q, k, v, w0, eta, b)
        assert oracle.max_rel_err(z, zn) < 1e-13
        assert oracle.max_rel_err(wf, wn) < 1e-13


# -- P2: b = 1 is plain online gradient descent (03 §8) -----------------------

def test_b1_is_online_gd():
    q, k, v, w0, eta = _rand_f64(5, 2, 40, 8, eta_scale=0.2)
    z, wf = oracle.linear_primal(q, k, v, w0, eta, 1)
    for c in range(2):
        W = w0[c].copy()
        for t in range(40):
            W = W - eta[c, t] * 2.0 * np.outer(W @ k[c, t] - v[c, t], k[c, t])
            np.testing.assert_allclose(z[c, t], W @ q[c, t], rtol=0, atol=1e-14)
        np.testing.assert_allclose(wf[c], W, rtol=0, atol=1e-14)


# -- P3: eta = 0 leaves the state alone: Z = W0 Q, W_final = W0 ----------------

def test_eta_zero():
    q, k, v, w0, eta = _rand_f64(6, 2, 48, 8)
    z, wf = oracle.linear_primal(q, k, v, w0, np.zeros_like(eta), 16)
    np.testing.assert_array_equal(wf, w0)
    np.testing.assert_allclose(z, np.einsum("cij,ctj->cti", w0, q), rtol=0, atol=1e-15)


# -- P4: W0 = 0 with batch GD (b = T) is causal linear attention (03 §8) ------

def test_batch_gd_is_linear_attention_exact():
    rng = random.Random(4)
    d, T = 3, 6
    q, k, v, _, _ = _rand_case(rng, d, T, False)
    eta = Fraction(1, 8)
    w0 = [[Fraction(0)] * d for _ in range(d)]
    z, wf = oracle.linear_primal_exact(q, k, v, w0, [eta] * T, T)
    for t in range(T):
        expect = [sum(2 * eta * sum(q[t][j] * k[s][j] for j in range(d)) * v[s][i]
                      for s in range(t + 1)) for i in range(d)]
        assert z[t] == expect
    wexp = [[sum(2 * eta * v[s][i] * k[s][j] for s in range(T)) for j in range(d)] for i in range(d)]
    assert wf == wexp


def test_batch_gd_is_linear_attention_f64():
    q, k, v, _, _ = _rand_f64(8, 2, 32, 8)
    eta = np.full((2, 32), 1.0 / 64)
    z, wf = oracle.linear_primal(q, k, v, np.zeros((2, 8, 8)), eta, 32)
    for c in range(2):
        att = np.tril(q[c] @ k[c].T)                   # [t, s], s <= t, diagonal included
        np.testing.assert_allclose(z[c], 2.0 / 64 * att @ v[c], rtol=0, atol=1e-15)
        np.testing.assert_allclose(wf[c], 2.0 / 64 * v[c].T @ k[c], rtol=0, atol=1e-15)


# -- P5: the step is a gradient step of |W k - v|^2 (finite differences) -------

def test_step_is_gradient_of_reconstruction_loss():
    r = np.random.default_rng(9)
    d = 6
    W0 = r.standard_normal((d, d))
    k, v, q = r.standard_normal(d), r.standard_normal(d), r.standard_normal(d)
    eta = 0.03
    _, wf = oracle.linear_primal(q[None, None], k[None, None], v[None, None], W0[None],
                                 np.array([[eta]]), 1)
    grad_used = (W0 - wf[0]) / eta
    loss = lambda W: float(np.sum((W @ k - v) ** 2))  # noqa: E731
    fd = np.zeros((d, d))
    h = 1e-6
    for i in range(d):
        for j in range(d):
            Wp, Wm = W0.copy(), W0.copy()
            Wp[i, j] += h
            Wm[i, j] -= h
            fd[i, j] = (loss(Wp) - loss(Wm)) / (2 * h)
    np.testing.assert_allclose(grad_used, fd, rtol=1e-6, atol=1e-7)


# -- P6: orthogonal-key interpolation (boundary, diagonal, eta index) ----------

def _orthogonal_case(d, b, nmb, seed, exact):
    """Q = K; within a mini-batch k_s = c_s e_{pi(s)} on distinct axes, eta_s = 1/(2 c_s^2).

    Then every z_t equals v_t and W_final k_s = v_s for the last mini-batch.
    The axis set pi is the same in every mini-batch, so a misplaced boundary
    pairs non-orthogonal keys and breaks the identity.
    """
    rng = random.Random(seed)
    one = Fraction(1) if exact else 1.0
    axes = rng.sample(range(d), b)
    cs = [one * rng.choice([Fraction(1, 4), Fraction(1, 2), 1, 2]) for _ in range(b * nmb)]
    T = b * nmb
    k = []
    for t in range(T):
        row = [one * 0] * d
        row[axes[t % b]] = cs[t]
        k.append(row)
    v = [[one * rng.randint(-8, 8) / 4 for _ in range(d)] for _ in range(T)]
    w0 = [[one * rng.randint(-8, 8) / 8 for _ in range(d)] for _ in range(d)]
    eta = [1 / (2 * c * c) for c in cs]
    return k, v, w0, eta


def test_orthogonal_interpolation_exact():
    d, b, nmb = 5, 3, 4
    k, v, w0, eta = _orthogonal_case(d, b, nmb, 11, True)
    z, wf = oracle.linear_primal_exact(k, k, v, w0, eta, b)
    assert z == v
    for s in range(b * (nmb - 1), b * nmb):
        assert [sum(wf[i][j] * k[s][j] for j in range(d)) for i in range(d)] == v[s]
    # with the boundary one token off, the identity no longer holds
    z_bad, _ = oracle.linear_primal_exact(k, k, v, w0, eta, b + 1)
    assert z_bad != v


def test_orthogonal_interpolation_c_at_real_shape():
    d, b, nmb = 64, 16, 6
    k, v, w0, eta = _orthogonal_case(d, b, nmb, 12, False)
    k, v, w0 = np.array(k), np.array(v), np.array(w0)
    z, wf = oracle.linear_primal(k[None], k[None], v[None], w0[None], np.array(eta)[None], b)
    np.testing.assert_allclose(z[0], v, rtol=0, atol=1e-13)
    np.testing.assert_allclose(wf[0] @ k[-b:].T, v[-b:].T, rtol=0, atol=1e-13)


# -- P7: a state that already reconstructs V is a fixed point -------------------

def test_fixed_point():
    r = np.random.default_rng(13)
    d, T = 8, 48
    Ws = r.standard_normal((d, d)) * 0.1
    k = r.standard_normal((1, T, d))
    q = r.standard_normal((1, T, d))
    v = (k[0] @ Ws.T)[None]
    z, wf = oracle.linear_primal(q, k, v, Ws[None], np.full((1, T), 0.05), 16)
    np.testing.assert_allclose(wf[0], Ws, rtol=0, atol=1e-14)
    np.testing.assert_allclose(z[0], q[0] @ Ws.T, rtol=0, atol=1e-14)


# -- P8: (Z, W_final) is linear in (W0, V) jointly ------------------------------

def test_superposition_exact():
    rng = random.Random(21)
    d, T, b = 3, 6, 2
    q, k, v1, w1, eta = _rand_case(rng, d, T, True)
    _, _, v2, w2, _ = _rand_case(rng, d, T, True)
    a, c = Fraction(3, 2), Fraction(-2, 3)
    comb = lambda X, Y: [[a * x + c * y for x, y in zip(rx, ry)] for rx, ry in zip(X, Y)]  # noqa: E731
    z1, f1 = oracle.linear_primal_exact(q, k, v1, w1, eta, b)
    z2, f2 = oracle.linear_primal_exact(q, k, v2, w2, eta, b)
    z3, f3 = oracle.linear_primal_exact(q, k, comb(v1, v2), comb(w1, w2), eta, b)
    assert z3 == comb(z1, z2)
    assert f3 == comb(f1, f2)


# -- P9: state passing = checkpoint/resume at a mini-batch boundary -------------

@pytest.mark.parametrize("split", [16, 48, 64])
def test_state_passing_bitwise(split):
    q, k, v, w0, eta = _rand_f64(14, 2, 96, 16)
    z, wf = oracle.linear_primal(q, k, v, w0, eta, 16)
    za, wa = oracle.linear_primal(q[:, :split], k[:, :split], v[:, :split], w0, eta[:, :split], 16)
    zb, wb = oracle.linear_primal(q[:, split:], k[:, split:], v[:, split:], wa, eta[:, split:], 16)
    np.testing.assert_array_equal(z, np.concatenate([za, zb], axis=1))
    np.testing.assert_array_equal(wf, wb)


# -- P10: rows of the state are independent -------------------------------------

def test_row_permutation():
    q, k, v, w0, eta = _rand_f64(15, 2, 64, 8)
    perm = np.random.default_rng(1).permutation(8)
    z, wf = oracle.linear_primal(q, k, v, w0, eta, 16)
    zp, wp = oracle.linear_primal(q, k, v[:, :, perm], w0[:, perm, :], eta, 16)
    np.testing.assert_allclose(zp, z[:, :, perm], rtol=0, atol=1e-15)
    np.testing.assert_allclose(wp, wf[:, perm, :], rtol=0, atol=1e-15)


def test_chains_are_independent():
    q, k, v, w0, eta = _rand_f64(16, 4, 32, 8)
    z, wf = oracle.linear_primal(q, k, v, w0, eta, 8)
    for c in range(4):
        zc, wc = oracle.linear_primal(q[c:c + 1], k[c:c + 1], v[c:c + 1], w0[c:c + 1], eta[c:c + 1], 8)
        np.testing.assert_array_equal(zc[0], z[c])
        np.testing.assert_array_equal(wc[0], wf[c])


def test_threads_do_not_change_results():
    q, k, v, w0, eta = _rand_f64(17, 6, 64, 16)
    a = oracle.linear_primal(q, k, v, w0, eta, 16, threads=1)
    b = oracle.linear_primal(q, k, v, w0, eta, 16, threads=4)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# -- the error metric itself --------------------------------------------------

def test_max_rel_err_metric():
    ref = np.array([[1.0, -4.0], [0.5, 0.25]])
    x = ref + np.array([[0.0, 0.04], [0.0, 0.005]])
    # slice 0: 0.04 / 4 = 0.01; slice 1: 0.005 / 0.5 = 0.01
    assert abs(oracle.max_rel_err(x, ref) - 0.01) < 1e-15
    assert oracle.max_rel_err(ref, ref) == 0.0
