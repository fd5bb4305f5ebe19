"""GPU parity of TTT-MLP with layer norm and residual inside f,
f(x) = x + LN(W2 GELU(W1 x)), against the fp64 oracle (2e-3, bf16 inputs).

Pages: [TTT] news article, part 03 §9 (f always contains layer normalization
and a residual connection; TTT-MLP has two layers, hidden width 4d, GELU).
"""
import numpy as np
import pytest

import oracle
import ttt_inputs as ti
from ttt_testutil import max_rel, rows, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import test_sequence_layer_amd as m
    m.lib()
    return m


def _ln_params(H, d, seed):
    r = np.random.default_rng(seed)
    return (1.0 + 0.2 * r.standard_normal((H, d))).astype(np.float32), (0.1 * r.standard_normal((H, d))).astype(
        np.float32)


def _run(ttt, cfg, gamma, beta, eps=1e-6, chains=None, eta_override=None):
    inp = ti.generate(cfg)
    t = to_device(inp)
    eta = t["eta"] if eta_override is None else eta_override
    g, b = torch.from_numpy(gamma).cuda(), torch.from_numpy(beta).cuda()
    z, w1f, w2f = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], g, b, eta, cfg.b, eps=eps)
    torch.cuda.synchronize()
    return inp, t, z, w1f, w2f


def _oracle(inp, gamma, beta, eps=1e-6, eta_rows=None):
    cfg = inp.cfg
    heads = np.asarray(inp.chains) % cfg.H
    return oracle.mlp_ln_primal(inp.q, inp.k, inp.v, inp.w_rows(1), inp.w_rows(2), gamma[heads].astype(np.float64),
                                beta[heads].astype(np.float64),
                                inp.eta_rows() if eta_rows is None else eta_rows, cfg.b, eps)


@pytest.mark.parametrize("B,H,T", [(1, 1, 16), (2, 3, 48), (1, 2, 80)])
@pytest.mark.parametrize("eta_kind", ["scalar", "token"])
def test_small(ttt, B, H, T, eta_kind):
    cfg = ti.CONFIGS["mlp"].with_(B=B, H=H, T=T, eta_kind=eta_kind, eta_value=1.0 / 64, seed=90 + T + H)
    gamma, beta = _ln_params(H, 64, 5 + T)
    inp, _, z, w1f, w2f = _run(ttt, cfg, gamma, beta)
    zr, w1r, w2r = _oracle(inp, gamma, beta)
    errs = [max_rel(rows(x), r) for x, r in ((z, zr), (w1f, w1r), (w2f, w2r))]
    print(f"mlp+ln B{B} H{H} T{T} {eta_kind}: Z {errs[0]:.3e} W1 {errs[1]:.3e} W2 {errs[2]:.3e}", flush=True)
    assert max(errs) < 2e-3, errs


def test_large_step_and_eps(ttt):
    # a step size 8x the usual one and a large eps: the normalisation and its
    # backward away from the eps -> 0 regime
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=64, eta_value=8.0 / 64, seed=97)
    gamma, beta = _ln_params(2, 64, 11)
    inp, _, z, w1f, w2f = _run(ttt, cfg, gamma, beta, eps=0.05)
    zr, w1r, w2r = _oracle(inp, gamma, beta, eps=0.05)
    errs = [max_rel(rows(x), r) for x, r in ((z, zr), (w1f, w1r), (w2f, w2r))]
    print(f"mlp+ln large step, eps 0.05: {errs}", flush=True)
    assert max(errs) < 2e-3, errs


def test_config_mlp_sampled(ttt):
    """The full TTT-MLP shape (B16 H32 T2048), 3 sampled chains.

    With the workload's 0.02-std weights the pre-norm output of the layer has a
    variance of ~1e-5, only ~10x eps, so the layer-norm backward divides by a tiny
    scale and the recurrence amplifies rounding: an fp32 numpy implementation of
    the same dual form already differs from the fp64 oracle by 8e-3 at T = 2048
    (6e-6 at T = 80).  No fp32 implementation can meet 2e-3 there, so the full
    length is checked at a well-conditioned scale, W1 and W2 multiplied by 20
    and 5 (stds 0.4 and 0.1: the fp32 numpy form is within 6e-7 of fp64); the
    short-sequence tests above use the workload's own scale."""
    cfg = ti.CONFIGS["mlp"]
    gamma, beta = _ln_params(cfg.H, cfg.d, 12)
    inp = ti.generate(cfg)
    w1 = (inp.w1 * np.float32(20)).astype(np.float32)
    w2 = (inp.w2 * np.float32(5)).astype(np.float32)
    t = to_device(inp)
    g, b = torch.from_numpy(gamma).cuda(), torch.from_numpy(beta).cuda()
    z, w1f, w2f = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], torch.from_numpy(w1).cuda(), torch.from_numpy(w2).cuda(),
                                 g, b, t["eta"], cfg.b)
    torch.cuda.synchronize()
    ch = ti.sample_chains(cfg, 3)
    sub = ti.generate(cfg, chains=ch)
    heads = np.asarray(ch) % cfg.H
    zr, w1r, w2r = oracle.mlp_ln_primal(sub.q, sub.k, sub.v, w1[heads], w2[heads], gamma[heads], beta[heads],
                                        sub.eta_rows(), cfg.b, 1e-6)
    errs = [max_rel(rows(x, ch), r) for x, r in ((z, zr), (w1f, w1r), (w2f, w2r))]
    print(f"mlp+ln full shape, chains {list(ch)}: {errs}", flush=True)
    assert max(errs) < 2e-3, errs


def test_eta_zero(ttt):
    """eta = 0: the weights do not move (bitwise) and Z = Q + LN(W2 GELU(W1 Q))."""
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=2, T=32, seed=98)
    gamma, beta = _ln_params(2, 64, 13)
    inp, t, z, w1f, w2f = _run(ttt, cfg, gamma, beta, eta_override=0.0)
    assert torch.equal(w1f, t["w1"].unsqueeze(0).expand_as(w1f))
    assert torch.equal(w2f, t["w2"].unsqueeze(0).expand_as(w2f))
    zr, _, _ = _oracle(inp, gamma, beta, eta_rows=np.zeros((cfg.chains, cfg.T)))
    assert max_rel(rows(z), zr) < 2e-3


def test_zero_gamma(ttt):
    """gamma = 0: f(x) = x + beta does not depend on the weights, so they stay
    exactly where they are and Z = Q + beta exactly (fp32 sum of bf16 Q and beta)."""
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=3, T=48, seed=99)
    _, beta = _ln_params(3, 64, 14)
    gamma = np.zeros((3, 64), np.float32)
    _, t, z, w1f, w2f = _run(ttt, cfg, gamma, beta)
    assert torch.equal(w1f, t["w1"].unsqueeze(0).expand_as(w1f))
    assert torch.equal(w2f, t["w2"].unsqueeze(0).expand_as(w2f))
    expect = t["q"].float() + torch.from_numpy(beta).cuda()[None, :, None, :]
    assert torch.equal(z, expect)


def test_state_passing_and_determinism(ttt):
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=64, seed=100)
    gamma, beta = _ln_params(2, 64, 15)
    inp = ti.generate(cfg)
    t = to_device(inp)
    g, b = torch.from_numpy(gamma).cuda(), torch.from_numpy(beta).cuda()
    z, w1f, w2f = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], g, b, t["eta"], 16)
    z2, w1f2, w2f2 = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], g, b, t["eta"], 16)
    h = 32
    za, w1a, w2a = ttt.mlp_ln_fwd(t["q"][:, :, :h].contiguous(), t["k"][:, :, :h].contiguous(),
                                  t["v"][:, :, :h].contiguous(), t["w1"], t["w2"], g, b, t["eta"], 16)
    zb, w1b, w2b = ttt.mlp_ln_fwd(t["q"][:, :, h:].contiguous(), t["k"][:, :, h:].contiguous(),
                                  t["v"][:, :, h:].contiguous(), w1a, w2a, g, b, t["eta"], 16)
    torch.cuda.synchronize()
    assert torch.equal(z, z2) and torch.equal(w1f, w1f2) and torch.equal(w2f, w2f2)
    assert max_rel(rows(torch.cat([za, zb], dim=2)), rows(z)) < 1e-5
    assert max_rel(rows(w1b), rows(w1f)) < 1e-5 and max_rel(rows(w2b), rows(w2f)) < 1e-5


def test_errors(ttt):
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=16, seed=101)
    inp = ti.generate(cfg)
    t = to_device(inp)
    g = torch.ones(2, 64, device="cuda:0")
    b = torch.zeros(2, 64, device="cuda:0")
    with pytest.raises(ValueError):
        ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], g[:1], b, t["eta"], 16)
    with pytest.raises(ttt.TTTError, match="TTT_ERR_SHAPE"):
        ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], g, b, t["eta"], 16, eps=-1.0)
    z = torch.empty(1, 2, 16, 64, device="cuda:0")
    with pytest.raises(ttt.TTTError, match="TTT_ERR_ALIAS"):   # gamma inside Z
        ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], z.view(-1)[:128].view(2, 64), b, t["eta"], 16,
                       z=z)
