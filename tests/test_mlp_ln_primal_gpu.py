"""GPU tests of TTT-MLP with layer norm and residual inside f,
f(x) = x + LN(W2 GELU(W1 x)), in the primal form (token by token): the full
forward (ttt_mlp_ln_fwd with TTT_FLAG_PRIMAL) and decode (ttt_mlp_ln_decode),
through the C ABI, against the fp64 oracle (oracle.mlp_ln_primal).

Pages: [TTT] news article, part 03 §7 (the naive form), §9 (TTT-MLP; f always
holds a layer norm and a residual connection), part 04 §3 (generation is
sequential and uses the primal form).  The kernel computes in fp32 throughout.
Bars: the fp32 one, 1e-5, where the recurrence lets fp32 arithmetic meet it;
with the workload's 0.02-std weights and random gamma, beta the recurrence
amplifies rounding on some chains, so an fp32 numpy emulation of this primal loop is 1.6e-6 / 2.3e-6 from the fp64 oracle at
T = 48 / 80 (b = 16) but 1.8e-5 at T = 512 and 2.0e-5 at T = 64 with b = 5.
Those cases, and every case with a mini-batch size other than 16, run at the
rescaled weights the dual-form tests use (W1 x 20, W2 x 5, where the emulation
stays within 3.2e-6 on sampled chains).  At the full shape the tests take the
two settings that are well conditioned on every chain (see the test there).
"""
import numpy as np
import pytest

import oracle
import ttt_inputs as ti
from ttt_testutil import CONTRACT_FP32, errors, max_rel, rows, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

DEV = "cuda:0"


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


def _weights(inp, scaled):
    w1, w2 = inp.w1, inp.w2
    if scaled:
        w1, w2 = (w1 * np.float32(20)).astype(np.float32), (w2 * np.float32(5)).astype(np.float32)
    return w1, w2


def _oracle(cfg, w1, w2, gamma, beta, eps=1e-6, chains=None, eta_rows=None):
    chains = np.arange(cfg.chains) if chains is None else np.asarray(chains)
    sub = ti.generate(cfg, chains=chains)
    heads = chains % cfg.H
    return oracle.mlp_ln_primal(sub.q, sub.k, sub.v, w1[heads], w2[heads], gamma[heads], beta[heads],
                                sub.eta_rows() if eta_rows is None else eta_rows, cfg.b, eps)


def _report(label, pairs, tol=CONTRACT_FP32):
    errs = {n: errors(g, r) for n, g, r in pairs}
    print(f"[mlp ln primal {label}] " + "  ".join(f"{n}: max {e['max']:.2e} frob {e['frob']:.2e}"
                                                for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items() if not (e["max"] < tol and e["frob"] < tol)}
    assert not bad, bad


def _fwd(ttt, cfg, scaled, gamma, beta, eps=1e-6, **kw):
    inp = ti.generate(cfg)
    t = to_device(inp)
    w1, w2 = _weights(inp, scaled)
    z, f1, f2 = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], torch.from_numpy(w1).to(DEV), torch.from_numpy(w2).to(DEV),
                               torch.from_numpy(gamma).to(DEV), torch.from_numpy(beta).to(DEV), t["eta"], cfg.b,
                               eps, primal=True, **kw)
    torch.cuda.synchronize()
    return inp, t, w1, w2, z, f1, f2


@pytest.mark.parametrize("b,T,dtype,eta_kind,scaled", [
    (16, 16, "bf16", "scalar", False),
    (16, 48, "bf16", "token", False),
    (16, 80, "bf16", "scalar", False),
    (16, 64, "fp32", "head", False),
    (1, 12, "bf16", "token", True),      # online GD
    (5, 40, "fp32", "token", True),      # a mini-batch size the dual form does not take
    (64, 128, "bf16", "scalar", True),
])
def test_mlp_ln_primal_vs_oracle(ttt, b, T, dtype, eta_kind, scaled):
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=3, T=T, b=b, dtype=dtype, eta_kind=eta_kind, eta_value=1.0 / 64,
                                  seed=400 + b + T)
    gamma, beta = _ln_params(3, 64, T)
    assert ttt.mlp_ln_kernel_name(2, 3, T, 64, 256, b, primal=True) == "ttt_mlp_ln_primal_d64h256"
    inp, _, w1, w2, z, f1, f2 = _fwd(ttt, cfg, scaled, gamma, beta)
    zr, r1, r2 = _oracle(cfg, w1, w2, gamma, beta)
    _report(f"b{b} T{T} {dtype} {eta_kind}{' scaled' if scaled else ''}",
            [("Z", rows(z), zr), ("W1", rows(f1), r1), ("W2", rows(f2), r2)])


def test_mlp_ln_primal_large_step_and_eps(ttt):
    """A step size 8x the workload's and a large eps (0.05), at the workload's
    own weights: the normalisation and its backward away from eps -> 0."""
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=64, eta_value=8.0 / 64, seed=410)
    gamma, beta = _ln_params(2, 64, 11)
    _, _, w1, w2, z, f1, f2 = _fwd(ttt, cfg, False, gamma, beta, eps=0.05)
    zr, r1, r2 = _oracle(cfg, w1, w2, gamma, beta, eps=0.05)
    _report("eta 8/64, eps 0.05", [("Z", rows(z), zr), ("W1", rows(f1), r1), ("W2", rows(f2), r2)])


def test_mlp_ln_primal_zero_gamma_is_exact(ttt):
    """gamma = 0: f(k) = k + beta does not depend on the weights, every gradient
    is 0, so the weights stay exactly where they are and Z = Q + beta exactly."""
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=2, T=40, b=8, dtype="fp32", seed=411)
    inp = ti.generate(cfg)
    t = to_device(inp)
    beta = torch.randn((2, 64), device=DEV)
    z, f1, f2 = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], torch.zeros((2, 64), device=DEV), beta,
                               t["eta"], 8, primal=True)
    torch.cuda.synchronize()
    assert torch.equal(f1, t["w1"].unsqueeze(0).expand_as(f1))
    assert torch.equal(f2, t["w2"].unsqueeze(0).expand_as(f2))
    assert torch.equal(z, t["q"] + beta[None, :, None, :])


def test_mlp_ln_primal_bf16_output(ttt):
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=32, seed=412)
    t = to_device(ti.generate(cfg))
    g, be = (torch.from_numpy(x).to(DEV) for x in _ln_params(2, 64, 12))
    z32, a1, a2 = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], g, be, t["eta"], 16, primal=True)
    z16, c1, c2 = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], g, be, t["eta"], 16, primal=True,
                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(z16, z32.to(torch.bfloat16)) and torch.equal(a1, c1) and torch.equal(a2, c2)


@pytest.mark.parametrize("case", ["unit gamma, workload weights, T2048", "random gamma, scaled weights, T512"])
def test_mlp_ln_primal_full_shape_vs_dual_and_oracle(ttt, case):
    """The TTT-MLP workload's batch and heads (B16 H32) token by token, in the
    two settings where the recurrence is well conditioned on every chain (see
    tests/test_mlp_ln_gpu.py): the workload's own weights at the full length
    with gamma = 1, beta = 0, and random gamma, beta with W1 x 20, W2 x 5 at
    T = 512.  Against the oracle on sampled chains (and chain 118, the dual
    form's worst in the second setting) at the fp32 bar, and against the
    dual-form layer-norm kernel on all chains (measured 2.7e-5 and 2.6e-4)."""
    unit = case.startswith("unit")
    cfg = ti.CONFIGS["mlp"].with_(T=2048 if unit else 512)
    if unit:
        gamma, beta = np.ones((cfg.H, 64), np.float32), np.zeros((cfg.H, 64), np.float32)
    else:
        gamma, beta = _ln_params(cfg.H, 64, 12)
    inp, t, w1, w2, z, f1, f2 = _fwd(ttt, cfg, not unit, gamma, beta)
    zd, d1, d2 = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], torch.from_numpy(w1).to(DEV), torch.from_numpy(w2).to(DEV),
                                torch.from_numpy(gamma).to(DEV), torch.from_numpy(beta).to(DEV), t["eta"], cfg.b)
    torch.cuda.synchronize()
    ch = np.unique(np.concatenate([ti.sample_chains(cfg, 4), [118]]))
    zr, r1, r2 = _oracle(cfg, w1, w2, gamma, beta, chains=ch)
    _report(case, [("Z", rows(z, ch), zr), ("W1", rows(f1, ch), r1), ("W2", rows(f2, ch), r2)])
    e = max(max_rel(rows(z), rows(zd)), max_rel(rows(f1), rows(d1)), max_rel(rows(f2), rows(d2)))
    print(f"[mlp ln primal vs dual, all chains, {case}] {e:.2e}", flush=True)
    assert e < (1e-4 if unit else 5e-4)


def _decode_in_chunks(ttt, t, w1, w2, gamma, beta, cuts, b, eps=1e-6):
    B, H, T, d = t["q"].shape
    s1 = torch.from_numpy(w1).to(DEV).unsqueeze(0).expand(B, -1, -1, -1).contiguous()
    s2 = torch.from_numpy(w2).to(DEV).unsqueeze(0).expand(B, -1, -1, -1).contiguous()
    s1b, s2b = s1.clone(), s2.clone()
    zs, pos = [], 0
    for c in cuts:
        sl = lambda x: x[:, :, pos:pos + c].contiguous()  # noqa: E731
        e = sl(t["eta"]) if t["eta"].dim() == 3 else t["eta"]
        zs.append(ttt.mlp_decode(sl(t["q"]), sl(t["k"]), sl(t["v"]), e, s1, s2, s1b, s2b, pos, b,
                                 ln=(gamma, beta, eps)))
        pos += c
    assert pos == T
    return torch.cat(zs, dim=2), s1, s2


@pytest.mark.parametrize("cuts", [[1] * 40, [5, 11, 16, 3, 5], [40], [17, 23]])
def test_mlp_ln_decode_matches_forward_and_oracle(ttt, cuts):
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=2, T=40, b=8, eta_kind="token", seed=413)
    inp = ti.generate(cfg)
    t = to_device(inp)
    w1, w2 = _weights(inp, True)
    g, be = _ln_params(2, 64, 14)
    gd, bd = torch.from_numpy(g).to(DEV), torch.from_numpy(be).to(DEV)
    z, s1, s2 = _decode_in_chunks(ttt, t, w1, w2, gd, bd, cuts, 8)
    zf, f1, f2 = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], torch.from_numpy(w1).to(DEV), torch.from_numpy(w2).to(DEV),
                                gd, bd, t["eta"], 8, primal=True)
    torch.cuda.synchronize()
    zr, r1, r2 = _oracle(cfg, w1, w2, g, be)
    _report(f"decode cuts={cuts[:5]}", [("Z", rows(z), zr), ("W1", rows(s1), r1), ("W2", rows(s2), r2)])
    assert max_rel(rows(z), rows(zf)) < 1e-5 and max_rel(rows(s1), rows(f1)) < 1e-5


def test_mlp_ln_decode_ragged_length(ttt):
    """37 tokens, b = 16: the last mini-batch is short (the oracle's reading)."""
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=3, T=37, seed=414)
    inp = ti.generate(cfg)
    t = to_device(inp)
    w1, w2 = _weights(inp, False)
    g, be = _ln_params(3, 64, 15)
    z, s1, s2 = _decode_in_chunks(ttt, t, w1, w2, torch.from_numpy(g).to(DEV), torch.from_numpy(be).to(DEV),
                                  [20, 17], 16)
    torch.cuda.synchronize()
    zr, r1, r2 = _oracle(cfg, w1, w2, g, be)
    _report("ragged", [("Z", rows(z), zr), ("W1", rows(s1), r1), ("W2", rows(s2), r2)])


def test_mlp_ln_decode_batch_512(ttt):
    """Generation at the pages' batch (512 sequences x 32 heads), one token per
    call across a mini-batch boundary, against the oracle on sampled chains."""
    cfg = ti.CONFIGS["mlp"].with_(B=512, H=32, T=18, seed=415)
    inp = ti.generate(cfg)
    t = to_device(inp)
    w1, w2 = _weights(inp, False)
    g, be = _ln_params(32, 64, 16)
    z, s1, s2 = _decode_in_chunks(ttt, t, w1, w2, torch.from_numpy(g).to(DEV), torch.from_numpy(be).to(DEV),
                                  [1] * 18, 16)
    torch.cuda.synchronize()
    ch = ti.sample_chains(cfg, 12)
    zr, r1, r2 = _oracle(cfg, w1, w2, g, be, chains=ch)
    _report("decode batch 512", [("Z", rows(z, ch), zr), ("W1", rows(s1, ch), r1), ("W2", rows(s2, ch), r2)])


def test_mlp_ln_decode_errors(ttt):
    x = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16, device=DEV)
    w1 = torch.zeros((1, 1, 256, 64), device=DEV)
    w2 = torch.zeros((1, 1, 64, 256), device=DEV)
    g = torch.ones((1, 64), device=DEV)
    with pytest.raises(ttt.TTTError) as ei:                          # eps < 0
        ttt.mlp_decode(x, x, x, 0.1, w1, w2, w1.clone(), w2.clone(), 0, 16, ln=(g, g.clone(), -1.0))
    assert ei.value.status == 2
    with pytest.raises(ValueError):
        ttt.mlp_decode(x, x, x, 0.1, w1, w2, w1.clone(), w2.clone(), 0, 16, ln=(g[:, :32], g.clone(), 1e-6))
