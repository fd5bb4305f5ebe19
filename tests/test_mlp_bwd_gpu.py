"""GPU parity of the TTT-MLP backward (ttt_mlp_bwd, through the C ABI) against
the oracle's reverse pass of the primal loop (oracle.mlp_primal_grads, which
the CPU tests pin to finite differences, torch fp64 autograd and the eta = 0
closed form).

Pages: [TTT] news article, part 03 §4 (the layer is trained end to end), §6
(mini-batch GD), §9 (TTT-MLP).  The kernel computes in fp32 throughout; every
gradient is compared per chain (max|x - ref| / max|ref|, max over chains)
against the 2e-3 contract and the regression bound below, and the errors are
printed.  Measured on MI355X, the primal form (fp32 throughout): at most
9.4e-7 on the small shapes and 4.7e-6 (dW1) on the TTT-MLP workload's sampled
chains, bound 2e-5; the dual form (matrix-core products of split bf16
operands): at most 1.02e-5 (deta, T = 16) and 6.5e-6 on the workload, bound 5e-5.
"""
import numpy as np
import pytest

import oracle
import ttt_inputs as ti
from ttt_testutil import CONTRACT_BF16, errors, rows, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "deta", "dw1", "dw2")
REGRESS_MLP_BWD = 2e-5   # the primal form (fp32 throughout)
REGRESS_DUAL = 5e-5      # the dual form (matrix cores, split bf16 operands)


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import test_sequence_layer_amd as m
    m.lib()
    return m


def _upstream(cfg, seed, with_dwf=True):
    r = np.random.default_rng(seed)
    dz = r.standard_normal((cfg.B, cfg.H, cfg.T, cfg.d)).astype(np.float32)
    d1 = r.standard_normal((cfg.B, cfg.H, cfg.dh, cfg.d)).astype(np.float32) if with_dwf else None
    d2 = r.standard_normal((cfg.B, cfg.H, cfg.d, cfg.dh)).astype(np.float32) if with_dwf else None
    return dz, d1, d2


def _run(ttt, cfg, seed=0, with_dwf=True, scale=None, chains=None, eta_override=None, primal=False):
    inp = ti.generate(cfg)
    t = to_device(inp)
    w1, w2 = inp.w1, inp.w2
    if scale:
        w1, w2 = (w1 * np.float32(scale[0])).astype(np.float32), (w2 * np.float32(scale[1])).astype(np.float32)
    dz, d1, d2 = _upstream(cfg, seed, with_dwf)
    dev = lambda x: None if x is None else torch.from_numpy(x).to(DEV)  # noqa: E731
    eta = t["eta"] if eta_override is None else eta_override
    got = ttt.mlp_bwd(t["q"], t["k"], t["v"], dev(w1), dev(w2), eta, cfg.b, dev(dz), dev(d1), dev(d2),
                      primal=primal)
    torch.cuda.synchronize()
    got = dict(zip(NAMES, got))
    chains = np.arange(cfg.chains) if chains is None else np.asarray(chains)
    sub = inp if len(chains) == cfg.chains else ti.generate(cfg, chains=chains)
    heads = chains % cfg.H
    flat = lambda x, s: None if x is None else x.reshape((cfg.chains,) + s)[chains]  # noqa: E731
    eta_rows = sub.eta_rows() if eta_override is None else np.zeros((len(chains), cfg.T))
    ref = dict(zip(NAMES, oracle.mlp_primal_grads(sub.q, sub.k, sub.v, w1[heads], w2[heads], eta_rows, cfg.b,
                                                  flat(dz, (cfg.T, cfg.d)), flat(d1, (cfg.dh, cfg.d)),
                                                  flat(d2, (cfg.d, cfg.dh)))))
    return got, ref, chains


def _check(label, got, ref, chains, regress=REGRESS_MLP_BWD):
    errs = {n: errors(rows(got[n], chains), ref[n]) for n in NAMES}
    print(f"[mlp bwd {label}] " + "  ".join(f"{n}: max {e['max']:.2e} frob {e['frob']:.2e}"
                                          for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items()
           if not (e["max"] < CONTRACT_BF16 and e["frob"] < CONTRACT_BF16 and e["max"] < regress)}
    assert not bad, bad


@pytest.mark.parametrize("b,T,dtype,eta_kind", [
    (16, 16, "bf16", "scalar"),
    (16, 48, "bf16", "token"),
    (16, 37, "fp32", "head"),     # a short last mini-batch
    (8, 40, "bf16", "token"),
    (5, 23, "fp32", "scalar"),
    (1, 9, "bf16", "token"),      # online GD
])
def test_mlp_bwd_vs_oracle(ttt, b, T, dtype, eta_kind):
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=3, T=T, b=b, dtype=dtype, eta_kind=eta_kind, eta_value=1.0 / 64,
                                  seed=500 + b + T)
    dual = b == 16 and T % 16 == 0 and dtype == "bf16"
    assert ttt.mlp_bwd_kernel_name(2, 3, T, 64, 256, b, in_dtype=1 if dtype == "bf16" else 0) == \
        ("ttt_mlp_bwd_d64h256b16" if dual else "ttt_mlp_bwd_d64h256")
    got, ref, ch = _run(ttt, cfg, seed=T)
    _check(f"b{b} T{T} {dtype} {eta_kind}", got, ref, ch, REGRESS_DUAL if dual else REGRESS_MLP_BWD)
    if dual:  # the same call in the primal form
        got_p, _, _ = _run(ttt, cfg, seed=T, primal=True)
        _check(f"b{b} T{T} {dtype} {eta_kind} primal", got_p, ref, ch)


@pytest.mark.parametrize("primal", [False, True])
def test_mlp_bwd_no_final_gradients_and_large_step(ttt, primal):
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=64, eta_value=8.0 / 64, seed=510)
    got, ref, ch = _run(ttt, cfg, seed=1, with_dwf=False, primal=primal)
    _check(f"dW_final = 0, eta 8/64{' primal' if primal else ''}", got, ref, ch,
           REGRESS_MLP_BWD if primal else REGRESS_DUAL)


def test_mlp_bwd_per_sequence_initial_state(ttt):
    """W0 given per sequence ([B, H, dh, d]): the gradients are per sequence too."""
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=2, T=32, seed=511)
    inp = ti.generate(cfg)
    t = to_device(inp)
    r = np.random.default_rng(3)
    w1 = (0.02 * r.standard_normal((2, 2, 256, 64))).astype(np.float32)
    w2 = (0.02 * r.standard_normal((2, 2, 64, 256))).astype(np.float32)
    dz, d1, d2 = _upstream(cfg, 4)
    got = ttt.mlp_bwd(t["q"], t["k"], t["v"], torch.from_numpy(w1).to(DEV), torch.from_numpy(w2).to(DEV), t["eta"],
                      16, torch.from_numpy(dz).to(DEV), torch.from_numpy(d1).to(DEV), torch.from_numpy(d2).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.mlp_primal_grads(inp.q, inp.k, inp.v, w1.reshape(4, 256, 64), w2.reshape(4, 64, 256),
                                  inp.eta_rows(), 16, dz.reshape(4, 32, 64), d1.reshape(4, 256, 64),
                                  d2.reshape(4, 64, 256))
    _check("per-sequence W0", dict(zip(NAMES, got)), dict(zip(NAMES, ref)), np.arange(4), REGRESS_DUAL)


@pytest.mark.parametrize("primal", [False, True])
def test_mlp_bwd_eta_zero(ttt, primal):
    """eta = 0: every path into K and V carries eta, so dK = dV = 0 exactly."""
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=32, seed=512)
    got, ref, ch = _run(ttt, cfg, seed=2, eta_override=torch.zeros((1,), device=DEV), primal=primal)
    assert float(got["dk"].abs().max()) == 0.0 and float(got["dv"].abs().max()) == 0.0
    _check(f"eta = 0{' primal' if primal else ''}", got, ref, ch, REGRESS_MLP_BWD if primal else REGRESS_DUAL)


def test_mlp_bwd_dual_short_and_empty(ttt):
    """One mini-batch (T = 16), and T = 0 (the gradients of W0 are the final-state ones)."""
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=2, T=16, seed=513)
    got, ref, ch = _run(ttt, cfg, seed=3)
    _check("T = 16", got, ref, ch, REGRESS_DUAL)
    q = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    w1 = torch.randn((2, 256, 64), device=DEV) * 0.02
    w2 = torch.randn((2, 64, 256), device=DEV) * 0.02
    d1 = torch.randn((1, 2, 256, 64), device=DEV)
    d2 = torch.randn((1, 2, 64, 256), device=DEV)
    out = ttt.mlp_bwd(q, q, q, w1, w2, torch.full((1,), 1 / 64, device=DEV), 16,
                      torch.zeros((1, 2, 0, 64), device=DEV), d1, d2)
    torch.cuda.synchronize()
    assert torch.equal(out[4], d1) and torch.equal(out[5], d2)


@pytest.mark.parametrize("primal", [False, True])
def test_mlp_bwd_full_shape_sampled(ttt, primal):
    """The TTT-MLP workload (B16 H32 T2048, scalar eta 1/64), sampled chains."""
    cfg = ti.CONFIGS["mlp"]
    assert ttt.mlp_bwd_kernel_name(cfg.B, cfg.H, cfg.T, 64, 256, 16, primal=primal) == \
        ("ttt_mlp_bwd_d64h256" if primal else "ttt_mlp_bwd_d64h256b16")
    got, ref, ch = _run(ttt, cfg, seed=5, chains=ti.sample_chains(cfg, 6), primal=primal)
    _check(f"TTT-MLP workload {'primal' if primal else 'dual'}", got, ref, ch,
           REGRESS_MLP_BWD if primal else REGRESS_DUAL)
