"""GPU parity of TTT-MLP (f(x) = W2 GELU(W1 x), d=64, dh=256, b=16) against the fp64 oracle.

Tolerance: 2e-3 max relative error (bf16 inputs, fp32 Z and state) per output
tensor and chain, and the 5e-5 regression bound of the split-bf16 arithmetic
(tests/ttt_testutil.py); every test prints the errors it measured.
"""
import numpy as np
import pytest
from scipy.stats import norm

import oracle
import ttt_inputs as ti
from ttt_testutil import CONTRACT_BF16, REGRESS_MFMA, max_rel, parity, rows, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import test_sequence_layer_amd as m
    m.lib()
    return m


def _run(ttt, inp):
    t = to_device(inp)
    z, f1, f2 = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], inp.cfg.b)
    torch.cuda.synchronize()
    return z, f1, f2, t


def _check(ttt, cfg, chains=None, tol=CONTRACT_BF16, regress=REGRESS_MFMA, label=""):
    full = ti.generate(cfg)
    z, f1, f2, _ = _run(ttt, full)
    if chains is None:
        chains = np.arange(cfg.chains)
        zr, r1, r2 = oracle.run_inputs(full)
    else:
        zr, r1, r2 = oracle.run_inputs(ti.generate(cfg, chains=chains))
    parity(f"{label or cfg.name} chains={len(chains)}",
           [("Z", rows(z, chains), zr), ("W1", rows(f1, chains), r1), ("W2", rows(f2, chains), r2)], tol, regress)


def test_kernel_name(ttt):
    assert ttt.mlp_kernel_name(16, 32, 2048, 64, 256, 16) == "ttt_mlp_fwd_d64h256b16"
    assert ttt.mlp_kernel_name(16, 32, 2048, 64, 128, 16) is None


@pytest.mark.parametrize("B,H,T", [(1, 1, 16), (2, 3, 48), (1, 2, 80)])
@pytest.mark.parametrize("eta_kind", ["scalar", "token"])
def test_small(ttt, B, H, T, eta_kind):
    cfg = ti.CONFIGS["mlp"].with_(B=B, H=H, T=T, eta_kind=eta_kind, seed=31 + T)
    _check(ttt, cfg, label=f"mlp B{B} H{H} T{T} {eta_kind}")


def test_large_step_size(ttt):
    """A step size 16x the workload's makes the state move far from W0 within
    a few mini-batches, so the dual-form corrections dominate the outputs."""
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=128, eta_value=0.25, seed=3)
    _check(ttt, cfg, label="mlp eta=0.25")


def test_config_mlp_all_chains(ttt):
    """The TTT-MLP workload (B16 H32 T2048), every chain against the oracle."""
    _check(ttt, ti.CONFIGS["mlp"])


def test_eta_zero(ttt):
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=2, T=64, eta_value=0.0)
    inp = ti.generate(cfg)
    z, f1, f2, _ = _run(ttt, inp)
    np.testing.assert_array_equal(rows(f1), inp.w_rows(1))
    np.testing.assert_array_equal(rows(f2), inp.w_rows(2))
    w1, w2 = inp.w_rows(1).astype(np.float64), inp.w_rows(2).astype(np.float64)
    hid = np.einsum("cjd,ctd->ctj", w1, inp.q.astype(np.float64))
    ref = np.einsum("cij,ctj->cti", w2, hid * norm.cdf(hid))
    err = max_rel(rows(z), ref)
    print(f"eta=0: Z vs W2 GELU(W1 Q): {err:.3e}", flush=True)
    assert err < 1e-5


def test_zero_second_layer_single_minibatch(ttt):
    """W2_0 = 0 and one mini-batch: W1 does not move and Z is causal linear
    attention with the feature map GELU(W1 x)."""
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=16, eta_value=0.05, seed=4)
    inp = ti.generate(cfg)
    t = to_device(inp)
    w2 = torch.zeros_like(t["w2"])
    z, f1, f2 = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], w2, t["eta"], 16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(rows(f1), inp.w_rows(1))
    for c in range(2):
        w1 = inp.w_rows(1)[c].astype(np.float64)
        hk, hq = inp.k[c] @ w1.T, inp.q[c] @ w1.T
        fk, fq = hk * norm.cdf(hk), hq * norm.cdf(hq)
        ref = (np.tril(fq @ fk.T) * 2 * 0.05) @ inp.v[c].astype(np.float64)
        err = np.abs(z[0, c].cpu().numpy() - ref).max() / np.abs(ref).max()
        print(f"W2=0: chain {c} err {err:.3e}", flush=True)
        assert err < 1e-4


def test_state_passing_and_determinism(ttt):
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=2, T=96, seed=6)
    inp = ti.generate(cfg)
    z, f1, f2, t = _run(ttt, inp)
    z2, g1, g2 = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16)
    torch.cuda.synchronize()
    assert torch.equal(z, z2) and torch.equal(f1, g1) and torch.equal(f2, g2)
    s1 = t["w1"].unsqueeze(0).expand(2, -1, -1, -1).contiguous()
    s2 = t["w2"].unsqueeze(0).expand(2, -1, -1, -1).contiguous()
    sl = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
    za, _, _ = ttt.mlp_fwd(sl(t["q"], 0, 48), sl(t["k"], 0, 48), sl(t["v"], 0, 48), s1, s2, t["eta"], 16,
                           w1_final=s1, w2_final=s2)
    zb, _, _ = ttt.mlp_fwd(sl(t["q"], 48, 96), sl(t["k"], 48, 96), sl(t["v"], 48, 96), s1, s2, t["eta"], 16,
                           w1_final=s1, w2_final=s2)
    torch.cuda.synchronize()
    assert torch.equal(z, torch.cat([za, zb], dim=2))
    assert torch.equal(f1, s1) and torch.equal(f2, s2)


def test_host_errors(ttt):
    x = torch.zeros((1, 1, 32, 64), dtype=torch.bfloat16, device="cuda:0")
    w1 = torch.zeros((1, 128, 64), device="cuda:0")
    w2 = torch.zeros((1, 64, 128), device="cuda:0")
    with pytest.raises(ttt.TTTError) as ei:
        ttt.mlp_fwd(x, x, x, w1, w2, 0.1, 16)
    assert ei.value.status == 4
    x = torch.zeros((1, 1, 40, 64), dtype=torch.bfloat16, device="cuda:0")
    w1 = torch.zeros((1, 256, 64), device="cuda:0")
    w2 = torch.zeros((1, 64, 256), device="cuda:0")
    with pytest.raises(ttt.TTTError) as ei:
        ttt.mlp_fwd(x, x, x, w1, w2, 0.1, 16)
    assert ei.value.status == 2
