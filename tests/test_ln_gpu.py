"""GPU parity of TTT-Linear with layer norm and residual inside f (f(x) = x + LN(W x)).

Pages: [TTT] news article, part 03 §9 (f always contains LN and a residual
connection).  Compared with the fp64 oracle; tolerance 2e-3 (bf16 inputs) and
the 5e-5 regression bound of the split-bf16 arithmetic (tests/ttt_testutil.py).
"""
import numpy as np
import pytest

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


def _ln_params(H, d, seed, kind="random"):
    r = np.random.default_rng(seed)
    if kind == "unit":
        return np.ones((H, d), np.float32), np.zeros((H, d), np.float32)
    return ((1.0 + 0.3 * r.standard_normal((H, d))).astype(np.float32),
            (0.1 * r.standard_normal((H, d))).astype(np.float32))


def _check(ttt, cfg, gamma, beta, chains=None, eps=1e-6, tol=CONTRACT_BF16, regress=REGRESS_MFMA, label=""):
    full = ti.generate(cfg)
    t = to_device(full)
    dev = "cuda:0"
    z, wf = ttt.linear_ln_fwd(t["q"], t["k"], t["v"], t["w1"], torch.from_numpy(gamma).to(dev),
                              torch.from_numpy(beta).to(dev), t["eta"], cfg.b, eps)
    torch.cuda.synchronize()
    chains = np.arange(cfg.chains) if chains is None else np.asarray(chains)
    sub = full if len(chains) == cfg.chains else ti.generate(cfg, chains=chains)
    heads = chains % cfg.H
    zr, wr = oracle.linear_ln_primal(sub.q, sub.k, sub.v, sub.w_rows(), gamma[heads], beta[heads],
                                     sub.eta_rows(), cfg.b, eps)
    parity(f"LN {label or cfg.name}", [("Z", rows(z, chains), zr), ("W_final", rows(wf, chains), wr)], tol, regress)
    return z, wf, t


@pytest.mark.parametrize("B,H,T", [(1, 1, 16), (2, 3, 112), (1, 2, 256)])
@pytest.mark.parametrize("eta_kind", ["scalar", "token"])
def test_ln_small(ttt, B, H, T, eta_kind):
    cfg = ti.CONFIGS["l1p3b"].with_(B=B, H=H, T=T, eta_kind=eta_kind, eta_value=1.0 / 64, seed=60 + T)
    g, b = _ln_params(H, 64, T)
    _check(ttt, cfg, g, b, label=f"B{B} H{H} T{T} {eta_kind}")


def test_ln_large_step(ttt):
    """A large step size drives the state (and the LN statistics) far from W0."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=1, H=2, T=256, eta_kind="scalar", eta_value=0.5, seed=62)
    g, b = _ln_params(2, 64, 5)
    _check(ttt, cfg, g, b, label="eta=0.5")


def test_ln_full_shape_all_chains(ttt):
    cfg = ti.CONFIGS["l1p3b"]
    g, b = _ln_params(cfg.H, 64, 7, "unit")
    z, _, t = _check(ttt, cfg, g, b, label="1.3B shape, gamma=1 beta=0, all chains")
    # with gamma = 1, beta = 0 every z_t - q_t is normalised over its 64 entries
    dz = (z.float() - t["q"].float()).reshape(-1, 64)
    assert float(dz.mean(dim=1).abs().max()) < 1e-5


def test_ln_zero_gamma_freezes_state(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=64, seed=63)
    inp = ti.generate(cfg)
    t = to_device(inp)
    beta = torch.randn((2, 64), device="cuda:0")
    z, wf = ttt.linear_ln_fwd(t["q"], t["k"], t["v"], t["w1"], torch.zeros((2, 64), device="cuda:0"), beta,
                              t["eta"], 16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(rows(wf), inp.w_rows())
    ref = t["q"].float() + beta[None, :, None, :]
    assert float((z - ref).abs().max()) < 1e-6


def test_ln_errors(ttt):
    x = torch.zeros((1, 1, 32, 64), dtype=torch.bfloat16, device="cuda:0")
    w0 = torch.zeros((1, 64, 64), device="cuda:0")
    g = torch.ones((1, 64), device="cuda:0")
    xf = torch.zeros((1, 1, 32, 64), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_ln_fwd(xf, xf, xf, w0, g, g, 0.1, 16)      # fp32 inputs: no LN kernel
    assert ei.value.status == 4
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_ln_fwd(x, x, x, w0, g, g, 0.1, 16, eps=-1.0)
    assert ei.value.status == 2
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_ln_fwd(x, x, x, w0, g, g, 0.1, 16, eps=float("nan"))
    assert ei.value.status == 2
    z = torch.empty((1, 1, 32, 64), device="cuda:0")
    with pytest.raises(ttt.TTTError, match="TTT_ERR_ALIAS"):  # gamma inside Z
        ttt.linear_ln_fwd(x, x, x, w0, z.view(-1)[:64].view(1, 64), g, 0.1, 16, z=z)
    wf = torch.empty((1, 1, 64, 64), device="cuda:0")
    with pytest.raises(ttt.TTTError, match="TTT_ERR_ALIAS"):  # beta inside W_final
        ttt.linear_ln_fwd(x, x, x, w0, g, wf.view(-1)[64:128].view(1, 64), 0.1, 16, w_final=wf)
    # flags (here a row-block count) are not taken: through the C ABI directly
    import ctypes
    desc = ttt.linear_desc(1, 1, 32, 64, 16, 1, 0, 0, (0, 0, 0), ttt.TTT_FLAG_ROWS[2])
    eta = torch.full((1,), 0.1, device="cuda:0")
    zz = torch.empty((1, 1, 32, 64), device="cuda:0")
    st = ttt.lib().ttt_linear_ln_fwd(ctypes.byref(desc), x.data_ptr(), x.data_ptr(), x.data_ptr(), w0.data_ptr(),
                                     g.data_ptr(), g.data_ptr(), ctypes.c_float(1e-6), eta.data_ptr(),
                                     zz.data_ptr(), wf.data_ptr(), None)
    assert st == 4


def test_ln_bf16_output_is_rounded_fp32(ttt):
    """bf16 Z: the same kernel arithmetic, rounded to bf16 (nearest even) at the
    store, so it equals the fp32 output rounded by torch, bit for bit."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=3, T=96, seed=64)
    t = to_device(ti.generate(cfg))
    g, b = (torch.from_numpy(x).cuda() for x in _ln_params(3, 64, 8))
    z32, w32 = ttt.linear_ln_fwd(t["q"], t["k"], t["v"], t["w1"], g, b, t["eta"], 16)
    z16, w16 = ttt.linear_ln_fwd(t["q"], t["k"], t["v"], t["w1"], g, b, t["eta"], 16, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert z16.dtype == torch.bfloat16
    assert torch.equal(z16, z32.to(torch.bfloat16))
    assert torch.equal(w16, w32)


def test_ln_state_passing_and_in_place_carry(ttt):
    """fwd(T) == fwd(T1) then fwd(T - T1) from its final state (bitwise: the
    per-step arithmetic does not depend on the position), here with a
    per-sequence W0 [B, H, d, d] carried in place (W_final aliasing W0)."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=128, eta_kind="token", seed=65)
    inp = ti.generate(cfg)
    t = to_device(inp)
    g, b = (torch.from_numpy(x).cuda() for x in _ln_params(2, 64, 9))
    w0 = t["w1"].unsqueeze(0).expand(2, -1, -1, -1).contiguous()
    z, wf = ttt.linear_ln_fwd(t["q"], t["k"], t["v"], w0, g, b, t["eta"], 16)
    h = 48
    state = w0.clone()
    parts = []
    for lo, hi in ((0, h), (h, cfg.T)):
        sl = lambda x: x[:, :, lo:hi].contiguous()  # noqa: E731
        zp, _ = ttt.linear_ln_fwd(sl(t["q"]), sl(t["k"]), sl(t["v"]), state, g, b, sl(t["eta"]), 16,
                                  w_final=state)
        parts.append(zp)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, dim=2), z)
    assert torch.equal(state, wf)


def test_ln_eta_zero(ttt):
    """eta = 0: the state does not move (bitwise) and Z = Q + LN(W0 Q)."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=1, H=2, T=64, seed=66)
    inp = ti.generate(cfg)
    t = to_device(inp)
    gamma, beta = _ln_params(2, 64, 10)
    z, wf = ttt.linear_ln_fwd(t["q"], t["k"], t["v"], t["w1"], torch.from_numpy(gamma).cuda(),
                              torch.from_numpy(beta).cuda(), 0.0, 16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(rows(wf), inp.w_rows())
    heads = np.arange(cfg.chains) % cfg.H
    zr, _ = oracle.linear_ln_primal(inp.q, inp.k, inp.v, inp.w_rows(), gamma[heads], beta[heads],
                                    np.zeros((cfg.chains, cfg.T)), 16, 1e-6)
    parity("LN eta=0", [("Z", rows(z), zr)], CONTRACT_BF16, REGRESS_MFMA)


def test_ln_empty(ttt):
    """B = 0 or T = 0: nothing to do, no launch; W_final = W0 when T = 0."""
    dev = "cuda:0"
    g = torch.ones((3, 64), device=dev)
    b = torch.zeros((3, 64), device=dev)
    w0 = torch.randn((3, 64, 64), device=dev)
    e = torch.empty((0, 3, 32, 64), dtype=torch.bfloat16, device=dev)
    z, wf = ttt.linear_ln_fwd(e, e, e, w0, g, b, 0.1, 16)
    assert z.shape == (0, 3, 32, 64) and wf.shape == (0, 3, 64, 64)
    e = torch.empty((2, 3, 0, 64), dtype=torch.bfloat16, device=dev)
    z, wf = ttt.linear_ln_fwd(e, e, e, w0, g, b, 0.1, 16)
    torch.cuda.synchronize()
    assert z.shape == (2, 3, 0, 64)
    assert torch.equal(wf, w0.unsqueeze(0).expand(2, -1, -1, -1))
