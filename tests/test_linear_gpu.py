"""GPU parity of TTT-Linear (libttt.so through its C ABI) against the fp64 oracle.

Tolerances (max over chains of max|x - ref| / max|ref|): 1e-5 for fp32
inputs, 2e-3 for bf16 inputs (fp32 Z), and for bf16 inputs also the 5e-5
regression bound of the hi+lo split-bf16 arithmetic (tests/ttt_testutil.py);
each test prints the max-norm, elementwise and Frobenius errors.
"""
import numpy as np
import pytest

import oracle
import ttt_inputs as ti
from ttt_testutil import CONTRACT_BF16, CONTRACT_FP32, REGRESS_MFMA, max_rel, parity, rows, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import test_sequence_layer_amd as m
    m.lib()
    return m


def _run(ttt, inp, generic=False, out_dtype=None, dtype=None):
    cfg = inp.cfg
    t = to_device(inp, dtype=dtype)
    z, wf = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, out_dtype=out_dtype,
                           generic=generic)
    torch.cuda.synchronize()
    return z, wf, t


def _check(ttt, cfg, tol, chains=None, generic=False, out_dtype=None, label=""):
    full = ti.generate(cfg)
    z, wf, _ = _run(ttt, full, generic=generic, out_dtype=out_dtype)
    if chains is None:
        chains = np.arange(cfg.chains)
        sub = full
    else:
        sub = ti.generate(cfg, chains=chains)
    zr, wr = oracle.run_inputs(sub)
    name = ttt.linear_kernel_name(cfg.B, cfg.H, cfg.T, cfg.d, cfg.b,
                                  1 if cfg.dtype == "bf16" else 0, 0, full.eta_strides, generic)
    e = parity(f"{label or cfg.name} kernel={name} chains={len(chains)}",
               [("Z", rows(z, chains), zr), ("W_final", rows(wf, chains), wr)], tol,
               REGRESS_MFMA if cfg.dtype == "bf16" and out_dtype in (None, torch.float32) else None)
    return e["Z"]["max"], e["W_final"]["max"]


def test_tiny_fp32(ttt):
    _check(ttt, ti.CONFIGS["tiny"], CONTRACT_FP32)


@pytest.mark.parametrize("B,H,T", [(1, 1, 16), (2, 3, 112), (3, 5, 256), (1, 2, 80)])
@pytest.mark.parametrize("eta_kind", ["scalar", "head", "token"])
def test_bf16_mfma_small(ttt, B, H, T, eta_kind):
    cfg = ti.CONFIGS["l1p3b"].with_(B=B, H=H, T=T, eta_kind=eta_kind, eta_value=1.0 / 64, seed=7 + T)
    assert ttt.linear_kernel_name(B, H, T, 64, 16) == "ttt_linear_mfma_d64b16"
    _check(ttt, cfg, CONTRACT_BF16, label=f"mfma B{B} H{H} T{T} {eta_kind}")


@pytest.mark.parametrize("B,H,T,eta_kind", [(2, 3, 112, "token"), (1, 2, 64, "scalar")])
def test_bf16_generic_small(ttt, B, H, T, eta_kind):
    cfg = ti.CONFIGS["l1p3b"].with_(B=B, H=H, T=T, eta_kind=eta_kind, eta_value=1.0 / 64, seed=11 + T)
    _check(ttt, cfg, CONTRACT_BF16, generic=True, label=f"generic B{B} H{H} T{T} {eta_kind}")


@pytest.mark.parametrize("d,b,T", [(64, 16, 128), (32, 8, 96), (16, 4, 64), (64, 32, 64), (16, 1, 20)])
def test_fp32_generic(ttt, d, b, T):
    cfg = ti.CONFIGS["tiny"].with_(B=2, H=3, d=d, b=b, T=T, eta_value=0.05, seed=d * b + T)
    _check(ttt, cfg, CONTRACT_FP32, generic=True, label=f"fp32 d{d} b{b} T{T}")


# ---- fp32 Q/K/V on the matrix cores (d = 64, b = 16) ----------------------------------

@pytest.mark.parametrize("B,H,T", [(1, 1, 16), (2, 3, 112), (1, 2, 256)])
@pytest.mark.parametrize("eta_kind", ["scalar", "head", "token"])
def test_fp32_mfma_small(ttt, B, H, T, eta_kind):
    cfg = ti.CONFIGS["l1p3b"].with_(B=B, H=H, T=T, dtype="fp32", eta_kind=eta_kind, eta_value=1.0 / 64,
                                   seed=300 + T)
    assert ttt.linear_kernel_name(B, H, T, 64, 16, in_dtype=0) == "ttt_linear_mfma_f32_d64b16"
    _check(ttt, cfg, CONTRACT_FP32, label=f"fp32 mfma B{B} H{H} T{T} {eta_kind}")


@pytest.mark.parametrize("name,sample", [("l125m", 12), ("l1p3b", 6), ("long", 3)])
def test_fp32_mfma_workloads(ttt, name, sample):
    """The 125M, 1.3B and long workload shapes with fp32 Q/K/V (the support
    matrix's fp32 rows), against the oracle on sampled chains at the fp32 bar."""
    cfg = ti.CONFIGS[name].with_(dtype="fp32")
    _check(ttt, cfg, CONTRACT_FP32, chains=ti.sample_chains(cfg, sample), label=f"fp32 {name}")


def test_fp32_mfma_vs_generic_and_bf16_output(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=3, T=192, dtype="fp32", seed=310)
    inp = ti.generate(cfg)
    z1, w1, _ = _run(ttt, inp)
    z2, w2, _ = _run(ttt, inp, generic=True)
    zb, wb, _ = _run(ttt, inp, out_dtype=torch.bfloat16)
    e = max(max_rel(rows(z1), rows(z2)), max_rel(rows(w1), rows(w2)))
    print(f"fp32 mfma vs generic: {e:.2e}", flush=True)
    assert e < 1e-5
    assert torch.equal(zb, z1.to(torch.bfloat16)) and torch.equal(wb, w1)


def test_mfma_vs_generic(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=4, T=320, seed=21)
    inp = ti.generate(cfg)
    z1, w1, _ = _run(ttt, inp)
    z2, w2, _ = _run(ttt, inp, generic=True)
    ez = max_rel(rows(z1), rows(z2))
    ew = max_rel(rows(w1), rows(w2))
    print(f"mfma vs generic: Z {ez:.3e} W {ew:.3e}", flush=True)
    assert ez < 1e-4 and ew < 1e-4


# ---- the workloads at full size, in the launch configuration the benchmark times ----

def test_config_l125m_all_chains(ttt):
    _check(ttt, ti.CONFIGS["l125m"], CONTRACT_BF16)


def test_config_l1p3b_all_chains(ttt):
    """The headline workload (B16 H32 T8192, per-token eta), every output of
    every chain against the oracle (about a second of 16 host threads)."""
    _check(ttt, ti.CONFIGS["l1p3b"], CONTRACT_BF16)


def test_config_long_all_chains(ttt):
    """The long-context workload (B2 H32 T32768), every chain."""
    _check(ttt, ti.CONFIGS["long"], CONTRACT_BF16)


# ---- pins that need no oracle ----

def test_eta_zero(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=64, eta_kind="scalar", eta_value=0.0)
    inp = ti.generate(cfg)
    z, wf, t = _run(ttt, inp)
    w0 = inp.w_rows()
    np.testing.assert_array_equal(rows(wf), w0)          # the state never moves
    ref = np.einsum("cij,ctj->cti", w0.astype(np.float64), inp.q.astype(np.float64))
    assert max_rel(rows(z), ref) < 1e-5


def test_orthogonal_interpolation(ttt):
    """Q = K with orthogonal keys inside every mini-batch, eta_s = 1/(2 c_s^2): Z = V."""
    rng = np.random.default_rng(3)
    B, H, T, d, b = 2, 2, 96, 64, 16
    axes = rng.permutation(d)[:b]
    cs = rng.choice([0.25, 0.5, 1.0, 2.0], size=(B, H, T))
    k = np.zeros((B, H, T, d), np.float32)
    for t in range(T):
        k[:, :, t, axes[t % b]] = cs[:, :, t]
    v, _ = ti.bf16_round(rng.standard_normal((B, H, T, d)).astype(np.float32) / 8)
    eta = (1.0 / (2.0 * cs * cs)).astype(np.float32)
    w0 = (rng.standard_normal((H, d, d)) * 0.02).astype(np.float32)
    dev = "cuda:0"
    bf = lambda x: torch.from_numpy(ti.bf16_round(x)[1].view(np.int16)).view(torch.bfloat16).to(dev)  # noqa
    kt = bf(k)
    z, wf = ttt.linear_fwd(kt, kt, bf(v), torch.from_numpy(w0).to(dev), torch.from_numpy(eta).to(dev), b)
    torch.cuda.synchronize()
    err = np.abs(z.cpu().numpy() - v).max() / np.abs(v).max()
    print(f"orthogonal interpolation: max |Z - V| / max|V| = {err:.3e}", flush=True)
    # The state maps a key of size c_s = 1/4 to v_s, so |W_b k_t| reaches ~8 max|V| for
    # c_t = 2; hi+lo bf16 operands carry up to 2^-16 relative error on those products
    # (~1.5e-5 * 8 before the fp32 sums): bound 1e-4.
    assert err < 1e-4
    # the final state maps the last mini-batch's keys to their values
    wk = np.einsum("bhij,bhtj->bhti", wf.cpu().numpy().astype(np.float64), k[:, :, -b:].astype(np.float64))
    assert np.abs(wk - v[:, :, -b:]).max() / np.abs(v).max() < 1e-4


@pytest.mark.parametrize("generic", [False, True])
def test_batch_gd_is_linear_attention(ttt, generic):
    """W0 = 0 and one mini-batch (b = T): E = -V, so z_t = 2 sum_{s <= t} eta_s (q_t . k_s) v_s
    (causal linear attention, [TTT] 03 §8) and W_final = 2 sum_s eta_s v_s k_s^T.
    Closed form in fp64 on the stored input values."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=3, T=16, eta_kind="token", seed=21)
    inp = ti.generate(cfg)
    t = to_device(inp)
    dev = "cuda:0"
    w0 = torch.zeros((cfg.H, 64, 64), device=dev)
    z, wf = ttt.linear_fwd(t["q"], t["k"], t["v"], w0, t["eta"], 16, generic=generic)
    torch.cuda.synchronize()
    q, k, v = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v))
    eta = inp.eta_rows().astype(np.float64)
    scores = np.einsum("ntc,nsc->nts", q, k) * eta[:, None, :] * np.tril(np.ones((16, 16)))[None]
    z_ref = 2.0 * np.einsum("nts,nsi->nti", scores, v)
    w_ref = 2.0 * np.einsum("ns,nsi,nsc->nic", eta, v, k)
    ez, ew = max_rel(rows(z), z_ref), max_rel(rows(wf), w_ref)
    print(f"linear attention (generic={generic}): err Z={ez:.3e} W_final={ew:.3e}", flush=True)
    assert ez < 1e-5 and ew < 1e-5


def test_fixed_point_exact(ttt):
    """V = W* K with W0 = W*: every gradient is zero, so W_final = W* and Z = W* Q.
    With W* = 1/2 times a permutation, W* K is exact in bf16 and E is exactly zero
    in the kernel, so both hold bit for bit."""
    rng = np.random.default_rng(22)
    B, H, T, d = 2, 3, 64, 64
    perm = np.stack([rng.permutation(d) for _ in range(H)])
    wstar = np.zeros((H, d, d), np.float32)
    for h in range(H):
        wstar[h, np.arange(d), perm[h]] = 0.5
    k, _ = ti.bf16_round(rng.standard_normal((B, H, T, d)).astype(np.float32) / 8)
    q, _ = ti.bf16_round(rng.standard_normal((B, H, T, d)).astype(np.float32) / 8)
    v = np.einsum("hij,bhtj->bhti", wstar, k).astype(np.float32)   # exact: one term of 0.5 * bf16
    dev = "cuda:0"
    bf = lambda x: torch.from_numpy(ti.bf16_round(x)[1].view(np.int16)).view(torch.bfloat16).to(dev)  # noqa
    eta = torch.full((B, H, T), 0.03, device=dev)
    z, wf = ttt.linear_fwd(bf(q), bf(k), bf(v), torch.from_numpy(wstar).to(dev), eta, 16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(wf.cpu().numpy(), np.broadcast_to(wstar, (B, H, d, d)))
    np.testing.assert_array_equal(z.cpu().numpy(), np.einsum("hij,bhtj->bhti", wstar, q))


def test_output_row_permutation(ttt):
    """Permuting the output rows of W0 and V permutes the rows of Z and W_final
    (rows of the state are independent, [TTT] 03 §9 with f = W x): bit for bit."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=128, seed=23)
    inp = ti.generate(cfg)
    t = to_device(inp)
    perm = torch.from_numpy(np.random.default_rng(24).permutation(64)).to("cuda:0")
    z, wf = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    zp, wfp = ttt.linear_fwd(t["q"], t["k"], t["v"][..., perm].contiguous(), t["w1"][:, perm].contiguous(),
                             t["eta"], 16)
    torch.cuda.synchronize()
    assert torch.equal(zp, z[..., perm])
    assert torch.equal(wfp, wf[:, :, perm])


def test_state_passing_and_inplace_carry(ttt):
    """fwd(T) == fwd(T1) then fwd(T - T1) from W_final (bitwise), with the state
    carried in place (W_final written over a per-sequence W0)."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=3, T=160, seed=5)
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, wf = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    T1 = 96
    state = t["w1"].unsqueeze(0).expand(cfg.B, -1, -1, -1).contiguous()
    sl = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
    za, _ = ttt.linear_fwd(sl(t["q"], 0, T1), sl(t["k"], 0, T1), sl(t["v"], 0, T1), state,
                           sl(t["eta"], 0, T1), 16, w_final=state)
    zb, _ = ttt.linear_fwd(sl(t["q"], T1, 160), sl(t["k"], T1, 160), sl(t["v"], T1, 160), state,
                           sl(t["eta"], T1, 160), 16, w_final=state)
    torch.cuda.synchronize()
    assert torch.equal(z, torch.cat([za, zb], dim=2))
    assert torch.equal(wf, state)


def test_deterministic(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=4, H=8, T=256, seed=9)
    inp = ti.generate(cfg)
    z1, w1, t = _run(ttt, inp)
    z2, w2 = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    torch.cuda.synchronize()
    assert torch.equal(z1, z2) and torch.equal(w1, w2)


def test_bf16_output(ttt):
    # bf16 has 8 significant bits: rounding Z adds up to 2^-8 relative to each element,
    # so the fp32-Z bound of 2e-3 cannot hold here; the bound is 2^-8 plus the compute error.
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=128, seed=13)
    _check(ttt, cfg, 2.0 ** -8 + 2e-4, out_dtype=torch.bfloat16, label="bf16 Z")


def test_empty_and_zero_length(ttt):
    dev = "cuda:0"
    e = torch.empty((0, 3, 32, 64), dtype=torch.bfloat16, device=dev)
    z, wf = ttt.linear_fwd(e, e, e, torch.zeros((3, 64, 64), device=dev), 0.1, 16)
    assert z.shape == (0, 3, 32, 64) and wf.shape == (0, 3, 64, 64)
    e = torch.empty((2, 3, 0, 64), dtype=torch.bfloat16, device=dev)
    w0 = torch.randn((3, 64, 64), device=dev)
    z, wf = ttt.linear_fwd(e, e, e, w0, 0.1, 16)
    torch.cuda.synchronize()
    assert torch.equal(wf, w0.unsqueeze(0).expand(2, -1, -1, -1))


def test_host_errors(ttt):
    dev = "cuda:0"
    x = torch.zeros((1, 1, 24, 64), dtype=torch.bfloat16, device=dev)
    w0 = torch.zeros((1, 64, 64), device=dev)
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_fwd(x, x, x, w0, 0.1, 16)            # T % b != 0
    assert ei.value.status == 2
    x = torch.zeros((1, 1, 32, 48), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_fwd(x, x, x, torch.zeros((1, 48, 48), device=dev), 0.1, 16)   # d = 48
    assert ei.value.status == 4
    x = torch.zeros((1, 1, 32, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_fwd(x, x, x, w0, 0.1, 16, z=x)       # Z aliases Q
    assert ei.value.status in (5, 3)
