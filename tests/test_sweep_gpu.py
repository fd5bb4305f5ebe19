"""Seeded random sweep of small shapes through every matrix-core kernel
against the fp64 oracle: batch, heads and length (up to 9 mini-batches),
step-size layout and magnitude, and output dtype drawn at random.  Same
bounds as the family tests: 2e-3 for bf16 inputs and the 5e-5 regression bound
of the split-bf16 arithmetic for fp32 outputs (tests/ttt_testutil.py); bf16
outputs add their own rounding, 2^-8."""
import numpy as np
import pytest

import oracle
import ttt_inputs as ti
from ttt_testutil import CONTRACT_BF16, REGRESS_MFMA, parity, rows, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = CONTRACT_BF16
BF16_OUT_TOL = 2.0 ** -8 + 2e-4


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import test_sequence_layer_amd as m
    m.lib()
    return m


def _draw(i, base):
    r = np.random.default_rng(1000 + i)
    cfg = ti.CONFIGS[base].with_(B=int(r.integers(1, 4)), H=int(r.integers(1, 5)), T=16 * int(r.integers(1, 10)),
                                 eta_kind=str(r.choice(["scalar", "head", "token"])),
                                 eta_value=float(r.choice([1.0 / 64, 1.0 / 16, 0.25])), seed=2000 + i)
    out_bf16 = bool(r.integers(0, 2))
    return cfg, out_bf16


@pytest.mark.parametrize("i", range(10))
def test_linear_forward(ttt, i):
    cfg, out_bf16 = _draw(i, "l1p3b")
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, wf = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b,
                           out_dtype=torch.bfloat16 if out_bf16 else None)
    torch.cuda.synchronize()
    zr, wr = oracle.run_inputs(inp)
    lab = f"sweep fwd {i} B{cfg.B} H{cfg.H} T{cfg.T} {cfg.eta_kind} eta {cfg.eta_value}"
    parity(lab, [("W_final", rows(wf), wr)], TOL, REGRESS_MFMA)
    parity(lab + (" bf16 Z" if out_bf16 else ""), [("Z", rows(z), zr)], BF16_OUT_TOL if out_bf16 else TOL,
           None if out_bf16 else REGRESS_MFMA)


@pytest.mark.parametrize("i", range(8))
def test_linear_layer_norm(ttt, i):
    cfg, out_bf16 = _draw(100 + i, "l1p3b")
    r = np.random.default_rng(3000 + i)
    gamma = (1.0 + 0.3 * r.standard_normal((cfg.H, cfg.d))).astype(np.float32)
    beta = (0.1 * r.standard_normal((cfg.H, cfg.d))).astype(np.float32)
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, wf = ttt.linear_ln_fwd(t["q"], t["k"], t["v"], t["w1"], torch.from_numpy(gamma).cuda(),
                              torch.from_numpy(beta).cuda(), t["eta"], cfg.b,
                              out_dtype=torch.bfloat16 if out_bf16 else None)
    torch.cuda.synchronize()
    heads = np.arange(cfg.chains) % cfg.H
    zr, wr = oracle.linear_ln_primal(inp.q, inp.k, inp.v, inp.w_rows(), gamma[heads], beta[heads],
                                     inp.eta_rows(), cfg.b, 1e-6)
    lab = f"sweep ln {i} B{cfg.B} H{cfg.H} T{cfg.T} {cfg.eta_kind} eta {cfg.eta_value}"
    parity(lab, [("W_final", rows(wf), wr)], TOL, REGRESS_MFMA)
    parity(lab + (" bf16 Z" if out_bf16 else ""), [("Z", rows(z), zr)], BF16_OUT_TOL if out_bf16 else TOL,
           None if out_bf16 else REGRESS_MFMA)


@pytest.mark.parametrize("i", range(6))
def test_mlp_forward(ttt, i):
    cfg, _ = _draw(200 + i, "mlp")
    cfg = cfg.with_(eta_value=min(cfg.eta_value, 1.0 / 16))
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, w1f, w2f = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], cfg.b)
    torch.cuda.synchronize()
    zr, w1r, w2r = oracle.run_inputs(inp)
    parity(f"sweep mlp {i} B{cfg.B} H{cfg.H} T{cfg.T} {cfg.eta_kind} eta {cfg.eta_value}",
           [("Z", rows(z), zr), ("W1", rows(w1f), w1r), ("W2", rows(w2f), w2r)], TOL, REGRESS_MFMA)


@pytest.mark.parametrize("i", range(6))
def test_linear_backward(ttt, i):
    cfg, out_bf16 = _draw(300 + i, "l1p3b")
    inp = ti.generate(cfg)
    t = to_device(inp)
    grad_dtype = "bf16" if out_bf16 else "fp32"
    z, wf, e = ttt.linear_fwd_save(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b)
    dz, dwf = ti.upstream_grads(cfg, dtype=grad_dtype)
    tdt = torch.bfloat16 if out_bf16 else torch.float32
    dz_t = torch.from_numpy(dz).reshape(cfg.B, cfg.H, cfg.T, cfg.d).to("cuda:0").to(tdt)
    dwf_t = torch.from_numpy(dwf).reshape(cfg.B, cfg.H, cfg.d, cfg.d).to("cuda:0")
    got = ttt.linear_bwd(t["q"], t["k"], t["eta"], wf, e, dz_t, cfg.b, dw_final=dwf_t)
    torch.cuda.synchronize()
    ref = oracle.linear_primal_grads(inp.q, inp.k, inp.v, inp.w_rows(), inp.eta_rows(), cfg.b, dz, dwf)
    lab = f"sweep bwd {i} B{cfg.B} H{cfg.H} T{cfg.T} {cfg.eta_kind} eta {cfg.eta_value} {grad_dtype}"
    for name, x, r in zip(("dq", "dk", "dv", "deta", "dw0"), got, ref):
        bf = x.dtype == torch.bfloat16
        parity(f"{lab} {name}", [(name, rows(x), r)], BF16_OUT_TOL if bf else TOL, None if bf else REGRESS_MFMA)
