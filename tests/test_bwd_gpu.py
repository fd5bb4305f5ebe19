"""GPU parity of the TTT-Linear backward (ttt_linear_fwd_save + ttt_linear_bwd,
through the C ABI) against the fp64 oracle.

Pages: [TTT] news article, part 03 §4 (the layer is trained end to end), §7
(the dual form serves the backward too).  Tolerances (max over chains of
max|x - ref| / max|ref|, per output): 2e-3 for bf16 inputs, 1e-5 for fp32
inputs -- the forward's bars; each test prints its errors.  The reference is
the oracle's C reverse pass of the primal loop (oracle.linear_primal_grads),
which the CPU tests pin to finite differences and to torch fp64 autograd.
"""
import numpy as np
import pytest

import oracle
import ttt_inputs as ti
from ttt_testutil import CONTRACT_BF16, CONTRACT_FP32, REGRESS_MFMA, errors, max_rel, rows, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

NAMES = ("dq", "dk", "dv", "deta", "dw0")


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import test_sequence_layer_amd as m
    m.lib()
    return m


def _grads_dev(cfg, dz, dwf, grad_dtype, with_dwf):
    tdt = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
    dz_t = torch.from_numpy(dz).reshape(cfg.B, cfg.H, cfg.T, cfg.d).to("cuda:0").to(tdt)
    dwf_t = torch.from_numpy(dwf).reshape(cfg.B, cfg.H, cfg.d, cfg.d).to("cuda:0") if with_dwf else None
    return dz_t, dwf_t


def _gpu(ttt, cfg, generic=False, grad_dtype="fp32", with_dwf=True, dwf_scale=1.0):
    full = ti.generate(cfg)
    t = to_device(full)
    out_dtype = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
    z, wf, e = ttt.linear_fwd_save(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, generic=generic)
    dz_np, dwf_np = ti.upstream_grads(cfg, dtype=grad_dtype, dwf_scale=dwf_scale)
    dz, dwf = _grads_dev(cfg, dz_np, dwf_np, grad_dtype, with_dwf)
    assert dz.dtype == out_dtype
    g = ttt.linear_bwd(t["q"], t["k"], t["eta"], wf, e, dz, cfg.b, dw_final=dwf, generic=generic)
    torch.cuda.synchronize()
    return dict(zip(NAMES, g)), (z, wf, e), t, (full, dz_np, dwf_np)


def _oracle(cfg, chains, grad_dtype="fp32", with_dwf=True, dwf_scale=1.0, host=None):
    """host: (inputs, dZ, dW_final) of every chain, reused when chains is all of them."""
    if host is not None and len(chains) == cfg.chains:
        sub, dz, dwf = host
    else:
        sub = ti.generate(cfg, chains=chains)
        dz, dwf = ti.upstream_grads(cfg, chains=chains, dtype=grad_dtype, dwf_scale=dwf_scale)
    ref = oracle.linear_primal_grads(sub.q, sub.k, sub.v, sub.w_rows(), sub.eta_rows(), cfg.b, dz,
                                     dwf if with_dwf else None)
    return dict(zip(NAMES, ref))


# bf16 outputs (dq, dk, dv when dZ is bf16): rounding to 8 significant bits
# alone is up to 2^-8 relative, plus the kernel's own error
BF16_OUT_TOL = 2.0 ** -8 + 2e-4


def _compare(got, ref, chains, tol, label, regress=None):
    """Each gradient against the oracle: max-norm error below ``tol`` (bf16
    outputs: their rounding bar) and below ``regress`` for fp32 outputs; the
    elementwise and Frobenius errors are printed beside it."""
    full = {n: errors(rows(got[n], chains), ref[n]) for n in NAMES}
    print(f"[bwd {label}] " + "  ".join(f"{n}: max {e['max']:.2e} elem {e['elem']:.2e} frob {e['frob']:.2e}"
                                        for n, e in full.items()), flush=True)
    bad = {}
    for n, e in full.items():
        bf = got[n].dtype == torch.bfloat16
        if not e["max"] < (BF16_OUT_TOL if bf else tol) or not e["frob"] < (BF16_OUT_TOL if bf else tol):
            bad[n] = e
        elif regress is not None and not bf and not e["max"] < regress:
            bad[n] = (e, "regression bound", regress)
    assert not bad, bad
    return {n: e["max"] for n, e in full.items()}


def _check(ttt, cfg, tol, chains=None, generic=False, grad_dtype="fp32", with_dwf=True, dwf_scale=1.0, label="",
           regress=None):
    got, _, _, host = _gpu(ttt, cfg, generic, grad_dtype, with_dwf, dwf_scale)
    chains = np.arange(cfg.chains) if chains is None else np.asarray(chains)
    ref = _oracle(cfg, chains, grad_dtype, with_dwf, dwf_scale, host)
    name = ttt.linear_bwd_kernel_name(cfg.B, cfg.H, cfg.T, cfg.d, cfg.b, 1 if cfg.dtype == "bf16" else 0,
                                      1 if grad_dtype == "bf16" else 0, generic=generic)
    if regress is None and cfg.dtype == "bf16":
        regress = REGRESS_MFMA
    return _compare(got, ref, chains, tol, f"{label or cfg.name} {name}", regress)


# ---- MFMA kernel (d = 64, b = 16, bf16 Q/K) ---------------------------------------

@pytest.mark.parametrize("B,H,T", [(1, 1, 16), (2, 3, 112), (1, 2, 256)])
@pytest.mark.parametrize("eta_kind", ["scalar", "head", "token"])
def test_mfma_small(ttt, B, H, T, eta_kind):
    cfg = ti.CONFIGS["l1p3b"].with_(B=B, H=H, T=T, eta_kind=eta_kind, eta_value=1.0 / 64, seed=90 + T)
    _check(ttt, cfg, CONTRACT_BF16, label=f"B{B} H{H} T{T} {eta_kind}")


def test_mfma_no_dwf_and_bf16_grads(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=128, seed=91)
    _check(ttt, cfg, CONTRACT_BF16, with_dwf=False, label="dW_final = 0")
    _check(ttt, cfg, CONTRACT_BF16, grad_dtype="bf16", label="bf16 dZ / outputs")


def test_mfma_large_step(ttt):
    """eta = 0.5: the inner steps move the state far from W0 (the rebuilt states must follow)."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=1, H=2, T=256, eta_kind="scalar", eta_value=0.5, seed=92)
    _check(ttt, cfg, CONTRACT_BF16, label="eta=0.5")


def test_mfma_matches_generic(ttt):
    """The two GPU backward kernels agree on the same saved forward."""
    cfg = ti.CONFIGS["l125m"].with_(B=2, H=3, T=256, seed=93)
    a, _, _, _ = _gpu(ttt, cfg, generic=False)
    b, _, _, _ = _gpu(ttt, cfg, generic=True)
    errs = {n: max_rel(rows(a[n]), rows(b[n])) for n in NAMES}
    print("[bwd mfma vs generic] " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    assert max(errs.values()) < 1e-4, errs


def test_mfma_eta_zero(ttt):
    """eta = 0 (closed form): dQ = W0^T dZ, dW0 = sum_t dz_t q_t^T + dW_final, dK = dV = 0."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=1, H=2, T=64, eta_kind="scalar", eta_value=0.0, seed=94)
    got, _, t, _ = _gpu(ttt, cfg)
    assert float(got["dk"].abs().max()) == 0.0 and float(got["dv"].abs().max()) == 0.0
    dz, dwf = ti.upstream_grads(cfg)
    inp = ti.generate(cfg)
    w0 = inp.w_rows().astype(np.float64)
    q = inp.q.astype(np.float64)
    dq_ref = np.einsum("nij,nti->ntj", w0, dz)
    dw0_ref = np.einsum("nti,ntj->nij", dz, q) + dwf
    assert max_rel(rows(got["dq"]), dq_ref) < 1e-5
    assert max_rel(rows(got["dw0"]), dw0_ref) < 1e-5


def test_mfma_1p3b_all_chains(ttt):
    """The 1.3B-layer shape (B16 H32 T8192, per-token eta) in the launch the
    benchmark times, every gradient of every chain against the oracle's
    reverse pass."""
    _check(ttt, ti.CONFIGS["l1p3b"], CONTRACT_BF16, label="1.3B shape, all chains")


def test_mfma_long_all_chains(ttt):
    """2048 mini-batches: the state is rebuilt backward over the whole
    sequence; every chain."""
    _check(ttt, ti.CONFIGS["long"], CONTRACT_BF16, label="long, all chains")


# ---- portable fp32 kernel ------------------------------------------------------------

def test_generic_tiny_fp32(ttt):
    _check(ttt, ti.CONFIGS["tiny"], 1e-5, generic=True)


@pytest.mark.parametrize("d,b,T", [(32, 8, 96), (64, 16, 64), (16, 64, 128)])
def test_generic_fp32_shapes(ttt, d, b, T):
    cfg = ti.CONFIGS["tiny"].with_(B=2, H=2, d=d, b=b, T=T, eta_value=0.05, seed=95 + d)
    _check(ttt, cfg, 1e-5, generic=True, label=f"fp32 d{d} b{b}")


def test_generic_bf16(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=1, H=3, T=96, seed=96)
    _check(ttt, cfg, CONTRACT_BF16, generic=True, label="generic bf16")


# ---- edge cases ------------------------------------------------------------------------

def test_empty_sequence(ttt):
    """T = 0: no tokens; dW0 = dW_final."""
    dev = "cuda:0"
    q = torch.zeros((2, 3, 0, 64), dtype=torch.bfloat16, device=dev)
    wf = torch.randn((2, 3, 64, 64), device=dev)
    dwf = torch.randn((2, 3, 64, 64), device=dev)
    e = torch.zeros((2, 3, 0, 64), device=dev)
    dz = torch.zeros((2, 3, 0, 64), device=dev)
    dq, dk, dv, deta, dw0 = ttt.linear_bwd(q, q, 0.1, wf, e, dz, 16, dw_final=dwf)
    torch.cuda.synchronize()
    assert torch.equal(dw0, dwf)


def test_errors(ttt):
    dev = "cuda:0"
    x = torch.zeros((1, 1, 32, 64), dtype=torch.bfloat16, device=dev)
    e = torch.zeros((1, 1, 32, 64), device=dev)
    wf = torch.zeros((1, 1, 64, 64), device=dev)
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_bwd(x, x, 0.1, wf, e, e, 24)   # T % b != 0
    assert ei.value.status == 2
    with pytest.raises(ttt.TTTError) as ei:       # dV over E
        ttt.linear_bwd(x, x, 0.1, wf, e, e.clone(), 16,
                       out=(e.clone(), e.clone(), e, torch.zeros((1, 1, 32), device=dev), wf.clone()))
    assert ei.value.status == 5
