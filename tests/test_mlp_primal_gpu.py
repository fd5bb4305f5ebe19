"""GPU tests of the TTT-MLP primal form (token by token): the full-sequence
forward (ttt_mlp_fwd with TTT_FLAG_PRIMAL) and decode (ttt_mlp_decode), through
the C ABI, against the fp64 oracle.

Pages: [TTT] news article, part 03 §7 (the naive form), §9 (TTT-MLP), part 04
§3 (generation is sequential and uses the primal form; Fig 15 compares TTT-MLP
generation with TTT-Linear).  The kernel computes in fp32 throughout, so the
bar is the fp32 one: 1e-5 max relative error per output tensor and chain
(fp32 or bf16 inputs; bf16 Z is checked against its own rounding).
"""
import numpy as np
import pytest

import oracle
import ttt_inputs as ti
from ttt_testutil import CONTRACT_FP32, errors, max_rel, rows, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

BF16_OUT_TOL = 2.0 ** -8 + 1e-5


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import test_sequence_layer_amd as m
    m.lib()
    return m


def _report(label, pairs, tol=CONTRACT_FP32):
    errs = {n: errors(g, r) for n, g, r in pairs}
    print(f"[mlp primal {label}] " + "  ".join(f"{n}: max {e['max']:.2e} frob {e['frob']:.2e}"
                                              for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items() if not (e["max"] < tol and e["frob"] < tol)}
    assert not bad, bad


@pytest.mark.parametrize("b,T,dtype,eta_kind", [
    (16, 48, "bf16", "scalar"),
    (16, 64, "bf16", "token"),
    (1, 12, "bf16", "token"),        # online GD
    (5, 40, "fp32", "token"),        # a mini-batch size the dual form does not take
    (64, 128, "fp32", "scalar"),
    (16, 32, "fp32", "head"),
])
def test_primal_vs_oracle(ttt, b, T, dtype, eta_kind):
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=3, T=T, b=b, dtype=dtype, eta_kind=eta_kind, eta_value=1.0 / 64,
                                  seed=200 + b + T)
    inp = ti.generate(cfg)
    t = to_device(inp)
    assert ttt.mlp_kernel_name(2, 3, T, 64, 256, b, primal=True) == "ttt_mlp_primal_d64h256"
    z, f1, f2 = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], b, primal=True)
    torch.cuda.synchronize()
    zr, r1, r2 = oracle.run_inputs(inp)
    _report(f"b{b} T{T} {dtype} {eta_kind}", [("Z", rows(z), zr), ("W1", rows(f1), r1), ("W2", rows(f2), r2)])


def test_primal_bf16_output(ttt):
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=32, seed=210)
    inp = ti.generate(cfg)
    t = to_device(inp)
    z32, a1, a2 = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16, primal=True)
    z16, b1, b2 = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16, primal=True,
                              out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(z16, z32.to(torch.bfloat16)) and torch.equal(a1, b1) and torch.equal(a2, b2)


def test_primal_large_step(ttt):
    """eta 16x the workload's: the state moves far from W0."""
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=128, eta_value=0.25, seed=211)
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, f1, f2 = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16, primal=True)
    torch.cuda.synchronize()
    zr, r1, r2 = oracle.run_inputs(inp)
    _report("eta=0.25", [("Z", rows(z), zr), ("W1", rows(f1), r1), ("W2", rows(f2), r2)])


def test_primal_full_mlp_shape_sampled(ttt):
    """The TTT-MLP workload (B16 H32 T2048) token by token, against the oracle
    on sampled chains and against the dual-form kernel on all of them."""
    cfg = ti.CONFIGS["mlp"]
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, f1, f2 = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16, primal=True)
    zd, d1, d2 = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16)
    torch.cuda.synchronize()
    ch = ti.sample_chains(cfg, 8)
    zr, r1, r2 = oracle.run_inputs(ti.generate(cfg, chains=ch))
    _report("MLP shape", [("Z", rows(z, ch), zr), ("W1", rows(f1, ch), r1), ("W2", rows(f2, ch), r2)])
    e = max(max_rel(rows(z), rows(zd)), max_rel(rows(f1), rows(d1)), max_rel(rows(f2), rows(d2)))
    print(f"[mlp primal vs dual, all chains] {e:.2e}", flush=True)
    assert e < 1e-4


def _decode_in_chunks(ttt, t, cuts, b):
    B, H, T, d = t["q"].shape
    w1 = t["w1"].unsqueeze(0).expand(B, -1, -1, -1).contiguous()
    w2 = t["w2"].unsqueeze(0).expand(B, -1, -1, -1).contiguous()
    w1b, w2b = w1.clone(), w2.clone()
    zs, pos = [], 0
    for c in cuts:
        sl = lambda x: x[:, :, pos:pos + c].contiguous()  # noqa: E731
        e = sl(t["eta"]) if t["eta"].dim() == 3 else t["eta"]
        zs.append(ttt.mlp_decode(sl(t["q"]), sl(t["k"]), sl(t["v"]), e, w1, w2, w1b, w2b, pos, b))
        pos += c
    assert pos == T
    return torch.cat(zs, dim=2), w1, w2


@pytest.mark.parametrize("cuts", [[1] * 40, [5, 11, 16, 3, 5], [40], [17, 23]])
def test_decode_matches_forward_and_oracle(ttt, cuts):
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=2, T=40, b=8, eta_kind="token", seed=212)
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, w1, w2 = _decode_in_chunks(ttt, t, cuts, 8)
    zf, f1, f2 = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 8, primal=True)
    torch.cuda.synchronize()
    zr, r1, r2 = oracle.run_inputs(inp)
    _report(f"decode cuts={cuts[:5]}", [("Z", rows(z), zr), ("W1", rows(w1), r1), ("W2", rows(w2), r2)])
    assert max_rel(rows(z), rows(zf)) < 1e-5


def test_decode_ragged_length(ttt):
    """37 tokens, b = 16: the last mini-batch is short (the oracle's reading)."""
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=3, T=37, seed=213)
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, w1, w2 = _decode_in_chunks(ttt, t, [20, 17], 16)
    torch.cuda.synchronize()
    zr, r1, r2 = oracle.run_inputs(inp)
    _report("ragged", [("Z", rows(z), zr), ("W1", rows(w1), r1), ("W2", rows(w2), r2)])


def test_decode_batch_512(ttt):
    """Generation at the pages' batch (512 sequences x 32 heads), one token per
    call across a mini-batch boundary, against the oracle on sampled chains."""
    cfg = ti.CONFIGS["mlp"].with_(B=512, H=32, T=18, seed=214)
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, w1, w2 = _decode_in_chunks(ttt, t, [1] * 18, 16)
    torch.cuda.synchronize()
    ch = ti.sample_chains(cfg, 12)
    zr, r1, r2 = oracle.run_inputs(ti.generate(cfg, chains=ch))
    _report("decode batch 512", [("Z", rows(z, ch), zr), ("W1", rows(w1, ch), r1), ("W2", rows(w2, ch), r2)])


def test_decode_errors(ttt):
    dev = "cuda:0"
    x = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16, device=dev)
    w1 = torch.zeros((1, 1, 256, 64), device=dev)
    w2 = torch.zeros((1, 1, 64, 256), device=dev)
    with pytest.raises(ttt.TTTError) as ei:
        ttt.mlp_decode(x, x, x, 0.1, w1, w2, w1.clone(), w2.clone(), -1, 16)
    assert ei.value.status == 10
    with pytest.raises(ttt.TTTError) as ei:                          # W1b is W1
        ttt.mlp_decode(x, x, x, 0.1, w1, w2, w1, w2.clone(), 0, 16)
    assert ei.value.status == 5
