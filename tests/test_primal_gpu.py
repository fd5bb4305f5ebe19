"""GPU tests of the primal-form TTT-Linear kernel (token by token) and the decode entry point.

Pages: [TTT] news article, part 03 §7 (the naive form the dual form replaces)
and part 04 §3 (decoding is sequential and uses the primal form).
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


def _oracle(inp):
    return oracle.run_inputs(inp)


@pytest.mark.parametrize("d,b,T,dtype,eta_kind", [
    (16, 4, 64, "fp32", "scalar"),      # the tiny workload
    (64, 16, 128, "bf16", "token"),
    (64, 1, 24, "bf16", "head"),
    (64, 5, 45, "fp32", "token"),
    (32, 8, 96, "bf16", "scalar"),
    (64, 64, 128, "bf16", "token"),     # b larger than any dual-form kernel takes
    (16, 16, 80, "fp32", "token"),      # unrolled 16-token pieces at d = 16, 32, 64
    (64, 16, 112, "fp32", "head"),      # fp32 inputs, three 32-token blocks and a 16-token tail
    (32, 32, 128, "bf16", "head"),
])
def test_primal_vs_oracle(ttt, d, b, T, dtype, eta_kind):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=3, d=d, b=b, T=T, dtype=dtype, eta_kind=eta_kind,
                                   eta_value=0.05, seed=d + b + T)
    inp = ti.generate(cfg)
    t = to_device(inp)
    assert ttt.linear_kernel_name(2, 3, T, d, b, primal=True) == f"ttt_linear_primal_kernel<{d}>"
    z, wf = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], b, primal=True)
    torch.cuda.synchronize()
    zr, wr = _oracle(inp)
    ez, ew = max_rel(rows(z), zr), max_rel(rows(wf), wr)
    print(f"primal d{d} b{b} T{T} {dtype} {eta_kind}: Z {ez:.3e} W {ew:.3e}", flush=True)
    assert ez < 1e-5 and ew < 1e-5


def test_primal_full_125m_shape(ttt):
    cfg = ti.CONFIGS["l125m"]
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, wf = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16, primal=True)
    zd, wd = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    torch.cuda.synchronize()
    ch = ti.sample_chains(cfg, 12)
    zr, wr = _oracle(ti.generate(cfg, chains=ch))
    ez, ew = max_rel(rows(z, ch), zr), max_rel(rows(wf, ch), wr)
    print(f"primal 125M shape: Z {ez:.3e} W {ew:.3e}; vs dual Z {max_rel(rows(z), rows(zd)):.3e}", flush=True)
    assert ez < 1e-5 and ew < 1e-5
    assert max_rel(rows(z), rows(zd)) < 1e-4


def _decode_in_chunks(ttt, t, cuts, b, w0_bh):
    B, H, T, d = t["q"].shape
    w = w0_bh.clone()
    wb = w0_bh.clone()
    zs = []
    pos = 0
    eta = t["eta"]
    for c in cuts:
        sl = lambda x: x[:, :, pos:pos + c].contiguous()  # noqa: E731
        e = sl(eta) if eta.dim() == 3 else eta
        zs.append(ttt.linear_decode(sl(t["q"]), sl(t["k"]), sl(t["v"]), e, w, wb, pos, b))
        pos += c
    assert pos == T
    return torch.cat(zs, dim=2), w


@pytest.mark.parametrize("cuts", [[1] * 48, [5, 11, 16, 3, 13], [48], [5, 40, 3], [16, 32]])
def test_decode_matches_forward(ttt, cuts):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=48, seed=17)
    inp = ti.generate(cfg)
    t = to_device(inp)
    w0 = t["w1"].unsqueeze(0).expand(2, -1, -1, -1).contiguous()
    z, w = _decode_in_chunks(ttt, t, cuts, 16, w0)
    zf, wf = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    torch.cuda.synchronize()
    zr, wr = _oracle(inp)
    print(f"decode cuts={cuts[:6]}: vs oracle Z {max_rel(rows(z), zr):.3e} W {max_rel(rows(w), wr):.3e}; "
          f"vs dual Z {max_rel(rows(z), rows(zf)):.3e}", flush=True)
    assert max_rel(rows(z), zr) < 1e-5 and max_rel(rows(w), wr) < 1e-5
    assert max_rel(rows(z), rows(zf)) < 1e-4 and max_rel(rows(w), rows(wf)) < 1e-4


def test_decode_batch_512(ttt):
    """Generation at the pages' batch (512 sequences x 32 heads = 16,384 chains,
    [TTT] 04 §3), one token per call with positions advancing over a mini-batch
    boundary, against the oracle on sampled chains."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=512, H=32, T=20, seed=23)
    inp = ti.generate(cfg)
    t = to_device(inp)
    w0 = t["w1"].unsqueeze(0).expand(cfg.B, -1, -1, -1).contiguous()
    z, w = _decode_in_chunks(ttt, t, [1] * 20, 16, w0)
    torch.cuda.synchronize()
    ch = ti.sample_chains(cfg, 16)
    zr, wr = _oracle(ti.generate(cfg, chains=ch))
    ez, ew = max_rel(rows(z, ch), zr), max_rel(rows(w, ch), wr)
    print(f"decode batch 512: vs oracle Z {ez:.3e} W {ew:.3e}", flush=True)
    assert ez < 1e-5 and ew < 1e-5


def test_decode_ragged_length(ttt):
    """37 tokens with b = 16: the last mini-batch is short (the oracle's reading of a
    ragged tail); the dual-form forward rejects T % b != 0, decode does not."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=1, H=3, T=37, seed=19)
    inp = ti.generate(cfg)
    t = to_device(inp)
    w0 = t["w1"].unsqueeze(0).contiguous()
    z, w = _decode_in_chunks(ttt, t, [20, 17], 16, w0)
    torch.cuda.synchronize()
    zr, wr = _oracle(inp)
    assert max_rel(rows(z), zr) < 1e-5 and max_rel(rows(w), wr) < 1e-5
    with pytest.raises(ttt.TTTError):
        ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)


def test_decode_errors(ttt):
    x = torch.zeros((1, 1, 1, 64), dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros((1, 1, 64, 64), device="cuda:0")
    wb = torch.zeros((1, 1, 64, 64), device="cuda:0")
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_decode(x, x, x, 0.1, w, wb, -1, 16)
    assert ei.value.status == 10
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_decode(x, x, x, 0.1, w, w, 0, 16)   # W and Wb alias
    assert ei.value.status == 5
