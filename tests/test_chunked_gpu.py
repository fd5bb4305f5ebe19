"""GPU tests of the chunked TTT-Linear forward (chunk maps + scan + parallel chunks).

Each mini-batch maps the state affinely (W -> W P + R), so splitting a sequence
into chunks, composing each chunk's map, scanning the maps and running the
chunks in parallel must reproduce the sequential result (to rounding).
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


# 16 mini-batches: equal chunks (2, 4, 8, 16) and unequal ones (3, 5, 7: chunk c
# starts at mini-batch c * 16 // n)
@pytest.mark.parametrize("nchunks", [2, 3, 4, 5, 7, 8, 16])
@pytest.mark.parametrize("eta_kind", ["scalar", "head", "token"])
def test_chunked_small(ttt, nchunks, eta_kind):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=3, T=256, eta_kind=eta_kind, eta_value=1.0 / 64, seed=40 + nchunks)
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, wf = ttt.linear_fwd_chunked(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16, nchunks)
    zp, wp = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    torch.cuda.synchronize()
    zr, wr = oracle.run_inputs(inp)
    parity(f"chunked n={nchunks} {eta_kind}", [("Z", rows(z), zr), ("W_final", rows(wf), wr)], CONTRACT_BF16,
           REGRESS_MFMA)
    print(f"chunked n={nchunks} {eta_kind}: vs plain Z {max_rel(rows(z), rows(zp)):.3e}", flush=True)
    assert max_rel(rows(z), rows(zp)) < 1e-4 and max_rel(rows(wf), rows(wp)) < 1e-4


def test_chunked_long_config(ttt):
    """The long workload (64 chains x 2,048 mini-batches) with 5 chunks (the
    benchmark's split: chunk 0 a little longer) and 8, every chain against the
    oracle."""
    cfg = ti.CONFIGS["long"]
    inp = ti.generate(cfg)
    t = to_device(inp)
    ch = np.arange(cfg.chains)
    zr, wr = oracle.run_inputs(inp)
    for n in (5, 8):
        z, wf = ttt.linear_fwd_chunked(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16, n)
        torch.cuda.synchronize()
        parity(f"chunked long ({n} chunks)", [("Z", rows(z, ch), zr), ("W_final", rows(wf, ch), wr)],
               CONTRACT_BF16, REGRESS_MFMA)


def test_chunked_inplace_state_and_workspace_reuse(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=128, seed=43)
    inp = ti.generate(cfg)
    t = to_device(inp)
    ref_z, ref_w = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    state = t["w1"].unsqueeze(0).expand(2, -1, -1, -1).contiguous()
    ws = torch.empty(ttt.linear_chunked_workspace_bytes(2, 2, 128, 64, 16, 4), dtype=torch.uint8, device="cuda:0")
    ws.fill_(0xFF)  # garbage in the workspace must not matter
    z, _ = ttt.linear_fwd_chunked(t["q"], t["k"], t["v"], state, t["eta"], 16, 4, workspace=ws, w_final=state)
    torch.cuda.synchronize()
    assert max_rel(rows(z), rows(ref_z)) < 1e-4 and max_rel(rows(state), rows(ref_w)) < 1e-4


def test_chunked_errors(ttt):
    x = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda:0")
    w0 = torch.zeros((2, 64, 64), device="cuda:0")
    with pytest.raises(ttt.TTTError) as ei:                      # 8 chunks, 4 mini-batches
        ttt.linear_fwd_chunked(x, x, x, w0, 0.1, 16, 8)
    assert ei.value.status == 2
    small = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_fwd_chunked(x, x, x, w0, 0.1, 16, 2, workspace=small)
    assert ei.value.status == 11
    xf = torch.zeros((1, 2, 64, 64), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ttt.TTTError) as ei:                      # fp32 inputs: no MFMA path
        ttt.linear_fwd_chunked(xf, xf, xf, w0, 0.1, 16, 2)
    assert ei.value.status == 4
