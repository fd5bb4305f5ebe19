"""GPU test of ttt_linear_fwd_chunked_noalloc, the chunked TTT-Linear forward
for callers that cannot allocate: its maps and start states live in the
library's static device scratch instead of a caller workspace.

Two calls in a row, the second with a smaller input (so the scratch still
holds the first call's maps), each checked bit for bit against
ttt_linear_fwd_chunked with a workspace (the same kernels), and against the
fp64 oracle on sampled chains at the parity bar (2e-3 for bf16 inputs).
"""
import numpy as np
import pytest

import oracle
import ttt_inputs as ti
from ttt_testutil import CONTRACT_BF16, REGRESS_MFMA, parity, rows, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import test_sequence_layer_amd as m
    m.lib()
    return m


def _case(ttt, cfg, nchunks):
    inp = ti.generate(cfg)
    t = to_device(inp)
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    z = torch.full((B, H, T, d), float("nan"), device="cuda:0")
    wf = torch.full((B, H, d, d), float("nan"), device="cuda:0")
    print(f"noalloc: {cfg.name} B{B} H{H} T{T} eta {cfg.eta_kind}, {nchunks} chunks", flush=True)
    ttt.linear_fwd_chunked_noalloc(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, nchunks, z=z, w_final=wf)
    zr, wr = ttt.linear_fwd_chunked(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, nchunks)
    torch.cuda.synchronize()
    assert torch.equal(z, zr) and torch.equal(wf, wr)
    ch = ti.sample_chains(cfg, 4)
    zo, wo = oracle.run_inputs(ti.generate(cfg, chains=ch))
    parity("noalloc vs oracle", [("Z", rows(z, ch), zo), ("W_final", rows(wf, ch), wo)], CONTRACT_BF16, REGRESS_MFMA)


def test_noalloc_two_calls_second_smaller(ttt):
    big = ti.CONFIGS["long"].with_(B=1, H=32, T=8192, eta_kind="token", seed=71)
    small = ti.CONFIGS["long"].with_(B=1, H=6, T=1024, seed=72)
    assert ttt.linear_chunked_workspace_bytes(1, 32, 8192, 64, 16, 8) <= ttt.NOALLOC_SCRATCH_BYTES
    _case(ttt, big, 8)
    _case(ttt, small, 4)


def test_noalloc_rejects_more_than_the_scratch(ttt):
    x = torch.zeros((16, 32, 64, 64), dtype=torch.bfloat16, device="cuda:0")
    w0 = torch.zeros((32, 64, 64), device="cuda:0")
    assert ttt.linear_chunked_workspace_bytes(16, 32, 64, 64, 16, 4) > ttt.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ttt.TTTError) as ei:
        ttt.linear_fwd_chunked_noalloc(x, x, x, w0, 0.1, 16, 4)
    assert ei.value.status == 12
