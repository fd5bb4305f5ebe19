"""GPU tests of the row-block split of the matrix-core TTT-Linear forward.

Rows of W evolve independently (row i of the next state and of Z needs only
row i of W, column i of V and all of K, Q, eta), so one (sequence, head) may be
computed by 1, 2 or 4 workgroups of 64, 32 or 16 rows.  Every row goes through
the same arithmetic whichever workgroup holds it, so the three counts must
agree bit for bit -- a row or column placed in the wrong block, a V column
staged from the wrong offset or a Z piece written to the wrong place changes
values -- and each must match the fp64 oracle (2e-3, bf16 inputs).
"""
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


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


# (B, H): 6 and 11 units leave a last group of fewer than 8 (the XCD packing's
# ragged case), 16 fills two groups exactly
@pytest.mark.parametrize("B,H,T,eta_kind", [(2, 3, 112, "token"), (1, 11, 80, "scalar"), (4, 4, 64, "head")])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_row_blocks_agree_and_match_oracle(ttt, B, H, T, eta_kind, out_dtype):
    cfg = ti.CONFIGS["l1p3b"].with_(B=B, H=H, T=T, eta_kind=eta_kind, eta_value=1.0 / 64, seed=60 + T + H)
    inp = ti.generate(cfg)
    t = to_device(inp)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    res = {}
    for r in (1, 2, 4):
        assert ttt.linear_kernel_name(B, H, T, 64, 16, eta_strides=inp.eta_strides, rows=r).startswith(
            "ttt_linear_mfma_d64b16")
        res[r] = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16, out_dtype=od, rows=r)
    torch.cuda.synchronize()
    zr, wr = oracle.run_inputs(inp)
    bf = out_dtype != "f32"
    tol = 2.0 ** -8 + 2e-4 if bf else CONTRACT_BF16  # bf16 Z: its own rounding, up to 2^-8 relative
    for r, (z, wf) in res.items():
        lab = f"rows={r} B{B} H{H} T{T} {eta_kind} {out_dtype}"
        parity(lab, [("W_final", rows(wf), wr)], CONTRACT_BF16, REGRESS_MFMA)
        parity(lab, [("Z", rows(z), zr)], tol, None if bf else REGRESS_MFMA)
    assert _same(res[1], res[2]) and _same(res[1], res[4])


def test_row_blocks_default_is_one(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=3, T=96, seed=71)
    inp = ti.generate(cfg)
    t = to_device(inp)
    assert ttt.linear_kernel_name(2, 3, 96, 64, 16, eta_strides=inp.eta_strides) == "ttt_linear_mfma_d64b16"
    a = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    b = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16, rows=4)
    torch.cuda.synchronize()
    assert _same(a, b)


@pytest.mark.parametrize("rows_", [2, 4])
def test_row_blocks_save_for_backward(ttt, rows_):
    cfg = ti.CONFIGS["l1p3b"].with_(B=1, H=5, T=128, seed=72)
    inp = ti.generate(cfg)
    t = to_device(inp)
    ref = ttt.linear_fwd_save(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16, rows=1)
    got = ttt.linear_fwd_save(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16, rows=rows_)
    torch.cuda.synchronize()
    assert _same(ref, got)


@pytest.mark.parametrize("nchunks", [2, 5])
@pytest.mark.parametrize("rows_", [1, 2, 4])
def test_row_blocks_chunked(ttt, nchunks, rows_):
    cfg = ti.CONFIGS["l1p3b"].with_(B=1, H=3, T=160, eta_kind="token", seed=73 + nchunks)
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, wf = ttt.linear_fwd_chunked(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16, nchunks, rows=rows_)
    z1, w1 = ttt.linear_fwd_chunked(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16, nchunks, rows=1)
    torch.cuda.synchronize()
    zr, wr = oracle.run_inputs(inp)
    parity(f"chunked n={nchunks} rows={rows_}", [("Z", rows(z), zr), ("W_final", rows(wf), wr)], CONTRACT_BF16,
           REGRESS_MFMA)
    assert torch.equal(z, z1) and torch.equal(wf, w1)


def test_row_blocks_long_config_sampled(ttt):
    # the long shape (64 chains x 2,048 mini-batches) with 2 and 4 row blocks
    cfg = ti.CONFIGS["long"]
    inp = ti.generate(cfg)
    t = to_device(inp)
    z, wf = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, rows=2)
    torch.cuda.synchronize()
    ch = ti.sample_chains(cfg, 3)
    zr, wr = oracle.run_inputs(ti.generate(cfg, chains=ch))
    parity(f"long rows=2 chains {list(ch)}", [("Z", rows(z, ch), zr), ("W_final", rows(wf, ch), wr)],
           CONTRACT_BF16, REGRESS_MFMA)
    z4, w4 = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, rows=4)
    torch.cuda.synchronize()
    assert torch.equal(z, z4) and torch.equal(wf, w4)


def test_row_blocks_inplace_carry(ttt):
    # W_final == W0 (per-sequence state carried in place) with 4 row blocks:
    # each block reads its own rows of W0 before it writes them
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=64, seed=74)
    inp = ti.generate(cfg)
    t = to_device(inp)
    w = t["w1"].unsqueeze(0).expand(cfg.B, -1, -1, -1).contiguous()
    ref = ttt.linear_fwd(t["q"], t["k"], t["v"], w.clone(), t["eta"], 16, rows=1)
    z, wf = ttt.linear_fwd(t["q"], t["k"], t["v"], w, t["eta"], 16, w_final=w, rows=4)
    torch.cuda.synchronize()
    assert wf.data_ptr() == w.data_ptr()
    assert torch.equal(z, ref[0]) and torch.equal(w, ref[1])
