"""Every entry point runs on the stream it is given: torch's current stream by
default (so `with torch.cuda.stream(s)` works), or an explicit ``stream=``.
Results on a side stream equal the default stream's bit for bit, including
when the inputs are produced on that side stream just before the call."""
import pytest

import ttt_inputs as ti
from ttt_testutil import to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ttt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import test_sequence_layer_amd as m
    m.lib()
    return m


def test_forward_on_side_stream(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=4, T=256, eta_kind="token", seed=120)
    t = to_device(ti.generate(cfg))
    z0, w0 = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(s):
        # inputs made on the side stream right before the call: the call must be
        # ordered after them on that stream
        q = t["q"].clone()
        z1, w1 = ttt.linear_fwd(q, t["k"], t["v"], t["w1"], t["eta"], 16)
    s.synchronize()
    assert torch.equal(z0, z1) and torch.equal(w0, w1)
    # the explicit argument
    z2 = torch.empty_like(z0)
    w2 = torch.empty_like(w0)
    with torch.cuda.stream(s):
        k = t["k"].clone()
    ttt.linear_fwd(t["q"], k, t["v"], t["w1"], t["eta"], 16, z=z2, w_final=w2, stream=s)
    s.synchronize()
    assert torch.equal(z0, z2) and torch.equal(w0, w2)


def test_mlp_layer_norm_and_backward_on_side_stream(ttt):
    s = torch.cuda.Stream()
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=64, seed=121)
    t = to_device(ti.generate(cfg))
    g = torch.ones((2, 64), device="cuda:0")
    b = torch.zeros((2, 64), device="cuda:0")
    ref = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16)
    ref_ln = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], g, b, t["eta"], 16)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16)
        out_ln = ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], g, b, t["eta"], 16)
    s.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(ref, out))
    assert all(torch.equal(x, y) for x, y in zip(ref_ln, out_ln))

    cfg = ti.CONFIGS["l1p3b"].with_(B=1, H=3, T=128, seed=122)
    t = to_device(ti.generate(cfg))
    z, wf, e = ttt.linear_fwd_save(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    dz = torch.randn_like(z)
    ref = ttt.linear_bwd(t["q"], t["k"], t["eta"], wf, e, dz, 16)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        got = ttt.linear_bwd(t["q"], t["k"], t["eta"], wf, e, dz, 16)
    s.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(ref, got))


def test_decode_on_side_stream(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=32, seed=123)
    t = to_device(ti.generate(cfg))

    def run(stream):
        w = t["w1"].unsqueeze(0).expand(2, -1, -1, -1).contiguous()
        wb = w.clone()
        zs = []
        for i in range(cfg.T):
            sl = lambda x: x[:, :, i:i + 1].contiguous()  # noqa: E731
            zs.append(ttt.linear_decode(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["eta"]), w, wb, i, 16,
                                        stream=stream))
        return torch.cat(zs, dim=2), w

    z0, w0 = run(None)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    z1, w1 = run(s)
    s.synchronize()
    assert torch.equal(z0, z1) and torch.equal(w0, w1)


def test_mlp_backward_on_side_stream(ttt):
    """ttt_mlp_bwd (dual form: two launches) on a side stream, after inputs made on it."""
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=2, T=32, seed=150)
    t = to_device(ti.generate(cfg))
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(151)
    dz = torch.randn((2, 2, 32, 64), generator=gen, device="cuda:0")
    ref = ttt.mlp_bwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16, dz)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(s):
        dz2 = dz.clone()
        got = ttt.mlp_bwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16, dz2)
    s.synchronize()
    for x, r in zip(got, ref):
        assert torch.equal(x, r)
