"""The entry points allocate nothing and only launch kernels on the caller's
stream, so they can be captured in a HIP graph.  Each test captures calls on a
side stream, replays the graph several times with eager work and
synchronisations in between, and checks every replay against the eager
result, bit for bit."""
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


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the graph (first-call setup)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def test_forward_graph_replays(ttt):
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=4, T=256, eta_kind="token", seed=130)
    t = to_device(ti.generate(cfg))
    z_ref, w_ref = ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16)
    zl_ref, wl_ref = ttt.linear_ln_fwd(t["q"], t["k"], t["v"], t["w1"], torch.ones((4, 64), device="cuda:0"),
                                       torch.zeros((4, 64), device="cuda:0"), t["eta"], 16)
    z, w = torch.empty_like(z_ref), torch.empty_like(w_ref)
    zl, wl = torch.empty_like(zl_ref), torch.empty_like(wl_ref)
    g1 = torch.ones((4, 64), device="cuda:0")
    b1 = torch.zeros((4, 64), device="cuda:0")

    def calls():
        ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], 16, z=z, w_final=w)
        ttt.linear_ln_fwd(t["q"], t["k"], t["v"], t["w1"], g1, b1, t["eta"], 16, z=zl, w_final=wl)

    g = _capture(calls)
    for i in range(3):
        for x in (z, w, zl, wl):
            x.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(z, z_ref) and torch.equal(w, w_ref), f"replay {i}"
        assert torch.equal(zl, zl_ref) and torch.equal(wl, wl_ref), f"replay {i}"


def test_mlp_and_chunked_graph_replays(ttt):
    cfg = ti.CONFIGS["mlp"].with_(B=1, H=2, T=64, seed=131)
    t = to_device(ti.generate(cfg))
    ref = ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16)
    out = [torch.empty_like(x) for x in ref]
    cfg2 = ti.CONFIGS["l1p3b"].with_(B=1, H=3, T=256, seed=132)
    t2 = to_device(ti.generate(cfg2))
    zc_ref, wc_ref = ttt.linear_fwd_chunked(t2["q"], t2["k"], t2["v"], t2["w1"], t2["eta"], 16, 4)
    ws = torch.empty(ttt.linear_chunked_workspace_bytes(1, 3, 256, 64, 16, 4), dtype=torch.uint8, device="cuda:0")
    zc, wc = torch.empty_like(zc_ref), torch.empty_like(wc_ref)

    def calls():
        ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16, z=out[0], w1_final=out[1],
                    w2_final=out[2])
        ttt.linear_fwd_chunked(t2["q"], t2["k"], t2["v"], t2["w1"], t2["eta"], 16, 4, workspace=ws, z=zc,
                               w_final=wc)

    g = _capture(calls)
    for i in range(3):
        for x in out + [zc, wc, ws]:
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(out, ref)), f"replay {i}"
        assert torch.equal(zc, zc_ref) and torch.equal(wc, wc_ref), f"replay {i}"


def test_decode_graph_replays(ttt):
    """A graph of one mini-batch of one-token decode calls (positions 0..15),
    replayed twice, continues the state exactly as the same calls made eagerly
    twice."""
    cfg = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=16, eta_kind="token", seed=133)
    t = to_device(ti.generate(cfg))
    toks = [tuple(x[:, :, i:i + 1].contiguous() for x in (t["q"], t["k"], t["v"], t["eta"])) for i in range(16)]
    w0 = t["w1"].unsqueeze(0).expand(2, -1, -1, -1).contiguous()

    def calls(w, wb, z):
        for i in range(16):
            ttt.linear_decode(*toks[i], w, wb, i, 16, z=z[i])

    w_e, wb_e = w0.clone(), w0.clone()
    z_e = [torch.empty((2, 2, 1, 64), device="cuda:0") for _ in range(16)]
    zs = []
    for _ in range(2):
        calls(w_e, wb_e, z_e)
        zs.append(torch.cat(z_e, dim=2))
    torch.cuda.synchronize()

    w_g, wb_g = w0.clone(), w0.clone()
    z_g = [torch.empty((2, 2, 1, 64), device="cuda:0") for _ in range(16)]
    g = _capture(lambda: calls(w_g, wb_g, z_g))
    # the warm-up inside _capture ran the calls once already: start over
    w_g.copy_(w0)
    wb_g.copy_(w0)
    torch.cuda.synchronize()
    for r in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.cat(z_g, dim=2), zs[r]), f"replay {r}"
    assert torch.equal(w_g, w_e) and torch.equal(wb_g, wb_e)


def test_layer_norm_decode_graph_replays(ttt):
    """The same for the layer-norm decode entry points of TTT-Linear and
    TTT-MLP, captured together in one graph of 16 one-token calls each."""
    dev = "cuda:0"
    cl = ti.CONFIGS["l1p3b"].with_(B=2, H=2, T=16, eta_kind="token", seed=134)
    cm = ti.CONFIGS["mlp"].with_(B=2, H=2, T=16, seed=135)
    tl, tm = to_device(ti.generate(cl)), to_device(ti.generate(cm))
    g = torch.Generator(device="cpu").manual_seed(7)
    gam = (1.0 + 0.2 * torch.randn((2, 64), generator=g)).to(dev)
    bet = (0.1 * torch.randn((2, 64), generator=g)).to(dev)
    lt = [tuple(x[:, :, i:i + 1].contiguous() for x in (tl["q"], tl["k"], tl["v"], tl["eta"])) for i in range(16)]
    mt = [tuple(x[:, :, i:i + 1].contiguous() for x in (tm["q"], tm["k"], tm["v"])) for i in range(16)]
    w0 = tl["w1"].unsqueeze(0).expand(2, -1, -1, -1).contiguous()
    m1 = tm["w1"].unsqueeze(0).expand(2, -1, -1, -1).contiguous()
    m2 = tm["w2"].unsqueeze(0).expand(2, -1, -1, -1).contiguous()

    def calls(s, zl, zm):
        w, wb, a1, a2, a1b, a2b = s
        for i in range(16):
            ttt.linear_ln_decode(*lt[i], gam, bet, w, wb, i, 16, z=zl[i])
            ttt.mlp_decode(*mt[i], tm["eta"], a1, a2, a1b, a2b, i, 16, z=zm[i], ln=(gam, bet, 1e-6))

    def fresh():
        return [w0.clone(), w0.clone(), m1.clone(), m2.clone(), m1.clone(), m2.clone()]

    def outs():
        return ([torch.empty((2, 2, 1, 64), device=dev) for _ in range(16)],
                [torch.empty((2, 2, 1, 64), device=dev) for _ in range(16)])

    s_e, (zl_e, zm_e) = fresh(), outs()
    ref = []
    for _ in range(2):
        calls(s_e, zl_e, zm_e)
        ref.append((torch.cat(zl_e, dim=2), torch.cat(zm_e, dim=2)))
    torch.cuda.synchronize()

    s_g, (zl_g, zm_g) = fresh(), outs()
    graph = _capture(lambda: calls(s_g, zl_g, zm_g))
    for x, x0 in zip(s_g, fresh()):   # the warm-up inside _capture ran the calls once: start over
        x.copy_(x0)
    torch.cuda.synchronize()
    for r in range(2):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.cat(zl_g, dim=2), ref[r][0]), f"linear, replay {r}"
        assert torch.equal(torch.cat(zm_g, dim=2), ref[r][1]), f"mlp, replay {r}"
    assert all(torch.equal(a, b) for a, b in zip(s_g, s_e))


@pytest.mark.parametrize("primal", [False, True])
def test_mlp_backward_graph_replays(ttt, primal):
    """ttt_mlp_bwd: the dual form's two launches (checkpointing forward, reverse
    pass) and the primal form's one, with the caller's workspace."""
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=2, T=64, eta_kind="token", seed=140)
    t = to_device(ti.generate(cfg))
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(141)
    dz = torch.randn((2, 2, 64, 64), generator=gen, device="cuda:0")
    d1 = torch.randn((2, 2, 256, 64), generator=gen, device="cuda:0")
    d2 = torch.randn((2, 2, 64, 256), generator=gen, device="cuda:0")
    ws = torch.empty(ttt.mlp_bwd_workspace_bytes(2, 2, 64, 64, 256, 16), dtype=torch.uint8, device="cuda:0")
    ref = ttt.mlp_bwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16, dz, d1, d2, workspace=ws,
                      primal=primal)
    torch.cuda.synchronize()
    out = tuple(torch.empty_like(x) for x in ref)

    def calls():
        ttt.mlp_bwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], 16, dz, d1, d2, workspace=ws, out=out,
                    primal=primal)

    g = _capture(calls)
    for i in range(3):
        for x in out:
            x.fill_(float("nan"))
        ws.fill_(255)  # the workspace holds nothing between calls
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("dq", "dk", "dv", "deta", "dw1", "dw2"), out, ref):
            assert torch.equal(x, r), f"replay {i}: {name}"
