"""The seeded input generator: determinism, bf16 rounding, distributions, chain subsets."""
import hashlib

import numpy as np
import pytest
import torch

import ttt_inputs as ti


def _digest(inp):
    h = hashlib.sha256()
    for a in (inp.q, inp.k, inp.v, inp.w1, inp.eta_buf):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_deterministic():
    cfg = ti.CONFIGS["tiny"]
    assert _digest(ti.generate(cfg)) == _digest(ti.generate(cfg))
    other = ti.generate(cfg.with_(seed=cfg.seed + 1))
    assert _digest(other) != _digest(ti.generate(cfg))


def test_bf16_round_matches_torch_rne():
    r = np.random.default_rng(0)
    x = (r.standard_normal(100000) * 10.0 ** r.integers(-6, 6, 100000)).astype(np.float32)
    # exact ties: low 16 bits = 0x8000, both parities of the kept bit
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, 1.0, 3.0e38], np.float32)])
    vals, bits = ti.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16)
    np.testing.assert_array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(vals, ref.float().numpy())


def test_bf16_values_are_representable():
    inp = ti.generate(ti.CONFIGS["l125m"], chains=[0, 5])
    for a in (inp.q, inp.k, inp.v):
        assert np.all(a.view(np.uint32) & 0xFFFF == 0)
    assert inp.bits("q").dtype == np.uint16


@pytest.mark.parametrize("name", ["l125m", "l1p3b", "mlp"])
def test_distributions(name):
    cfg = ti.CONFIGS[name]
    inp = ti.generate(cfg, chains=ti.sample_chains(cfg, 4))
    for a in (inp.q, inp.k, inp.v):
        assert abs(a.std() * np.sqrt(cfg.d) - 1.0) < 0.02
        assert abs(a.mean()) < 0.01
    assert abs(inp.w1.std() / 0.02 - 1.0) < 0.05
    if cfg.is_mlp:
        assert inp.w1.shape == (cfg.H, cfg.dh, cfg.d) and inp.w2.shape == (cfg.H, cfg.d, cfg.dh)
    else:
        assert inp.w1.shape == (cfg.H, cfg.d, cfg.d) and inp.w2 is None
    eta = inp.eta_rows()
    assert eta.shape == (len(inp.chains), cfg.T)
    if cfg.eta_kind == "token":
        assert eta.min() > 0 and eta.max() < 1.0 / cfg.d
        assert abs(eta.mean() * cfg.d - 0.5) < 0.01
    else:
        assert np.all(eta == np.float32(cfg.eta_value))


def test_chain_subset_matches_full():
    cfg = ti.CONFIGS["l1p3b"].with_(T=64, B=2, H=3)
    full = ti.generate(cfg)
    sub = ti.generate(cfg, chains=[1, 4])
    np.testing.assert_array_equal(sub.q, full.q[[1, 4]])
    np.testing.assert_array_equal(sub.v, full.v[[1, 4]])
    np.testing.assert_array_equal(sub.eta_rows(), full.eta_rows()[[1, 4]])
    np.testing.assert_array_equal(sub.w_rows(), full.w_rows()[[1, 4]])


def test_eta_strides():
    cfg = ti.CONFIGS["l1p3b"].with_(T=8, B=2, H=3)
    inp = ti.generate(cfg)
    assert inp.eta_strides == (3 * 8, 8, 1)
    np.testing.assert_array_equal(inp.eta_chain(4), inp.eta_buf[32:40])
    assert ti.generate(ti.CONFIGS["l125m"].with_(T=16), chains=[0]).eta_strides == (0, 1, 0)
    assert ti.generate(ti.CONFIGS["tiny"]).eta_strides == (0, 0, 0)
    assert ti.generate(ti.CONFIGS["tiny"]).eta_buf[0] == np.float32(0.1)


def test_sample_chains():
    cfg = ti.CONFIGS["l1p3b"]
    s = ti.sample_chains(cfg, 32)
    assert len(s) == 32 and s[0] == 0 and s[-1] == cfg.chains - 1
    assert np.all(np.diff(s) > 0)
    np.testing.assert_array_equal(s, ti.sample_chains(cfg, 32))
