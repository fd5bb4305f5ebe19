"""Seeded synthetic inputs for the TTT-Linear / TTT-MLP forward pass.

This module is shared by the fp64 oracle (``oracle/``) and by the HIP path's
tests and benchmark.  It holds none of the method's arithmetic: it only draws
random numbers, rounds them to the storage dtype and lays them out.

Workloads (the layer shapes of the TTT article's 125M / 1.3B language models,
its long-context runs, and the TTT-MLP variant; the pages are
[TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer",
aharts.cn / itmax.cn, part 04 "experiments" §1-§3):

  name    B   H   d   dh   T      b   Q/K/V dtype  eta
  tiny    1   1   16  -    64     4   fp32         scalar fp32(0.1)
  l125m   8   12  64  -    2048   16  bf16         per head, 1/d
  l1p3b   16  32  64  -    8192   16  bf16         per token, fp32(sigmoid(g)/d), g ~ N(0,1)
  long    2   32  64  -    32768  16  bf16         scalar 1/d
  mlp     16  32  64  256  2048   16  bf16         scalar 1/d

Recipe (identical bits on both sides):
  * Every random tensor of every (batch, head) chain has its own PCG64 stream,
    seeded by SeedSequence(seed, spawn_key=(tensor_id, index)), so a subset of
    chains can be regenerated without drawing the rest.
  * Q, K, V ~ N(0, 1/d) (variance 1/d, so |k|^2 ~ 1), drawn in fp64, cast to
    fp32, then (bf16 configs) rounded to bf16 with round-to-nearest-even.
  * W0 (or W1, W2) ~ N(0, 0.02^2) per head, fp64 -> fp32.  W0 is [H, d, d],
    row-major, shared by every sequence of the batch; z = W q.
  * eta as listed; per-token g ~ N(0, 1) per chain, eta = fp32(sigmoid(g)/d).
  * Backward: upstream gradients dZ ~ N(0, 1) per element ([n, T, d], fp32,
    or rounded to bf16) and dW_final ~ N(0, 1) ([n, d, d], fp32), each chain
    with its own stream as above.

Layouts: Q, K, V are [B, H, T, d] (token-major).  eta is described by a
buffer plus element strides (stride_b, stride_h, stride_t).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

# tensor ids used in the stream keys
_TID_Q, _TID_K, _TID_V, _TID_W1, _TID_W2, _TID_G = 0, 1, 2, 3, 4, 5
_TID_DZ, _TID_DWF = 6, 7


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    d: int
    T: int
    b: int
    dtype: str              # "fp32" or "bf16" (storage dtype of Q, K, V)
    eta_kind: str           # "scalar", "head", "token"
    eta_value: float = 0.0  # for scalar / head kinds (stored as fp32)
    seed: int = 0
    dh: int = 0             # hidden width for the MLP variant, 0 = TTT-Linear

    @property
    def is_mlp(self) -> bool:
        return self.dh > 0

    @property
    def chains(self) -> int:
        return self.B * self.H

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": Config("tiny", 1, 1, 16, 64, 4, "fp32", "scalar", 0.1, seed=1001),
    "l125m": Config("l125m", 8, 12, 64, 2048, 16, "bf16", "head", 1.0 / 64, seed=1002),
    "l1p3b": Config("l1p3b", 16, 32, 64, 8192, 16, "bf16", "token", seed=1003),
    "long": Config("long", 2, 32, 64, 32768, 16, "bf16", "scalar", 1.0 / 64, seed=1004),
    "mlp": Config("mlp", 16, 32, 64, 2048, 16, "bf16", "scalar", 1.0 / 64, seed=1005, dh=256),
}


def bf16_round(x: np.ndarray):
    """Round fp32 values to bf16, round-to-nearest-even.

    Returns (values as fp32, raw bf16 bits as uint16).  Inputs are finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    hi = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    vals = (hi.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return vals, hi


def _rng(seed: int, tid: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tid, index))))


def _qkv_chain(cfg: Config, tid: int, chain: int) -> np.ndarray:
    std = 1.0 / np.sqrt(cfg.d)
    x = (_rng(cfg.seed, tid, chain).standard_normal((cfg.T, cfg.d)) * std).astype(np.float32)
    if cfg.dtype == "bf16":
        x, _ = bf16_round(x)
    return x


def _eta_token_chain(cfg: Config, chain: int) -> np.ndarray:
    g = _rng(cfg.seed, _TID_G, chain).standard_normal(cfg.T)
    return (1.0 / (1.0 + np.exp(-g)) / cfg.d).astype(np.float32)


@dataclasses.dataclass
class Inputs:
    """Inputs of one workload, as fp32 arrays holding exactly the stored values.

    q, k, v : [n, T, d] for the selected chains (n = B*H when all chains)
    chains  : the flat chain ids (bi*H + h) these rows belong to
    w1      : [H, dh or d, d] fp32 (W0 for TTT-Linear)
    w2      : [H, d, dh] fp32 or None
    eta_buf : 1-D fp32 buffer addressed by eta_strides (elements)
    eta_strides : (stride_b, stride_h, stride_t)
    """
    cfg: Config
    chains: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    w1: np.ndarray
    w2: Optional[np.ndarray]
    eta_buf: np.ndarray
    eta_strides: tuple

    def eta_chain(self, chain: int) -> np.ndarray:
        """eta for every token of one chain (length T), read through the strides."""
        bi, h = divmod(int(chain), self.cfg.H)
        sb, sh, st = self.eta_strides
        idx = bi * sb + h * sh + np.arange(self.cfg.T) * st
        return self.eta_buf[idx]

    def eta_rows(self) -> np.ndarray:
        """[n, T] eta for the selected chains."""
        return np.stack([self.eta_chain(c) for c in self.chains]) if len(self.chains) else \
            np.zeros((0, self.cfg.T), np.float32)

    def w_rows(self, which: int = 1) -> np.ndarray:
        """Initial weights expanded to the selected chains: [n, ...]."""
        w = self.w1 if which == 1 else self.w2
        heads = np.asarray(self.chains) % self.cfg.H
        return w[heads]

    def bits(self, name: str) -> np.ndarray:
        """bf16 bits (uint16) of q/k/v for a bf16 config."""
        assert self.cfg.dtype == "bf16"
        return bf16_round(getattr(self, name))[1]


def generate(cfg: Config, chains: Optional[Sequence[int]] = None) -> Inputs:
    """Draw the inputs of ``cfg`` for ``chains`` (default: all B*H chains)."""
    if chains is None:
        chains = np.arange(cfg.chains)
    chains = np.asarray(chains, dtype=np.int64)
    n, T, d = len(chains), cfg.T, cfg.d
    q = np.empty((n, T, d), np.float32)
    k = np.empty((n, T, d), np.float32)
    v = np.empty((n, T, d), np.float32)
    for i, c in enumerate(chains):
        q[i] = _qkv_chain(cfg, _TID_Q, int(c))
        k[i] = _qkv_chain(cfg, _TID_K, int(c))
        v[i] = _qkv_chain(cfg, _TID_V, int(c))
    rows = cfg.dh if cfg.is_mlp else d
    w1 = np.stack([(_rng(cfg.seed, _TID_W1, h).standard_normal((rows, d)) * 0.02).astype(np.float32)
                   for h in range(cfg.H)])
    w2 = None
    if cfg.is_mlp:
        w2 = np.stack([(_rng(cfg.seed, _TID_W2, h).standard_normal((d, cfg.dh)) * 0.02).astype(np.float32)
                       for h in range(cfg.H)])
    if cfg.eta_kind == "scalar":
        eta_buf = np.array([cfg.eta_value], np.float32)
        strides = (0, 0, 0)
    elif cfg.eta_kind == "head":
        eta_buf = np.full(cfg.H, cfg.eta_value, np.float32)
        strides = (0, 1, 0)
    elif cfg.eta_kind == "token":
        # only the selected chains are drawn; the others stay zero
        eta_buf = np.zeros(cfg.B * cfg.H * T, np.float32)
        for c in chains:
            eta_buf[int(c) * T:(int(c) + 1) * T] = _eta_token_chain(cfg, int(c))
        strides = (cfg.H * T, T, 1)
    else:
        raise ValueError(cfg.eta_kind)
    return Inputs(cfg, chains, q, k, v, w1, w2, eta_buf, strides)


def upstream_grads(cfg: Config, chains: Optional[Sequence[int]] = None, dtype: str = "fp32",
                   dwf_scale: float = 1.0):
    """Seeded gradients of a loss with respect to Z and W_final, for the backward.

    returns (dz [n, T, d] fp32 holding the stored values -- bf16-rounded when
    dtype == "bf16" --, dwf [n, d, d] fp32 scaled by dwf_scale).
    """
    if chains is None:
        chains = np.arange(cfg.chains)
    chains = np.asarray(chains, dtype=np.int64)
    n, T, d = len(chains), cfg.T, cfg.d
    dz = np.empty((n, T, d), np.float32)
    dwf = np.empty((n, d, d), np.float32)
    for i, c in enumerate(chains):
        x = _rng(cfg.seed, _TID_DZ, int(c)).standard_normal((T, d)).astype(np.float32)
        dz[i] = bf16_round(x)[0] if dtype == "bf16" else x
        dwf[i] = (_rng(cfg.seed, _TID_DWF, int(c)).standard_normal((d, d)) * dwf_scale).astype(np.float32)
    return dz, dwf


def sample_chains(cfg: Config, count: int, seed: int = 7) -> np.ndarray:
    """A fixed, sorted sample of chain ids (always includes the first and last chain)."""
    n = cfg.chains
    if count >= n:
        return np.arange(n)
    rng = np.random.Generator(np.random.PCG64(seed))
    pick = set(rng.choice(n, size=max(count - 2, 0), replace=False).tolist())
    pick.update({0, n - 1})
    return np.array(sorted(pick), dtype=np.int64)


def to_device(inp: Inputs, device="cuda:0", dtype: Optional[str] = None) -> dict:
    """Upload a full-chain Inputs: dict(q, k, v, w1, w2, eta) of torch tensors.

    Q, K, V are [B, H, T, d] in the storage dtype (the exact bits the oracle
    reads); eta is shaped to match its strides: [1], [H] or [B, H, T].
    """
    import torch

    cfg = inp.cfg
    assert len(inp.chains) == cfg.chains and np.all(inp.chains == np.arange(cfg.chains))
    shape = (cfg.B, cfg.H, cfg.T, cfg.d)
    dtype = dtype or cfg.dtype

    def qkv(x):
        if dtype == "bf16":
            bits = bf16_round(x)[1]
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).reshape(shape).to(device)
        return torch.from_numpy(np.ascontiguousarray(x)).reshape(shape).to(device)

    out = dict(q=qkv(inp.q), k=qkv(inp.k), v=qkv(inp.v),
               w1=torch.from_numpy(inp.w1).to(device),
               w2=None if inp.w2 is None else torch.from_numpy(inp.w2).to(device))
    strides = tuple(inp.eta_strides)
    if strides == (0, 0, 0):
        out["eta"] = torch.from_numpy(inp.eta_buf[:1].copy()).to(device)
    elif strides == (0, 1, 0):
        out["eta"] = torch.from_numpy(inp.eta_buf.copy()).to(device)
    else:
        out["eta"] = torch.from_numpy(inp.eta_buf.reshape(cfg.B, cfg.H, cfg.T).copy()).to(device)
    return out
