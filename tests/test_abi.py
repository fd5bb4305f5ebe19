"""The C ABI without a GPU: libttt.so loads, exports every symbol include/ttt.h
declares, and its host-side validation returns the documented status codes.

Validation runs entirely on the host before any HIP call, so it is exercised
here through ttt_*_validate with fake (never dereferenced) device addresses.
"""
import ctypes
import os
import re
import subprocess

import pytest

import test_sequence_layer_amd as ttt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")

OK, NULL, SHAPE, DTYPE, UNSUP, ALIAS, ALIGN, HIP, STRIDE, FLAGS, POS, WORKSPACE, SCRATCH = range(13)
GB = 1 << 30


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ttt_[a-z_0-9]+)\s*\(", src, re.M)))


def test_header_and_binding_agree():
    assert sorted(ttt.EXPORTS) == _declared()


def test_library_exports_every_declared_symbol():
    L = ttt.lib()
    for sym in _declared():
        assert hasattr(L, sym), sym
    out = subprocess.run(["nm", "-D", "--defined-only", ttt.LIB_PATH], capture_output=True, text=True).stdout
    for sym in _declared():
        assert re.search(rf"\bT {sym}$", out, re.M), sym


def test_version_and_status_strings():
    assert ttt.abi_version() == 1
    for s in range(13):
        assert ttt.status_str(s) and ttt.status_str(s) != "unknown status"
    assert ttt.status_str(99) == "unknown status"


# ---- TTT-Linear validation -----------------------------------------------------

class Bufs:
    """Fake, well-separated, aligned device addresses for one problem."""

    def __init__(self):
        self.q, self.k, self.v = 1 * GB, 2 * GB, 3 * GB
        self.w0, self.eta, self.z, self.wf = 4 * GB, 5 * GB, 6 * GB, 7 * GB

    def args(self):
        return (self.q, self.k, self.v, self.w0, self.eta, self.z, self.wf)


def _desc(B=2, H=4, T=64, d=64, b=16, ind=1, outd=0, flags=0, wstride=0, est=(0, 0, 0)):
    return ttt.linear_desc(B, H, T, d, b, ind, outd, wstride, est, flags)


def _val(desc, bufs=None, **over):
    bufs = bufs or Bufs()
    for k, v in over.items():
        setattr(bufs, k, v)
    return ttt.lib().ttt_linear_validate(ctypes.byref(desc), *bufs.args())


def test_linear_ok():
    assert _val(_desc()) == OK
    assert _val(_desc(est=(4 * 64, 64, 1))) == OK
    assert _val(_desc(ind=0, d=16, b=4)) == OK


def test_linear_null():
    assert ttt.lib().ttt_linear_validate(None, *Bufs().args()) == NULL
    for name in ("q", "k", "v", "w0", "eta", "z", "wf"):
        assert _val(_desc(), **{name: None}) == NULL, name


def test_linear_empty_allows_null_tensors():
    assert _val(_desc(B=0), q=None, k=None, v=None, z=None, w0=None, wf=None, eta=None) == OK
    assert _val(_desc(T=0), q=None, k=None, v=None, z=None, eta=None) == OK
    assert _val(_desc(T=0), w0=None) == NULL


@pytest.mark.parametrize("kw", [dict(T=60), dict(b=0), dict(B=-1), dict(d=0), dict(T=-16)])
def test_linear_shape(kw):
    assert _val(_desc(**kw)) == SHAPE


def test_linear_dtype_flags_stride():
    assert _val(_desc(ind=2)) == DTYPE
    assert _val(_desc(outd=-1)) == DTYPE
    assert _val(_desc(flags=32)) == FLAGS
    assert _val(_desc(wstride=5)) == STRIDE
    assert _val(_desc(est=(0, -1, 0))) == STRIDE
    assert _val(_desc(wstride=4 * 64 * 64)) == OK


@pytest.mark.parametrize("kw", [dict(d=48), dict(d=128), dict(d=64, b=64), dict(d=16, b=65, T=130)])
def test_linear_unsupported(kw):
    assert _val(_desc(**kw)) == UNSUP


def test_linear_align():
    assert _val(_desc(), q=1 * GB + 8) == ALIGN
    assert _val(_desc(), wf=7 * GB + 4) == ALIGN
    assert _val(_desc(), eta=5 * GB + 2) == ALIGN
    assert _val(_desc(), eta=5 * GB + 4) == OK


def test_linear_alias():
    d = _desc()
    assert _val(d, z=1 * GB) == ALIAS                       # Z == Q
    assert _val(d, z=2 * GB + 4096) == ALIAS                # Z inside K
    assert _val(d, wf=3 * GB) == ALIAS                      # W_final == V
    assert _val(d, wf=4 * GB) == ALIAS                      # in place with a shared W0
    assert _val(_desc(wstride=4 * 64 * 64), wf=4 * GB) == OK      # in place, per-sequence W0
    assert _val(_desc(wstride=4 * 64 * 64), wf=4 * GB + 256) == ALIAS
    # Z directly after Q (no overlap) is fine: Q is 2*4*64*64*2 bytes
    assert _val(d, z=1 * GB + 2 * 4 * 64 * 64 * 2) == OK
    assert _val(d, z=1 * GB + 2 * 4 * 64 * 64 * 2 - 16) == ALIAS


def test_linear_row_block_flags():
    R1, R2, R4 = (ttt.TTT_FLAG_ROWS[r] for r in (1, 2, 4))
    for f in (R1, R2, R4):
        assert _val(_desc(flags=f)) == OK
    assert _val(_desc(flags=R1 | R2)) == FLAGS                       # at most one count
    assert _val(_desc(flags=R2 | R4)) == FLAGS
    assert _val(_desc(flags=R4 | ttt.TTT_FLAG_GENERIC)) == FLAGS
    assert _val(_desc(flags=R2 | ttt.TTT_FLAG_PRIMAL)) == FLAGS
    assert _val(_desc(flags=R4, ind=0, d=16, b=4)) == UNSUP           # matrix-core shapes only
    assert _val(_desc(flags=R2, ind=0)) == UNSUP
    # 2^29 sequence-heads x 4 row blocks: more workgroups than one launch takes
    assert _val(_desc(B=1 << 15, H=1 << 14, flags=R4)) == SHAPE
    with pytest.raises(ValueError):
        ttt.linear_kernel_name(1, 1, 64, 64, 16, rows=3)


def test_linear_row_block_choice():
    # one workgroup per (sequence, head) unless a flag asks for row blocks
    name = lambda B, H, **kw: ttt.linear_kernel_name(B, H, 8192, 64, 16, **kw)  # noqa: E731
    for B, H in ((16, 32), (2, 32), (8, 12), (1, 1)):
        assert name(B, H) == "ttt_linear_mfma_d64b16"
        assert name(B, H, rows=1) == "ttt_linear_mfma_d64b16"
        assert name(B, H, rows=2) == "ttt_linear_mfma_d64b16_r2"
        assert name(B, H, rows=4) == "ttt_linear_mfma_d64b16_r4"


def test_linear_kernel_selection():
    assert ttt.linear_kernel_name(16, 32, 8192, 64, 16) == "ttt_linear_mfma_d64b16"
    assert ttt.linear_kernel_name(16, 32, 8192, 64, 16, generic=True) == "ttt_linear_generic_kernel<64>"
    assert ttt.linear_kernel_name(1, 1, 64, 16, 4, in_dtype=0) == "ttt_linear_generic_kernel<16>"
    assert ttt.linear_kernel_name(1, 1, 64, 64, 16, in_dtype=0) == "ttt_linear_mfma_f32_d64b16"   # fp32 Q/K/V
    assert ttt.linear_kernel_name(1, 1, 64, 64, 16, in_dtype=0, generic=True) == "ttt_linear_generic_kernel<64>"
    assert ttt.linear_kernel_name(1, 1, 64, 64, 8, in_dtype=0) == "ttt_linear_generic_kernel<64>"
    assert ttt.linear_kernel_name(1, 1, 64, 48, 16) is None


# ---- TTT-MLP validation ----------------------------------------------------------

def _mdesc(B=2, H=4, T=64, d=64, dh=256, b=16, wstride=0, est=(0, 0, 0), in_dtype=1, out_dtype=0):
    return ttt.mlp_desc(B, H, T, d, dh, b, in_dtype, out_dtype, wstride, est)


def _mval(desc, **over):
    p = dict(q=1 * GB, k=2 * GB, v=3 * GB, w1=4 * GB, w2=5 * GB, eta=6 * GB, z=7 * GB, f1=8 * GB, f2=9 * GB)
    p.update(over)
    return ttt.lib().ttt_mlp_validate(ctypes.byref(desc), p["q"], p["k"], p["v"], p["w1"], p["w2"], p["eta"],
                                      p["z"], p["f1"], p["f2"])


def test_mlp_validation():
    if ttt.mlp_kernel_name(2, 4, 64, 64, 256, 16) is None:
        assert _mval(_mdesc()) == UNSUP
        pytest.skip("MLP kernel not built")
    assert _mval(_mdesc()) == OK
    assert _mval(_mdesc(T=40)) == SHAPE
    assert _mval(_mdesc(dh=128)) == UNSUP
    assert _mval(_mdesc(out_dtype=1)) == UNSUP    # Z is fp32 only
    assert _mval(_mdesc(in_dtype=0)) == UNSUP     # bf16 inputs only
    assert _mval(_mdesc(out_dtype=7)) == 3        # no such dtype: TTT_ERR_DTYPE
    assert _mval(_mdesc(), f1=None) == NULL
    assert _mval(_mdesc(), z=1 * GB) == ALIAS
    assert _mval(_mdesc(), f1=4 * GB) == ALIAS
    assert _mval(_mdesc(wstride=4 * 64 * 256), f1=4 * GB, f2=5 * GB) == OK
    assert _mval(_mdesc(), f2=9 * GB + 8) == ALIGN


def test_mlp_primal_flag_validation():
    P = ttt.TTT_FLAG_PRIMAL

    def d(T=64, dh=256, b=16, ind=1, outd=0, flags=P):
        return ttt.mlp_desc(2, 4, T, 64, dh, b, ind, outd, 0, (0, 0, 0), flags)

    assert _mval(d()) == OK
    assert _mval(d(b=1)) == OK and _mval(d(b=64)) == OK       # any mini-batch size
    assert _mval(d(ind=0, outd=1)) == OK                       # fp32 inputs, bf16 Z
    assert _mval(d(T=40)) == SHAPE                              # T % b != 0
    assert _mval(d(dh=128)) == UNSUP
    assert _mval(d(flags=P | 1)) == FLAGS
    assert ttt.mlp_kernel_name(2, 4, 64, 64, 256, 5, primal=True) == "ttt_mlp_primal_d64h256"
    assert ttt.mlp_kernel_name(2, 4, 64, 64, 128, 16, primal=True) is None


class MlpDecBufs:
    NAMES = ("q", "k", "v", "eta", "z", "w1", "w2", "w1b", "w2b")

    def __init__(self):
        for i, n in enumerate(self.NAMES):
            setattr(self, n, (i + 1) * GB)


def _mdval(desc, pos=0, **over):
    b = MlpDecBufs()
    for k, v in over.items():
        setattr(b, k, v)
    return ttt.lib().ttt_mlp_decode_validate(ctypes.byref(desc), *(getattr(b, n) for n in MlpDecBufs.NAMES),
                                             ctypes.c_int64(pos))


def test_mlp_decode_validation():
    assert _mdval(_mdesc(T=1)) == OK
    assert _mdval(_mdesc(T=37, b=16, in_dtype=0, out_dtype=1, est=(4 * 37, 37, 1)), pos=5) == OK  # ragged T
    assert ttt.lib().ttt_mlp_decode_validate(None, *(0,) * 9, ctypes.c_int64(0)) == NULL
    for name in MlpDecBufs.NAMES:
        assert _mdval(_mdesc(T=1), **{name: None}) == NULL, name
    assert _mdval(_mdesc(T=1), pos=-1) == POS
    assert _mdval(_mdesc(T=1, wstride=4 * 64 * 256)) == STRIDE
    assert _mdval(_mdesc(T=1, dh=128)) == UNSUP
    assert _mdval(_mdesc(T=1), w1b=6 * GB + 16) == ALIAS          # W1b inside W1
    assert _mdval(_mdesc(T=1), z=2 * GB) == ALIAS                 # Z over K
    assert _mdval(_mdesc(T=1), w2=7 * GB + 4) == ALIGN
    assert _mdval(_mdesc(B=0, T=1)) == OK
    assert _mdval(_mdesc(T=0), q=None, k=None, v=None, z=None, eta=None) == OK


def _mlndval(desc, pos=0, eps=1e-6, gamma=10 * GB, beta=11 * GB, **over):
    b = MlpDecBufs()
    for k, v in over.items():
        setattr(b, k, v)
    q, k, v, eta, z, w1, w2, w1b, w2b = (getattr(b, n) for n in MlpDecBufs.NAMES)
    return ttt.lib().ttt_mlp_ln_decode_validate(ctypes.byref(desc), q, k, v, eta, gamma, beta, ctypes.c_float(eps),
                                                z, w1, w2, w1b, w2b, ctypes.c_int64(pos))


def test_mlp_ln_decode_validation():
    assert _mlndval(_mdesc(T=1)) == OK
    assert _mlndval(_mdesc(T=37, b=5, in_dtype=0, out_dtype=1)) == OK     # any b, ragged T
    assert _mlndval(_mdesc(T=1), pos=-1) == POS
    assert _mlndval(_mdesc(T=1, dh=128)) == UNSUP
    assert _mlndval(_mdesc(T=1), eps=-1.0) == SHAPE
    assert _mlndval(_mdesc(T=1), gamma=None) == NULL
    assert _mlndval(_mdesc(T=0), q=None, k=None, v=None, z=None, eta=None, beta=None) == NULL
    assert _mlndval(_mdesc(B=0), gamma=None, beta=None) == OK
    assert _mlndval(_mdesc(T=1), beta=11 * GB + 2) == ALIGN
    assert _mlndval(_mdesc(T=1), gamma=6 * GB + 64) == ALIAS             # gamma inside W1
    assert _mlndval(_mdesc(T=1), beta=9 * GB) == ALIAS                   # beta over W2b
    assert _mlndval(_mdesc(T=1), w1b=6 * GB + 16) == ALIAS               # the plain decode checks still hold


def test_mlp_ln_fwd_primal_flag_host_errors():
    P = ttt.TTT_FLAG_PRIMAL
    f = ttt.lib().ttt_mlp_ln_fwd

    def call(desc, eps=1e-6, gamma=10 * GB):
        return f(ctypes.byref(desc), 1 * GB, 2 * GB, 3 * GB, 4 * GB, 5 * GB, gamma, 11 * GB, ctypes.c_float(eps),
                 6 * GB, 7 * GB, 8 * GB, 9 * GB, None)

    def d(dh=256, b=16, T=64, flags=P):
        return ttt.mlp_desc(2, 4, T, 64, dh, b, 1, 0, 0, (0, 0, 0), flags)
    assert call(d(dh=128)) == UNSUP
    assert call(d(flags=P | 1)) == FLAGS
    assert call(d(b=5, T=63)) == SHAPE
    assert call(d(), eps=-1.0) == SHAPE
    assert call(d(), gamma=None) == NULL
    assert call(d(), gamma=7 * GB) == ALIAS                             # gamma over Z
    assert ttt.mlp_ln_kernel_name(2, 4, 64, 64, 256, 16) == "ttt_mlp_fwd_d64h256b16 (layer norm)"
    assert ttt.mlp_ln_kernel_name(2, 4, 60, 64, 256, 5, primal=True) == "ttt_mlp_ln_primal_d64h256"
    assert ttt.mlp_ln_kernel_name(2, 4, 64, 64, 128, 16, primal=True) is None


class MlpBwdBufs:
    NAMES = ("q", "k", "v", "w1", "w2", "eta", "dz", "d1f", "d2f", "ws", "dq", "dk", "dv", "deta", "d1", "d2")

    def __init__(self):
        for i, n in enumerate(self.NAMES):
            setattr(self, n, (i + 1) * GB)


def _mbval(desc, ws_bytes=None, **over):
    b = MlpBwdBufs()
    for k, v in over.items():
        setattr(b, k, v)
    if ws_bytes is None:
        ws_bytes = max(ttt.lib().ttt_mlp_bwd_workspace_bytes(ctypes.byref(desc)), 0)
    v = [getattr(b, n) for n in MlpBwdBufs.NAMES]
    return ttt.lib().ttt_mlp_bwd_validate(ctypes.byref(desc), *v[:10], ctypes.c_int64(ws_bytes), *v[10:])


def test_mlp_bwd_validation():
    d = _mdesc(T=64, in_dtype=1, out_dtype=0)
    assert _mbval(d) == OK
    assert _mbval(_mdesc(T=37, b=5, in_dtype=0)) == OK                 # ragged T, any b <= 16
    assert _mbval(d, d1f=None, d2f=None) == OK                         # zero final-state gradients
    assert ttt.lib().ttt_mlp_bwd_validate(None, *(0,) * 10, ctypes.c_int64(0), *(0,) * 6) == NULL
    for name in ("q", "k", "v", "w1", "w2", "eta", "dz", "dq", "dk", "dv", "deta", "d1", "d2"):
        assert _mbval(d, **{name: None}) == NULL, name
    assert _mbval(d, ws=None) == WORKSPACE
    assert _mbval(d, ws_bytes=1024) == WORKSPACE
    assert _mbval(d, ws=10 * GB + 8) == WORKSPACE                       # misaligned
    assert _mbval(_mdesc(T=64, b=32)) == UNSUP
    assert _mbval(_mdesc(T=64, dh=128)) == UNSUP
    assert _mbval(_mdesc(T=64, out_dtype=1)) == UNSUP                  # dZ and gradients fp32 only
    assert _mbval(_mdesc(T=64, wstride=7)) == STRIDE
    assert _mbval(ttt.mlp_desc(2, 4, 64, 64, 256, 16, 1, 0, 0, (0, 0, 0), ttt.TTT_FLAG_PRIMAL)) == OK
    assert _mbval(ttt.mlp_desc(2, 4, 64, 64, 256, 16, 1, 0, 0, (0, 0, 0), ttt.TTT_FLAG_GENERIC)) == FLAGS
    assert _mbval(d, dq=11 * GB + 8) == ALIGN
    assert _mbval(d, d1=1 * GB) == ALIAS                               # dW1 over Q
    assert _mbval(d, dk=11 * GB) == ALIAS                              # dK over dQ
    assert _mbval(d, ws=16 * GB) == ALIAS                              # workspace over dW2
    assert _mbval(_mdesc(B=0, T=64), ws=None, ws_bytes=0) == OK
    assert _mbval(_mdesc(T=0), q=None, k=None, v=None, eta=None, dz=None, dq=None, dk=None, dv=None, deta=None,
                  ws=None, ws_bytes=0) == OK
    assert ttt.mlp_bwd_workspace_bytes(2, 4, 64, 64, 256, 16) == 2 * 4 * 4 * 2 * 64 * 256 * 4
    assert ttt.mlp_bwd_workspace_bytes(1, 1, 37, 64, 256, 16) == 3 * 2 * 64 * 256 * 4
    assert ttt.mlp_bwd_kernel_name(16, 32, 2048, 64, 256, 16) == "ttt_mlp_bwd_d64h256b16"           # dual form
    assert ttt.mlp_bwd_kernel_name(16, 32, 2048, 64, 256, 16, primal=True) == "ttt_mlp_bwd_d64h256"
    assert ttt.mlp_bwd_kernel_name(16, 32, 2048, 64, 256, 16, in_dtype=0) == "ttt_mlp_bwd_d64h256"  # fp32 inputs
    assert ttt.mlp_bwd_kernel_name(16, 32, 2040, 64, 256, 8) == "ttt_mlp_bwd_d64h256"
    assert ttt.mlp_bwd_kernel_name(1, 1, 37, 64, 256, 16) == "ttt_mlp_bwd_d64h256"                  # ragged T
    assert ttt.mlp_bwd_kernel_name(16, 32, 2048, 64, 256, 32) is None



def _mlnval(desc, eps=1e-6, ws_bytes=None, **over):
    """ttt_mlp_ln_bwd_validate with fake pointers: MlpBwdBufs plus gamma, beta,
    dgamma, dbeta at 17-20 GB."""
    b = MlpBwdBufs()
    extra = dict(gamma=17 * GB, beta=18 * GB, dg=19 * GB, db=20 * GB)
    for k, v in over.items():
        if k in extra:
            extra[k] = v
        else:
            setattr(b, k, v)
    if ws_bytes is None:
        ws_bytes = max(ttt.lib().ttt_mlp_bwd_workspace_bytes(ctypes.byref(desc)), 0)
    v = [getattr(b, n) for n in MlpBwdBufs.NAMES]
    return ttt.lib().ttt_mlp_ln_bwd_validate(ctypes.byref(desc), *v[:5], extra["gamma"], extra["beta"],
                                             ctypes.c_float(eps), *v[5:10], ctypes.c_int64(ws_bytes), *v[10:],
                                             extra["dg"], extra["db"])


def test_mlp_ln_bwd_validation():
    d = _mdesc(T=64, in_dtype=1, out_dtype=0)
    assert _mlnval(d) == OK
    assert _mlnval(_mdesc(T=37, b=5, in_dtype=0)) == OK                 # ragged T, any b <= 16
    assert _mlnval(d, d1f=None, d2f=None) == OK
    assert _mlnval(d, eps=-1.0) == SHAPE
    assert _mlnval(d, eps=float("nan")) == SHAPE
    for name in ("gamma", "beta", "dg", "db", "dq", "ws"):
        assert _mlnval(d, **{name: None}) in (NULL, WORKSPACE), name
    assert _mlnval(d, gamma=17 * GB + 2) == ALIGN
    assert _mlnval(d, dg=19 * GB + 2) == ALIGN
    assert _mlnval(d, gamma=11 * GB) == ALIAS                          # gamma over dQ
    assert _mlnval(d, dg=1 * GB) == ALIAS                              # dgamma over Q
    assert _mlnval(d, dg=11 * GB) == ALIAS                             # dgamma over dQ
    assert _mlnval(d, db=19 * GB) == ALIAS                             # dbeta over dgamma
    assert _mlnval(_mdesc(T=64, dh=128)) == UNSUP
    assert _mlnval(_mdesc(B=0, T=64), ws=None, ws_bytes=0, gamma=None, beta=None, dg=None, db=None) == OK
    assert ttt.mlp_ln_bwd_kernel_name(16, 32, 2048, 64, 256, 16) == "ttt_mlp_bwd_d64h256 (layer norm)"
    assert ttt.mlp_ln_bwd_kernel_name(16, 32, 2048, 64, 256, 32) is None


# ---- decode validation -------------------------------------------------------------

def _dval(desc, pos=0, **over):
    p = dict(q=1 * GB, k=2 * GB, v=3 * GB, eta=5 * GB, z=6 * GB, w=7 * GB, wb=8 * GB)
    p.update(over)
    return ttt.lib().ttt_linear_decode_validate(ctypes.byref(desc), p["q"], p["k"], p["v"], p["eta"], p["z"],
                                                p["w"], p["wb"], pos)


def test_decode_validation():
    POS = 10
    assert _dval(_desc(T=1)) == OK
    assert _dval(_desc(T=37)) == OK                # T need not be a multiple of b
    assert _dval(_desc(T=1), pos=-1) == POS
    assert _dval(_desc(T=1, flags=1)) == FLAGS
    assert _dval(_desc(T=1, wstride=4 * 64 * 64)) == STRIDE
    assert _dval(_desc(T=1, d=48)) == UNSUP
    assert _dval(_desc(T=1), wb=7 * GB) == ALIAS   # W and Wb alias
    assert _dval(_desc(T=1), w=1 * GB) == ALIAS    # W over Q
    assert _dval(_desc(T=1), z=None) == NULL
    assert _dval(_desc(T=0), q=None, k=None, v=None, z=None, eta=None) == OK


def test_primal_flag():
    assert _val(_desc(flags=2, b=7, T=63)) == OK   # any b with the primal form
    assert _val(_desc(flags=3)) == FLAGS            # generic and primal together
    assert ttt.linear_kernel_name(2, 4, 64, 64, 16, primal=True) == "ttt_linear_primal_kernel<64>"


def test_chunked_workspace_bytes():
    d = _desc(B=2, H=32, T=32768)
    assert ttt.lib().ttt_linear_chunked_workspace_bytes(ctypes.byref(d), 1) == 0
    # maps (P, R) of chunks 1 .. 6 and start states of chunks 1 .. 7
    assert ttt.lib().ttt_linear_chunked_workspace_bytes(ctypes.byref(d), 8) == 64 * (6 * 2 + 7) * 64 * 64 * 4
    assert ttt.lib().ttt_linear_chunked_workspace_bytes(ctypes.byref(d), 2) == 64 * 1 * 64 * 64 * 4
    assert ttt.lib().ttt_linear_chunked_workspace_bytes(ctypes.byref(d), 0) == -1
    assert ttt.lib().ttt_linear_chunked_workspace_bytes(None, 4) == -1


def test_chunked_noalloc_host_errors():
    """The allocation-free chunked forward's argument errors return before any
    HIP call (so they run without a GPU): bad shapes and flags as the chunked
    forward, and TTT_ERR_SCRATCH when the maps and start states would not fit
    the static scratch."""
    f = ttt.lib().ttt_linear_fwd_chunked_noalloc

    def call(desc, nchunks, **over):
        b = Bufs()
        for k_, v_ in over.items():
            setattr(b, k_, v_)
        return f(ctypes.byref(desc), nchunks, *b.args(), None)

    assert call(_desc(B=2, H=32, T=32768), 0) == SHAPE
    assert call(_desc(B=2, H=32, T=64), 5) == SHAPE             # more chunks than mini-batches
    assert call(_desc(B=2, H=32, T=32768, ind=0), 4) == UNSUP   # fp32 inputs: no matrix-core path
    assert call(_desc(B=2, H=32, T=32768, flags=1), 4) == UNSUP
    assert call(_desc(B=2, H=32, T=32768), 4, q=None) == NULL
    assert call(_desc(B=2, H=32, T=32768), 4, z=3 * GB) == ALIAS
    big = _desc(B=16, H=32, T=8192)                              # 512 chains x 4 chunks: 56 MiB of maps
    need = ttt.lib().ttt_linear_chunked_workspace_bytes(ctypes.byref(big), 4)
    assert need > ttt.NOALLOC_SCRATCH_BYTES
    assert call(big, 4) == SCRATCH
    assert "static scratch" in ttt.status_str(SCRATCH)
    assert f(None, 4, *Bufs().args(), None) == NULL


# ---- backward validation ----------------------------------------------------------

class BwdBufs:
    """Fake aligned, disjoint device addresses for the backward's 12 tensors."""

    NAMES = ("q", "k", "eta", "wf", "e", "dz", "dwf", "dq", "dk", "dv", "deta", "dw0")

    def __init__(self):
        for i, n in enumerate(self.NAMES):
            setattr(self, n, (i + 1) * GB)

    def args(self):
        return tuple(getattr(self, n) for n in self.NAMES)


def _bval(desc, **over):
    bufs = BwdBufs()
    for k, v in over.items():
        setattr(bufs, k, v)
    return ttt.lib().ttt_linear_bwd_validate(ctypes.byref(desc), *bufs.args())


def test_bwd_validation():
    assert _bval(_desc()) == OK
    assert _bval(_desc(est=(4 * 64, 64, 1))) == OK
    assert _bval(_desc(ind=0, d=16, b=4)) == OK
    assert _bval(_desc(), dwf=None) == OK                     # dW_final is optional
    assert ttt.lib().ttt_linear_bwd_validate(None, *BwdBufs().args()) == NULL
    for name in ("q", "k", "eta", "wf", "e", "dz", "dq", "dk", "dv", "deta", "dw0"):
        assert _bval(_desc(), **{name: None}) == NULL, name
    assert _bval(_desc(T=60)) == SHAPE
    assert _bval(_desc(flags=ttt.TTT_FLAG_PRIMAL)) == FLAGS   # no primal backward
    assert _bval(_desc(d=48)) == UNSUP
    assert _bval(_desc(d=64, b=32, ind=0)) == UNSUP           # generic backward: d = 64 needs b <= 16
    assert _bval(_desc(), e=1 * GB + 8) == ALIGN
    assert _bval(_desc(), dv=1 * GB) == ALIAS                 # output over an input
    assert _bval(_desc(), dk=8 * GB + 64) == ALIAS            # output over another output
    assert _bval(_desc(B=0)) == OK
    assert _bval(_desc(T=0), q=None, k=None, e=None, dz=None, dq=None, dk=None, dv=None, deta=None) == OK


def test_bwd_kernel_selection():
    assert ttt.linear_bwd_kernel_name(16, 32, 8192, 64, 16) == "ttt_linear_bwd_d64b16"
    assert ttt.linear_bwd_kernel_name(16, 32, 8192, 64, 16, generic=True) == "ttt_linear_bwd_generic_kernel<64>"
    assert ttt.linear_bwd_kernel_name(1, 1, 64, 16, 4, in_dtype=ttt.TTT_F32) == "ttt_linear_bwd_generic_kernel<16>"
    assert ttt.linear_bwd_kernel_name(1, 1, 64, 64, 32) is None


def test_fwd_save_rejects_primal():
    desc = _desc(flags=ttt.TTT_FLAG_PRIMAL)
    b = Bufs()
    st = ttt.lib().ttt_linear_fwd_save(ctypes.byref(desc), *b.args(), 9 * GB, None)
    assert st == FLAGS


# ---- layer-norm backward validation -------------------------------------------

class LnBwdBufs:
    """Fake aligned, disjoint device addresses for the layer-norm backward."""

    NAMES = ("q", "k", "v", "eta", "gamma", "beta", "wf", "dl", "dz", "dwf", "dq", "dk", "dv", "deta", "dw0",
             "dgamma", "dbeta")

    def __init__(self):
        for i, n in enumerate(self.NAMES):
            setattr(self, n, (i + 1) * GB)

    def args(self, eps):
        a = [getattr(self, n) for n in self.NAMES]
        return (*a[:6], ctypes.c_float(eps), *a[6:])


def _lbval(desc, eps=1e-6, **over):
    bufs = LnBwdBufs()
    for k, v in over.items():
        setattr(bufs, k, v)
    return ttt.lib().ttt_linear_ln_bwd_validate(ctypes.byref(desc), *bufs.args(eps))


def test_ln_bwd_validation():
    assert _lbval(_desc()) == OK
    assert _lbval(_desc(outd=1, est=(4 * 64, 64, 1))) == OK
    assert _lbval(_desc(), dwf=None) == OK
    assert ttt.lib().ttt_linear_ln_bwd_validate(None, *LnBwdBufs().args(1e-6)) == NULL
    for name in LnBwdBufs.NAMES:
        if name != "dwf":
            assert _lbval(_desc(), **{name: None}) == NULL, name
    assert _lbval(_desc(), eps=-1.0) == SHAPE
    assert _lbval(_desc(), eps=float("nan")) == SHAPE
    assert _lbval(_desc(ind=0)) == UNSUP                      # bf16 inputs only
    assert _lbval(_desc(b=8)) == UNSUP
    assert _lbval(_desc(flags=ttt.TTT_FLAG_GENERIC)) == OK
    assert _lbval(_desc(flags=ttt.TTT_FLAG_PRIMAL)) == FLAGS
    assert _lbval(_desc(), v=3 * GB + 8) == ALIGN
    assert _lbval(_desc(), gamma=5 * GB + 2) == ALIGN
    assert _lbval(_desc(), dgamma=1 * GB) == ALIAS            # output over an input
    assert _lbval(_desc(), dbeta=16 * GB + 64) == ALIAS       # output over another output
    assert _lbval(_desc(), dq=5 * GB) == ALIAS                # dq over gamma
    assert _lbval(_desc(B=0)) == OK
    assert _lbval(_desc(T=0), q=None, k=None, v=None, dl=None, dz=None, dq=None, dk=None, dv=None,
                  deta=None) == OK
    assert ttt.linear_ln_bwd_kernel_name(16, 32, 8192, 64, 16) == "ttt_linear_ln_bwd_d64b16"
    assert ttt.linear_ln_bwd_kernel_name(16, 32, 8192, 64, 16, generic=True) == "ttt_linear_ln_bwd_fp32"
    assert ttt.linear_ln_bwd_kernel_name(1, 1, 64, 64, 16, in_dtype=ttt.TTT_F32) is None


def test_ln_fwd_save_host_errors():
    desc = _desc()
    b = Bufs()
    f = ttt.lib().ttt_linear_ln_fwd_save
    gam, bet = 8 * GB, 9 * GB
    assert f(ctypes.byref(desc), b.q, b.k, b.v, b.w0, gam, bet, ctypes.c_float(1e-6), b.eta, b.z, b.wf,
             None, None) == NULL
    assert f(ctypes.byref(desc), b.q, b.k, b.v, b.w0, gam, bet, ctypes.c_float(1e-6), b.eta, b.z, b.wf,
             b.z, None) == ALIAS
    assert f(ctypes.byref(desc), b.q, b.k, b.v, b.w0, gam, bet, ctypes.c_float(1e-6), b.eta, b.z, b.wf,
             gam, None) == ALIAS
    assert f(ctypes.byref(desc), b.q, b.k, b.v, b.w0, gam, bet, ctypes.c_float(1e-6), b.eta, b.z, b.wf,
             10 * GB + 4, None) == ALIGN
    assert f(ctypes.byref(_desc(ind=0)), b.q, b.k, b.v, b.w0, gam, bet, ctypes.c_float(1e-6), b.eta, b.z, b.wf,
             10 * GB, None) == UNSUP


def _lnd(desc, pos=0, eps=1e-6, **over):
    p = dict(q=1 * GB, k=2 * GB, v=3 * GB, eta=5 * GB, gamma=10 * GB, beta=11 * GB, z=6 * GB, w=7 * GB, wb=8 * GB)
    p.update(over)
    return ttt.lib().ttt_linear_ln_decode_validate(ctypes.byref(desc), p["q"], p["k"], p["v"], p["eta"], p["gamma"],
                                                   p["beta"], ctypes.c_float(eps), p["z"], p["w"], p["wb"], pos)


def test_ln_decode_validation():
    POS = 10
    assert _lnd(_desc(T=1)) == OK
    assert _lnd(_desc(T=37, d=32, b=5, ind=0)) == OK     # any b, ragged T, fp32 inputs
    assert _lnd(_desc(T=1), pos=-1) == POS
    assert _lnd(_desc(T=1, flags=2)) == FLAGS
    assert _lnd(_desc(T=1, d=48)) == UNSUP
    assert _lnd(_desc(T=1), eps=-1.0) == SHAPE
    assert _lnd(_desc(T=1), eps=float("nan")) == SHAPE
    assert _lnd(_desc(T=1), gamma=None) == NULL
    assert _lnd(_desc(T=1), beta=None) == NULL
    assert _lnd(_desc(T=0), q=None, k=None, v=None, z=None, eta=None, gamma=None) == NULL  # the kernel reads gamma
    assert _lnd(_desc(B=0), gamma=None, beta=None) == OK
    assert _lnd(_desc(T=1), gamma=10 * GB + 2) == ALIGN
    assert _lnd(_desc(T=1), gamma=7 * GB + 64) == ALIAS   # gamma inside W
    assert _lnd(_desc(T=1), beta=6 * GB) == ALIAS         # beta over Z
    assert _lnd(_desc(T=1), wb=7 * GB) == ALIAS           # the plain decode checks still hold


def test_ln_fwd_primal_flag_host_errors():
    b = Bufs()
    f = ttt.lib().ttt_linear_ln_fwd
    gam, bet = 8 * GB, 9 * GB

    def call(desc, eps=1e-6, g=gam):
        return f(ctypes.byref(desc), b.q, b.k, b.v, b.w0, g, bet, ctypes.c_float(eps), b.eta, b.z, b.wf, None)
    assert call(_desc(flags=2, d=48)) == UNSUP
    assert call(_desc(flags=3)) == FLAGS
    assert call(_desc(flags=2, b=5, T=63)) == SHAPE      # T a multiple of b, as for ttt_linear_fwd
    assert call(_desc(flags=2), eps=-1.0) == SHAPE
    assert call(_desc(flags=2), g=None) == NULL
    assert call(_desc(flags=2), g=6 * GB) == ALIAS        # gamma over Z
    save = ttt.lib().ttt_linear_ln_fwd_save             # the primal kernel saves nothing
    assert save(ctypes.byref(_desc(flags=2)), b.q, b.k, b.v, b.w0, gam, bet, ctypes.c_float(1e-6), b.eta, b.z,
                b.wf, 10 * GB, None) == UNSUP
    assert ttt.linear_ln_kernel_name(2, 4, 64, 64, 16) == "ttt_linear_mfma_d64b16 (layer norm)"
    assert ttt.linear_ln_kernel_name(2, 4, 64, 64, 16, primal=True) == "ttt_linear_ln_primal_kernel<64>"
    assert ttt.linear_ln_kernel_name(2, 4, 60, 32, 5, primal=True) == "ttt_linear_ln_primal_kernel<32>"
    assert ttt.linear_ln_kernel_name(2, 4, 64, 48, 16, primal=True) is None
    assert ttt.linear_ln_kernel_name(2, 4, 64, 64, 16, in_dtype=ttt.TTT_F32) is None


def test_one_hip_runtime_per_process():
    # torch ships a HIP runtime under the same soname the library needs; the
    # binding imports torch before it loads libttt.so so that both use that one
    # runtime (the library loaded first would bind to the system's, and torch
    # would then bring a second runtime whose memory the first cannot use)
    code = ("import test_sequence_layer_amd as t; t.lib(); import torch; "
            "print(sorted(set(l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l)))")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr
    runtimes = eval(out.stdout.strip().splitlines()[-1])
    assert len(runtimes) == 1, runtimes


def test_status_check_and_debug_sync(monkeypatch):
    calls = []

    class FakeCuda:
        @staticmethod
        def synchronize():
            calls.append("sync")

    class FakeTorch:
        cuda = FakeCuda

    monkeypatch.setattr(ttt, "_torch", lambda: FakeTorch)
    monkeypatch.delenv("TTT_DEBUG_SYNC", raising=False)
    ttt._done(OK, "ttt_linear_fwd")
    assert calls == []
    with pytest.raises(ttt.TTTError, match="TTT_ERR_SHAPE"):
        ttt._done(SHAPE, "ttt_linear_fwd")
    monkeypatch.setenv("TTT_DEBUG_SYNC", "1")
    ttt._done(OK, "ttt_linear_fwd")
    assert calls == ["sync"]
    with pytest.raises(ttt.TTTError):
        ttt._done(ALIGN, "ttt_linear_fwd")
    assert calls == ["sync"]   # no wait after a rejected call: nothing was launched
