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

OK, NULL, SHAPE, DTYPE, UNSUP, ALIAS, ALIGN, HIP, STRIDE, FLAGS, POS, WORKSPACE = range(12)
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
    for s in range(12):
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
    assert ttt.linear_kernel_name(1, 1, 64, 64, 16, in_dtype=0) == "ttt_linear_generic_kernel<64>"
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
    assert ttt.lib().ttt_linear_chunked_workspace_bytes(ctypes.byref(d), 8) == 64 * (7 * 2 + 8) * 64 * 64 * 4
    assert ttt.lib().ttt_linear_chunked_workspace_bytes(ctypes.byref(d), 0) == -1
    assert ttt.lib().ttt_linear_chunked_workspace_bytes(None, 4) == -1


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
