"""MI355X (gfx950) TTT sequence layer (forward, and the TTT-Linear backward) -- Python binding.

Thin ctypes layer over libttt.so (C ABI in include/ttt.h).  It only checks and
marshals arguments: torch supplies device memory and the current HIP stream,
and every step of the computation runs in the library's HIP kernels.  There is
no CPU or PyTorch fallback: if libttt.so is missing, importing the ops raises.

    import test_sequence_layer_amd as ttt
    z, w_final = ttt.linear_fwd(q, k, v, w0, eta, b=16)
    z, w1_final, w2_final = ttt.mlp_fwd(q, k, v, w1, w2, eta, b=16)
    z, w_final, e = ttt.linear_fwd_save(q, k, v, w0, eta, b=16)          # training
    dq, dk, dv, deta, dw0 = ttt.linear_bwd(q, k, eta, w_final, e, dz, b=16)

Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
(aharts.cn / itmax.cn), part 03 §1-§9 (the TTT layer, mini-batch GD, the dual
form, TTT-Linear and TTT-MLP).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libttt.so")

TTT_OK = 0
TTT_F32, TTT_BF16 = 0, 1
TTT_FLAG_GENERIC = 1
TTT_FLAG_PRIMAL = 2
TTT_FLAG_ROWS = {1: 4, 2: 8, 4: 16}  # row blocks per (sequence, head) -> TTT_FLAG_ROWS1/2/4


def _rows_flag(rows) -> int:
    """flag bits forcing ``rows`` row blocks of the matrix-core forward (None: the library's choice)"""
    if rows is None:
        return 0
    if rows not in TTT_FLAG_ROWS:
        raise ValueError(f"rows must be None, 1, 2 or 4, not {rows!r}")
    return TTT_FLAG_ROWS[rows]

STATUS_NAMES = {
    0: "TTT_OK", 1: "TTT_ERR_NULL", 2: "TTT_ERR_SHAPE", 3: "TTT_ERR_DTYPE", 4: "TTT_ERR_UNSUPPORTED",
    5: "TTT_ERR_ALIAS", 6: "TTT_ERR_ALIGN", 7: "TTT_ERR_HIP", 8: "TTT_ERR_STRIDE", 9: "TTT_ERR_FLAGS",
    10: "TTT_ERR_POS", 11: "TTT_ERR_WORKSPACE", 12: "TTT_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # TTT_NOALLOC_SCRATCH_BYTES

# Every symbol include/ttt.h declares.
EXPORTS = (
    "ttt_linear_fwd", "ttt_linear_validate", "ttt_linear_kernel_name",
    "ttt_linear_decode", "ttt_linear_decode_validate",
    "ttt_linear_fwd_chunked", "ttt_linear_chunked_workspace_bytes", "ttt_linear_fwd_chunked_noalloc",
    "ttt_linear_ln_fwd", "ttt_linear_ln_fwd_save", "ttt_linear_ln_bwd", "ttt_linear_ln_bwd_validate",
    "ttt_linear_ln_bwd_kernel_name", "ttt_linear_ln_kernel_name", "ttt_linear_ln_decode",
    "ttt_linear_ln_decode_validate",
    "ttt_linear_fwd_save", "ttt_linear_bwd", "ttt_linear_bwd_validate", "ttt_linear_bwd_kernel_name",
    "ttt_mlp_fwd", "ttt_mlp_validate", "ttt_mlp_kernel_name", "ttt_mlp_ln_fwd",
    "ttt_mlp_decode", "ttt_mlp_decode_validate", "ttt_mlp_ln_decode", "ttt_mlp_ln_decode_validate",
    "ttt_mlp_ln_kernel_name", "ttt_mlp_bwd", "ttt_mlp_bwd_validate", "ttt_mlp_bwd_workspace_bytes",
    "ttt_mlp_bwd_kernel_name", "ttt_mlp_ln_bwd", "ttt_mlp_ln_bwd_validate", "ttt_mlp_ln_bwd_kernel_name",
    "ttt_status_str", "ttt_abi_version",
)


class LinearDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("d", ctypes.c_int32), ("b", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("w0_batch_stride", ctypes.c_int64),
        ("eta_stride_b", ctypes.c_int64), ("eta_stride_h", ctypes.c_int64), ("eta_stride_t", ctypes.c_int64),
    ]


class MlpDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("d", ctypes.c_int32), ("dh", ctypes.c_int32), ("b", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("reserved", ctypes.c_int32),
        ("w_batch_stride", ctypes.c_int64),
        ("eta_stride_b", ctypes.c_int64), ("eta_stride_h", ctypes.c_int64), ("eta_stride_t", ctypes.c_int64),
    ]


_lib = None


class TTTError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


def lib() -> ctypes.CDLL:
    """The loaded libttt.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    # torch ships its own HIP runtime under the soname libamdhip64.so.7, which
    # libttt.so also needs.  Loaded after torch, libttt.so binds to torch's
    # runtime; loaded first, it would bind to the system's and torch would then
    # load a second runtime whose device memory the first cannot use.  So torch
    # (when installed) is imported first.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, fp = ctypes.c_void_p, ctypes.c_void_p
    L.ttt_linear_fwd.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, fp, vp, fp, vp]
    L.ttt_linear_fwd.restype = ctypes.c_int
    L.ttt_linear_validate.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, fp, vp, fp]
    L.ttt_linear_validate.restype = ctypes.c_int
    L.ttt_linear_decode.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, vp, fp, fp, ctypes.c_int64, vp]
    L.ttt_linear_decode.restype = ctypes.c_int
    L.ttt_linear_decode_validate.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, vp, fp, fp, ctypes.c_int64]
    L.ttt_linear_decode_validate.restype = ctypes.c_int
    L.ttt_linear_fwd_chunked.argtypes = [ctypes.POINTER(LinearDesc), ctypes.c_int32, vp, vp, vp, fp, fp, vp, fp,
                                         vp, ctypes.c_int64, vp]
    L.ttt_linear_fwd_chunked.restype = ctypes.c_int
    L.ttt_linear_fwd_chunked_noalloc.argtypes = [ctypes.POINTER(LinearDesc), ctypes.c_int32, vp, vp, vp, fp, fp,
                                                 vp, fp, vp]
    L.ttt_linear_fwd_chunked_noalloc.restype = ctypes.c_int
    L.ttt_linear_chunked_workspace_bytes.argtypes = [ctypes.POINTER(LinearDesc), ctypes.c_int32]
    L.ttt_linear_chunked_workspace_bytes.restype = ctypes.c_int64
    L.ttt_linear_ln_fwd.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, fp, fp, ctypes.c_float, fp, vp, fp,
                                    vp]
    L.ttt_linear_ln_fwd.restype = ctypes.c_int
    L.ttt_linear_ln_fwd_save.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, fp, fp, ctypes.c_float, fp, vp,
                                         fp, fp, vp]
    L.ttt_linear_ln_fwd_save.restype = ctypes.c_int
    L.ttt_linear_ln_bwd.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, fp, fp, ctypes.c_float, fp, fp, vp,
                                    fp, vp, vp, vp, fp, fp, fp, fp, vp]
    L.ttt_linear_ln_bwd.restype = ctypes.c_int
    L.ttt_linear_ln_bwd_validate.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, fp, fp, ctypes.c_float,
                                             fp, fp, vp, fp, vp, vp, vp, fp, fp, fp, fp]
    L.ttt_linear_ln_bwd_validate.restype = ctypes.c_int
    L.ttt_linear_ln_bwd_kernel_name.argtypes = [ctypes.POINTER(LinearDesc)]
    L.ttt_linear_ln_bwd_kernel_name.restype = ctypes.c_char_p
    L.ttt_linear_ln_kernel_name.argtypes = [ctypes.POINTER(LinearDesc)]
    L.ttt_linear_ln_kernel_name.restype = ctypes.c_char_p
    L.ttt_linear_ln_decode.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, fp, fp, ctypes.c_float, vp, fp,
                                       fp, ctypes.c_int64, vp]
    L.ttt_linear_ln_decode.restype = ctypes.c_int
    L.ttt_linear_ln_decode_validate.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, fp, fp, ctypes.c_float,
                                                vp, fp, fp, ctypes.c_int64]
    L.ttt_linear_ln_decode_validate.restype = ctypes.c_int
    L.ttt_linear_fwd_save.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, vp, fp, fp, vp, fp, fp, vp]
    L.ttt_linear_fwd_save.restype = ctypes.c_int
    L.ttt_linear_bwd.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, fp, fp, fp, vp, fp, vp, vp, vp, fp, fp, vp]
    L.ttt_linear_bwd.restype = ctypes.c_int
    L.ttt_linear_bwd_validate.argtypes = [ctypes.POINTER(LinearDesc), vp, vp, fp, fp, fp, vp, fp, vp, vp, vp, fp,
                                          fp]
    L.ttt_linear_bwd_validate.restype = ctypes.c_int
    L.ttt_linear_bwd_kernel_name.argtypes = [ctypes.POINTER(LinearDesc)]
    L.ttt_linear_bwd_kernel_name.restype = ctypes.c_char_p
    L.ttt_linear_kernel_name.argtypes = [ctypes.POINTER(LinearDesc)]
    L.ttt_linear_kernel_name.restype = ctypes.c_char_p
    L.ttt_mlp_fwd.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, fp, fp, vp, fp, fp, vp]
    L.ttt_mlp_decode.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, vp, fp, fp, fp, fp, ctypes.c_int64, vp]
    L.ttt_mlp_decode.restype = ctypes.c_int
    L.ttt_mlp_decode_validate.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, vp, fp, fp, fp, fp,
                                          ctypes.c_int64]
    L.ttt_mlp_decode_validate.restype = ctypes.c_int
    L.ttt_mlp_fwd.restype = ctypes.c_int
    L.ttt_mlp_ln_fwd.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, fp, vp, fp,
                                 fp, vp]
    L.ttt_mlp_ln_fwd.restype = ctypes.c_int
    L.ttt_mlp_validate.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, fp, fp, vp, fp, fp]
    L.ttt_mlp_validate.restype = ctypes.c_int
    L.ttt_mlp_kernel_name.argtypes = [ctypes.POINTER(MlpDesc)]
    L.ttt_mlp_kernel_name.restype = ctypes.c_char_p
    L.ttt_mlp_ln_kernel_name.argtypes = [ctypes.POINTER(MlpDesc)]
    L.ttt_mlp_ln_kernel_name.restype = ctypes.c_char_p
    L.ttt_mlp_bwd.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, fp, fp, fp, fp, fp, vp, ctypes.c_int64,
                              fp, fp, fp, fp, fp, fp, vp]
    L.ttt_mlp_bwd.restype = ctypes.c_int
    L.ttt_mlp_bwd_validate.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, fp, fp, fp, fp, fp, vp,
                                       ctypes.c_int64, fp, fp, fp, fp, fp, fp]
    L.ttt_mlp_bwd_validate.restype = ctypes.c_int
    L.ttt_mlp_bwd_workspace_bytes.argtypes = [ctypes.POINTER(MlpDesc)]
    L.ttt_mlp_bwd_workspace_bytes.restype = ctypes.c_int64
    L.ttt_mlp_bwd_kernel_name.argtypes = [ctypes.POINTER(MlpDesc)]
    L.ttt_mlp_bwd_kernel_name.restype = ctypes.c_char_p
    L.ttt_mlp_ln_bwd.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, fp, fp, fp, fp,
                                 vp, ctypes.c_int64, fp, fp, fp, fp, fp, fp, fp, fp, vp]
    L.ttt_mlp_ln_bwd.restype = ctypes.c_int
    L.ttt_mlp_ln_bwd_validate.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, fp,
                                          fp, fp, fp, vp, ctypes.c_int64, fp, fp, fp, fp, fp, fp, fp, fp]
    L.ttt_mlp_ln_bwd_validate.restype = ctypes.c_int
    L.ttt_mlp_ln_bwd_kernel_name.argtypes = [ctypes.POINTER(MlpDesc)]
    L.ttt_mlp_ln_bwd_kernel_name.restype = ctypes.c_char_p
    L.ttt_mlp_ln_decode.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, fp, fp, ctypes.c_float, vp, fp, fp, fp,
                                    fp, ctypes.c_int64, vp]
    L.ttt_mlp_ln_decode.restype = ctypes.c_int
    L.ttt_mlp_ln_decode_validate.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, fp, fp, fp, ctypes.c_float, vp,
                                             fp, fp, fp, fp, ctypes.c_int64]
    L.ttt_mlp_ln_decode_validate.restype = ctypes.c_int
    L.ttt_status_str.argtypes = [ctypes.c_int]
    L.ttt_status_str.restype = ctypes.c_char_p
    L.ttt_abi_version.argtypes = []
    L.ttt_abi_version.restype = ctypes.c_int
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().ttt_status_str(int(status)).decode()


def abi_version() -> int:
    return int(lib().ttt_abi_version())


# ----------------------------------------------------------------- helpers --

def _torch():
    import torch
    return torch


def _done(status: int, what: str) -> None:
    """Raise on a non-OK status.  With TTT_DEBUG_SYNC=1 in the environment, also
    wait for the launched work and let torch raise any asynchronous kernel fault
    here, at the call that caused it, rather than at a later synchronization."""
    if status != TTT_OK:
        raise TTTError(status, what)
    if os.environ.get("TTT_DEBUG_SYNC") == "1":
        _torch().cuda.synchronize()


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return TTT_F32
    if dt == torch.bfloat16:
        return TTT_BF16
    raise TypeError(f"unsupported dtype {dt} (float32 or bfloat16)")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


_raw_stream = None


def _stream_handle(stream, dev: Optional[int] = None) -> Optional[int]:
    """hipStream_t of ``stream``, else of torch's current stream on device ``dev``
    (default: the current device).  torch's raw-stream query is used when it
    exists: building a Stream object costs ~3 us per call, which matters for
    one-token decode calls."""
    torch = _torch()
    if stream is not None:
        return stream.cuda_stream
    global _raw_stream
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_stream:
        return _raw_stream(torch.cuda.current_device() if dev is None else dev)
    return torch.cuda.current_stream().cuda_stream


def _check_dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("every tensor must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("every tensor must be contiguous")


def eta_layout(eta, B: int, H: int, T: int, device):
    """eta as (device fp32 tensor, (stride_b, stride_h, stride_t)).

    float / 1-element tensor -> scalar; [H] -> per head; [B, H, T] -> per token.
    """
    torch = _torch()
    if not torch.is_tensor(eta):
        return torch.tensor([float(eta)], dtype=torch.float32, device=device), (0, 0, 0)
    if eta.dtype != torch.float32:
        raise TypeError("eta must be float32")
    if eta.numel() == 1:
        return eta.reshape(1), (0, 0, 0)
    if tuple(eta.shape) == (H,):
        return eta, (0, 1, 0)
    if tuple(eta.shape) == (B, H, T):
        return eta, (H * T, T, 1)
    raise ValueError(f"eta shape {tuple(eta.shape)}: expected scalar, [H] or [B, H, T]")


# ------------------------------------------------------------- TTT-Linear --

def linear_desc(B, H, T, d, b, in_dtype, out_dtype, w0_batch_stride, eta_strides, flags=0) -> LinearDesc:
    return LinearDesc(B, H, T, d, b, in_dtype, out_dtype, flags, w0_batch_stride, *eta_strides)


def linear_fwd(q, k, v, w0, eta, b: int, out_dtype=None, w_final=None, z=None,
               generic: bool = False, primal: bool = False, rows=None, stream=None) -> Tuple["object", "object"]:
    """TTT-Linear forward (dual form) on the GPU.

    q, k, v : [B, H, T, d] bfloat16 or float32 (same dtype), contiguous, on the GPU
    w0      : [H, d, d] (shared over the batch) or [B, H, d, d] float32; z = W q
    eta     : float, [H] or [B, H, T] float32
    b       : mini-batch size (T % b == 0)
    returns (Z [B, H, T, d] of out_dtype (default float32), W_final [B, H, d, d] float32).
    ``w_final`` may be ``w0`` itself (in-place carry) when w0 is [B, H, d, d].
    ``generic`` forces the portable fp32 kernel; ``primal`` computes token by
    token (the primal form) instead of with the dual form; ``rows`` (1, 2, 4)
    forces the number of row-block workgroups per sequence and head of the
    matrix-core kernel (default 1).
    """
    torch = _torch()
    B, H, T, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same shape and dtype")
    if w0.dtype != torch.float32:
        raise TypeError("w0 must be float32")
    if tuple(w0.shape) == (H, d, d):
        wstride = 0
    elif tuple(w0.shape) == (B, H, d, d):
        wstride = H * d * d
    else:
        raise ValueError(f"w0 shape {tuple(w0.shape)}: expected [H,d,d] or [B,H,d,d]")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=out_dtype, device=q.device)
    if w_final is None:
        w_final = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    _check_dev(q, k, v, w0, eta_t, z, w_final)
    flags = (TTT_FLAG_GENERIC if generic else 0) | (TTT_FLAG_PRIMAL if primal else 0) | _rows_flag(rows)
    desc = linear_desc(B, H, T, d, b, _dtype_code(q.dtype), _dtype_code(z.dtype), wstride, est, flags)
    st = lib().ttt_linear_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w0), _ptr(eta_t),
                              _ptr(z), _ptr(w_final), _stream_handle(stream))
    _done(st, "ttt_linear_fwd")
    return z, w_final


def linear_fwd_save(q, k, v, w0, eta, b: int, out_dtype=None, w_final=None, z=None, e_saved=None,
                    generic: bool = False, rows=None, stream=None):
    """TTT-Linear forward for training: :func:`linear_fwd` plus the saved
    reconstruction errors E [B, H, T, d] float32 (e_t = W k_t - v_t at the
    mini-batch-start W) that :func:`linear_bwd` needs.

    returns (Z, W_final, E).
    """
    torch = _torch()
    B, H, T, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same shape and dtype")
    if w0.dtype != torch.float32:
        raise TypeError("w0 must be float32")
    wstride = _w0_stride(w0, B, H, d)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=out_dtype, device=q.device)
    if w_final is None:
        w_final = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    if e_saved is None:
        e_saved = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    _check_dev(q, k, v, w0, eta_t, z, w_final, e_saved)
    flags = (TTT_FLAG_GENERIC if generic else 0) | _rows_flag(rows)
    desc = linear_desc(B, H, T, d, b, _dtype_code(q.dtype), _dtype_code(z.dtype), wstride, est, flags)
    st = lib().ttt_linear_fwd_save(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w0), _ptr(eta_t),
                                   _ptr(z), _ptr(w_final), _ptr(e_saved), _stream_handle(stream))
    _done(st, "ttt_linear_fwd_save")
    return z, w_final, e_saved


def linear_bwd(q, k, eta, w_final, e_saved, dz, b: int, dw_final=None, generic: bool = False, out=None,
               stream=None):
    """TTT-Linear backward (dual form).

    q, k     : the forward's [B, H, T, d] inputs (v is not needed)
    eta      : as given to the forward
    w_final, e_saved : from :func:`linear_fwd_save`
    dz       : [B, H, T, d] gradient of the loss with respect to Z (its dtype
               is the dtype of dq, dk, dv)
    dw_final : [B, H, d, d] float32 gradient with respect to W_final, or None (zero)
    out      : optional (dq, dk, dv, deta, dw0) preallocated outputs
    returns (dq, dk, dv, deta [B, H, T] per token, dw0 [B, H, d, d] per sequence).
    """
    torch = _torch()
    B, H, T, d = q.shape
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q, k must have the same shape and dtype")
    if dz.shape != q.shape or tuple(e_saved.shape) != tuple(q.shape) or tuple(w_final.shape) != (B, H, d, d):
        raise ValueError("dz, e_saved must be [B, H, T, d] and w_final [B, H, d, d]")
    if e_saved.dtype != torch.float32 or w_final.dtype != torch.float32:
        raise TypeError("e_saved and w_final must be float32")
    if dw_final is not None and (tuple(dw_final.shape) != (B, H, d, d) or dw_final.dtype != torch.float32):
        raise ValueError("dw_final must be [B, H, d, d] float32")
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if out is None:
        dev = q.device
        out = (torch.empty((B, H, T, d), dtype=dz.dtype, device=dev),
               torch.empty((B, H, T, d), dtype=dz.dtype, device=dev),
               torch.empty((B, H, T, d), dtype=dz.dtype, device=dev),
               torch.empty((B, H, T), dtype=torch.float32, device=dev),
               torch.empty((B, H, d, d), dtype=torch.float32, device=dev))
    dq, dk, dv, deta, dw0 = out
    _check_dev(q, k, eta_t, w_final, e_saved, dz, dw_final, dq, dk, dv, deta, dw0)
    flags = TTT_FLAG_GENERIC if generic else 0
    desc = linear_desc(B, H, T, d, b, _dtype_code(q.dtype), _dtype_code(dz.dtype), 0, est, flags)
    st = lib().ttt_linear_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(eta_t), _ptr(w_final), _ptr(e_saved),
                              _ptr(dz), _ptr(dw_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta), _ptr(dw0),
                              _stream_handle(stream))
    _done(st, "ttt_linear_bwd")
    return dq, dk, dv, deta, dw0


def linear_bwd_kernel_name(B, H, T, d, b, in_dtype=TTT_BF16, out_dtype=TTT_F32, eta_strides=(0, 0, 0),
                           generic=False) -> Optional[str]:
    desc = linear_desc(B, H, T, d, b, in_dtype, out_dtype, 0, eta_strides, TTT_FLAG_GENERIC if generic else 0)
    name = lib().ttt_linear_bwd_kernel_name(ctypes.byref(desc))
    return None if name is None else name.decode()


def _w0_stride(w0, B, H, d) -> int:
    if tuple(w0.shape) == (H, d, d):
        return 0
    if tuple(w0.shape) == (B, H, d, d):
        return H * d * d
    raise ValueError(f"w0 shape {tuple(w0.shape)}: expected [H,d,d] or [B,H,d,d]")


def linear_kernel_name(B, H, T, d, b, in_dtype=TTT_BF16, out_dtype=TTT_F32, eta_strides=(0, 0, 0),
                       generic=False, primal=False, rows=None) -> Optional[str]:
    flags = (TTT_FLAG_GENERIC if generic else 0) | (TTT_FLAG_PRIMAL if primal else 0) | _rows_flag(rows)
    desc = linear_desc(B, H, T, d, b, in_dtype, out_dtype, 0, eta_strides, flags)
    name = lib().ttt_linear_kernel_name(ctypes.byref(desc))
    return None if name is None else name.decode()


def linear_fwd_chunked(q, k, v, w0, eta, b: int, nchunks: int, workspace=None, out_dtype=None,
                       w_final=None, z=None, rows=None, stream=None):
    """TTT-Linear forward with the sequence split into ``nchunks`` chunks run in parallel.

    Same arguments and result as :func:`linear_fwd` (to rounding).  ``workspace``
    is a uint8 device tensor of at least :func:`linear_chunked_workspace_bytes`
    bytes; one is allocated when omitted.
    """
    torch = _torch()
    B, H, T, d = q.shape
    if tuple(w0.shape) == (H, d, d):
        wstride = 0
    elif tuple(w0.shape) == (B, H, d, d):
        wstride = H * d * d
    else:
        raise ValueError(f"w0 shape {tuple(w0.shape)}: expected [H,d,d] or [B,H,d,d]")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=out_dtype, device=q.device)
    if w_final is None:
        w_final = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    desc = linear_desc(B, H, T, d, b, _dtype_code(q.dtype), _dtype_code(z.dtype), wstride, est, _rows_flag(rows))
    need = int(lib().ttt_linear_chunked_workspace_bytes(ctypes.byref(desc), int(nchunks)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check_dev(q, k, v, w0, eta_t, z, w_final, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ttt_linear_fwd_chunked(ctypes.byref(desc), int(nchunks), _ptr(q), _ptr(k), _ptr(v), _ptr(w0),
                                      _ptr(eta_t), _ptr(z), _ptr(w_final), _ptr(workspace), wbytes,
                                      _stream_handle(stream))
    _done(st, "ttt_linear_fwd_chunked")
    return z, w_final


def linear_fwd_chunked_noalloc(q, k, v, w0, eta, b: int, nchunks: int, out_dtype=None, w_final=None, z=None,
                               rows=None, stream=None):
    """:func:`linear_fwd_chunked` with the library's static scratch in place of a
    workspace (ttt_linear_fwd_chunked_noalloc: the call allocates no device
    memory; calls that overlap on one GPU race).  ``z`` and ``w_final`` are
    allocated here when omitted; pass them to keep the call allocation-free."""
    torch = _torch()
    B, H, T, d = q.shape
    wstride = _w0_stride(w0, B, H, d)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=out_dtype, device=q.device)
    if w_final is None:
        w_final = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    _check_dev(q, k, v, w0, eta_t, z, w_final)
    desc = linear_desc(B, H, T, d, b, _dtype_code(q.dtype), _dtype_code(z.dtype), wstride, est, _rows_flag(rows))
    st = lib().ttt_linear_fwd_chunked_noalloc(ctypes.byref(desc), int(nchunks), _ptr(q), _ptr(k), _ptr(v), _ptr(w0),
                                              _ptr(eta_t), _ptr(z), _ptr(w_final), _stream_handle(stream))
    _done(st, "ttt_linear_fwd_chunked_noalloc")
    return z, w_final


def linear_ln_fwd(q, k, v, w0, gamma, beta, eta, b: int, eps: float = 1e-6, out_dtype=None, w_final=None,
                  z=None, stream=None, g_saved=None, save: bool = False, primal: bool = False):
    """TTT-Linear with layer norm and residual inside f: f(x) = x + LN(W x).

    gamma, beta : [H, d] float32 (per head).  Other arguments as :func:`linear_fwd`.
    save / g_saved : also write G [B, H, T, d] float32, each token's update
    factor -eta delta as the forward applied it (delta the gradient of the
    token's loss with respect to W k at its mini-batch-start W), the input of
    :func:`linear_ln_bwd`; then returns (Z, W_final, G).
    primal : compute token by token (the primal form; any b, d in {16, 32, 64}).
    """
    torch = _torch()
    B, H, T, d = q.shape
    if tuple(gamma.shape) != (H, d) or tuple(beta.shape) != (H, d):
        raise ValueError("gamma and beta must be [H, d]")
    if gamma.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("gamma and beta must be float32")
    wstride = _w0_stride(w0, B, H, d)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=out_dtype, device=q.device)
    if w_final is None:
        w_final = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    save = save or g_saved is not None
    if save and g_saved is None:
        g_saved = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    _check_dev(q, k, v, w0, gamma, beta, eta_t, z, w_final, g_saved)
    desc = linear_desc(B, H, T, d, b, _dtype_code(q.dtype), _dtype_code(z.dtype), wstride, est,
                       TTT_FLAG_PRIMAL if primal else 0)
    if save:
        st = lib().ttt_linear_ln_fwd_save(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w0), _ptr(gamma),
                                          _ptr(beta), float(eps), _ptr(eta_t), _ptr(z), _ptr(w_final),
                                          _ptr(g_saved), _stream_handle(stream))
        _done(st, "ttt_linear_ln_fwd_save")
        return z, w_final, g_saved
    st = lib().ttt_linear_ln_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w0), _ptr(gamma),
                                 _ptr(beta), float(eps), _ptr(eta_t), _ptr(z), _ptr(w_final), _stream_handle(stream))
    _done(st, "ttt_linear_ln_fwd")
    return z, w_final


def linear_ln_bwd(q, k, v, eta, gamma, beta, w_final, g_saved, dz, b: int, eps: float = 1e-6,
                  dw_final=None, out=None, stream=None, generic: bool = False):
    """Backward of :func:`linear_ln_fwd`.

    q, k, v, eta, gamma, beta, eps : as given to the forward
    w_final, g_saved : from :func:`linear_ln_fwd` with save=True
    dz       : [B, H, T, d] gradient with respect to Z (its dtype is that of dq, dk, dv)
    dw_final : [B, H, d, d] float32 gradient with respect to W_final, or None (zero)
    out      : optional (dq, dk, dv, deta, dw0, dgamma, dbeta) preallocated outputs
    generic  : run the fp32 kernel (the cross-check) instead of the matrix-core one
    returns (dq, dk, dv, deta [B, H, T], dw0 [B, H, d, d], dgamma [B, H, d], dbeta [B, H, d]),
    the last three per sequence.
    """
    torch = _torch()
    B, H, T, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same shape and dtype")
    if tuple(gamma.shape) != (H, d) or tuple(beta.shape) != (H, d):
        raise ValueError("gamma and beta must be [H, d]")
    if gamma.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("gamma and beta must be float32")
    if dz.shape != q.shape or tuple(g_saved.shape) != tuple(q.shape) or tuple(w_final.shape) != (B, H, d, d):
        raise ValueError("dz, g_saved must be [B, H, T, d] and w_final [B, H, d, d]")
    if g_saved.dtype != torch.float32 or w_final.dtype != torch.float32:
        raise TypeError("g_saved and w_final must be float32")
    if dw_final is not None and (tuple(dw_final.shape) != (B, H, d, d) or dw_final.dtype != torch.float32):
        raise ValueError("dw_final must be [B, H, d, d] float32")
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if out is None:
        dev = q.device
        out = (torch.empty((B, H, T, d), dtype=dz.dtype, device=dev),
               torch.empty((B, H, T, d), dtype=dz.dtype, device=dev),
               torch.empty((B, H, T, d), dtype=dz.dtype, device=dev),
               torch.empty((B, H, T), dtype=torch.float32, device=dev),
               torch.empty((B, H, d, d), dtype=torch.float32, device=dev),
               torch.empty((B, H, d), dtype=torch.float32, device=dev),
               torch.empty((B, H, d), dtype=torch.float32, device=dev))
    dq, dk, dv, deta, dw0, dgamma, dbeta = out
    _check_dev(q, k, v, eta_t, gamma, beta, w_final, g_saved, dz, dw_final, *out)
    desc = linear_desc(B, H, T, d, b, _dtype_code(q.dtype), _dtype_code(dz.dtype), 0, est,
                       TTT_FLAG_GENERIC if generic else 0)
    st = lib().ttt_linear_ln_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(eta_t), _ptr(gamma),
                                 _ptr(beta), float(eps), _ptr(w_final), _ptr(g_saved), _ptr(dz),
                                 _ptr(dw_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta), _ptr(dw0),
                                 _ptr(dgamma), _ptr(dbeta), _stream_handle(stream))
    _done(st, "ttt_linear_ln_bwd")
    return dq, dk, dv, deta, dw0, dgamma, dbeta


def linear_ln_bwd_kernel_name(B, H, T, d, b, in_dtype=TTT_BF16, out_dtype=TTT_F32,
                              eta_strides=(0, 0, 0), generic: bool = False) -> Optional[str]:
    desc = linear_desc(B, H, T, d, b, in_dtype, out_dtype, 0, eta_strides, TTT_FLAG_GENERIC if generic else 0)
    name = lib().ttt_linear_ln_bwd_kernel_name(ctypes.byref(desc))
    return None if name is None else name.decode()


def linear_ln_kernel_name(B, H, T, d, b, in_dtype=TTT_BF16, out_dtype=TTT_F32, eta_strides=(0, 0, 0),
                          primal: bool = False) -> Optional[str]:
    desc = linear_desc(B, H, T, d, b, in_dtype, out_dtype, 0, eta_strides, TTT_FLAG_PRIMAL if primal else 0)
    name = lib().ttt_linear_ln_kernel_name(ctypes.byref(desc))
    return None if name is None else name.decode()


def linear_chunked_workspace_bytes(B, H, T, d, b, nchunks) -> int:
    desc = linear_desc(B, H, T, d, b, TTT_BF16, TTT_F32, 0, (0, 0, 0), 0)
    return int(lib().ttt_linear_chunked_workspace_bytes(ctypes.byref(desc), int(nchunks)))


def linear_decode(q, k, v, eta, w, wb, pos: int, b: int, out_dtype=None, z=None, stream=None):
    """Continue B*H sequences by T new tokens (primal form), state carried in place.

    q, k, v : [B, H, T, d];  w, wb : [B, H, d, d] float32 -- the state and the
    mini-batch-start state after ``pos`` tokens, both updated in place.
    eta     : float, [H] or [B, H, T] (indexed by the new tokens).
    returns Z [B, H, T, d].
    """
    torch = _torch()
    B, H, T, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same shape and dtype")
    if tuple(w.shape) != (B, H, d, d) or tuple(wb.shape) != (B, H, d, d):
        raise ValueError("w and wb must be [B, H, d, d]")
    if w.dtype != torch.float32 or wb.dtype != torch.float32:
        raise TypeError("w and wb must be float32")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=out_dtype, device=q.device)
    _check_dev(q, k, v, eta_t, z, w, wb)
    desc = linear_desc(B, H, T, d, b, _dtype_code(q.dtype), _dtype_code(z.dtype), 0, est, 0)
    st = lib().ttt_linear_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(eta_t), _ptr(z),
                                 _ptr(w), _ptr(wb), int(pos), _stream_handle(stream))
    _done(st, "ttt_linear_decode")
    return z


def linear_ln_decode(q, k, v, eta, gamma, beta, w, wb, pos: int, b: int, eps: float = 1e-6, out_dtype=None,
                     z=None, stream=None):
    """:func:`linear_decode` with f(x) = x + LN(W x); gamma, beta [H, d] float32."""
    torch = _torch()
    B, H, T, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same shape and dtype")
    if tuple(w.shape) != (B, H, d, d) or tuple(wb.shape) != (B, H, d, d):
        raise ValueError("w and wb must be [B, H, d, d]")
    if w.dtype != torch.float32 or wb.dtype != torch.float32:
        raise TypeError("w and wb must be float32")
    if tuple(gamma.shape) != (H, d) or tuple(beta.shape) != (H, d):
        raise ValueError("gamma and beta must be [H, d]")
    if gamma.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("gamma and beta must be float32")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=out_dtype, device=q.device)
    _check_dev(q, k, v, eta_t, gamma, beta, z, w, wb)
    desc = linear_desc(B, H, T, d, b, _dtype_code(q.dtype), _dtype_code(z.dtype), 0, est, 0)
    st = lib().ttt_linear_ln_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(eta_t), _ptr(gamma),
                                    _ptr(beta), float(eps), _ptr(z), _ptr(w), _ptr(wb), int(pos),
                                    _stream_handle(stream))
    _done(st, "ttt_linear_ln_decode")
    return z


# ---------------------------------------------------------------- TTT-MLP --

def mlp_desc(B, H, T, d, dh, b, in_dtype, out_dtype, w_batch_stride, eta_strides, flags=0) -> MlpDesc:
    return MlpDesc(B, H, T, d, dh, b, in_dtype, out_dtype, flags, 0, w_batch_stride, *eta_strides)


def mlp_fwd(q, k, v, w1, w2, eta, b: int, out_dtype=None, w1_final=None, w2_final=None, z=None,
            stream=None, primal: bool = False):
    """TTT-MLP forward: f(x) = W2 GELU(W1 x).

    w1 : [H, dh, d] or [B, H, dh, d] float32;  w2 : [H, d, dh] or [B, H, d, dh] float32
    primal : compute token by token (the primal form) instead of the dual form
    returns (Z, W1_final [B,H,dh,d], W2_final [B,H,d,dh]).
    """
    return _mlp_call(q, k, v, w1, w2, eta, b, out_dtype, w1_final, w2_final, z, stream,
                     flags=TTT_FLAG_PRIMAL if primal else 0)


def mlp_ln_fwd(q, k, v, w1, w2, gamma, beta, eta, b: int, eps: float = 1e-6, out_dtype=None, w1_final=None,
               w2_final=None, z=None, stream=None, primal: bool = False):
    """TTT-MLP with layer norm and residual inside f: f(x) = x + LN(W2 GELU(W1 x)).

    gamma, beta : [H, d] float32 (per head).  Other arguments as :func:`mlp_fwd`.
    primal : compute token by token (the primal form) instead of the dual form.
    """
    torch = _torch()
    H, d = q.shape[1], q.shape[3]
    if tuple(gamma.shape) != (H, d) or tuple(beta.shape) != (H, d):
        raise ValueError("gamma and beta must be [H, d]")
    if gamma.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("gamma and beta must be float32")
    return _mlp_call(q, k, v, w1, w2, eta, b, out_dtype, w1_final, w2_final, z, stream, ln=(gamma, beta, eps),
                     flags=TTT_FLAG_PRIMAL if primal else 0)


def _mlp_call(q, k, v, w1, w2, eta, b, out_dtype, w1_final, w2_final, z, stream, ln=None, flags=0):
    torch = _torch()
    B, H, T, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same shape and dtype")
    dh = w1.shape[-2]
    if w1.dtype != torch.float32 or w2.dtype != torch.float32:
        raise TypeError("w1, w2 must be float32")
    if tuple(w1.shape) == (H, dh, d) and tuple(w2.shape) == (H, d, dh):
        wstride = 0
    elif tuple(w1.shape) == (B, H, dh, d) and tuple(w2.shape) == (B, H, d, dh):
        wstride = H * dh * d
    else:
        raise ValueError("w1/w2 shapes: expected [H,dh,d]/[H,d,dh] or [B,H,dh,d]/[B,H,d,dh]")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=out_dtype, device=q.device)
    if w1_final is None:
        w1_final = torch.empty((B, H, dh, d), dtype=torch.float32, device=q.device)
    if w2_final is None:
        w2_final = torch.empty((B, H, d, dh), dtype=torch.float32, device=q.device)
    _check_dev(q, k, v, w1, w2, eta_t, z, w1_final, w2_final, *(ln[:2] if ln else ()))
    desc = mlp_desc(B, H, T, d, dh, b, _dtype_code(q.dtype), _dtype_code(z.dtype), wstride, est, flags)
    if ln is None:
        st = lib().ttt_mlp_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w1), _ptr(w2), _ptr(eta_t),
                               _ptr(z), _ptr(w1_final), _ptr(w2_final), _stream_handle(stream))
        _done(st, "ttt_mlp_fwd")
    else:
        gamma, beta, eps = ln
        st = lib().ttt_mlp_ln_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w1), _ptr(w2), _ptr(gamma),
                                  _ptr(beta), float(eps), _ptr(eta_t), _ptr(z), _ptr(w1_final), _ptr(w2_final),
                                  _stream_handle(stream))
        _done(st, "ttt_mlp_ln_fwd")
    return z, w1_final, w2_final


def mlp_kernel_name(B, H, T, d, dh, b, in_dtype=TTT_BF16, out_dtype=TTT_F32, eta_strides=(0, 0, 0),
                    primal: bool = False):
    desc = mlp_desc(B, H, T, d, dh, b, in_dtype, out_dtype, 0, eta_strides, TTT_FLAG_PRIMAL if primal else 0)
    name = lib().ttt_mlp_kernel_name(ctypes.byref(desc))
    return None if name is None else name.decode()


def mlp_ln_kernel_name(B, H, T, d, dh, b, in_dtype=TTT_BF16, out_dtype=TTT_F32, eta_strides=(0, 0, 0),
                       primal: bool = False):
    desc = mlp_desc(B, H, T, d, dh, b, in_dtype, out_dtype, 0, eta_strides, TTT_FLAG_PRIMAL if primal else 0)
    name = lib().ttt_mlp_ln_kernel_name(ctypes.byref(desc))
    return None if name is None else name.decode()


def mlp_bwd_workspace_bytes(B, H, T, d, dh, b) -> int:
    return int(lib().ttt_mlp_bwd_workspace_bytes(ctypes.byref(mlp_desc(B, H, T, d, dh, b, TTT_BF16, TTT_F32, 0,
                                                                         (0, 0, 0)))))


def mlp_bwd_kernel_name(B, H, T, d, dh, b, in_dtype=TTT_BF16, primal: bool = False) -> Optional[str]:
    """ttt_mlp_bwd_d64h256b16 (dual form, matrix cores) or ttt_mlp_bwd_d64h256 (primal form)."""
    desc = mlp_desc(B, H, T, d, dh, b, in_dtype, TTT_F32, 0, (0, 0, 0), TTT_FLAG_PRIMAL if primal else 0)
    name = lib().ttt_mlp_bwd_kernel_name(ctypes.byref(desc))
    return None if name is None else name.decode()


def mlp_bwd(q, k, v, w1, w2, eta, b: int, dz, dw1_final=None, dw2_final=None, workspace=None, out=None,
            stream=None, primal: bool = False):
    """Backward of :func:`mlp_fwd`: the gradients of L with respect to every
    input, given dz = dL/dZ and dw1_final, dw2_final = dL/dW1_final, dL/dW2_final
    (None for zero).  dz and the gradients are float32.  The dual form on the
    matrix cores runs where it applies (b = 16, T a multiple of 16, bf16
    inputs); primal=True, or any other shape, runs the primal form.

    workspace : uint8 device tensor of at least mlp_bwd_workspace_bytes bytes
    (allocated when omitted).  out : optional preallocated
    (dq, dk, dv, deta, dw1, dw2).
    returns (dq [B,H,T,d], dk, dv, deta [B,H,T], dw1 [B,H,dh,d], dw2 [B,H,d,dh]).
    """
    torch = _torch()
    B, H, T, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same shape and dtype")
    if tuple(dz.shape) != (B, H, T, d) or dz.dtype != torch.float32:
        raise ValueError("dz must be float32 [B, H, T, d]")
    dh = w1.shape[-2]
    if w1.dtype != torch.float32 or w2.dtype != torch.float32:
        raise TypeError("w1, w2 must be float32")
    if tuple(w1.shape) == (H, dh, d) and tuple(w2.shape) == (H, d, dh):
        wstride = 0
    elif tuple(w1.shape) == (B, H, dh, d) and tuple(w2.shape) == (B, H, d, dh):
        wstride = H * dh * d
    else:
        raise ValueError("w1/w2 shapes: expected [H,dh,d]/[H,d,dh] or [B,H,dh,d]/[B,H,d,dh]")
    for x, shape in ((dw1_final, (B, H, dh, d)), (dw2_final, (B, H, d, dh))):
        if x is not None and (tuple(x.shape) != shape or x.dtype != torch.float32):
            raise ValueError(f"final-state gradients must be float32 {shape}")
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    desc = mlp_desc(B, H, T, d, dh, b, _dtype_code(q.dtype), TTT_F32, wstride, est,
                    TTT_FLAG_PRIMAL if primal else 0)
    need = int(lib().ttt_mlp_bwd_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        f = dict(dtype=torch.float32, device=q.device)
        out = (torch.empty((B, H, T, d), **f), torch.empty((B, H, T, d), **f), torch.empty((B, H, T, d), **f),
               torch.empty((B, H, T), **f), torch.empty((B, H, dh, d), **f), torch.empty((B, H, d, dh), **f))
    dq, dk, dv, deta, dw1, dw2 = out
    _check_dev(q, k, v, w1, w2, eta_t, dz, dw1_final, dw2_final, workspace, *out)
    st = lib().ttt_mlp_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w1), _ptr(w2), _ptr(eta_t), _ptr(dz),
                           _ptr(dw1_final), _ptr(dw2_final), _ptr(workspace), workspace.numel(), _ptr(dq), _ptr(dk),
                           _ptr(dv), _ptr(deta), _ptr(dw1), _ptr(dw2), _stream_handle(stream))
    _done(st, "ttt_mlp_bwd")
    return dq, dk, dv, deta, dw1, dw2


def mlp_ln_bwd_kernel_name(B, H, T, d, dh, b, in_dtype=TTT_BF16) -> Optional[str]:
    name = lib().ttt_mlp_ln_bwd_kernel_name(ctypes.byref(mlp_desc(B, H, T, d, dh, b, in_dtype, TTT_F32, 0, (0, 0, 0))))
    return None if name is None else name.decode()


def mlp_ln_bwd(q, k, v, w1, w2, gamma, beta, eps: float, eta, b: int, dz, dw1_final=None, dw2_final=None,
               workspace=None, out=None, stream=None):
    """Backward of :func:`mlp_ln_fwd` (f(x) = x + LN(W2 GELU(W1 x))): as
    :func:`mlp_bwd`, with gamma, beta [H, d] float32 and eps the forward's.
    out : optional preallocated (dq, dk, dv, deta, dw1, dw2, dgamma, dbeta).
    returns (dq, dk, dv, deta, dw1, dw2, dgamma [B,H,d], dbeta [B,H,d]).
    """
    torch = _torch()
    B, H, T, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same shape and dtype")
    if tuple(dz.shape) != (B, H, T, d) or dz.dtype != torch.float32:
        raise ValueError("dz must be float32 [B, H, T, d]")
    dh = w1.shape[-2]
    if w1.dtype != torch.float32 or w2.dtype != torch.float32:
        raise TypeError("w1, w2 must be float32")
    if tuple(w1.shape) == (H, dh, d) and tuple(w2.shape) == (H, d, dh):
        wstride = 0
    elif tuple(w1.shape) == (B, H, dh, d) and tuple(w2.shape) == (B, H, d, dh):
        wstride = H * dh * d
    else:
        raise ValueError("w1/w2 shapes: expected [H,dh,d]/[H,d,dh] or [B,H,dh,d]/[B,H,d,dh]")
    if tuple(gamma.shape) != (H, d) or tuple(beta.shape) != (H, d):
        raise ValueError("gamma and beta must be [H, d]")
    if gamma.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("gamma and beta must be float32")
    for x, shape in ((dw1_final, (B, H, dh, d)), (dw2_final, (B, H, d, dh))):
        if x is not None and (tuple(x.shape) != shape or x.dtype != torch.float32):
            raise ValueError(f"final-state gradients must be float32 {shape}")
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    desc = mlp_desc(B, H, T, d, dh, b, _dtype_code(q.dtype), TTT_F32, wstride, est)
    need = int(lib().ttt_mlp_bwd_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        f = dict(dtype=torch.float32, device=q.device)
        out = (torch.empty((B, H, T, d), **f), torch.empty((B, H, T, d), **f), torch.empty((B, H, T, d), **f),
               torch.empty((B, H, T), **f), torch.empty((B, H, dh, d), **f), torch.empty((B, H, d, dh), **f),
               torch.empty((B, H, d), **f), torch.empty((B, H, d), **f))
    dq, dk, dv, deta, dw1, dw2, dg, db = out
    _check_dev(q, k, v, w1, w2, gamma, beta, eta_t, dz, dw1_final, dw2_final, workspace, *out)
    st = lib().ttt_mlp_ln_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w1), _ptr(w2), _ptr(gamma),
                              _ptr(beta), float(eps), _ptr(eta_t), _ptr(dz), _ptr(dw1_final), _ptr(dw2_final),
                              _ptr(workspace), workspace.numel(), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta),
                              _ptr(dw1), _ptr(dw2), _ptr(dg), _ptr(db), _stream_handle(stream))
    _done(st, "ttt_mlp_ln_bwd")
    return dq, dk, dv, deta, dw1, dw2, dg, db


def mlp_decode(q, k, v, eta, w1, w2, w1b, w2b, pos: int, b: int, out_dtype=None, z=None, stream=None, ln=None):
    """Continue B*H TTT-MLP sequences by T new tokens (primal form), state carried in place.

    q, k, v : [B, H, T, d];  w1, w1b : [B, H, dh, d], w2, w2b : [B, H, d, dh]
    float32 -- the state and the mini-batch-start state after ``pos`` tokens,
    all updated in place.  eta : float, [H] or [B, H, T] (indexed by the new tokens).
    ln : (gamma, beta, eps) for f(x) = x + LN(W2 GELU(W1 x)) (ttt_mlp_ln_decode),
    gamma and beta [H, d] float32.
    returns Z [B, H, T, d].
    """
    torch = _torch()
    B, H, T, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same shape and dtype")
    dh = w1.shape[-2]
    if (tuple(w1.shape) != (B, H, dh, d) or tuple(w1b.shape) != (B, H, dh, d) or
            tuple(w2.shape) != (B, H, d, dh) or tuple(w2b.shape) != (B, H, d, dh)):
        raise ValueError("w1, w1b must be [B, H, dh, d] and w2, w2b [B, H, d, dh]")
    if any(x.dtype != torch.float32 for x in (w1, w2, w1b, w2b)):
        raise TypeError("the states must be float32")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    eta_t, est = eta_layout(eta, B, H, T, q.device)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=out_dtype, device=q.device)
    desc = mlp_desc(B, H, T, d, dh, b, _dtype_code(q.dtype), _dtype_code(z.dtype), 0, est)
    if ln is not None:
        gamma, beta, eps = ln
        if tuple(gamma.shape) != (H, d) or tuple(beta.shape) != (H, d):
            raise ValueError("gamma and beta must be [H, d]")
        if gamma.dtype != torch.float32 or beta.dtype != torch.float32:
            raise TypeError("gamma and beta must be float32")
        _check_dev(q, k, v, eta_t, z, w1, w2, w1b, w2b, gamma, beta)
        st = lib().ttt_mlp_ln_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(eta_t), _ptr(gamma),
                                     _ptr(beta), float(eps), _ptr(z), _ptr(w1), _ptr(w2), _ptr(w1b), _ptr(w2b),
                                     int(pos), _stream_handle(stream))
        _done(st, "ttt_mlp_ln_decode")
        return z
    _check_dev(q, k, v, eta_t, z, w1, w2, w1b, w2b)
    st = lib().ttt_mlp_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(eta_t), _ptr(z), _ptr(w1),
                              _ptr(w2), _ptr(w1b), _ptr(w2b), int(pos), _stream_handle(stream))
    _done(st, "ttt_mlp_decode")
    return z
