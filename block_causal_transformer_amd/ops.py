"""Python binding of the C ABI in include/bca.h (argument marshalling only).

Every attention step runs in the HIP kernels of ``libbca.so``; torch only
provides device memory (``tensor.data_ptr()``) and streams
(``torch.cuda.current_stream().cuda_stream``).  There is no fallback: if the
library is not built, or a call fails, an exception is raised.

Raw entry points carry the C names and arguments:
``space_attn_fwd``, ``space_attn_bwd``, ``time_attn_fwd``, ``time_attn_bwd``,
``time_attn_bwd_noalloc``, ``time_attn_decode_fwd``, ``rmsnorm_qkv_fwd``, ``out_proj_fwd``,
``bca_bwd_workspace_bytes``, ``bca_qkv_workspace_bytes``, ``bca_status_string``,
``bca_last_error``, ``bca_abi_version``.  ``attn_fwd`` / ``attn_bwd`` /
``attn_decode_fwd`` / ``qkv_proj`` / ``out_proj`` allocate the outputs with
torch and call them.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbca.so")

BCA_OK, BCA_ERR_INVALID_ARG, BCA_ERR_UNSUPPORTED, BCA_ERR_HIP = 0, 1, 2, 3
BCA_BF16, BCA_F32 = 0, 1
BCA_OP_SPACE, BCA_OP_TIME = 0, 1
ABI_VERSION = 4


class BcaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("N", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class BcaMask(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int32), ("window", ctypes.c_int32),
                ("agent_begin", ctypes.c_int32), ("agent_count", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class BcaProjShape(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("d_model", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32)]


class BcaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__("%s: %s (%s)" % (where, _STATUS.get(status, status), detail))
        self.status = status


_STATUS = {0: "BCA_OK", 1: "BCA_ERR_INVALID_ARG", 2: "BCA_ERR_UNSUPPORTED", 3: "BCA_ERR_HIP"}
_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None

EXPORTED = ["space_attn_fwd", "space_attn_bwd", "time_attn_fwd", "time_attn_bwd",
            "time_attn_bwd_noalloc", "time_attn_decode_fwd", "rmsnorm_qkv_fwd", "out_proj_fwd", "bca_bwd_workspace_bytes",
            "bca_qkv_workspace_bytes", "bca_status_string", "bca_last_error", "bca_abi_version"]


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbca.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libbca.so not found at %s: build it with "
                               "`python -m block_causal_transformer_amd.build`" % path)
        h = ctypes.CDLL(path)
        P = ctypes.c_void_p
        SP = ctypes.POINTER(BcaShape)
        MP = ctypes.POINTER(BcaMask)
        for name in ("space_attn_fwd", "time_attn_fwd"):
            f = getattr(h, name)
            f.argtypes = [SP, MP, P, P, P, P, P, P]
            f.restype = ctypes.c_int
        for name in ("space_attn_bwd", "time_attn_bwd"):
            f = getattr(h, name)
            f.argtypes = [SP, MP, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
            f.restype = ctypes.c_int
        h.time_attn_bwd_noalloc.argtypes = [SP, MP, P, P, P, P, P, P, P, P, P, P]
        h.time_attn_bwd_noalloc.restype = ctypes.c_int
        h.time_attn_decode_fwd.argtypes = [SP, MP, P, P, P, ctypes.c_int32, ctypes.c_int32, P, P, P]
        h.time_attn_decode_fwd.restype = ctypes.c_int
        PP = ctypes.POINTER(BcaProjShape)
        h.rmsnorm_qkv_fwd.argtypes = [PP, P, P, ctypes.c_float, P, P, P, P, P, P, ctypes.c_size_t, P]
        h.rmsnorm_qkv_fwd.restype = ctypes.c_int
        h.out_proj_fwd.argtypes = [PP, P, P, P, P, P]
        h.out_proj_fwd.restype = ctypes.c_int
        h.bca_qkv_workspace_bytes.argtypes = [PP]
        h.bca_qkv_workspace_bytes.restype = ctypes.c_size_t
        h.bca_bwd_workspace_bytes.argtypes = [ctypes.c_int, SP]
        h.bca_bwd_workspace_bytes.restype = ctypes.c_size_t
        h.bca_status_string.argtypes = [ctypes.c_int]
        h.bca_status_string.restype = ctypes.c_char_p
        h.bca_last_error.argtypes = []
        h.bca_last_error.restype = ctypes.c_char_p
        h.bca_abi_version.argtypes = []
        h.bca_abi_version.restype = ctypes.c_int
        if h.bca_abi_version() != ABI_VERSION:
            raise RuntimeError("libbca.so ABI version %d, binding expects %d"
                               % (h.bca_abi_version(), ABI_VERSION))
        _lib = h
        return h


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _ref(x):
    return None if x is None else ctypes.byref(x)


def _check(rc: int, where: str):
    if rc != BCA_OK:
        raise BcaError(rc, where, bca_last_error())


# ------------------------------------------------------------ raw C names

def space_attn_fwd(shape: BcaShape, mask: BcaMask, q, k, v, o, lse, stream=None) -> int:
    return load().space_attn_fwd(_ref(shape), _ref(mask), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(o), _ptr(lse), stream)


def time_attn_fwd(shape: BcaShape, mask: BcaMask, q, k, v, o, lse, stream=None) -> int:
    return load().time_attn_fwd(_ref(shape), _ref(mask), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(o), _ptr(lse), stream)


def space_attn_bwd(shape: BcaShape, mask: BcaMask, q, k, v, o, lse, dout, dq, dk, dv,
                   workspace=None, workspace_bytes: int = 0, stream=None) -> int:
    return load().space_attn_bwd(_ref(shape), _ref(mask), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(workspace), workspace_bytes, stream)


def time_attn_bwd(shape: BcaShape, mask: BcaMask, q, k, v, o, lse, dout, dq, dk, dv,
                  workspace=None, workspace_bytes: int = 0, stream=None) -> int:
    return load().time_attn_bwd(_ref(shape), _ref(mask), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(workspace), workspace_bytes, stream)


def time_attn_bwd_noalloc(shape: BcaShape, mask: BcaMask, q, k, v, o, lse, dout, dq, dk, dv,
                          stream=None) -> int:
    return load().time_attn_bwd_noalloc(_ref(shape), _ref(mask), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                        _ptr(dv), stream)


def time_attn_decode_fwd(shape: BcaShape, mask: BcaMask, q, k_cache, v_cache, cache_frames: int,
                         q_frame0: int, o, lse, stream=None) -> int:
    return load().time_attn_decode_fwd(_ref(shape), _ref(mask), _ptr(q), _ptr(k_cache),
                                       _ptr(v_cache), cache_frames, q_frame0, _ptr(o), _ptr(lse),
                                       stream)


def rmsnorm_qkv_fwd(shape: BcaProjShape, x, gain, eps: float, w_qkv, q, k, v, rstd, workspace,
                    workspace_bytes: int, stream=None) -> int:
    return load().rmsnorm_qkv_fwd(_ref(shape), _ptr(x), _ptr(gain), eps, _ptr(w_qkv), _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(rstd), _ptr(workspace), workspace_bytes,
                                  stream)


def out_proj_fwd(shape: BcaProjShape, o, w_o, residual, y, stream=None) -> int:
    return load().out_proj_fwd(_ref(shape), _ptr(o), _ptr(w_o), _ptr(residual), _ptr(y), stream)


def bca_qkv_workspace_bytes(shape: BcaProjShape) -> int:
    return int(load().bca_qkv_workspace_bytes(_ref(shape)))


def bca_bwd_workspace_bytes(op: int, shape: BcaShape) -> int:
    return int(load().bca_bwd_workspace_bytes(op, _ref(shape)))


def bca_status_string(status: int) -> str:
    return load().bca_status_string(status).decode()


def bca_last_error() -> str:
    return load().bca_last_error().decode()


def bca_abi_version() -> int:
    return int(load().bca_abi_version())


# ------------------------------------------------------- torch conveniences

def make_shape(q, k) -> BcaShape:
    import torch
    B, T, N, Hq, D = q.shape
    dt = {torch.bfloat16: BCA_BF16, torch.float32: BCA_F32}.get(q.dtype)
    if dt is None:
        raise TypeError("q must be bfloat16 or float32, got %s" % q.dtype)
    return BcaShape(B, T, N, Hq, k.shape[3], D, dt)


def make_mask(op: str, window: int = 0, agent_begin: int = 0, agent_count: int = 0,
              scale: float = 0.0) -> BcaMask:
    if op == "space":
        return BcaMask(0, 0, agent_begin, agent_count, scale)
    return BcaMask(1, window, 0, 0, scale)


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def attn_fwd(op: str, q, k, v, window: int = 0, agent_begin: int = 0, agent_count: int = 0,
             scale: float = 0.0, out: Optional[Tuple] = None, stream=None):
    """Forward of space or time attention on torch device tensors.
    Returns (o, lse); ``out`` may pass preallocated (o, lse)."""
    import torch
    shape = make_shape(q, k)
    mask = make_mask(op, window, agent_begin, agent_count, scale)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:4], dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    f = space_attn_fwd if op == "space" else time_attn_fwd
    _check(f(shape, mask, q, k, v, o, lse, _stream(stream)), op + "_attn_fwd")
    return o, lse


def attn_bwd(op: str, q, k, v, o, lse, dout, window: int = 0, agent_begin: int = 0,
             agent_count: int = 0, scale: float = 0.0, out: Optional[Tuple] = None,
             workspace=None, stream=None):
    """Backward of space or time attention.  Returns (dq, dk, dv)."""
    import torch
    shape = make_shape(q, k)
    mask = make_mask(op, window, agent_begin, agent_count, scale)
    opc = BCA_OP_SPACE if op == "space" else BCA_OP_TIME
    need = bca_bwd_workspace_bytes(opc, shape)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
    f = space_attn_bwd if op == "space" else time_attn_bwd
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(f(shape, mask, q, k, v, o, lse, dout, dq, dk, dv, workspace if need else None,
             ws_bytes if need else 0, _stream(stream)), op + "_attn_bwd")
    return dq, dk, dv


def attn_decode_fwd(q, k_cache, v_cache, q_frame0: int, window: int = 0, scale: float = 0.0,
                    out: Optional[Tuple] = None, stream=None):
    """Rollout decode of time attention: q (B, Tq, N, Hq, D) are the frames
    q_frame0 .. q_frame0 + Tq - 1; k_cache, v_cache (B, C, N, Hkv, D) hold
    absolute frame f at position f % C.  Returns (o, lse)."""
    import torch
    shape = make_shape(q, k_cache)
    mask = make_mask("time", window, 0, 0, scale)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:4], dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    _check(time_attn_decode_fwd(shape, mask, q, k_cache, v_cache, k_cache.shape[1], q_frame0,
                                o, lse, _stream(stream)), "time_attn_decode_fwd")
    return o, lse


def qkv_proj(x, gain, w_qkv, Hq: int, Hkv: int, D: int, eps: float = 1e-6, out=None,
             workspace=None, stream=None):
    """RMS norm + QKV projection on torch tensors: x (M, d_model) bf16, gain
    (d_model) fp32, w_qkv ((Hq+2Hkv)*D, d_model) bf16.  Returns (q (M, Hq*D),
    k (M, Hkv*D), v (M, Hkv*D), rstd (M,))."""
    import torch
    M, dm = x.shape
    shape = BcaProjShape(M, dm, Hq, Hkv, D)
    need = bca_qkv_workspace_bytes(shape)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if out is None:
        q = torch.empty((M, Hq * D), dtype=torch.bfloat16, device=x.device)
        k = torch.empty((M, Hkv * D), dtype=torch.bfloat16, device=x.device)
        v = torch.empty_like(k)
        rstd = torch.empty(M, dtype=torch.float32, device=x.device)
    else:
        q, k, v, rstd = out
    _check(rmsnorm_qkv_fwd(shape, x, gain, eps, w_qkv, q, k, v, rstd, workspace,
                           workspace.numel() * workspace.element_size(), _stream(stream)),
           "rmsnorm_qkv_fwd")
    return q, k, v, rstd


def out_proj(o, w_o, residual=None, Hq: int = 0, D: int = 0, out=None, stream=None):
    """y = residual + o w_o^T on torch tensors: o (M, Hq*D), w_o (d_model,
    Hq*D) bf16, residual (M, d_model) bf16 or None."""
    import torch
    M, din = o.shape
    dm = w_o.shape[0]
    if not Hq or not D:
        D = 64 if din % 64 == 0 else 8
        Hq = din // D
    shape = BcaProjShape(M, dm, Hq, 1, D)
    y = torch.empty((M, dm), dtype=torch.bfloat16, device=o.device) if out is None else out
    _check(out_proj_fwd(shape, o, w_o, residual, y, _stream(stream)), "out_proj_fwd")
    return y


def workload_kwargs(w) -> dict:
    """Mask keyword arguments of a configs.Workload."""
    if w.op == "space":
        return {"agent_begin": w.agent_begin, "agent_count": w.agent_count}
    return {"window": w.window}
