"""ctypes wrapper of the fp64 oracle (test infrastructure only).

Inputs may be any real numpy arrays of the documented shapes; they are widened
to contiguous float64.  Outputs are float64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_OUT_DIR, "liboracle.so")
_lock = threading.Lock()
_handle: Optional[ctypes.CDLL] = None


def lib_path() -> str:
    return _LIB


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle C source with gcc (-O2, OpenMP) into a shared library."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_DP = ctypes.POINTER(ctypes.c_double)


def _declare(h: ctypes.CDLL) -> ctypes.CDLL:
    i = ctypes.c_int
    d = ctypes.c_double
    h.oracle_space_fwd.argtypes = [i] * 6 + [i, i, d] + [_DP] * 5
    h.oracle_space_bwd.argtypes = [i] * 6 + [i, i, d] + [_DP] * 7
    h.oracle_time_fwd.argtypes = [i] * 6 + [i, d] + [_DP] * 5
    h.oracle_time_bwd.argtypes = [i] * 6 + [i, d] + [_DP] * 7
    h.oracle_time_decode_fwd.argtypes = [i] * 7 + [d, i, i] + [_DP] * 5
    L = ctypes.c_long
    h.oracle_rmsnorm_qkv_fwd.argtypes = [L, i, i, i, i, d] + [_DP] * 7
    h.oracle_rmsnorm_qkv_fwd.restype = ctypes.c_int
    h.oracle_out_proj_fwd.argtypes = [L, i, i, _DP, _DP, _DP, _DP]
    h.oracle_out_proj_fwd.restype = ctypes.c_int
    for f in (h.oracle_space_fwd, h.oracle_space_bwd, h.oracle_time_fwd, h.oracle_time_bwd,
              h.oracle_time_decode_fwd):
        f.restype = ctypes.c_int
    h.oracle_set_threads.argtypes = [i]
    h.oracle_set_threads.restype = None
    h.oracle_max_threads.argtypes = []
    h.oracle_max_threads.restype = ctypes.c_int
    return h


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the oracle library (building it first if it does not exist).
    With ``path`` given, load that file instead (used by planted-mistake tests)."""
    global _handle
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _handle is None:
            if not os.path.exists(_LIB):
                build()
            _handle = _declare(ctypes.CDLL(_LIB))
        return _handle


def set_threads(n: int) -> None:
    load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(load().oracle_max_threads())


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_DP)


def _dims(q, k):
    B, T, N, Hq, D = q.shape
    Hkv = k.shape[3]
    if k.shape != (B, T, N, Hkv, D):
        raise ValueError("k shape %s does not match q shape %s" % (k.shape, q.shape))
    return B, T, N, Hq, Hkv, D


def _check(rc: int, what: str):
    if rc == -1:
        raise ValueError("oracle %s: invalid arguments" % what)
    if rc == -2:
        raise ValueError("oracle %s: a query sees no key" % what)
    if rc != 0:
        raise RuntimeError("oracle %s: rc=%d" % (what, rc))


def space_fwd(q, k, v, agent_begin: int = 0, agent_count: int = 0, scale: float = 0.0,
              lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Space attention forward: returns (o, lse) in float64."""
    h = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, N, Hq, Hkv, D = _dims(q, k)
    o = np.zeros_like(q)
    lse = np.zeros((B, T, N, Hq))
    _check(h.oracle_space_fwd(B, T, N, Hq, Hkv, D, agent_begin, agent_count, scale,
                              _p(q), _p(k), _p(v), _p(o), _p(lse)), "space_fwd")
    return o, lse


def space_bwd(q, k, v, dout, agent_begin: int = 0, agent_count: int = 0, scale: float = 0.0,
              lib: Optional[ctypes.CDLL] = None):
    """Space attention backward: returns (dq, dk, dv) in float64."""
    h = lib or load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, T, N, Hq, Hkv, D = _dims(q, k)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    _check(h.oracle_space_bwd(B, T, N, Hq, Hkv, D, agent_begin, agent_count, scale,
                              _p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk), _p(dv)), "space_bwd")
    return dq, dk, dv


def time_fwd(q, k, v, window: int = 0, scale: float = 0.0,
             lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Causal sliding-window time attention forward: returns (o, lse)."""
    h = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, N, Hq, Hkv, D = _dims(q, k)
    o = np.zeros_like(q)
    lse = np.zeros((B, T, N, Hq))
    _check(h.oracle_time_fwd(B, T, N, Hq, Hkv, D, window, scale,
                             _p(q), _p(k), _p(v), _p(o), _p(lse)), "time_fwd")
    return o, lse


def time_bwd(q, k, v, dout, window: int = 0, scale: float = 0.0,
             lib: Optional[ctypes.CDLL] = None):
    """Causal sliding-window time attention backward: returns (dq, dk, dv)."""
    h = lib or load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, T, N, Hq, Hkv, D = _dims(q, k)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    _check(h.oracle_time_bwd(B, T, N, Hq, Hkv, D, window, scale,
                             _p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk), _p(dv)), "time_bwd")
    return dq, dk, dv


def time_decode_fwd(q, kc, vc, q_frame0: int, window: int = 0, scale: float = 0.0,
                    lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Rollout decode of time attention: queries are the frames q_frame0 ..
    q_frame0 + Tq - 1 (q is (B,Tq,N,Hq,D)); kc, vc (B,C,N,Hkv,D) hold absolute
    frame f at ring position f % C.  Returns (o, lse) in float64."""
    h = lib or load()
    q, kc, vc = _f64(q), _f64(kc), _f64(vc)
    B, Tq, N, Hq, D = q.shape
    C, Hkv = kc.shape[1], kc.shape[3]
    if kc.shape != (B, C, N, Hkv, D) or vc.shape != kc.shape:
        raise ValueError("cache shape %s does not match q shape %s" % (kc.shape, q.shape))
    o = np.zeros_like(q)
    lse = np.zeros((B, Tq, N, Hq))
    _check(h.oracle_time_decode_fwd(B, Tq, N, Hq, Hkv, D, window, scale, C, q_frame0,
                                    _p(q), _p(kc), _p(vc), _p(o), _p(lse)), "time_decode_fwd")
    return o, lse


def fwd(w, q, k, v, scale: float = 0.0, lib=None):
    """Forward of workload ``w`` (a configs.Workload-like object)."""
    if w.op == "space":
        return space_fwd(q, k, v, w.agent_begin, w.agent_count, scale, lib=lib)
    return time_fwd(q, k, v, w.window, scale, lib=lib)


def bwd(w, q, k, v, dout, scale: float = 0.0, lib=None):
    """Backward of workload ``w``."""
    if w.op == "space":
        return space_bwd(q, k, v, dout, w.agent_begin, w.agent_count, scale, lib=lib)
    return time_bwd(q, k, v, dout, w.window, scale, lib=lib)


def rmsnorm_qkv_fwd(x, gamma, w, Hq: int, Hkv: int, D: int, eps: float = 1e-6,
                    lib: Optional[ctypes.CDLL] = None):
    """RMS norm (fp64, gain ``gamma``), then the QKV projection with weight
    ``w`` ((Hq+2Hkv)*D, dm), with no rounding in between.  x is (M, dm).
    Returns (q (M, Hq*D), k (M, Hkv*D), v (M, Hkv*D), rstd (M,))."""
    h = lib or load()
    x, gamma, w = _f64(x), _f64(gamma), _f64(w)
    M, dm = x.shape
    if gamma.shape != (dm,) or w.shape != ((Hq + 2 * Hkv) * D, dm):
        raise ValueError("shapes x %s gamma %s w %s" % (x.shape, gamma.shape, w.shape))
    q = np.zeros((M, Hq * D))
    k = np.zeros((M, Hkv * D))
    v = np.zeros((M, Hkv * D))
    rstd = np.zeros(M)
    _check(h.oracle_rmsnorm_qkv_fwd(M, dm, Hq, Hkv, D, eps, _p(x), _p(gamma), _p(w),
                                    _p(q), _p(k), _p(v), _p(rstd)), "rmsnorm_qkv_fwd")
    return q, k, v, rstd


def out_proj_fwd(o, w, residual=None, lib: Optional[ctypes.CDLL] = None):
    """y = residual + o w^T: o (M, din), w (dm, din), residual (M, dm) or None."""
    h = lib or load()
    o, w = _f64(o), _f64(w)
    M, din = o.shape
    dm = w.shape[0]
    if w.shape != (dm, din):
        raise ValueError("w shape %s" % (w.shape,))
    y = np.zeros((M, dm))
    res = None if residual is None else _f64(residual)
    if res is not None and res.shape != (M, dm):
        raise ValueError("residual shape %s" % (res.shape,))
    rp = ctypes.cast(None, _DP) if res is None else _p(res)
    _check(h.oracle_out_proj_fwd(M, dm, din, _p(o), _p(w), rp, _p(y)), "out_proj_fwd")
    return y
