"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, the bench and the smoke check.  It draws
random numbers and rounds them to the storage precision; it holds none of the
attention arithmetic.

Recipe (one workload = one ``configs.Workload``):

* ``SeedSequence(w.seed + variant)`` is spawned into five child streams, in
  order: q, k, v, dO, and an auxiliary stream for structure choices.
* Each of q, k, v, dO is ``standard_normal(float32)`` of its full shape,
  multiplied by ``w.value_scale`` (CoinRun inputs are scaled by 1/sqrt(64);
  dO by ``w.dout_scale``, 1 unless a test keeps its gradients small),
  then rounded to bf16 with round-to-nearest-even when the workload is bf16.
  fp32 workloads keep the fp32 draws.
* Tokenizer encoder workloads (``w.shared_rows``): in every frame a seeded
  random choice of ``count`` of the patch slots ``[begin, begin+patches)``
  stands for MAE-masked patches; those slots all carry one shared q/k/v row
  per head (the shared mask token after projection).  This changes values
  only, never shapes or work.

Arrays are returned as float32 numpy arrays whose values are exactly
representable in the storage dtype; ``to_bf16_bits`` gives the bf16 bit
patterns for upload.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .configs import DecodeWorkload, ProjWorkload, Workload


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Finite inputs only (the generator never produces inf or NaN)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even); returns fp32."""
    return bf16_to_f32(bf16_bits(x))


def _draw(rng: np.random.Generator, shape, scale: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == "bf16":
        x = bf16_round(x)
    return x


def make_inputs(w: Workload, variant: int = 0, with_dout: bool = True) -> Dict[str, np.ndarray]:
    """Draw q, k, v (and dO) for workload ``w``.

    Returns a dict of float32 arrays: q, dout of shape (B,T,N,Hq,D); k, v of
    shape (B,T,N,Hkv,D).  Same (w, variant) -> bitwise the same arrays.
    """
    ss = np.random.SeedSequence(w.seed + variant)
    rq, rk, rv, rd, raux = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5)]
    q = _draw(rq, w.q_shape(), w.value_scale, w.dtype)
    k = _draw(rk, w.kv_shape(), w.value_scale, w.dtype)
    v = _draw(rv, w.kv_shape(), w.value_scale, w.dtype)
    out = {"q": q, "k": k, "v": v}
    if w.shared_rows is not None:
        begin, count = w.shared_rows
        patches = 920 if w.N >= 920 else w.N  # 368x640 frame in 16x16 patches
        shared_q = _draw(raux, (w.Hq, w.D), w.value_scale, w.dtype)
        shared_k = _draw(raux, (w.Hkv, w.D), w.value_scale, w.dtype)
        shared_v = _draw(raux, (w.Hkv, w.D), w.value_scale, w.dtype)
        for b in range(w.B):
            for t in range(w.T):
                slots = begin + raux.choice(patches, size=count, replace=False)
                q[b, t, slots] = shared_q
                k[b, t, slots] = shared_k
                v[b, t, slots] = shared_v
    if with_dout:
        out["dout"] = _draw(rd, w.q_shape(), w.dout_scale, w.dtype)
    return out


def masked_slots(w: Workload, variant: int = 0) -> Optional[np.ndarray]:
    """For shared-row workloads, the (B*T, count) slot indices that carry the
    shared row (recomputed from the same auxiliary stream)."""
    if w.shared_rows is None:
        return None
    ss = np.random.SeedSequence(w.seed + variant)
    raux = np.random.Generator(np.random.PCG64(ss.spawn(5)[4]))
    begin, count = w.shared_rows
    patches = 920 if w.N >= 920 else w.N
    _draw(raux, (w.Hq, w.D), w.value_scale, w.dtype)
    _draw(raux, (w.Hkv, w.D), w.value_scale, w.dtype)
    _draw(raux, (w.Hkv, w.D), w.value_scale, w.dtype)
    rows = []
    for _ in range(w.B * w.T):
        rows.append(begin + raux.choice(patches, size=count, replace=False))
    return np.stack(rows)


def make_decode_inputs(w: DecodeWorkload, variant: int = 0) -> Dict[str, np.ndarray]:
    """Draw q (B,Tq,N,Hq,D) and the ring caches k_cache, v_cache (B,C,N,Hkv,D)
    of a decode workload: ``SeedSequence(w.seed + variant)`` spawned into q, k,
    v streams, standard normal, rounded like ``make_inputs``.  Every ring
    position is filled (positions the queries do not read carry values too)."""
    ss = np.random.SeedSequence(w.seed + variant)
    rq, rk, rv = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]
    return {"q": _draw(rq, w.q_shape(), 1.0, w.dtype),
            "k_cache": _draw(rk, w.cache_shape(), 1.0, w.dtype),
            "v_cache": _draw(rv, w.cache_shape(), 1.0, w.dtype)}


def make_proj_inputs(w: ProjWorkload, variant: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of the projections: ``SeedSequence(w.seed + variant)`` spawned into
    six streams, in order x, gain, w_qkv, o, w_o, residual.  x, o, residual are
    N(0,1) rounded to bf16; the gain is 1 + N(0, 0.1^2) in fp32; the weights
    are N(0, 1/in_features) rounded to bf16 (unit-variance outputs)."""
    ss = np.random.SeedSequence(w.seed + variant)
    r = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(6)]
    din = w.Hq * w.D
    return {
        "x": _draw(r[0], (w.M, w.d_model), 1.0, "bf16"),
        "gain": (1.0 + 0.1 * r[1].standard_normal(w.d_model, dtype=np.float32)).astype(np.float32),
        "w_qkv": _draw(r[2], (w.n_qkv, w.d_model), float(1.0 / np.sqrt(w.d_model)), "bf16"),
        "o": _draw(r[3], (w.M, din), 1.0, "bf16"),
        "w_o": _draw(r[4], (w.d_model, din), float(1.0 / np.sqrt(din)), "bf16"),
        "residual": _draw(r[5], (w.M, w.d_model), 1.0, "bf16"),
    }
