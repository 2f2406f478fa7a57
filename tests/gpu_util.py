"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the fp64 oracle on the same seeded inputs, compare."""
from __future__ import annotations

import math
import os
from typing import Dict, Optional, Sequence

import numpy as np

from block_causal_transformer_amd import configs as C
from block_causal_transformer_amd import gen, ops
from oracle import oracle as O

# Tolerances (per output tensor, over the whole compared tensor):
#  bf16 path: relative L2 <= 5e-3, and per element both
#             |got - bf16(want)| <= max(2e-2, ulp_bf16(want))     (a)
#             |got - want| - ulp_bf16(want)/2 <= 2e-2             (b)
#             where bf16(want) is the oracle rounded to nearest even.  (a)
#             is the 2e-2 bar against the best bf16 result there is; where
#             one bf16 step is larger than the bar (|want| >= 4) it allows
#             that one step, since an fp32 result a hair from a rounding
#             midpoint may round either way.  (b) bounds the distance to the
#             exact value beyond the output's own rounding.  Time-attention
#             dV reaches |16| at the dynamics shape, where one step is
#             0.0625, so even the exactly rounded fp64 result misses a bare
#             |got - want| <= 2e-2.
#             LSE (fp32): max-abs <= 1e-3.
#  fp32 path: max-abs <= 1e-5 and relative L2 <= 1e-5; LSE max-abs <= 1e-5.
TOL = {
    "bf16": {"max_abs": 2e-2, "rel_l2": 5e-3, "lse": 1e-3, "storage_ulp": True},
    "f32": {"max_abs": 1e-5, "rel_l2": 1e-5, "lse": 1e-5, "storage_ulp": False},
}


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (8 significant bits, ties to even), as
    float64; magnitudes stay far inside bf16's exponent range here."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def torch_dtype(w):
    import torch
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def to_dev(x: np.ndarray, w):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(torch_dtype(w))


def to_np(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def run_hip(w, inp: Dict[str, np.ndarray], bwd: bool = True, scale: float = 0.0):
    """Forward (and backward) through the C ABI; returns numpy float64 arrays."""
    import torch
    q, k, v = to_dev(inp["q"], w), to_dev(inp["k"], w), to_dev(inp["v"], w)
    kw = ops.workload_kwargs(w)
    o, lse = ops.attn_fwd(w.op, q, k, v, scale=scale, **kw)
    out = {"o": o, "lse": lse}
    if bwd:
        do = to_dev(inp["dout"], w)
        dq, dk, dv = ops.attn_bwd(w.op, q, k, v, o, lse, do, scale=scale, **kw)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {key: to_np(val) for key, val in out.items()}


def run_oracle(w, inp: Dict[str, np.ndarray], bwd: bool = True, scale: float = 0.0):
    o, lse = O.fwd(w, inp["q"], inp["k"], inp["v"], scale=scale)
    out = {"o": o, "lse": lse}
    if bwd:
        dq, dk, dv = O.bwd(w, inp["q"], inp["k"], inp["v"], inp["dout"], scale=scale)
        out.update(dq=dq, dk=dk, dv=dv)
    return out


def err_metrics(got: np.ndarray, want: np.ndarray):
    d = got - want
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    den = float(np.linalg.norm(want.ravel()))
    rel = float(np.linalg.norm(d.ravel())) / den if den > 0 else float(np.linalg.norm(d.ravel()))
    return max_abs, rel


def excess_over_storage(got: np.ndarray, want: np.ndarray) -> float:
    """max(|got - want| - ulp_bf16(want)/2): the error beyond output rounding."""
    if not got.size:
        return 0.0
    return float(np.max(np.abs(got - want) - half_ulp_bf16(want)))


def bf16_metrics(got: np.ndarray, want: np.ndarray) -> dict:
    """Error figures of a bf16 output against the fp64 oracle."""
    if not got.size:
        return {"max_abs": 0.0, "vs_rounded": 0.0, "vs_rounded_excess": -1.0, "beyond_rounding": 0.0,
                "rel_l2": 0.0, "floor_rel_l2": 0.0, "max_abs_want": 0.0}
    r = bf16_round(want)
    ma, rl = err_metrics(got, want)
    _, floor_rl = err_metrics(r, want)
    d = np.abs(got - r)
    return {
        "max_abs": ma,                                   # raw |got - want|
        "vs_rounded": float(np.max(d)),                  # |got - bf16(want)|
        # (a): |got - bf16(want)| - max(2e-2, ulp); must be <= 0
        "vs_rounded_excess": float(np.max(d - np.maximum(2e-2, 2 * half_ulp_bf16(want)))),
        "beyond_rounding": excess_over_storage(got, want),   # (b)
        "rel_l2": rl,
        "floor_rel_l2": floor_rl,                        # bf16(want) vs want
        "max_abs_want": float(np.max(np.abs(want))),
    }


def _report_sink(label: str, key: str, met: dict):
    """Appends the figures as a JSON line to $BCA_PARITY_REPORT when set."""
    path = os.environ.get("BCA_PARITY_REPORT")
    if not path:
        return
    import json
    with open(path, "a") as f:
        f.write(json.dumps(dict(case=label, tensor=key, **met)) + "\n")


# How far a kernel's bf16 result may sit beyond the precision floor of the
# method itself (see assert_close's ``floor``).
FLOOR_MARGIN = 2e-3


def load_floor(name: str):
    """Stored precision floor of workload ``name`` (tests/golden/precision_floor.json,
    written by tests/golden/precision_floor.py), or None."""
    import json
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "precision_floor.json")
    if not os.path.exists(path):
        return None
    return json.load(open(path)).get(name)


def assert_close(w, got: Dict[str, np.ndarray], want: Dict[str, np.ndarray], label: str = "",
                 floor=None):
    """Asserts the bf16 / fp32 bars above.  ``floor`` (bf16 only): per tensor,
    the error figures of an fp64 computation whose only roundings are the
    method's bf16 matmul operands (tests/golden/precision_floor.py); where
    that floor itself exceeds a max-abs bar, the bar for the tensor becomes
    the floor plus FLOOR_MARGIN, i.e. the kernel may add at most 2e-3 to the
    error the method's precision already makes.  Relative L2 is never
    relaxed."""
    tol = TOL[w.dtype]
    report = []
    for key in ("o", "lse", "dq", "dk", "dv"):
        if key not in got or key not in want:
            continue
        g, r = got[key], want[key]
        assert g.shape == r.shape, (key, g.shape, r.shape)
        assert np.all(np.isfinite(g)), "%s %s: non-finite values" % (label, key)
        ma, rl = err_metrics(g, r)
        if key == "lse":
            report.append("lse max_abs=%.3g" % ma)
            _report_sink(label, key, {"max_abs": ma})
            assert ma <= tol["lse"], "%s lse max_abs %.3g > %.3g" % (label, ma, tol["lse"])
            continue
        if not tol["storage_ulp"]:
            report.append("%s max_abs=%.3g rel_l2=%.3g" % (key, ma, rl))
            _report_sink(label, key, {"max_abs": ma, "rel_l2": rl})
            assert ma <= tol["max_abs"], "%s %s max_abs %.3g > %.3g" % (label, key, ma, tol["max_abs"])
            assert rl <= tol["rel_l2"], "%s %s rel_l2 %.3g > %.3g" % (label, key, rl, tol["rel_l2"])
            continue
        met = bf16_metrics(g, r)
        _report_sink(label, key, met)
        report.append("%s max_abs=%.3g vs_bf16(want)=%.3g beyond_rounding=%.3g rel_l2=%.3g (floor %.3g)" % (
            key, ma, met["vs_rounded"], met["beyond_rounding"], rl, met["floor_rel_l2"]))
        bar_a, bar_b = 0.0, tol["max_abs"]
        if floor and key in floor:
            bar_a = max(bar_a, floor[key]["vs_rounded_excess"] + FLOOR_MARGIN)
            bar_b = max(bar_b, floor[key]["beyond_rounding"] + FLOOR_MARGIN)
        assert met["vs_rounded_excess"] <= bar_a, \
            "%s %s |got - bf16(want)| %.3g exceeds max(%.3g, one bf16 step) by %.3g (allowed %.3g)" % (
                label, key, met["vs_rounded"], tol["max_abs"], met["vs_rounded_excess"], bar_a)
        assert met["beyond_rounding"] <= bar_b, \
            "%s %s max_abs %.3g (beyond output rounding %.3g) > %.3g" % (
                label, key, ma, met["beyond_rounding"], bar_b)
        assert rl <= tol["rel_l2"], "%s %s rel_l2 %.3g > %.3g" % (label, key, rl, tol["rel_l2"])
    return report


def sample_units(w, got: Dict[str, np.ndarray], inp: Dict[str, np.ndarray], units: Sequence[int]):
    """Slice the sampled units out of full-size inputs and HIP outputs.
    Space units are (b, t) blocks -> a (n, 1, N, H, D) batch; time units are
    slots n -> a (B, T, n, H, D) batch (all batches of the chosen slots)."""
    if w.op == "space":
        bs = [u // w.T for u in units]
        ts = [u % w.T for u in units]
        sl = lambda x: x[bs, ts][:, None]
        ws = w.with_(B=len(units), T=1)
    else:
        slots = sorted(set(u % w.N for u in units))
        sl = lambda x: x[:, :, slots]
        ws = w.with_(N=len(slots))
    return ws, {k: np.ascontiguousarray(sl(v)) for k, v in inp.items()}, \
        {k: np.ascontiguousarray(sl(v)) for k, v in got.items()}
