"""Precision floor of the bf16 method at full size: writes precision_floor.json.

    python tests/golden/precision_floor.py [3 4 ...]

Test infrastructure.  For each named workload it evaluates, in float64 with
numpy, attention whose only roundings are the bf16 ones the method's mixed
precision puts on matmul operands (Open Dreamer articles, pro.edgex.exchange
fr-FR edition, section "Ingénierie de la stabilité", item 3: bf16 matmul
inputs, fp32 statistics): the unnormalised probabilities before P V, the
probabilities before P^T dO, dS before dS K and dS^T Q, and O before
Delta = rowsum(dO * O), and every output rounded to bf16.  Everything else is
exact.  It then compares that against the fp64 oracle (oracle/) with the
error figures of the GPU parity tests and stores the worst per tensor.

No HIP code is involved: the figures say how far from the exact result a
computation that makes only those roundings lands, on the same seeded
inputs, i.e. what part of the error is the method's and not a kernel's.
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

from block_causal_transformer_amd import configs as C  # noqa: E402
from block_causal_transformer_amd import gen  # noqa: E402
from oracle import oracle as O  # noqa: E402

import gpu_util as U  # noqa: E402  (bf16 rounding and the error figures)

OUT = os.path.join(HERE, "precision_floor.json")


def _problems(w, x):
    """Per (unit, KV head) views: q, dO (L*G rows = position-major, head
    minor), k, v (L keys) as float64, plus the visibility matrix [L*G, L]."""
    G = w.G
    if w.op == "space":
        units = [(b, t) for b in range(w.B) for t in range(w.T)]
        sel = lambda a, u: a[u[0], u[1]]          # (N, H, D)
        L = w.N
        j = np.arange(L)
        ag = (j >= w.agent_begin) & (j < w.agent_begin + w.agent_count)
        vis = ~(ag[None, :] & ~ag[:, None])
    else:
        units = [(b, n) for b in range(w.B) for n in range(w.N)]
        sel = lambda a, u: a[u[0], :, u[1]]       # (T, H, D)
        L = w.T
        t = np.arange(L)
        d = t[:, None] - t[None, :]
        vis = (d >= 0) & ((w.window == 0) | (d < max(w.window, 1)))
    vis_rows = np.repeat(vis, G, axis=0)
    return units, sel, vis_rows


def emulate(w, x, scale=0.0):
    s = scale if scale > 0 else 1.0 / np.sqrt(w.D)
    G = w.G
    r16 = U.bf16_round
    out = {k: np.zeros(x[k2].shape) for k, k2 in (("o", "q"), ("dq", "q"), ("dk", "k"), ("dv", "v"))}
    units, sel, vis = _problems(w, x)
    for u in units:
        for g in range(w.Hkv):
            q = sel(x["q"], u)[:, g * G:(g + 1) * G].reshape(-1, w.D).astype(np.float64)
            do = sel(x["dout"], u)[:, g * G:(g + 1) * G].reshape(-1, w.D).astype(np.float64)
            k = sel(x["k"], u)[:, g].astype(np.float64)
            v = sel(x["v"], u)[:, g].astype(np.float64)
            z = np.where(vis, (q @ k.T) * s, -np.inf)
            m = z.max(axis=1, keepdims=True)
            p = np.exp(z - m)
            l = p.sum(axis=1, keepdims=True)
            o = (r16(p) @ v) / l
            ob = r16(o)
            P = p / l
            delta = np.sum(do * ob, axis=1, keepdims=True)
            ds = P * (do @ v.T - delta)
            dv = r16(P).T @ do
            dk = (r16(ds).T @ q) * s
            dq = (r16(ds) @ k) * s
            shp = sel(out["o"], u)[:, g * G:(g + 1) * G].shape
            sel(out["o"], u)[:, g * G:(g + 1) * G] = ob.reshape(shp)
            sel(out["dq"], u)[:, g * G:(g + 1) * G] = r16(dq).reshape(shp)
            sel(out["dk"], u)[:, g] = r16(dk)
            sel(out["dv"], u)[:, g] = r16(dv)
    return out


def floor_of(name):
    w = C.get(name)
    x = gen.make_inputs(w)
    t0 = time.time()
    em = emulate(w, x)
    ro, _ = O.fwd(w, x["q"], x["k"], x["v"])
    rdq, rdk, rdv = O.bwd(w, x["q"], x["k"], x["v"], x["dout"])
    res = {}
    for key, want in (("o", ro), ("dq", rdq), ("dk", rdk), ("dv", rdv)):
        met = U.bf16_metrics(em[key], want)
        res[key] = {a: met[a] for a in ("max_abs", "vs_rounded", "vs_rounded_excess",
                                          "beyond_rounding", "rel_l2")}
    print(name, "%.0f s" % (time.time() - t0), json.dumps(res))
    return res


def main(names):
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for n in names:
        data[n] = floor_of(n)
    data["_about"] = ("worst error per output tensor of an fp64 computation whose only roundings are "
                      "the method's bf16 matmul operands (P, dS, O before Delta) and bf16 outputs, "
                      "against the fp64 oracle; written by tests/golden/precision_floor.py")
    with open(OUT, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["3", "4"])
