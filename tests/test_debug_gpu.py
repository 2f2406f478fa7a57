"""GPU checks of the documented failure behaviour and debug switches:

* non-finite inputs: a NaN or infinity in the data of one problem (one
  (unit, KV head) pair) leaves every other problem's outputs bitwise those of
  a clean run, and nothing faults;
* BCA_DEBUG_LDS_POISON=1 fills the kernels' LDS with NaN bit patterns before
  staging; every kernel family returns bitwise the same results with it, so
  no kernel reads LDS that no thread wrote;
* BCA_SYNC=1 synchronizes after every call and still returns the same
  results.
"""
import os

import numpy as np
import pytest

from block_causal_transformer_amd import configs as C
from block_causal_transformer_amd import gen, ops

import gpu_util as U

pytestmark = pytest.mark.gpu


def _needs_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(w, inp, **env):
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        return U.run_hip(w, inp)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _problem_views(w, out, b, unit, g):
    """The outputs of problem (unit, KV head g) as a dict of arrays."""
    G = w.G
    if w.op == "space":
        t = unit
        sq = (b, t, slice(None), slice(g * G, (g + 1) * G))
        sk = (b, t, slice(None), g)
    else:
        n = unit
        sq = (b, slice(None), n, slice(g * G, (g + 1) * G))
        sk = (b, slice(None), n, g)
    return {"o": out["o"][sq], "lse": out["lse"][sq], "dq": out["dq"][sq],
            "dk": out["dk"][sk], "dv": out["dv"][sk]}


NONFINITE = [
    # (workload, tensor, index (b, t, n, head, d), value)
    (C.get("3").with_(B=1, T=3), "q", (0, 1, 7, 4, 5), np.nan),
    (C.get("3").with_(B=1, T=3), "k", (0, 2, 100, 2, 0), np.inf),
    (C.get("4").with_(N=3), "v", (0, 100, 1, 1, 9), np.nan),
    (C.get("4").with_(N=3), "dout", (0, 5, 2, 29, 63), -np.inf),
    (C.get("5c").with_(N=4), "k", (0, 3, 1, 7, 1), np.nan),          # short-problem kernels
    (C.get("5a").with_(T=2, Hq=4, Hkv=4), "v", (0, 1, 900, 3, 2), np.inf),  # several key blocks
]


@pytest.mark.parametrize("w,tensor,idx,val", NONFINITE,
                         ids=["%s_%s_%s" % (c[0].name, c[1], "nan" if np.isnan(c[3]) else "inf")
                              for c in NONFINITE])
def test_nonfinite_input_stays_in_its_problem(w, tensor, idx, val):
    _needs_gpu()
    print("case", w.name, tensor, idx, val, flush=True)
    inp = gen.make_inputs(w)
    clean = U.run_hip(w, inp)
    bad = {k: v.copy() for k, v in inp.items()}
    bad[tensor][idx] = val
    got = U.run_hip(w, bad)
    b, t, n, h, _ = idx
    g = h // w.G if tensor in ("q", "dout") else h
    hit = (b, t if w.op == "space" else n, g)
    units = w.T if w.op == "space" else w.N
    checked = 0
    for bb in range(w.B):
        for u in range(units):
            for gg in range(w.Hkv):
                if (bb, u, gg) == hit:
                    continue
                a = _problem_views(w, got, bb, u, gg)
                c = _problem_views(w, clean, bb, u, gg)
                for key in a:
                    assert np.array_equal(a[key], c[key]), (bb, u, gg, key)
                checked += 1
    assert checked == w.B * units * w.Hkv - 1


DEBUG_CASES = [
    C.get("3").with_(B=1, T=2),
    C.get("4").with_(N=3),
    C.get("2s").with_(B=1, T=2),
    C.get("5c").with_(N=3),
    C.Workload("space_N641", "space", 1, 1, 641, 6, 2, 64, "bf16", 0, 640, 1, 1.0, 9010),
    C.Workload("time_T300_W192", "time", 1, 300, 2, 6, 2, 64, "bf16", 192, 0, 0, 1.0, 9016),
    C.Workload("short_space_N21_G3_agent_mid", "space", 2, 2, 21, 9, 3, 64, "bf16", 0, 5, 3, 1.0, 9025),
    C.Workload("time_d64_f32", "time", 1, 12, 2, 4, 1, 64, "f32", 5, 0, 0, 1.0, 9008),
]


@pytest.mark.parametrize("w", DEBUG_CASES, ids=[w.name for w in DEBUG_CASES])
def test_lds_poison_and_sync_change_nothing(w):
    _needs_gpu()
    print("case", w.name, flush=True)
    inp = gen.make_inputs(w)
    ref = U.run_hip(w, inp)
    poisoned = _run(w, inp, BCA_DEBUG_LDS_POISON="1")
    synced = _run(w, inp, BCA_SYNC="1")
    for key in ref:
        assert np.array_equal(ref[key], poisoned[key]), "LDS poison changed %s" % key
        assert np.array_equal(ref[key], synced[key]), "BCA_SYNC changed %s" % key


def test_lds_poison_decode():
    _needs_gpu()
    import torch
    w = C.DECODE_CONFIGS["dec"].with_(N=5, seed=6160)
    x = gen.make_decode_inputs(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)
    q, kc, vc = dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"])
    o1, l1 = ops.attn_decode_fwd(q, kc, vc, w.q_frame0, window=w.window)
    os.environ["BCA_DEBUG_LDS_POISON"] = "1"
    try:
        o2, l2 = ops.attn_decode_fwd(q, kc, vc, w.q_frame0, window=w.window)
    finally:
        os.environ.pop("BCA_DEBUG_LDS_POISON", None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
