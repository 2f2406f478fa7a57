"""The precision-floor emulation (tests/golden/precision_floor.py) computes
attention: with its bf16 roundings replaced by the identity it equals the
fp64 oracle, and with them it stays within the bf16 error bars on a small
case."""
import importlib.util
import os

import numpy as np

from block_causal_transformer_amd import configs as C
from block_causal_transformer_amd import gen
from oracle import oracle as O

import gpu_util as U

HERE = os.path.dirname(os.path.abspath(__file__))


def _module():
    spec = importlib.util.spec_from_file_location("precision_floor", os.path.join(HERE, "golden", "precision_floor.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _cases():
    return [C.get("3").with_(B=1, T=1, N=40, agent_begin=39), C.get("4").with_(N=2, T=70, window=16)]


def test_emulation_without_rounding_is_the_oracle(monkeypatch):
    m = _module()
    monkeypatch.setattr(U, "bf16_round", lambda x: np.asarray(x, dtype=np.float64))
    for w in _cases():
        x = gen.make_inputs(w)
        em = m.emulate(w, x)
        ro, _ = O.fwd(w, x["q"], x["k"], x["v"])
        rdq, rdk, rdv = O.bwd(w, x["q"], x["k"], x["v"], x["dout"])
        for key, want in (("o", ro), ("dq", rdq), ("dk", rdk), ("dv", rdv)):
            np.testing.assert_allclose(em[key], want, rtol=1e-10, atol=1e-12, err_msg=key)


def test_emulation_with_rounding_is_within_the_bars():
    m = _module()
    for w in _cases():
        x = gen.make_inputs(w)
        em = m.emulate(w, x)
        want = U.run_oracle(w, x)
        for key in ("o", "dq", "dk", "dv"):
            met = U.bf16_metrics(em[key], want[key])
            assert 0 < met["rel_l2"] < 5e-3 and met["beyond_rounding"] < 2e-2, (w.name, key, met)


def test_stored_floor_covers_the_full_size_workloads():
    for name in ("3", "4"):
        f = U.load_floor(name)
        assert f and set(f) == {"o", "dq", "dk", "dv"}
        for key in f:
            assert f[key]["rel_l2"] < 5e-3
