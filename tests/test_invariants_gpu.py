"""GPU invariants of the HIP kernels (through the C ABI):

* bitwise determinism: two runs give identical bits (no atomics anywhere);
* agent isolation: changing the agent token's K/V leaves every world token's
  O, LSE and dQ bitwise unchanged (space attention);
* causality and window: changing frames after t, or at least W frames before
  t, leaves frame t's O, LSE and dQ bitwise unchanged (time attention);
* GQA equals attention on K/V heads replicated to Hq heads (within the bf16
  tolerance; dK/dV of the replicated run summed over each group).
"""
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


def _run(w, x, bwd=True):
    import torch
    q, k, v = (U.to_dev(x[n], w) for n in ("q", "k", "v"))
    kw = ops.workload_kwargs(w)
    o, lse = ops.attn_fwd(w.op, q, k, v, **kw)
    out = {"o": o, "lse": lse}
    if bwd:
        dq, dk, dv = ops.attn_bwd(w.op, q, k, v, o, lse, U.to_dev(x["dout"], w), **kw)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: t.detach().cpu() for n, t in out.items()}


@pytest.mark.parametrize("name", ["3", "4", "5c", "5d"])
def test_bitwise_determinism(name):
    _needs_gpu()
    w = {"3": C.get("3").with_(B=1, T=3), "4": C.get("4").with_(N=3),
         "5c": C.get("5c").with_(N=2), "5d": C.get("5d").with_(N=2)}[name]
    x = gen.make_inputs(w)
    a, b = _run(w, x), _run(w, x)
    for n in a:
        assert _bits_equal(a[n], b[n]), "%s %s differs between runs" % (name, n)


def _bits_equal(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).equal(b.view(torch.int16))
    return a.view(torch.int32).equal(b.view(torch.int32))


@pytest.mark.parametrize("agent", [(289, 1), (0, 1), (100, 3)])
def test_agent_isolation_bitwise(agent):
    _needs_gpu()
    ab, ac = agent
    w = C.get("3").with_(B=1, T=2, agent_begin=ab, agent_count=ac)
    x = gen.make_inputs(w)
    y = {n: v.copy() for n, v in x.items()}
    rng = np.random.default_rng(5)
    y["k"][:, :, ab:ab + ac] = gen.bf16_round(rng.standard_normal(y["k"][:, :, ab:ab + ac].shape).astype(np.float32) * 3)
    y["v"][:, :, ab:ab + ac] = gen.bf16_round(rng.standard_normal(y["v"][:, :, ab:ab + ac].shape).astype(np.float32) * 3)
    a, b = _run(w, x), _run(w, y)
    world = [j for j in range(w.N) if not (ab <= j < ab + ac)]
    for n in ("o", "lse", "dq"):
        assert _bits_equal(a[n][:, :, world], b[n][:, :, world]), "world %s changed with agent K/V" % n
    assert not _bits_equal(a["o"][:, :, ab], b["o"][:, :, ab]), "agent output should change"


@pytest.mark.parametrize("t,window", [(100, 192), (200, 192), (31, 16), (130, 0)])
def test_causal_window_bitwise(t, window):
    _needs_gpu()
    w = C.get("4").with_(N=3, window=window)
    x = gen.make_inputs(w)
    y = {n: v.copy() for n, v in x.items()}
    rng = np.random.default_rng(6)
    lo = t - window + 1 if window > 0 else 0
    for n in ("k", "v"):
        y[n][:, t + 1:] = gen.bf16_round(rng.standard_normal(y[n][:, t + 1:].shape).astype(np.float32) * 2)
        if lo > 0:
            y[n][:, :lo] = gen.bf16_round(rng.standard_normal(y[n][:, :lo].shape).astype(np.float32) * 2)
    a, b = _run(w, x), _run(w, y)
    for n in ("o", "lse", "dq"):
        assert _bits_equal(a[n][:, t], b[n][:, t]), "frame %d %s changed" % (t, n)
    assert not _bits_equal(a["o"][:, t + 1], b["o"][:, t + 1]), "a later frame should change"


@pytest.mark.parametrize("name", ["3", "4"])
def test_gqa_equals_replicated_kv(name):
    _needs_gpu()
    w = {"3": C.get("3").with_(B=1, T=2), "4": C.get("4").with_(N=2)}[name]
    x = gen.make_inputs(w)
    G = w.Hq // w.Hkv
    wr = w.with_(Hkv=w.Hq)
    xr = dict(x, k=np.repeat(x["k"], G, axis=3), v=np.repeat(x["v"], G, axis=3))
    a = {n: t.double().numpy() for n, t in _run(w, x).items()}
    b = {n: t.double().numpy() for n, t in _run(wr, xr).items()}
    B, T, N = w.B, w.T, w.N
    # O, LSE, dQ: one rounding on each side -> the usual bf16 bar
    print(U.assert_close(w, {n: a[n] for n in ("o", "lse", "dq")},
                         {n: b[n] for n in ("o", "lse", "dq")}, "gqa vs replicated"))
    # dK, dV: the replicated side is a sum of G separately rounded heads, so
    # its own rounding (G half-ulps) widens the bar beside the usual one
    for n in ("dk", "dv"):
        per_head = b[n].reshape(B, T, N, w.Hkv, G, w.D)
        ref = per_head.sum(4)
        slack = U.half_ulp_bf16(per_head).sum(4) + U.half_ulp_bf16(ref)
        excess = float(np.max(np.abs(a[n] - ref) - slack))
        _, rel = U.err_metrics(a[n], ref)
        print(n, "excess beyond rounding", excess, "rel_l2", rel)
        assert excess <= 2e-2 and rel <= 5e-3, (n, excess, rel)
