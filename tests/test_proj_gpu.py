"""GPU parity of the projections beside attention (rmsnorm_qkv_fwd,
out_proj_fwd) against the fp64 oracle, through the C ABI: the dynamics
layer's widths at a few hundred rows, ragged sizes (rows, features and
output columns that do not fill a 128 x 128 x 64 or 256 x 256 x 64 tile),
and the full 74,240 rows with the oracle on sampled rows."""
import numpy as np
import pytest

from block_causal_transformer_amd import configs as C
from block_causal_transformer_amd import gen, ops
from oracle import oracle as O

import gpu_util as U

pytestmark = pytest.mark.gpu

BASE = C.PROJ_CONFIGS["proj"]
CASES = {
    "dyn_rows300": BASE.with_(M=300, seed=7100),
    "one_row": BASE.with_(M=1, seed=7101),
    "ragged": BASE.with_(M=129, d_model=72, Hq=2, Hkv=1, D=8, seed=7102),
    "mha_k136": BASE.with_(M=257, d_model=136, Hq=4, Hkv=4, D=16, seed=7103),
    "eps_large": BASE.with_(M=64, eps=0.5, seed=7104),
    # the 256 x 256 tile path (rows and columns multiples of 8, K of 64):
    # rows that end inside a tile, problems smaller than one tile, and K of
    # one, two and three 64-wide steps (the loop's prologue and tail)
    "rows272": BASE.with_(M=272, seed=7105),
    "rows16_small": BASE.with_(M=16, d_model=128, Hq=2, Hkv=1, D=32, seed=7106),
    "k64_one_step": BASE.with_(M=48, d_model=64, Hq=1, Hkv=1, D=64, seed=7107),
    "k192_three_steps": BASE.with_(M=24, d_model=192, Hq=3, Hkv=1, D=64, seed=7108),
    # rows wider than the norm kernel keeps in registers (2048 features)
    "wide_rows": BASE.with_(M=40, d_model=2304, Hq=4, Hkv=2, D=64, seed=7109),
}


def _needs_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(got, want, label):
    """bf16 outputs: per element |got - want| - ulp(want)/2 <= 2e-2, rel-L2 <= 5e-3."""
    ex = U.excess_over_storage(got, want)
    ma, rl = U.err_metrics(got, want)
    print("%s max_abs=%.3g beyond_rounding=%.3g rel_l2=%.3g" % (label, ma, ex, rl))
    assert ex <= 2e-2 and rl <= 5e-3, (label, ma, ex, rl)


def _dev(a, dt=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    return t.to(dt) if dt is not None else t


def _run(w, x):
    import torch
    bf = torch.bfloat16
    q, k, v, rstd = ops.qkv_proj(_dev(x["x"], bf), _dev(x["gain"]), _dev(x["w_qkv"], bf),
                                 w.Hq, w.Hkv, w.D, eps=w.eps)
    y = ops.out_proj(_dev(x["o"], bf), _dev(x["w_o"], bf), _dev(x["residual"], bf), w.Hq, w.D)
    y0 = ops.out_proj(_dev(x["o"], bf), _dev(x["w_o"], bf), None, w.Hq, w.D)
    torch.cuda.synchronize()
    return {n: U.to_np(t) for n, t in (("q", q), ("k", k), ("v", v), ("rstd", rstd), ("y", y), ("y0", y0))}


def _oracle(w, x, rows=None):
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    q, k, v, rstd = O.rmsnorm_qkv_fwd(sel(x["x"]), x["gain"], x["w_qkv"], w.Hq, w.Hkv, w.D, w.eps)
    y = O.out_proj_fwd(sel(x["o"]), x["w_o"], sel(x["residual"]))
    y0 = O.out_proj_fwd(sel(x["o"]), x["w_o"], None)
    return {"q": q, "k": k, "v": v, "rstd": rstd, "y": y, "y0": y0}


def _compare(got, want, label, rows=None):
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    for n in ("q", "k", "v", "y", "y0"):
        _check(sel(got[n]), want[n], "%s %s" % (label, n))
    r = sel(got["rstd"])
    assert np.max(np.abs(r - want["rstd"]) / want["rstd"]) <= 1e-5, label + " rstd"


@pytest.mark.parametrize("name", list(CASES))
def test_projections_match_oracle(name):
    _needs_gpu()
    w = CASES[name]
    print("proj case", name, w, flush=True)
    x = gen.make_proj_inputs(w)
    _compare(_run(w, x), _oracle(w, x), name)


def test_projections_full_size_sampled_rows():
    _needs_gpu()
    w = BASE
    x = gen.make_proj_inputs(w)
    got = _run(w, x)
    rows = np.unique(np.concatenate([np.arange(0, 3), np.random.default_rng(7).integers(0, w.M, 40),
                                     np.arange(w.M - 3, w.M)]))
    _compare(got, _oracle(w, x, rows), "full", rows)
