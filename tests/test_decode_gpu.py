"""GPU parity of the rollout decode entry point (time_attn_decode_fwd) against
the fp64 oracle, through the C ABI: the Minecraft rollout shape in steady
state (wrapped ring) and at its first frames, several new frames at once, a
cache larger than the window, an unbounded window longer than one LDS key
block, 40 query heads per KV head (several row chunks per new frame),
head_dim 32 and fp32 (the generic kernel), and decode of frame t
against row t of the full-sequence time attention kernel; also the space
attention of the rollout's new block, whose tiny grid the forward launcher
splits differently from every training shape."""
import types

import numpy as np
import pytest

from block_causal_transformer_amd import configs as C
from block_causal_transformer_amd import gen, ops
from oracle import oracle as O

import gpu_util as U

pytestmark = pytest.mark.gpu

BASE = C.DECODE_CONFIGS["dec"]
CASES = {
    "steady": BASE,
    "first_frame": BASE.with_(q_frame0=0, seed=6100),
    "early": BASE.with_(q_frame0=7, seed=6101),
    "window_edge": BASE.with_(q_frame0=191, seed=6102),
    "four_new_frames": BASE.with_(Tq=4, cache_frames=200, q_frame0=300, N=37, seed=6103),
    "cache_larger": BASE.with_(cache_frames=256, q_frame0=777, N=41, seed=6104),
    "unbounded_long": BASE.with_(window=0, cache_frames=401, q_frame0=400, N=5, seed=6105),
    "batch2_mha": BASE.with_(B=2, Hq=4, Hkv=4, N=9, window=16, cache_frames=20, q_frame0=50, seed=6106),
    "d32": BASE.with_(D=32, N=11, Hq=8, Hkv=2, window=8, cache_frames=8, q_frame0=20, seed=6107),
    "fp32": BASE.with_(dtype="f32", N=6, Hq=4, Hkv=2, D=32, window=4, cache_frames=5, q_frame0=9, seed=6108),
    "g40": BASE.with_(Hq=40, Hkv=1, N=3, window=8, cache_frames=8, q_frame0=20, seed=6109),
}


def _needs_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tol(w):
    return types.SimpleNamespace(dtype=w.dtype)


def _run(w, x):
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    o, lse = ops.attn_decode_fwd(dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]),
                                 w.q_frame0, window=w.window)
    torch.cuda.synchronize()
    return {"o": U.to_np(o), "lse": U.to_np(lse)}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name):
    _needs_gpu()
    w = CASES[name]
    x = gen.make_decode_inputs(w)
    print("decode case", name, w, flush=True)
    got = _run(w, x)
    o, lse = O.time_decode_fwd(x["q"], x["k_cache"], x["v_cache"], w.q_frame0, w.window)
    print(U.assert_close(_tol(w), got, {"o": o, "lse": lse}, name))


def test_decode_equals_full_sequence_rows():
    """Frame t decoded from a ring filled with frames <= t equals row t of the
    time attention kernel over the whole sequence (both on the GPU)."""
    _needs_gpu()
    import torch
    w = C.get("4").with_(N=7, T=230)
    x = gen.make_inputs(w, with_dout=False)
    q, k, v = (U.to_dev(x[n], w) for n in ("q", "k", "v"))
    o_full, lse_full = ops.attn_fwd("time", q, k, v, window=w.window)
    Cf = 192
    for t in (0, 100, 191, 229):
        kc = torch.zeros((w.B, Cf, w.N, w.Hkv, w.D), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        for f in range(max(0, t - Cf + 1), t + 1):
            kc[:, f % Cf] = k[:, f]
            vc[:, f % Cf] = v[:, f]
        o, lse = ops.attn_decode_fwd(q[:, t:t + 1].contiguous(), kc, vc, t, window=w.window)
        torch.cuda.synchronize()
        got = {"o": U.to_np(o)[:, 0], "lse": U.to_np(lse)[:, 0]}
        want = {"o": U.to_np(o_full)[:, t], "lse": U.to_np(lse_full)[:, t]}
        print(t, U.assert_close(w, got, want, "frame %d" % t))


def test_decode_graph_replays_match_eager():
    """A decode call captured in a HIP graph gives the eager result on every
    replay, with eager work and synchronizations between the replays."""
    _needs_gpu()
    import torch
    w = CASES["four_new_frames"]
    x = gen.make_decode_inputs(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)
    q, kc, vc = dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"])
    o_ref, l_ref = ops.attn_decode_fwd(q, kc, vc, w.q_frame0, window=w.window)
    o = torch.zeros_like(o_ref)
    lse = torch.zeros_like(l_ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.attn_decode_fwd(q, kc, vc, w.q_frame0, window=w.window, out=(o, lse))
    for r in range(4):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "replay %d o" % r
        assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), "replay %d lse" % r
        ops.attn_decode_fwd(q, kc, vc, w.q_frame0, window=w.window)  # eager work between


@pytest.mark.parametrize("B", [1, 8])
def test_rollout_space_block_matches_oracle(B):
    """The rollout step's other half: space attention (agent isolation) over
    the new 290-token block of each environment, forward only.  With so few
    problems the forward launcher splits each one into 2-chunk workgroups
    (46 per problem, the last chunk 20 rows), a grid no training shape uses."""
    _needs_gpu()
    w = C.get("3").with_(B=B, T=1, seed=6200 + B)
    x = gen.make_inputs(w, with_dout=False)
    print("rollout space block", w, flush=True)
    got = U.run_hip(w, x, bwd=False)
    want = U.run_oracle(w, x, bwd=False)
    print(U.assert_close(w, got, want, "rollout space block B=%d" % B))
