"""Seeded generator and workload table (host only)."""
import numpy as np
import torch

from block_causal_transformer_amd import configs as C
from block_causal_transformer_amd import gen


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30])])
    ours = gen.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(gen.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_inputs_seeded_and_bf16_exact():
    w = C.get("1s").with_(dtype="bf16")
    a = gen.make_inputs(w)
    b = gen.make_inputs(w)
    for key in ("q", "k", "v", "dout"):
        assert np.array_equal(a[key], b[key])
        assert np.array_equal(gen.bf16_round(a[key]), a[key])
    c = gen.make_inputs(w, variant=1)
    assert not np.array_equal(a["q"], c["q"])
    assert a["q"].shape == w.q_shape() and a["k"].shape == w.kv_shape()


def test_scaled_inputs():
    w = C.get("2s").with_(B=1, T=2)
    x = gen.make_inputs(w)["q"]
    assert 0.08 < float(x.std()) < 0.17


def test_shared_mask_token_rows():
    w = C.get("5a").with_(T=2, Hq=2, Hkv=2)
    x = gen.make_inputs(w)
    slots = gen.masked_slots(w)
    assert slots.shape == (2, 828)
    for bt in range(2):
        s = slots[bt]
        assert len(set(s.tolist())) == 828 and s.max() < 920
        rows = x["k"][0, bt, s]
        assert np.all(rows == rows[0])
        rest = np.setdiff1d(np.arange(1432), s)
        assert not np.all(x["k"][0, bt, rest] == rows[0])


def test_visible_pairs_closed_forms():
    assert C.visible_pairs(C.get("3")) // (256 * 30) == 83811
    assert C.visible_pairs(C.get("4")) // (290 * 30) == 30816
    assert C.flops(C.get("3"), "fwd") == 4 * 64 * 83811 * 256 * 30
    assert abs(C.min_bytes(C.get("3"), "fwd") - 636.1e6) < 0.1e6
    assert abs(C.min_bytes(C.get("3"), "bwd") - 1263.3e6) < 0.1e6
