"""Pins for the CPU fp64 oracle: checks against things other than the oracle.

Each ``pin_*`` takes an oracle library handle (``oracle.oracle.load()`` or a
deliberately broken build of it) and raises AssertionError when the oracle
disagrees with what the mathematics or the pages fix:

* library routine: torch CPU fp64 ``scaled_dot_product_attention`` with an
  explicit boolean mask (and ``enable_gqa``), gradients from torch autograd,
  LSE from ``torch.logsumexp``;
* closed forms: identical keys, q = 0 (LSE = ln of the visible count, counts
  from tests/golden/visible_counts.txt), window 1, constant values;
* backward identities: sum of dK over keys is 0, sum of dV equals the sum of
  dO over the group; central finite differences of sum(O * dO);
* invariants: future / out-of-window frames and agent keys do not reach the
  outputs they may not reach; GQA equals replicated KV heads; a common key
  shift leaves O unchanged and shifts LSE by s<q, c>; permuting world tokens
  permutes outputs; units are independent;
* rollout decode: torch SDPA over the ring positions with a mask built from
  the frame each position holds, and row t of time attention over the whole
  sequence;
* projections: torch fp64 ``F.rms_norm`` and a matmul; the
  RMS norm's exact invariance to a power-of-two input scale; identity
  weights.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers

def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def to_units(x: np.ndarray, op: str) -> np.ndarray:
    """(B,T,N,H,D) -> (U,H,L,D): U units (blocks or slots), L positions."""
    B, T, N, H, D = x.shape
    if op == "space":
        return x.reshape(B * T, N, H, D).transpose(0, 2, 1, 3)
    return x.transpose(0, 2, 1, 3, 4).reshape(B * N, T, H, D).transpose(0, 2, 1, 3)


def from_units(y: np.ndarray, op: str, shape) -> np.ndarray:
    B, T, N, H, D = shape
    if op == "space":
        return y.transpose(0, 2, 1, 3).reshape(B, T, N, H, D)
    return y.transpose(0, 2, 1, 3).reshape(B, N, T, H, D).transpose(0, 2, 1, 3, 4)


def lse_from_units(y: np.ndarray, op: str, shape) -> np.ndarray:
    B, T, N, H = shape
    if op == "space":
        return y.transpose(0, 2, 1).reshape(B, T, N, H)
    return y.transpose(0, 2, 1).reshape(B, N, T, H).transpose(0, 2, 1, 3)


def vis_matrix(op, L, window=0, agent_begin=0, agent_count=0) -> np.ndarray:
    """Dense boolean (L, L) matrix, [query, key] -> visible."""
    a = np.arange(L)[:, None]
    b = np.arange(L)[None, :]
    if op == "time":
        m = b <= a
        if window > 0:
            m &= (a - b) <= window - 1
        return m
    ag = (np.arange(L) >= agent_begin) & (np.arange(L) < agent_begin + agent_count)
    return ~(ag[None, :] & ~ag[:, None])


def call_fwd(lib, op, q, k, v, window=0, ab=0, ac=0, scale=0.0):
    if op == "space":
        return O.space_fwd(q, k, v, ab, ac, scale, lib=lib)
    return O.time_fwd(q, k, v, window, scale, lib=lib)


def call_bwd(lib, op, q, k, v, do, window=0, ab=0, ac=0, scale=0.0):
    if op == "space":
        return O.space_bwd(q, k, v, do, ab, ac, scale, lib=lib)
    return O.time_bwd(q, k, v, do, window, scale, lib=lib)


def torch_ref(op, q, k, v, do, window=0, ab=0, ac=0, scale=0.0):
    """Library reference: torch CPU fp64 SDPA with a boolean mask + autograd."""
    B, T, N, Hq, D = q.shape
    Hkv = k.shape[3]
    L = N if op == "space" else T
    s = scale if scale > 0 else 1.0 / math.sqrt(D)
    qt = torch.tensor(to_units(q, op).copy(), dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(to_units(k, op).copy(), dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(to_units(v, op).copy(), dtype=torch.float64, requires_grad=True)
    dt = torch.tensor(to_units(do, op).copy(), dtype=torch.float64)
    m = torch.tensor(vis_matrix(op, L, window, ab, ac))
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=s, enable_gqa=(Hq != Hkv))
    (o * dt).sum().backward()
    with torch.no_grad():
        kr = kt.repeat_interleave(Hq // Hkv, dim=1)
        z = torch.matmul(qt, kr.transpose(-1, -2).contiguous()) * s
        z = z.masked_fill(~m, float("-inf"))
        lse = torch.logsumexp(z, dim=-1)
    return (from_units(o.detach().numpy(), op, q.shape),
            lse_from_units(lse.numpy(), op, (B, T, N, Hq)),
            from_units(qt.grad.numpy(), op, q.shape),
            from_units(kt.grad.numpy(), op, k.shape),
            from_units(vt.grad.numpy(), op, v.shape))


def close(a, b, tol=1e-10, what=""):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert err <= tol * ref, "%s: max err %.3e (ref %.3e)" % (what, err, ref)


# ---------------------------------------------------- library-routine pins

SPACE_CASES = [
    # (B, T, N, Hq, Hkv, D, agent_begin, agent_count)
    (1, 2, 7, 4, 2, 8, 6, 1),     # agent last
    (2, 1, 9, 3, 1, 5, 0, 1),     # agent first, MQA
    (1, 3, 6, 2, 2, 4, 2, 2),     # two agents in the middle, MHA
    (1, 1, 5, 6, 3, 3, 0, 0),     # no isolation (dense)
    (1, 2, 16, 4, 2, 32, 15, 1),  # tiny fp32 workload shape
]
TIME_CASES = [
    # (B, T, N, Hq, Hkv, D, window)
    (1, 8, 3, 4, 2, 8, 4),
    (2, 6, 2, 3, 1, 5, 1),
    (1, 7, 2, 2, 2, 4, 0),
    (1, 5, 2, 6, 3, 3, 9),       # window longer than the sequence
    (1, 8, 4, 4, 2, 32, 4),      # tiny fp32 workload shape
]


def pin_sdpa_space(lib):
    for i, (B, T, N, Hq, Hkv, D, ab, ac) in enumerate(SPACE_CASES):
        q = rnd((B, T, N, Hq, D), 10 + i)
        k = rnd((B, T, N, Hkv, D), 20 + i)
        v = rnd((B, T, N, Hkv, D), 30 + i)
        do = rnd((B, T, N, Hq, D), 40 + i)
        sc = 0.0 if i % 2 == 0 else 0.37
        o, lse = call_fwd(lib, "space", q, k, v, 0, ab, ac, sc)
        dq, dk, dv = call_bwd(lib, "space", q, k, v, do, 0, ab, ac, sc)
        ro, rl, rdq, rdk, rdv = torch_ref("space", q, k, v, do, 0, ab, ac, sc)
        for a, b, n in ((o, ro, "o"), (lse, rl, "lse"), (dq, rdq, "dq"), (dk, rdk, "dk"), (dv, rdv, "dv")):
            close(a, b, 1e-10, "space case %d %s" % (i, n))


def pin_sdpa_time(lib):
    for i, (B, T, N, Hq, Hkv, D, W) in enumerate(TIME_CASES):
        q = rnd((B, T, N, Hq, D), 110 + i)
        k = rnd((B, T, N, Hkv, D), 120 + i)
        v = rnd((B, T, N, Hkv, D), 130 + i)
        do = rnd((B, T, N, Hq, D), 140 + i)
        sc = 0.0 if i % 2 == 0 else 0.29
        o, lse = call_fwd(lib, "time", q, k, v, W, 0, 0, sc)
        dq, dk, dv = call_bwd(lib, "time", q, k, v, do, W, 0, 0, sc)
        ro, rl, rdq, rdk, rdv = torch_ref("time", q, k, v, do, W, 0, 0, sc)
        for a, b, n in ((o, ro, "o"), (lse, rl, "lse"), (dq, rdq, "dq"), (dk, rdk, "dk"), (dv, rdv, "dv")):
            close(a, b, 1e-10, "time case %d %s" % (i, n))


# ----------------------------------------------------------- closed forms

def pin_identical_keys(lib):
    """All keys of a unit equal -> uniform weights over the visible set:
    o_i = mean of visible v_j, LSE_i = s<q_i, k> + ln|vis(i)|."""
    for op, (B, T, N, Hq, Hkv, D), W, ab, ac in (
            ("space", (1, 2, 9, 4, 2, 8), 0, 8, 1),
            ("space", (1, 1, 7, 2, 1, 4), 0, 2, 3),
            ("time", (1, 9, 2, 4, 2, 8), 3, 0, 0),
            ("time", (2, 5, 1, 2, 2, 4), 0, 0, 0)):
        q = rnd((B, T, N, Hq, D), 1)
        k = np.broadcast_to(rnd((1, 1, 1, Hkv, D), 2), (B, T, N, Hkv, D)).copy()
        v = rnd((B, T, N, Hkv, D), 3)
        o, lse = call_fwd(lib, op, q, k, v, W, ab, ac)
        G = Hq // Hkv
        L = N if op == "space" else T
        M = vis_matrix(op, L, W, ab, ac)
        s = 1.0 / math.sqrt(D)
        qu, vu = to_units(q, op), to_units(v, op)
        ou, lu = to_units(o, op), lse.reshape(-1)  # lse checked via per-element loop below
        lse_u = to_units(lse[..., None], op)[..., 0]
        k0 = k[0, 0, 0]
        for u in range(qu.shape[0]):
            for h in range(Hq):
                g = h // G
                for a in range(L):
                    sel = M[a]
                    want_o = vu[u, g, sel].mean(axis=0)
                    want_l = s * float(qu[u, h, a] @ k0[g]) + math.log(sel.sum())
                    close(ou[u, h, a], want_o, 1e-12, "identical keys o")
                    close(lse_u[u, h, a], want_l, 1e-12, "identical keys lse")
        del lu


def read_golden_counts():
    rows = []
    with open(os.path.join(GOLDEN, "visible_counts.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            op, N, T, W, ab, ac, kind, pos, cnt = line.split()
            rows.append((op, int(N), int(T), int(W), int(ab), int(ac), kind, int(pos), int(cnt)))
    return rows


def pin_q_zero_golden(lib):
    """q = 0: every score is 0, LSE = ln(count) with the counts of the golden
    fixture at the page shapes, and o = mean of the visible values."""
    for op, N, T, W, ab, ac, kind, pos, cnt in read_golden_counts():
        Hq, Hkv, D = 2, 1, 4
        q = np.zeros((1, T, N, Hq, D))
        k = rnd((1, T, N, Hkv, D), 7)
        v = rnd((1, T, N, Hkv, D), 8)
        o, lse = call_fwd(lib, op, q, k, v, W, ab, ac)
        if op == "space":
            got_l = lse[0, 0, pos]
            got_o = o[0, 0, pos, 0]
            vis = [j for j in range(N) if not (ab <= j < ab + ac) or (ab <= pos < ab + ac)]
            want_o = v[0, 0, vis, 0].mean(axis=0)
        else:
            got_l = lse[0, pos, 0]
            got_o = o[0, pos, 0, 0]
            lo = max(0, pos - W + 1) if W > 0 else 0
            want_o = v[0, lo:pos + 1, 0, 0].mean(axis=0)
        close(got_l, np.full(Hq, math.log(cnt)), 1e-12, "q=0 lse %s %s" % (op, pos))
        close(got_o, want_o, 1e-12, "q=0 o %s %s" % (op, pos))


def pin_window_one(lib):
    """W = 1: frame t sees only itself: o_t = v_t, LSE = s<q_t, k_t>,
    dQ = 0, dK = 0 (a single key has dS = 0), dV_t = sum over the group of dO_t."""
    B, T, N, Hq, Hkv, D = 2, 6, 3, 4, 2, 8
    q, k, v, do = (rnd((B, T, N, h, D), s) for h, s in ((Hq, 1), (Hkv, 2), (Hkv, 3), (Hq, 4)))
    o, lse = call_fwd(lib, "time", q, k, v, 1)
    dq, dk, dv = call_bwd(lib, "time", q, k, v, do, 1)
    G = Hq // Hkv
    kr = np.repeat(k, G, axis=3)
    vr = np.repeat(v, G, axis=3)
    close(o, vr, 1e-12, "W=1 o")
    close(lse, (q * kr).sum(-1) / math.sqrt(D), 1e-12, "W=1 lse")
    close(dq, np.zeros_like(dq), 1e-12, "W=1 dq")
    close(dk, np.zeros_like(dk), 1e-12, "W=1 dk")
    close(dv, do.reshape(B, T, N, Hkv, G, D).sum(4), 1e-12, "W=1 dv")


def pin_constant_values(lib):
    """v_j = c for every key: o = c whatever the weights."""
    for op, W, ab, ac in (("space", 0, 4, 1), ("time", 3, 0, 0)):
        B, T, N, Hq, Hkv, D = 1, 5, 6, 4, 2, 8
        q = rnd((B, T, N, Hq, D), 11, 2.0)
        k = rnd((B, T, N, Hkv, D), 12, 2.0)
        c = rnd((Hkv, D), 13)
        v = np.broadcast_to(c, (B, T, N, Hkv, D)).copy()
        o, _ = call_fwd(lib, op, q, k, v, W, ab, ac)
        close(o, np.repeat(v, Hq // Hkv, axis=3), 1e-12, "const v " + op)


# --------------------------------------------------- backward identities

def pin_backward_sums(lib):
    """sum_j dS_ij = 0  =>  sum_j dK_j = 0 per unit and KV head;
    sum_j dV_j = sum over the group's heads and all queries of dO."""
    for op, W, ab, ac in (("space", 0, 7, 1), ("time", 4, 0, 0), ("time", 0, 0, 0)):
        B, T, N, Hq, Hkv, D = 1, 6, 8, 6, 2, 8
        q, k, v, do = (rnd((B, T, N, h, D), s) for h, s in ((Hq, 21), (Hkv, 22), (Hkv, 23), (Hq, 24)))
        dq, dk, dv = call_bwd(lib, op, q, k, v, do, W, ab, ac)
        dku = to_units(dk, op)   # (U, Hkv, L, D)
        dvu = to_units(dv, op)
        dou = to_units(do, op)   # (U, Hq, L, D)
        close(dku.sum(2), np.zeros_like(dku.sum(2)), 1e-11, "sum dK " + op)
        want = dou.reshape(dou.shape[0], Hkv, Hq // Hkv, dou.shape[2], D).sum((2, 3))
        close(dvu.sum(2), want, 1e-11, "sum dV " + op)


def pin_finite_differences(lib):
    """Central differences of L = sum(O * dO) match the analytic gradients
    (tiny workload shape: 16 tokens, 8 frames, 4 q heads over 2 KV heads, D 32)."""
    B, T, N, Hq, Hkv, D = 1, 8, 16, 4, 2, 32
    for op, W, ab, ac in (("space", 0, 15, 1), ("time", 4, 0, 0)):
        q, k, v, do = (rnd((B, T, N, h, D), s) for h, s in ((Hq, 31), (Hkv, 32), (Hkv, 33), (Hq, 34)))
        dq, dk, dv = call_bwd(lib, op, q, k, v, do, W, ab, ac)
        rng = np.random.default_rng(35)
        eps = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            flat = x.reshape(-1)
            for idx in rng.choice(flat.size, size=24, replace=False):
                old = flat[idx]
                flat[idx] = old + eps
                lp = (call_fwd(lib, op, q, k, v, W, ab, ac)[0] * do).sum()
                flat[idx] = old - eps
                lm = (call_fwd(lib, op, q, k, v, W, ab, ac)[0] * do).sum()
                flat[idx] = old
                fd = (lp - lm) / (2 * eps)
                an = g.reshape(-1)[idx]
                assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), \
                    "FD %s %s[%d]: fd %.9g analytic %.9g" % (op, name, idx, fd, an)


# ------------------------------------------------------------- invariants

def pin_future_and_window_invariance(lib):
    """Perturbing frames t' > t, or frames t' <= t - W, leaves o_t (and LSE_t)
    bitwise unchanged."""
    B, T, N, Hq, Hkv, D, W = 1, 10, 2, 4, 2, 8, 3
    q, k, v = (rnd((B, T, N, h, D), s) for h, s in ((Hq, 41), (Hkv, 42), (Hkv, 43)))
    o, lse = call_fwd(lib, "time", q, k, v, W)
    t = 5
    k2, v2 = k.copy(), v.copy()
    k2[:, t + 1:] += 3.0
    v2[:, t + 1:] -= 2.0
    k2[:, :t - W + 1] *= -1.5
    v2[:, :t - W + 1] += 7.0
    o2, lse2 = call_fwd(lib, "time", q, k2, v2, W)
    assert np.array_equal(o[:, t], o2[:, t]) and np.array_equal(lse[:, t], lse2[:, t]), \
        "frame t changed when future / out-of-window frames changed"
    assert not np.array_equal(o[:, t + 1], o2[:, t + 1]), "future frame should change"


def pin_agent_invariance(lib):
    """Perturbing the agent token's K/V leaves every world token's outputs
    bitwise unchanged; the agent token's own output does change."""
    B, T, N, Hq, Hkv, D = 1, 3, 9, 4, 2, 8
    for ab, ac in ((8, 1), (0, 1), (3, 2)):
        q, k, v = (rnd((B, T, N, h, D), s) for h, s in ((Hq, 51), (Hkv, 52), (Hkv, 53)))
        o, lse = call_fwd(lib, "space", q, k, v, 0, ab, ac)
        k2, v2 = k.copy(), v.copy()
        k2[:, :, ab:ab + ac] += 5.0
        v2[:, :, ab:ab + ac] -= 3.0
        o2, lse2 = call_fwd(lib, "space", q, k2, v2, 0, ab, ac)
        world = [j for j in range(N) if not (ab <= j < ab + ac)]
        assert np.array_equal(o[:, :, world], o2[:, :, world]), "world O changed with agent K/V"
        assert np.array_equal(lse[:, :, world], lse2[:, :, world]), "world LSE changed"
        assert not np.array_equal(o[:, :, ab], o2[:, :, ab]), "agent O should change"


def pin_gqa_equals_replicated(lib):
    """GQA with head h -> KV head h // G equals the op on KV heads replicated to
    Hq heads (dK, dV of the replicated op summed over each group)."""
    for op, W, ab, ac in (("space", 0, 6, 1), ("time", 3, 0, 0)):
        B, T, N, Hq, Hkv, D = 1, 5, 7, 6, 2, 8
        G = Hq // Hkv
        q, k, v, do = (rnd((B, T, N, h, D), s) for h, s in ((Hq, 61), (Hkv, 62), (Hkv, 63), (Hq, 64)))
        kr, vr = np.repeat(k, G, axis=3), np.repeat(v, G, axis=3)
        o, lse = call_fwd(lib, op, q, k, v, W, ab, ac)
        o2, lse2 = call_fwd(lib, op, q, kr, vr, W, ab, ac)
        close(o, o2, 1e-13, "gqa o")
        close(lse, lse2, 1e-13, "gqa lse")
        dq, dk, dv = call_bwd(lib, op, q, k, v, do, W, ab, ac)
        dq2, dk2, dv2 = call_bwd(lib, op, q, kr, vr, do, W, ab, ac)
        close(dq, dq2, 1e-12, "gqa dq")
        close(dk, dk2.reshape(B, T, N, Hkv, G, D).sum(4), 1e-12, "gqa dk")
        close(dv, dv2.reshape(B, T, N, Hkv, G, D).sum(4), 1e-12, "gqa dv")


def pin_key_shift(lib):
    """k_j += c for every key of a unit: O unchanged, LSE_i shifts by s<q_i, c>."""
    for op, W, ab, ac in (("space", 0, 5, 1), ("time", 4, 0, 0)):
        B, T, N, Hq, Hkv, D = 1, 6, 6, 4, 2, 8
        q, k, v = (rnd((B, T, N, h, D), s) for h, s in ((Hq, 71), (Hkv, 72), (Hkv, 73)))
        c = rnd((Hkv, D), 74)
        o, lse = call_fwd(lib, op, q, k, v, W, ab, ac)
        o2, lse2 = call_fwd(lib, op, q, k + c, v, W, ab, ac)
        close(o, o2, 1e-11, "shift o")
        shift = (q * np.repeat(c, Hq // Hkv, axis=0)).sum(-1) / math.sqrt(D)
        close(lse2 - lse, shift, 1e-11, "shift lse")


def pin_permute_world_tokens(lib):
    """Permuting the world tokens of a block permutes the outputs."""
    B, T, N, Hq, Hkv, D, ab = 1, 2, 8, 4, 2, 8, 7
    q, k, v, do = (rnd((B, T, N, h, D), s) for h, s in ((Hq, 81), (Hkv, 82), (Hkv, 83), (Hq, 84)))
    perm = np.concatenate([np.random.default_rng(85).permutation(7), [7]])
    o, lse = call_fwd(lib, "space", q, k, v, 0, ab, 1)
    dq, dk, dv = call_bwd(lib, "space", q, k, v, do, 0, ab, 1)
    P = lambda x: x[:, :, perm]
    o2, lse2 = call_fwd(lib, "space", P(q), P(k), P(v), 0, ab, 1)
    dq2, dk2, dv2 = call_bwd(lib, "space", P(q), P(k), P(v), P(do), 0, ab, 1)
    close(o2, P(o), 1e-12, "perm o")
    close(lse2, P(lse), 1e-12, "perm lse")
    close(dq2, P(dq), 1e-12, "perm dq")
    close(dk2, P(dk), 1e-12, "perm dk")
    close(dv2, P(dv), 1e-12, "perm dv")


def pin_units_independent(lib):
    """Shuffling blocks (space) or slots (time) shuffles the outputs."""
    for op, W, ab, ac in (("space", 0, 4, 1), ("time", 3, 0, 0)):
        B, T, N, Hq, Hkv, D = 2, 4, 5, 2, 1, 4
        q, k, v = (rnd((B, T, N, h, D), s) for h, s in ((Hq, 91), (Hkv, 92), (Hkv, 93)))
        o, lse = call_fwd(lib, op, q, k, v, W, ab, ac)
        if op == "space":
            pb, pt = np.random.default_rng(94).permutation(B), np.random.default_rng(95).permutation(T)
            S = lambda x: x[pb][:, pt]
        else:
            pb, pn = np.random.default_rng(96).permutation(B), np.random.default_rng(97).permutation(N)
            S = lambda x: x[pb][:, :, pn]
        o2, lse2 = call_fwd(lib, op, S(q), S(k), S(v), W, ab, ac)
        close(o2, S(o), 1e-13, "units o " + op)
        close(lse2, S(lse), 1e-13, "units lse " + op)


# ------------------------------------------------------- rollout decode

def ring_frames(C, last):
    """Absolute frame held by each ring position after frames up to ``last``
    were written at f % C (-1: never written)."""
    out = np.full(C, -1)
    for f in range(max(0, last - C + 1), last + 1):
        out[f % C] = f
    return out


# (B, Tq, N, Hq, Hkv, D, W, C, q_frame0)
DECODE_CASES = [
    (1, 1, 3, 4, 2, 8, 4, 4, 10),   # steady state, ring wrapped, C = W
    (2, 1, 2, 3, 1, 5, 3, 5, 1),    # second frame: partial history, C > W
    (1, 3, 2, 2, 2, 4, 0, 7, 4),    # unbounded window, three new frames fill the ring
    (1, 2, 2, 6, 3, 3, 5, 6, 20),   # two new frames, C = W + 1
    (1, 1, 2, 4, 2, 16, 1, 3, 7),   # window 1
]


def decode_ref(q, kc, vc, q_frame0, W, scale=0.0):
    """torch fp64 SDPA over the ring positions, masked by which frame each
    position holds; LSE from torch.logsumexp."""
    B, Tq, N, Hq, D = q.shape
    C, Hkv = kc.shape[1], kc.shape[3]
    s = scale if scale > 0 else 1.0 / math.sqrt(D)
    held = ring_frames(C, q_frame0 + Tq - 1)
    a = (q_frame0 + np.arange(Tq))[:, None]
    f = held[None, :]
    m = (f >= 0) & (f <= a)
    if W > 0:
        m &= (a - f) <= W - 1
    mt = torch.tensor(m)
    qt = torch.tensor(q.transpose(0, 2, 3, 1, 4).reshape(B * N, Hq, Tq, D))
    kt = torch.tensor(kc.transpose(0, 2, 3, 1, 4).reshape(B * N, Hkv, C, D))
    vt = torch.tensor(vc.transpose(0, 2, 3, 1, 4).reshape(B * N, Hkv, C, D))
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=s, enable_gqa=(Hq != Hkv))
    kr = kt.repeat_interleave(Hq // Hkv, dim=1)
    z = (torch.matmul(qt, kr.transpose(-1, -2).contiguous()) * s).masked_fill(~mt, float("-inf"))
    lse = torch.logsumexp(z, dim=-1)
    o = o.numpy().reshape(B, N, Hq, Tq, D).transpose(0, 3, 1, 2, 4)
    lse = lse.numpy().reshape(B, N, Hq, Tq).transpose(0, 3, 1, 2)
    return o, lse


def pin_decode_sdpa(lib):
    """Decode against a library routine over the ring positions."""
    for i, (B, Tq, N, Hq, Hkv, D, W, C, t0) in enumerate(DECODE_CASES):
        q = rnd((B, Tq, N, Hq, D), 510 + i)
        kc = rnd((B, C, N, Hkv, D), 520 + i)
        vc = rnd((B, C, N, Hkv, D), 530 + i)
        sc = 0.0 if i % 2 == 0 else 0.41
        o, lse = O.time_decode_fwd(q, kc, vc, t0, W, sc, lib=lib)
        ro, rl = decode_ref(q, kc, vc, t0, W, sc)
        close(o, ro, 1e-10, "decode case %d o" % i)
        close(lse, rl, 1e-10, "decode case %d lse" % i)


def pin_decode_matches_full_sequence(lib):
    """Decoding frame t from a ring filled with frames <= t reproduces row t
    of time attention over the whole sequence (the training op)."""
    B, T, N, Hq, Hkv, D = 1, 11, 3, 4, 2, 8
    q = rnd((B, T, N, Hq, D), 541)
    k = rnd((B, T, N, Hkv, D), 542)
    v = rnd((B, T, N, Hkv, D), 543)
    for W, C in ((4, 4), (4, 6), (0, 11)):
        o_full, lse_full = O.time_fwd(q, k, v, W, lib=lib)
        for t in (0, 2, 5, 10):
            held = ring_frames(C, t)
            kc = np.zeros((B, C, N, Hkv, D))
            vc = np.zeros((B, C, N, Hkv, D))
            for pos, f in enumerate(held):
                if f >= 0:
                    kc[:, pos], vc[:, pos] = k[:, f], v[:, f]
            o, lse = O.time_decode_fwd(q[:, t:t + 1], kc, vc, t, W, lib=lib)
            close(o[:, 0], o_full[:, t], 1e-12, "decode vs full o W=%d C=%d t=%d" % (W, C, t))
            close(lse[:, 0], lse_full[:, t], 1e-12, "decode vs full lse W=%d C=%d t=%d" % (W, C, t))


# ---------------------------------------------------------- projections

def pin_rmsnorm_qkv_torch(lib):
    """RMS norm + QKV projection against torch fp64 (F.rms_norm, a matmul)."""
    for i, (M, dm, Hq, Hkv, D, eps) in enumerate(((7, 48, 4, 2, 8, 1e-6), (5, 40, 3, 1, 8, 1e-3),
                                                  (3, 64, 2, 2, 16, 0.0))):
        x = rnd((M, dm), 610 + i, 3.0)
        g = rnd((dm,), 620 + i)
        w = rnd(((Hq + 2 * Hkv) * D, dm), 630 + i, 0.2)
        q, k, v, rstd = O.rmsnorm_qkv_fwd(x, g, w, Hq, Hkv, D, eps, lib=lib)
        xt = torch.tensor(x)
        y = F.rms_norm(xt, (dm,), torch.tensor(g), eps=eps)
        out = (y @ torch.tensor(w).T).numpy()
        close(q, out[:, :Hq * D], 1e-12, "qkv case %d q" % i)
        close(k, out[:, Hq * D:(Hq + Hkv) * D], 1e-12, "qkv case %d k" % i)
        close(v, out[:, (Hq + Hkv) * D:], 1e-12, "qkv case %d v" % i)
        close(rstd, torch.rsqrt((xt * xt).mean(-1) + eps).numpy(), 1e-12, "qkv case %d rstd" % i)


def pin_rmsnorm_scale_invariance(lib):
    """With eps = 0 the RMS norm ignores a power-of-two scale of its input
    exactly, so every output is bitwise the same."""
    M, dm, Hq, Hkv, D = 6, 32, 2, 1, 8
    x = rnd((M, dm), 641)
    g = rnd((dm,), 642)
    w = rnd(((Hq + 2 * Hkv) * D, dm), 643)
    a = O.rmsnorm_qkv_fwd(x, g, w, Hq, Hkv, D, 0.0, lib=lib)
    b = O.rmsnorm_qkv_fwd(x * 8.0, g, w, Hq, Hkv, D, 0.0, lib=lib)
    for u, t, n in zip(a[:3], b[:3], "qkv"):
        close(u, t, 0.0, "scale invariance " + n)


def pin_out_proj(lib):
    """Output projection + residual against a torch fp64 matmul; identity
    weights return the input plus the residual exactly."""
    M, din, dm = 9, 24, 16
    o = rnd((M, din), 651)
    w = rnd((dm, din), 652)
    r = rnd((M, dm), 653)
    y = O.out_proj_fwd(o, w, r, lib=lib)
    close(y, r + (torch.tensor(o) @ torch.tensor(w).T).numpy(), 1e-12, "out proj")
    close(O.out_proj_fwd(o, w, None, lib=lib), (torch.tensor(o) @ torch.tensor(w).T).numpy(), 1e-12,
          "out proj no residual")
    eye = np.eye(dm, din)
    close(O.out_proj_fwd(o, eye, r, lib=lib), o[:, :dm] + r, 0.0, "out proj identity")


ALL_PINS = [
    pin_sdpa_space, pin_sdpa_time, pin_identical_keys, pin_q_zero_golden, pin_window_one,
    pin_constant_values, pin_backward_sums, pin_finite_differences,
    pin_future_and_window_invariance, pin_agent_invariance, pin_gqa_equals_replicated,
    pin_key_shift, pin_permute_world_tokens, pin_units_independent,
    pin_decode_sdpa, pin_decode_matches_full_sequence,
    pin_rmsnorm_qkv_torch, pin_rmsnorm_scale_invariance, pin_out_proj,
]
