"""Page-shaped attention workloads (shapes, mask descriptors, value recipes).

Every shape below is taken from, or derived from, the Open Dreamer articles
(pro.edgex.exchange "Open Dreamer ... Dreamer 4 world model", fr-FR / es-LA /
ja-JP editions, and the 7minutos.es edition):

* dynamics model, section "Configuration d'entraînement": 30 attention heads
  over 3 KV heads (GQA) at d_model 1920, so head_dim 64; 32 learned register
  tokens per timestep; packing factor 2 (512 tokenizer latents -> 256 spatial
  tokens); time attention in a 192-step sliding window.
* section "Architecture": each timestep block holds (previous action, state,
  policy); world tokens may not read the agent token.
* tokenizer, section "Configuration d'entraînement": 368x640 frames in 16x16
  patches (920 patches), 512 latent tokens per frame, encoder d_model 1536,
  decoder d_model 1024; MAE masking up to 0.9.

Token order inside a block (the pages fix none of it): action first, then the
spatial tokens, then registers, agent token last (policy is last in the
block's tuple).  Only the agent slot matters to the arithmetic.

This module holds no attention arithmetic; it only describes workloads.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

SPACE = "space"
TIME = "time"


@dataclass(frozen=True)
class Workload:
    name: str
    op: str                 # "space" or "time"
    B: int
    T: int
    N: int
    Hq: int
    Hkv: int
    D: int
    dtype: str = "bf16"     # "bf16" or "f32"
    window: int = 0         # time op: 0 = unbounded causal, else sliding window
    agent_begin: int = 0    # space op: first agent slot
    agent_count: int = 0    # space op: 0 = no isolation
    value_scale: float = 1.0  # multiply the N(0,1) draws before rounding
    seed: int = 0           # SeedSequence entropy
    shared_rows: Optional[Tuple[int, int]] = None  # (slot_begin, count): MAE mask-token rows
    note: str = ""
    dout_scale: float = 1.0  # multiply the dO draws before rounding

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def units(self) -> int:
        """Independent attention problems per head: blocks (space) or slots (time)."""
        return self.B * self.T if self.op == SPACE else self.B * self.N

    @property
    def seq_len(self) -> int:
        """Positions inside one problem: tokens (space) or frames (time)."""
        return self.N if self.op == SPACE else self.T

    def q_shape(self):
        return (self.B, self.T, self.N, self.Hq, self.D)

    def kv_shape(self):
        return (self.B, self.T, self.N, self.Hkv, self.D)

    def lse_shape(self):
        return (self.B, self.T, self.N, self.Hq)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def visible_pairs(w: Workload) -> int:
    """Number of visible (query, key) pairs summed over units and query heads.

    Space: (N - A)^2 + A*N per block-head (world queries skip the A agent keys,
    agent queries read all N).  Time: sum_t min(t + 1, W) per slot-head.
    This is the count the FLOP figures use; masked or padded work is never
    counted.
    """
    if w.op == SPACE:
        A = w.agent_count
        per = (w.N - A) * (w.N - A) + A * w.N
        return per * w.units * w.Hq
    W = w.window if w.window > 0 else w.T
    per = sum(min(t + 1, W) for t in range(w.T))
    return per * w.units * w.Hq


def flops(w: Workload, direction: str) -> float:
    """Algorithmic FLOPs: 4*D per visible pair forward (QK^T and PV), 10*D
    backward (S recompute, dP, dV, dQ, dK)."""
    per = 4 if direction == "fwd" else 10
    return float(per * w.D * visible_pairs(w))


def min_bytes(w: Workload, direction: str) -> float:
    """Minimum HBM bytes the op must move.

    fwd: read Q, K, V; write O and LSE.
    bwd: read Q, K, V, O, dO, LSE; write dQ, dK, dV.
    """
    es = 2 if w.dtype == "bf16" else 4
    nq = w.B * w.T * w.N * w.Hq * w.D
    nkv = w.B * w.T * w.N * w.Hkv * w.D
    nl = w.B * w.T * w.N * w.Hq
    if direction == "fwd":
        return float(es * (nq + 2 * nkv + nq) + 4 * nl)
    return float(es * (nq + 2 * nkv + nq + nq) + 4 * nl + es * (nq + 2 * nkv))


def _mk() -> Dict[str, Workload]:
    c: Dict[str, Workload] = {}
    # 1: tiny fp32 case; 13 spatial + 2 registers + agent at slot 15.
    c["1s"] = Workload("1s", SPACE, 1, 8, 16, 4, 2, 32, "f32", 0, 15, 1, 1.0, 1000,
                       note="tiny fp32 space attention")
    c["1t"] = Workload("1t", TIME, 1, 8, 16, 4, 2, 32, "f32", 4, 0, 0, 1.0, 1000,
                       note="tiny fp32 time attention, window 4")
    # 2: CoinRun-scale: action@0, 64 spatial, 8 registers, agent@73; d_model 512.
    c["2s"] = Workload("2s", SPACE, 8, 64, 74, 8, 2, 64, "bf16", 0, 73, 1, 0.125, 2000,
                       note="CoinRun space layer, inputs scaled by 1/8")
    c["2t"] = Workload("2t", TIME, 8, 64, 74, 8, 2, 64, "bf16", 64, 0, 0, 0.125, 2000,
                       note="CoinRun time layer, window 64, inputs scaled by 1/8")
    c["2su"] = c["2s"].with_(name="2su", value_scale=1.0, seed=2001,
                             note="CoinRun space layer, unscaled inputs (parity only)")
    c["2tu"] = c["2t"].with_(name="2tu", value_scale=1.0, seed=2001,
                             note="CoinRun time layer, unscaled inputs (parity only)")
    # 3: Minecraft dynamics space layer: 256 frames = 4 x 64; 290-token blocks.
    c["3"] = Workload("3", SPACE, 4, 64, 290, 30, 3, 64, "bf16", 0, 289, 1, 1.0, 3000,
                      note="Minecraft dynamics space layer")
    # 4: Minecraft dynamics time layer: 256 frames, 290 slots, window 192.
    c["4"] = Workload("4", TIME, 1, 256, 290, 30, 3, 64, "bf16", 192, 0, 0, 1.0, 4000,
                      note="Minecraft dynamics time layer")
    # 5: tokenizer: 920 patches + 512 latents = 1432 tokens per frame, 16 frames.
    c["5a"] = Workload("5a", SPACE, 1, 16, 1432, 24, 24, 64, "bf16", 0, 0, 0, 1.0, 5000,
                       shared_rows=(0, 828),
                       note="tokenizer encoder space layer, 90% of patches share the mask token")
    c["5b"] = Workload("5b", SPACE, 1, 16, 1432, 16, 16, 64, "bf16", 0, 0, 0, 1.0, 5001,
                       note="tokenizer decoder space layer")
    c["5c"] = Workload("5c", TIME, 1, 16, 1432, 16, 16, 64, "bf16", 16, 0, 0, 1.0, 5002,
                       note="tokenizer decoder time layer, window 16")
    c["5d"] = Workload("5d", TIME, 1, 16, 1432, 24, 24, 64, "bf16", 16, 0, 0, 1.0, 5003,
                       note="tokenizer encoder time layer (24 heads, MHA), window 16")
    return c


CONFIGS: Dict[str, Workload] = _mk()

# The bench step: one pass of the dynamics model's attention hot path at the
# Minecraft shape, the space layer (3) and the time layer (4), fwd + bwd.
BENCH_STEP: List[str] = ["3", "4"]


def get(name: str) -> Workload:
    return CONFIGS[name]


# ------------------------------------------------------------ rollout decode

@dataclass(frozen=True)
class DecodeWorkload:
    """Time attention of Tq new frames against a ring-buffer K/V cache of C
    frames (absolute frame f at ring position f % C); the queries are the
    absolute frames q_frame0 .. q_frame0 + Tq - 1."""
    name: str
    B: int
    Tq: int
    N: int
    Hq: int
    Hkv: int
    D: int
    window: int
    cache_frames: int
    q_frame0: int
    dtype: str = "bf16"
    seed: int = 0
    note: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def q_shape(self):
        return (self.B, self.Tq, self.N, self.Hq, self.D)

    def cache_shape(self):
        return (self.B, self.cache_frames, self.N, self.Hkv, self.D)

    def key_frames(self) -> Tuple[int, int]:
        """Absolute frames [first, last] the queries read."""
        last = self.q_frame0 + self.Tq - 1
        first = max(0, self.q_frame0 - self.window + 1) if self.window > 0 else 0
        return first, last

    def with_(self, **kw) -> "DecodeWorkload":
        return replace(self, **kw)


def decode_visible_pairs(w: DecodeWorkload) -> int:
    per = 0
    for t in range(w.Tq):
        a = w.q_frame0 + t
        per += min(a + 1, w.window) if w.window > 0 else a + 1
    return per * w.B * w.N * w.Hq


def decode_flops(w: DecodeWorkload) -> float:
    """4*D per visible pair (QK^T and PV)."""
    return float(4 * w.D * decode_visible_pairs(w))


def decode_min_bytes(w: DecodeWorkload) -> float:
    """Read Q and the cached K, V frames the queries see; write O and LSE."""
    es = 2 if w.dtype == "bf16" else 4
    first, last = w.key_frames()
    nq = w.B * w.Tq * w.N * w.Hq * w.D
    nkv = w.B * (last - first + 1) * w.N * w.Hkv * w.D
    return float(es * (2 * nq + 2 * nkv) + 4 * w.B * w.Tq * w.N * w.Hq)


# Rollout of the Minecraft dynamics model (frame-by-frame generation, section
# "Artefacts publiés"): one new frame of 290 slots, 30 / 3 heads, window 192,
# the ring holding the 192 frames the window reads, steady state (wrapped).
DECODE_CONFIGS: Dict[str, DecodeWorkload] = {
    "dec": DecodeWorkload("dec", 1, 1, 290, 30, 3, 64, 192, 192, 1000, "bf16", 6000,
                          note="Minecraft rollout: one new frame, steady state"),
    "dec_b8": DecodeWorkload("dec_b8", 8, 1, 290, 30, 3, 64, 192, 192, 1000, "bf16", 6001,
                             note="Minecraft rollout, 8 environments"),
}


# --------------------------------------------------- projections beside attention

@dataclass(frozen=True)
class ProjWorkload:
    """RMS norm + QKV projection and output projection + residual over M token
    rows of a d_model-wide residual stream."""
    name: str
    M: int
    d_model: int
    Hq: int
    Hkv: int
    D: int
    eps: float = 1e-6
    seed: int = 0
    note: str = ""

    @property
    def n_qkv(self) -> int:
        return (self.Hq + 2 * self.Hkv) * self.D

    def with_(self, **kw) -> "ProjWorkload":
        return replace(self, **kw)


def proj_flops(w: ProjWorkload, which: str) -> float:
    """2*M*N*K of the GEMM ("qkv" or "out"); the norm is not counted."""
    if which == "qkv":
        return 2.0 * w.M * w.n_qkv * w.d_model
    return 2.0 * w.M * w.d_model * w.Hq * w.D


def proj_min_bytes(w: ProjWorkload, which: str) -> float:
    """qkv: read x, the gain and w_qkv, write q, k, v (and rstd); out: read o,
    w_o and the residual, write y."""
    if which == "qkv":
        return 2.0 * (w.M * w.d_model + w.n_qkv * w.d_model + w.M * w.n_qkv) + 4.0 * (w.d_model + w.M)
    din = w.Hq * w.D
    return 2.0 * (w.M * din + w.d_model * din + 2 * w.M * w.d_model)


# The dynamics model's layer at 256 frames per GPU: 74,240 token rows (4 x 64
# blocks of 290 tokens), d_model 1920, 30 / 3 heads of 64.
PROJ_CONFIGS: Dict[str, ProjWorkload] = {
    "proj": ProjWorkload("proj", 4 * 64 * 290, 1920, 30, 3, 64, 1e-6, 7000,
                         note="Minecraft dynamics projections, 256 frames per GPU"),
}
