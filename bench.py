#!/usr/bin/env python3
"""Benchmark of the block-causal attention hot path on one MI355X.

One step = one pass of the dynamics model's attention at the Minecraft shape
(Open Dreamer articles, pro.edgex.exchange fr-FR edition, sections
"Architecture" and "Configuration d'entraînement"; 256 frames per GPU from
section "Performance de calcul et stratégie mémoire"):

  space layer: 256 blocks (4 sequences x 64 frames) of 290 tokens, 30 query
               heads over 3 KV heads, head_dim 64, agent-token isolation:
               forward + backward;
  time layer:  256 frames x 290 token slots, causal, 192-step window, same
               heads: forward + backward.

Inputs are seeded synthetic bf16 tensors resident in HBM before the timed
region.  ``value`` is algorithmic TFLOP/s over the whole step: 4*D FLOPs per
visible (query, key, head) pair forward and 10*D backward; masked and padded
work is never counted.  Per-op kernel durations come from HIP events on the
stream the kernels run on.

    python bench.py [--gpus 1] [--steps 200] [--warmup 100] [--spinup-ms 300] [--no-cpu-baseline]

Before the warm-up steps, untimed steps run for ``--spinup-ms`` of wall time
(the GPU raises its clock over the first tens of milliseconds of work); the
JSON line reports that phase as ``spinup`` (wall ms and steps).

``--workload rollout_decode`` instead times one step of frame-by-frame
generation (section "Artefacts publiés": rollout generation, the demo
streaming the generated world frame by frame): space attention of the new
290-token block plus time attention of its 290 slots against a ring-buffer
cache of the 192 frames the window reads (``--decode-batch`` environments at
once); ``value`` is generated frames per second through that layer pair.

``--workload projections`` times the GEMMs either side of that attention at
the same 74,240 token rows (section "Configuration d'entraînement": d_model
1920; section "Ingénierie de la stabilité": fp32 norm, bf16 matmul inputs):
RMS norm + QKV projection (1920 -> 1920 + 2 x 192) and the output projection
+ residual; ``value`` is their GEMM TFLOP/s (2*M*N*K each, the norm not
counted).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
TRAFFIC_FILE_DECODE = os.path.join(ROOT, "profiles", "hbm_traffic_rollout_decode.txt")
TRAFFIC_FILE_PROJ = os.path.join(ROOT, "profiles", "hbm_traffic_projections.txt")
TRAFFIC_FILE_LONG = os.path.join(ROOT, "profiles", "hbm_traffic_long_time.txt")
UTIL_FILE = os.path.join(ROOT, "profiles", "mfma_utilisation.txt")


# kernel launches of each attention call (template argument 0 = space, 1 = time)
KERNELS = {
    "time_decode": "attn_fwd_kernel<2>",
    "time_decode_same_ring": "attn_fwd_kernel<2>",
    "space_fwd_block": "attn_fwd_kernel<0>",
    "space_fwd": "attn_fwd_kernel<0>",
    "time_fwd": "attn_fwd_kernel<1>",
    "space_bwd": "attn_bwd_dkv_kernel<0, TPW, FQ> [+ attn_bwd_dq_kernel<0> past 320 keys, "
                 "+ attn_bwd_split_reduce_kernel<0> when the last round is split]",
    "time_bwd": "attn_bwd_dkv_kernel<1, TPW, FQ> [+ attn_bwd_dq_kernel<1> past 320 keys, "
                "+ attn_bwd_split_reduce_kernel<1> when the last round is split]",
    "qkv_proj": "rstd_rows_kernel + fold_gain_kernel + gemm256_kernel<0, 8>",
    "out_proj": "gemm256_kernel<1, 6>",
}


def source_digest(files=None) -> str:
    """Digest of the kernel sources ``files`` (names in csrc/; all by default),
    comments and layout ignored: the one the counter summaries carry."""
    from block_causal_transformer_amd.rocprof_summary import source_digest as digest
    return digest(files)


def _read_summary(path: str):
    """key=value pairs of a committed counter summary, or None when absent or
    taken on kernel sources other than the current ones."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    files = vals.get("source_files")
    if vals.get("source_sha") != source_digest(files.split(",") if files else None):
        return None
    return vals


def read_util(kernel_key: str, path: str = UTIL_FILE):
    """MFMA / VALU busy figures of ``kernel_key`` from the committed rocprofv3
    utilisation summary, or None (absent, or other kernel sources)."""
    vals = _read_summary(path)
    if not vals or kernel_key + ".mfma_busy_pct" not in vals:
        return None
    return {k: float(vals[kernel_key + "." + k]) for k in
            ("mfma_busy_pct", "valu_busy_pct", "coexec_pct", "lds_active_pct")
            if kernel_key + "." + k in vals}


def read_traffic(kernel_key: str, path: str = TRAFFIC_FILE):
    """HBM bytes per launch of ``kernel_key`` from the committed rocprofv3
    counter summary, or None when absent or taken on other kernel sources."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    files = vals.get("source_files")
    if vals.get("source_sha") != source_digest(files.split(",") if files else None):
        return None
    v = vals.get(kernel_key + ".bytes")
    return float(v) if v else None


def cpu_baseline(target_s: float = 15.0):
    """Time the fp64 oracle on a bounded sample of the same step: n whole
    blocks of the space layer and n whole slots of the time layer, fwd + bwd,
    with n chosen from a short probe run so the sample takes ~target_s."""
    from block_causal_transformer_amd import configs as C, gen
    from oracle import oracle as O

    def run(n):
        ws = C.get("3").with_(B=1, T=n)
        wt = C.get("4").with_(N=n)
        xs, xt = gen.make_inputs(ws), gen.make_inputs(wt)
        t0 = time.perf_counter()
        O.fwd(ws, xs["q"], xs["k"], xs["v"])
        O.bwd(ws, xs["q"], xs["k"], xs["v"], xs["dout"])
        O.fwd(wt, xt["q"], xt["k"], xt["v"])
        O.bwd(wt, xt["q"], xt["k"], xt["v"], xt["dout"])
        dt = time.perf_counter() - t0
        fl = sum(C.flops(w, d) for w in (ws, wt) for d in ("fwd", "bwd"))
        return dt, fl

    dt, _ = run(4)
    n = max(4, min(256, int(4 * target_s / max(dt, 1e-3))))
    dt, fl = run(n)
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.max_threads(),
        "kind": "oracle",
        "sample": "%d space blocks (290 tokens, 30 q / 3 kv heads) + %d time slots (256 frames, "
                  "window 192), forward + backward, fp64, %.1f s" % (n, n, dt),
    }


def spread(samples):
    """Median, 10th and 90th percentile (ms) of per-step event durations."""
    import numpy as np
    a = np.asarray(samples, dtype=np.float64)
    return {"ms_median": round(float(np.median(a)), 5), "ms_p10": round(float(np.percentile(a, 10)), 5),
            "ms_p90": round(float(np.percentile(a, 90)), 5)}


def roofline_of(flop, min_bytes, ms):
    intensity = flop / min_bytes
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if intensity >= ridge:
        roof = {"bound": "mfma", "achieved": round(flop / ms / 1e9, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(min_bytes / ms / 1e6, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    return roof


def cpu_baseline_decode(B: int, target_s: float = 12.0):
    """The fp64 oracle on the decode step (the new block's space attention and
    the decode time attention of its slots), repeated for ~target_s."""
    from block_causal_transformer_amd import configs as C, gen
    from oracle import oracle as O

    wd = C.DECODE_CONFIGS["dec"].with_(B=B)
    ws = C.get("3").with_(B=B, T=1)
    xd, xs = gen.make_decode_inputs(wd), gen.make_inputs(ws, with_dout=False)

    def run(n):
        t0 = time.perf_counter()
        for _ in range(n):
            O.fwd(ws, xs["q"], xs["k"], xs["v"])
            O.time_decode_fwd(xd["q"], xd["k_cache"], xd["v_cache"], wd.q_frame0, wd.window)
        return time.perf_counter() - t0

    dt = run(1)
    n = max(1, min(1000, int(target_s / max(dt, 1e-3))))
    dt = run(n)
    return {
        "value": n * B / dt,
        "unit": "frames/s",
        "cores": O.max_threads(),
        "kind": "oracle",
        "sample": "%d decode steps of %d environment(s): space attention of the new 290-token "
                  "block + time attention of its slots over 192 cached frames, fp64, %.1f s"
                  % (n, B, dt),
    }


def spin_up(fn, ms):
    """Call fn() (one untimed step) until at least ms milliseconds have passed.

    The MI355X raises its clock over the first tens of milliseconds of work;
    a run with a handful of warm-up steps would otherwise time part of that
    ramp.  Returns {"ms": wall time spent, "steps": calls}."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "steps": n}


def main_decode(args):
    import torch
    from block_causal_transformer_amd import configs as C, gen, ops

    if not os.path.exists(ops.LIB_PATH):
        from block_causal_transformer_amd import build as hip_build
        hip_build.build()
    ops.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B = args.decode_batch
    wd = C.DECODE_CONFIGS["dec"].with_(B=B)
    ws = C.get("3").with_(B=B, T=1)
    xd, xs = gen.make_decode_inputs(wd), gen.make_inputs(ws, with_dout=False)
    t = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16)
    # A rollout keeps one K/V ring per time layer (seven for the dynamics
    # model), ~43 MB each per environment: together more than the 256 MB
    # MALL.  The timed step therefore rotates over RINGS independent copies
    # of the inputs (8 x 43 MB = 343 MB at one environment), so every call
    # reads its ring from HBM as the layers of a rollout would; the same-ring
    # figure (one ring re-read, resident in the MALL) is reported beside it.
    RINGS = 8
    dq = [t(xd["q"]) for _ in range(RINGS)]
    dk = [t(xd["k_cache"]) for _ in range(RINGS)]
    dvv = [t(xd["v_cache"]) for _ in range(RINGS)]
    sq = [t(xs["q"]) for _ in range(RINGS)]
    sk = [t(xs["k"]) for _ in range(RINGS)]
    sv = [t(xs["v"]) for _ in range(RINGS)]
    do = [torch.empty_like(dq[0]) for _ in range(RINGS)]
    dl = [torch.empty(dq[0].shape[:4], dtype=torch.float32, device=dev) for _ in range(RINGS)]
    so = [torch.empty_like(sq[0]) for _ in range(RINGS)]
    sl = [torch.empty(sq[0].shape[:4], dtype=torch.float32, device=dev) for _ in range(RINGS)]
    dshape, dmask = ops.make_shape(dq[0], dk[0]), ops.make_mask("time", window=wd.window)
    sshape, smask = ops.make_shape(sq[0], sk[0]), ops.make_mask("space", **ops.workload_kwargs(ws))
    stream = torch.cuda.current_stream()

    # A generation step is two small launches, so it is captured in a HIP
    # graph and replayed (the ABI calls take the capturing stream).
    def space_op(i=0):
        cs = torch.cuda.current_stream().cuda_stream
        if ops.space_attn_fwd(sshape, smask, sq[i], sk[i], sv[i], so[i], sl[i], cs):
            raise RuntimeError(ops.bca_last_error())

    def decode_op(i=0):
        cs = torch.cuda.current_stream().cuda_stream
        if ops.time_attn_decode_fwd(dshape, dmask, dq[i], dk[i], dvv[i], wd.cache_frames,
                                    wd.q_frame0, do[i], dl[i], cs):
            raise RuntimeError(ops.bca_last_error())

    def step(i=0):
        space_op(i)
        decode_op(i)

    spin = spin_up(step, args.spinup_ms)
    for i in range(args.warmup):
        step(i % RINGS)
    torch.cuda.synchronize()
    # graphs: "steps" = RINGS consecutive steps over the rotated copies; per
    # op, REPS back-to-back launches (rotated, and on one copy), so the graph
    # launch itself is amortized
    REPS = 24
    graphs = {}
    for key, fn, reps, rot in (("steps", step, RINGS, True),
                               ("space_fwd_block", space_op, REPS, True),
                               ("time_decode", decode_op, REPS, True),
                               ("time_decode_same_ring", decode_op, REPS, False)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(reps):
                fn(r % RINGS if rot else 0)
        graphs[key] = g
        for _ in range(3):
            g.replay()
    torch.cuda.synchronize()

    def timed(g, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    op_ms = {k: timed(graphs[k], max(1, args.steps // REPS)) / REPS
             for k in ("space_fwd_block", "time_decode", "time_decode_same_ring")}
    torch.cuda.synchronize()
    replays = max(1, args.steps // RINGS)
    t0 = time.perf_counter()
    for _ in range(replays):
        graphs["steps"].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    args.steps = replays * RINGS
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    ops_ = {}
    for key, fl, by in (("space_fwd_block", C.flops(ws, "fwd"), C.min_bytes(ws, "fwd")),
                        ("time_decode", C.decode_flops(wd), C.decode_min_bytes(wd)),
                        ("time_decode_same_ring", C.decode_flops(wd), C.decode_min_bytes(wd))):
        ms = op_ms[key]
        ops_[key] = {"ms": round(ms, 5), "tflops": round(fl / ms / 1e9, 2),
                     "gbps": round(by / ms / 1e6, 1),
                     "pct_hbm_peak": round(100.0 * by / ms / 1e6 / PEAK_HBM_GBPS, 2),
                     "flop": fl, "min_bytes": by}
    # the dominant op of the (rotated) step; the same-ring figure is context
    dom = max(("space_fwd_block", "time_decode"), key=lambda k: ops_[k]["ms"])
    d = ops_[dom]
    roof = roofline_of(d["flop"], d["min_bytes"], d["ms"])
    roof["kernel"] = dom + " (" + KERNELS[dom] + ", ring rotated over %d copies)" % RINGS
    # the committed counters were taken on the one-environment step
    roof["traffic"] = read_traffic(dom, TRAFFIC_FILE_DECODE) if B == 1 else None
    ms_step = elapsed / args.steps * 1e3
    out = {
        "metric": "rollout decode frames/s through one space + one time attention layer",
        "value": round(args.steps * B / elapsed, 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spinup": spin,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "timing": "HIP graph replays of %d consecutive steps, each on its own copy of the inputs "
                  "(8 rings of 43 MB per environment, more than the 256 MB MALL, as the seven "
                  "time layers of a rollout keep); per-op figures from graphs of %d back-to-back "
                  "launches rotated the same way; time_decode_same_ring re-reads one ring "
                  "(MALL-resident), context only" % (RINGS, REPS),
        "config": {
            "workload": "Minecraft rollout decode step: space attention of the new 290-token "
                        "block (30 q / 3 kv heads, d 64, agent isolation) + time attention of its "
                        "290 slots over a ring cache of the 192 frames the window reads, %d "
                        "environment(s)" % B,
            "B": B, "N": wd.N, "Hq": wd.Hq, "Hkv": wd.Hkv, "D": wd.D, "window": wd.window,
            "cache_frames": wd.cache_frames, "q_frame0": wd.q_frame0,
        },
        "ops": {k: {kk: vv for kk, vv in v.items() if kk not in ("flop", "min_bytes")}
                for k, v in ops_.items()},
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_decode(B),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_proj(w, target_s: float = 15.0):
    """The fp64 oracle's RMS norm + QKV projection and output projection +
    residual on a bounded sample of the rows (the full widths), scaled to the
    same GEMM TFLOP/s unit."""
    from block_causal_transformer_amd import configs as C, gen
    from oracle import oracle as O

    def run(n):
        ws = w.with_(M=n)
        x = gen.make_proj_inputs(ws)
        t0 = time.perf_counter()
        O.rmsnorm_qkv_fwd(x["x"], x["gain"], x["w_qkv"], ws.Hq, ws.Hkv, ws.D, ws.eps)
        O.out_proj_fwd(x["o"], x["w_o"], x["residual"])
        dt = time.perf_counter() - t0
        return dt, C.proj_flops(ws, "qkv") + C.proj_flops(ws, "out")

    dt, _ = run(512)
    n = max(512, min(w.M, int(512 * target_s / max(dt, 1e-3))))
    dt, fl = run(n)
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.max_threads(),
        "kind": "oracle",
        "sample": "%d token rows (d_model %d, %d q / %d kv heads of %d): RMS norm + QKV projection "
                  "and output projection + residual, fp64, %.1f s" % (n, w.d_model, w.Hq, w.Hkv, w.D, dt),
    }


def main_proj(args):
    import torch
    from block_causal_transformer_amd import configs as C, gen, ops

    if not os.path.exists(ops.LIB_PATH):
        from block_causal_transformer_amd import build as hip_build
        hip_build.build()
    ops.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = C.PROJ_CONFIGS["proj"]
    x = gen.make_proj_inputs(w)
    bf = torch.bfloat16
    d = {k: torch.from_numpy(v).to(dev) for k, v in x.items()}
    del x
    for k in ("x", "w_qkv", "o", "w_o", "residual"):
        d[k] = d[k].to(bf)
    shape = ops.BcaProjShape(w.M, w.d_model, w.Hq, w.Hkv, w.D)
    q = torch.empty((w.M, w.Hq * w.D), dtype=bf, device=dev)
    k = torch.empty((w.M, w.Hkv * w.D), dtype=bf, device=dev)
    v = torch.empty_like(k)
    rstd = torch.empty(w.M, dtype=torch.float32, device=dev)
    ws_bytes = ops.bca_qkv_workspace_bytes(shape)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    y = torch.empty((w.M, w.d_model), dtype=bf, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def qkv():
        if ops.rmsnorm_qkv_fwd(shape, d["x"], d["gain"], w.eps, d["w_qkv"], q, k, v, rstd, ws,
                               ws_bytes, sp):
            raise RuntimeError(ops.bca_last_error())

    def out():
        if ops.out_proj_fwd(shape, d["o"], d["w_o"], d["residual"], y, sp):
            raise RuntimeError(ops.bca_last_error())

    seq = (("qkv_proj", qkv), ("out_proj", out))

    def one_step():
        for _, fn in seq:
            fn()

    spin = spin_up(one_step, args.spinup_ms)
    for _ in range(args.warmup):
        for _, fn in seq:
            fn()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        evs[s_][0].record(stream)
        for i, (_, fn) in enumerate(seq):
            fn()
            evs[s_][i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    ops_ = {}
    total = 0.0
    for i, (name, _) in enumerate(seq):
        which = "qkv" if name == "qkv_proj" else "out"
        samples = [evs[s_][i].elapsed_time(evs[s_][i + 1]) for s_ in range(args.steps)]
        ms = sum(samples) / args.steps
        fl, by = C.proj_flops(w, which), C.proj_min_bytes(w, which)
        total += fl
        ops_[name] = {"ms": round(ms, 5), **spread(samples), "tflops": round(fl / ms / 1e9, 2),
                      "pct_mfma_peak": round(100.0 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
                      "gbps": round(by / ms / 1e6, 1), "flop": fl, "min_bytes": by}
    # the roofline is quoted on the output projection's GEMM: one launch per
    # call, so its event time is the kernel's duration (the QKV call also
    # runs the norm kernel)
    dm = ops_["out_proj"]
    roof = roofline_of(dm["flop"], dm["min_bytes"], dm["ms"])
    roof["kernel"] = "out_proj (" + KERNELS["out_proj"] + ")"
    roof["traffic"] = read_traffic("out_proj", TRAFFIC_FILE_PROJ)
    out_ = {
        "metric": "projection GEMM TFLOP/s beside the attention (QKV with RMS norm, output with "
                  "residual) and % of MI355X bf16 MFMA peak",
        "value": round(total * args.steps / elapsed / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spinup": spin,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Minecraft dynamics layer projections at 256 frames per GPU: RMS norm + QKV "
                        "projection (74,240 rows, 1920 -> 1920 + 2 x 192) and output projection "
                        "(1920 -> 1920) + residual",
            "M": w.M, "d_model": w.d_model, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "eps": w.eps,
            "flop_per_step": total,
        },
        "pct_mfma_peak": round(100.0 * total * args.steps / elapsed / 1e12 / PEAK_BF16_TFLOPS, 2),
        "ops": {k_: {kk: vv for kk, vv in v_.items() if kk not in ("flop", "min_bytes")}
                for k_, v_ in ops_.items()},
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_proj(w),
    }
    print(json.dumps(out_), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 200, enough to time the GPU at its steady clock)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 100; the clock ramps up over the first "
                         "few tens of milliseconds of work)")
    ap.add_argument("--spinup-ms", type=float, default=300.0,
                    help="untimed steps for at least this long before the warm-up steps, so that "
                         "the timed steps run at the GPU's steady clock (reported as spinup)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--workload", choices=("train_step", "tokenizer_step", "long_time", "rollout_decode",
                                           "projections"),
                    default="train_step")
    ap.add_argument("--decode-batch", type=int, default=1,
                    help="rollout_decode: environments generated at once")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(space attention shards by block and time attention by slot, with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.steps is None:
        args.steps = 200
    if args.warmup is None:
        args.warmup = 100
    if args.workload == "rollout_decode":
        return main_decode(args)
    if args.workload == "projections":
        return main_proj(args)

    return main_step(args)


def step_workloads(name):
    """(workloads, description, metric) of a fwd+bwd step workload."""
    from block_causal_transformer_amd import configs as C
    if name == "train_step":
        return ([C.get("3"), C.get("4")],
                "Minecraft dynamics attention step: space layer fwd+bwd (B=4 x T=64 blocks of 290 "
                "tokens, 30 q / 3 kv heads, d 64, agent isolation) + time layer fwd+bwd (T=256 "
                "frames x 290 slots, causal, window 192)",
                "block-causal attention TFLOP/s (fwd, fwd+bwd) and % of MI355X bf16 MFMA peak")
    if name == "tokenizer_step":
        return ([C.get("5a"), C.get("5d"), C.get("5b"), C.get("5c")],
                "Tokenizer attention step: encoder space layer (16 frames of 1432 tokens, 24 heads "
                "MHA, dense) + encoder time layer (1432 slots x 16 frames, 24 heads, causal, window "
                "16) + decoder space layer (16 heads) + decoder time layer (16 heads), each fwd+bwd",
                "tokenizer attention TFLOP/s (fwd+bwd) and % of MI355X bf16 MFMA peak")
    if name == "long_time":
        return ([C.get("4").with_(name="4L", T=1024, seed=4100)],
                "Long-sequence time layer fwd+bwd: T=1024 frames x 290 slots, 30 q / 3 kv heads, "
                "d 64, causal, window 192",
                "long-sequence time attention TFLOP/s (fwd+bwd) and % of MI355X bf16 MFMA peak")
    raise ValueError(name)


def main_step(args):
    import torch
    from block_causal_transformer_amd import configs as C, gen, ops

    if not os.path.exists(ops.LIB_PATH):
        from block_causal_transformer_amd import build as hip_build
        hip_build.build()
    ops.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wls, desc, metric = step_workloads(args.workload)
    bufs = {}
    for w in wls:
        x = gen.make_inputs(w)
        b = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in x.items()}
        del x
        b["o"] = torch.empty_like(b["q"])
        b["lse"] = torch.empty(w.lse_shape(), dtype=torch.float32, device=dev)
        b["dq"] = torch.empty_like(b["q"])
        b["dk"] = torch.empty_like(b["k"])
        b["dv"] = torch.empty_like(b["v"])
        b["shape"] = ops.make_shape(b["q"], b["k"])
        b["mask"] = ops.make_mask(w.op, **ops.workload_kwargs(w))
        need = ops.bca_bwd_workspace_bytes(ops.BCA_OP_SPACE if w.op == "space" else ops.BCA_OP_TIME,
                                           b["shape"])
        b["ws"] = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if need else None
        b["ws_bytes"] = need
        b["w"] = w
        bufs[w.name] = b
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def call(name, direction):
        b = bufs[name]
        w = b["w"]
        if direction == "fwd":
            f = ops.space_attn_fwd if w.op == "space" else ops.time_attn_fwd
            rc = f(b["shape"], b["mask"], b["q"], b["k"], b["v"], b["o"], b["lse"], sp)
        else:
            f = ops.space_attn_bwd if w.op == "space" else ops.time_attn_bwd
            rc = f(b["shape"], b["mask"], b["q"], b["k"], b["v"], b["o"], b["lse"], b["dout"],
                   b["dq"], b["dk"], b["dv"], b["ws"], b["ws_bytes"], sp)
        if rc != 0:
            raise RuntimeError("%s %s: %s" % (name, direction, ops.bca_last_error()))

    # Every layer's forward, then every backward in the same layer order: an
    # op's forward and backward are then separated by the other layers' ops,
    # which move far more than the 256 MB MALL, so no backward re-reads its
    # inputs (or the O its forward just wrote) from that cache; the next
    # step's forwards come after every other layer's backward.
    seq = [(w.name, "fwd") for w in wls] + [(w.name, "bwd") for w in wls]
    if args.workload == "train_step":
        labels = {("3", "fwd"): "space_fwd", ("3", "bwd"): "space_bwd",
                  ("4", "fwd"): "time_fwd", ("4", "bwd"): "time_bwd"}
    else:
        labels = {(n, d): "%s_%s_%s" % (n, bufs[n]["w"].op, d) for n, d in seq}

    def one_step():
        for name, d in seq:
            call(name, d)

    spin = spin_up(one_step, args.spinup_ms)
    for _ in range(args.warmup):
        for name, d in seq:
            call(name, d)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        evs[s_][0].record(stream)
        for i, (name, d) in enumerate(seq):
            call(name, d)
            evs[s_][i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    per_op = {}
    total_flops = 0.0
    for i, key in enumerate(seq):
        w = bufs[key[0]]["w"]
        samples = [evs[s_][i].elapsed_time(evs[s_][i + 1]) for s_ in range(args.steps)]
        ms = sum(samples) / args.steps
        fl = C.flops(w, key[1])
        by = C.min_bytes(w, key[1])
        total_flops += fl
        per_op[labels[key]] = {
            "ms": round(ms, 5),
            **spread(samples),
            "tflops": round(fl / ms / 1e9, 2),
            "pct_mfma_peak": round(100.0 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
            "gbps": round(by / ms / 1e6, 1),
            "pct_hbm_peak": round(100.0 * by / ms / 1e6 / PEAK_HBM_GBPS, 2),
            "flop": fl,
            "min_bytes": by,
            "op": "%s_%s" % (w.op, key[1]),
        }
    ms_step = elapsed / args.steps * 1e3
    value = total_flops * args.steps / elapsed / 1e12

    # dominant kernel: the op with the largest time share
    dom = max(per_op, key=lambda k: per_op[k]["ms"])
    d = per_op[dom]
    roof = roofline_of(d["flop"], d["min_bytes"], d["ms"])
    roof["kernel"] = dom + " (" + KERNELS[d["op"]] + ")"
    roof["traffic"] = (read_traffic(dom) if args.workload == "train_step" else
                       read_traffic(d["op"], TRAFFIC_FILE_LONG) if args.workload == "long_time" else None)
    if args.workload == "train_step":
        # rocprofv3 counters of the same kernels (MFMA busy share of the
        # SIMDs' cycles), from the committed summary when it matches the sources
        roof["counters"] = read_util(dom)

    cfg = {"workload": desc}
    for w in wls:
        cfg[w.name] = {"op": w.op, "B": w.B, "T": w.T, "N": w.N, "Hq": w.Hq, "Hkv": w.Hkv,
                       "D": w.D, "window": w.window, "agent_begin": w.agent_begin,
                       "agent_count": w.agent_count}
    cfg["flop_per_step"] = total_flops
    if args.workload == "train_step":
        cfg = {"workload": desc,
               "space": {k: v for k, v in cfg["3"].items() if k not in ("op", "window")},
               "time": {k: v for k, v in cfg["4"].items()
                        if k not in ("op", "agent_begin", "agent_count")},
               "flop_per_step": total_flops}
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spinup": spin,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": cfg,
        "order": [labels[k] for k in seq],
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "ops": {k: {kk: vv for kk, vv in v.items() if kk not in ("flop", "min_bytes", "op")}
                for k, v in per_op.items()},
        "roofline": roof,
    }
    if args.workload == "train_step":
        out["fwd_tflops"] = round((per_op["space_fwd"]["flop"] + per_op["time_fwd"]["flop"])
                                  / (per_op["space_fwd"]["ms"] + per_op["time_fwd"]["ms"]) / 1e9, 2)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline() if args.workload == "train_step" else cpu_baseline_ops(wls)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def cpu_baseline_ops(wls, target_s: float = 15.0):
    """The fp64 oracle on a bounded sample of each workload of the step (a few
    whole units of each, fwd + bwd), scaled to the same TFLOP/s unit."""
    from block_causal_transformer_amd import configs as C, gen
    from oracle import oracle as O

    def sample(w, n):
        return w.with_(B=1, T=n) if w.op == "space" else w.with_(B=1, N=n)

    def run(n):
        t0 = time.perf_counter()
        fl = 0.0
        for w in wls:
            ws_ = sample(w, n)
            x = gen.make_inputs(ws_)
            O.fwd(ws_, x["q"], x["k"], x["v"])
            O.bwd(ws_, x["q"], x["k"], x["v"], x["dout"])
            fl += C.flops(ws_, "fwd") + C.flops(ws_, "bwd")
        return time.perf_counter() - t0, fl

    dt, _ = run(1)
    n = max(1, min(64, int(target_s / max(dt, 1e-3))))
    dt, fl = run(n)
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.max_threads(),
        "kind": "oracle",
        "sample": "%d unit(s) (blocks / slots) of each of %s, forward + backward, fp64, %.1f s"
                  % (n, ", ".join(w.name for w in wls), dt),
    }


if __name__ == "__main__":
    main()
