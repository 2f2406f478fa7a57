"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

    python -m block_causal_transformer_amd.rocprof_summary stats \\
        KERNEL_STATS_CSV OUT_MD --cmd "the profiled command" [--bench-log LOG]
    python -m block_causal_transformer_amd.rocprof_summary traffic \\
        FETCH_COUNTER_CSV WRITE_COUNTER_CSV OUT_TXT --cmd "..." --sources a.hip,b.h

``stats`` lists every kernel of a ``--kernel-trace --stats`` run (calls,
average and total duration).  ``traffic`` reads two ``--pmc FETCH_SIZE`` /
``--pmc WRITE_SIZE`` runs of ``bench.py --copy-probe-mib M`` and writes HBM
bytes per launch of each op, each counter scaled by the factor
that makes it read the known byte count of the plain device copy of M MiB
that the same run performs; ``bench.py`` reads that file for the roofline's
``traffic`` field (and ignores it once one of the ``--sources`` files the
kernels are built from changes).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_causal_transformer_amd", "csrc")

# op of each kernel (attention: template argument 0 = space, 1 = time, 2 =
# decode; projections: 0 = QKV split, 1 = output + residual)
OPS = [
    (r"attn_fwd_kernel<2>", "time_decode"),
    (r"attn_fwd_kernel<0>", "space_fwd"),
    (r"attn_fwd_kernel<1>", "time_fwd"),
    (r"attn_bwd_dq_kernel<0[,>]", "space_bwd"),
    (r"attn_bwd_dkv_kernel<0[,>]", "space_bwd"),
    (r"attn_bwd_dq_kernel<1[,>]", "time_bwd"),
    (r"attn_bwd_dkv_kernel<1[,>]", "time_bwd"),
    (r"attn_bwd_split_reduce_kernel<0>", "space_bwd"),
    (r"attn_bwd_split_reduce_kernel<1>", "time_bwd"),
    (r"attn_bwd_seg_reduce_kernel", "time_bwd"),
    # one wave per short problem (template argument 0 = space, 1 = time)
    (r"short_fwd_kernel<0[,>]", "space_fwd"),
    (r"short_fwd_kernel<1[,>]", "time_fwd"),
    (r"short_bwd_kernel<0[,>]", "space_bwd"),
    (r"short_bwd_kernel<1[,>]", "time_bwd"),
    (r"rstd_rows_kernel", "qkv_proj"),
    (r"fold_gain_kernel", "qkv_proj"),
    (r"gemm256_kernel<0[,>]", "qkv_proj"),
    (r"gemm_nt_kernel<0>", "qkv_proj"),
    (r"gemm256_kernel<1[,>]", "out_proj"),
    (r"gemm_nt_kernel<1>", "out_proj"),
]
OP_ORDER = ("space_fwd", "space_bwd", "time_fwd", "time_bwd", "time_decode", "qkv_proj", "out_proj")


def strip_comments(src: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed, so
    that editing a comment does not change the digest (string and character
    literals are kept as they are)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest(files=None) -> str:
    """Digest of the kernel sources ``files`` (names in csrc/; all by default),
    comments and layout ignored."""
    h = hashlib.sha256()
    for name in sorted(files or os.listdir(CSRC)):
        path = os.path.join(CSRC, name)
        if not os.path.exists(path):
            return ""
        with open(path, encoding="utf-8") as f:
            h.update(name.encode())
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    k = kernel.replace("void ", "").replace("bca::(anonymous namespace)::", "")
    k = k.split("(bca::")[0]
    if len(k) > 90:
        k = k[:87] + "..."
    return k


def op_of(kernel: str):
    k = short_name(kernel)
    for pat, op in OPS:
        if re.match(pat, k):
            return op
    return None


def cmd_stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["# rocprofv3 kernel statistics", "",
           "Command (run from the repository root on one MI355X):", "",
           "    " + args.cmd, "",
           "| kernel | op | calls | average (us) | total (us) | share |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| `%s` | %s | %s | %.1f | %.1f | %.1f%% |" % (
            short_name(r["Name"]), op_of(r["Name"]) or "-", r["Calls"],
            float(r["AverageNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e3, float(r["Percentage"])))
    per_op = collections.defaultdict(float)
    for r in rows:
        op = op_of(r["Name"])
        if op:
            per_op[op] += float(r["AverageNs"]) / 1e3
    out += ["", "Average duration per op (sum over its kernels):", "",
            "| op | average (us) |", "|---|---|"]
    for op in OP_ORDER:
        if op in per_op:
            out.append("| %s | %.1f |" % (op, per_op[op]))
    if args.bench_log:
        # the bench's own HIP-event timing of each op in the same profiled run
        line = next((l for l in open(args.bench_log) if l.startswith("{")), None)
        if line:
            d = json.loads(line)
            out += ["", "`bench.py`'s HIP-event average per op in the same (profiled) run, "
                    "ms_per_step %.4f:" % d["ms_per_step"], "",
                    "| op | events (us) | kernel trace (us) |", "|---|---|---|"]
            bases = {}
            for op, v in d.get("ops", {}).items():
                # a workload's op names may carry its config as a prefix
                # ("4L_time_bwd"); the kernels' op is the rest
                base = {"space_fwd_block": "space_fwd"}.get(op, op)
                if base not in per_op and "_" in base and base.split("_", 1)[1] in per_op:
                    base = base.split("_", 1)[1]
                bases.setdefault(base, []).append((op, 1e3 * v["ms"]))
                kt = per_op.get(base)
                out.append("| %s | %.1f | %s |" % (op, 1e3 * v["ms"], "%.1f" % kt if kt else "-"))
            shared = {b: ev for b, ev in bases.items() if len(ev) > 1 and b in per_op}
            if shared:
                # several configs run the same kernels: the trace averages
                # over all their calls, so compare with the events' mean
                out += ["", "Ops whose kernels serve several configs (the kernel trace averages "
                        "over all their calls; the events' mean over those configs beside it):", "",
                        "| op | configs | events, mean (us) | kernel trace (us) |", "|---|---|---|---|"]
                for b, ev in shared.items():
                    out.append("| %s | %s | %.1f | %.1f |" % (
                        b, ", ".join(o for o, _ in ev), sum(t for _, t in ev) / len(ev), per_op[b]))
    out.append("")
    with open(args.out, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


def _counter(path, name):
    """(kernel name, value) per dispatch for counter ``name``."""
    res = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == name:
            res.append((r["Kernel_Name"], float(r["Counter_Value"]), int(r["Dispatch_Id"])))
    return res


def cmd_traffic(args):
    probe = args.copy_mib * (1 << 20)
    vals = {}
    for path, cname in ((args.fetch_csv, "FETCH_SIZE"), (args.write_csv, "WRITE_SIZE")):
        rows = _counter(path, cname)
        copies = [v for (k, v, _) in rows if "copy" in k.lower()]
        if not copies:
            sys.exit("no copy kernel found in %s" % path)
        # the probe is the largest plain copy of the run
        copy_kib = max(copies)
        factor = probe / (copy_kib * 1024.0)
        per_op = collections.defaultdict(list)
        per_disp = collections.defaultdict(float)
        for k, v, d in rows:
            op = op_of(k)
            if op:
                per_disp[(op, d)] += v
        # one launch of an op = its kernels' dispatches; average over launches
        for (op, d), v in per_disp.items():
            per_op[(op, short_name([k for k, _, dd in rows if dd == d][0]))].append(v)
        vals[cname] = (copy_kib, factor, per_op)
    out = ["# HBM traffic per launch, from rocprofv3 counters", "#",
           "# commands (from the repository root, one MI355X):",
           "#   " + args.cmd.replace("COUNTER", "FETCH_SIZE"),
           "#   " + args.cmd.replace("COUNTER", "WRITE_SIZE"),
           "# Each counter (KiB per dispatch) is scaled by the factor that makes it",
           "# read %d bytes for the plain %d MiB device copy in the same run." % (probe, args.copy_mib),
           "source_files=%s" % ",".join(sorted(args.sources.split(","))),
           "source_sha=%s" % source_digest(args.sources.split(",")),
           "copy_probe_bytes=%d" % probe]
    for cname, (ck, fac, _) in vals.items():
        out.append("%s.copy_kib=%.1f" % (cname.lower(), ck))
        out.append("%s.factor=%.4f" % (cname.lower(), fac))
    ops = collections.defaultdict(float)
    for cname, (_, fac, per_op) in vals.items():
        for (op, kname), vs in sorted(per_op.items()):
            avg = sum(vs) / len(vs)
            out.append("%s.%s.kib_per_dispatch=%.1f  # %s" % (op, cname.lower(), avg, kname))
            ops[op] += avg * 1024.0 * fac
    for op in OP_ORDER:
        if op in ops:
            out.append("%s.bytes=%.0f" % (op, ops[op]))
    out.append("")
    with open(args.out, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


# Counters of the utilisation summary and how each figure is formed (per
# dispatch, averaged over the dispatches of a kernel).  GRBM_GUI_ACTIVE is
# the dispatch's duration in GPU clocks; the SQ counters are summed over the
# 1024 SIMDs (MFMA busy, co-execution) or taken in quad-cycles over the 256
# CUs (VALU busy), as AMD's derived MfmaUtil, VALUBusy and LDSBankConflict
# define them.
UTIL_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU",
                 "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_LDS_BANK_CONFLICT",
                 "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE")
SIMDS, CUS, XCDS = 1024, 256, 8


def util_figures(c):
    """Utilisation figures from the per-dispatch averages ``c`` of UTIL_COUNTERS."""
    # GRBM_GUI_ACTIVE is reported per XCD and summed over the 8: one XCD's
    # count is the dispatch's duration in clocks
    gui = c["GRBM_GUI_ACTIVE"] / XCDS
    return {
        "mfma_busy_pct": 100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMDS),
        "coexec_pct": 100.0 * c["SQ_VALU_MFMA_COEXEC_CYCLES"] / (gui * SIMDS),
        "valu_busy_pct": 100.0 * c["SQ_ACTIVE_INST_VALU"] * 4 / (gui * SIMDS),
        "lds_bank_conflict_pct": 100.0 * c["SQ_LDS_BANK_CONFLICT"] / (gui * CUS),
        "lds_active_pct": 100.0 * c["SQ_LDS_IDX_ACTIVE"] / (gui * CUS),
        "valu_per_mfma": c["SQ_INSTS_VALU"] / max(c["SQ_INSTS_MFMA"], 1.0),
        "clocks": gui,
    }


def cmd_util(args):
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    names = {}
    for path in args.csv:
        for r in csv.DictReader(open(path)):
            k = short_name(r["Kernel_Name"])
            if r["Counter_Name"] in UTIL_COUNTERS:
                per[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
                names[k] = op_of(r["Kernel_Name"])
    out = ["# MFMA / VALU / LDS utilisation per kernel, from rocprofv3 counters", "#",
           "# command (from the repository root, one MI355X; one counter pass):",
           "#   " + args.cmd,
           "# figures per dispatch, averaged over the kernel's dispatches:",
           "#   mfma_busy_pct  = SQ_VALU_MFMA_BUSY_CYCLES / (clocks * 1024 SIMDs)",
           "#   coexec_pct     = SQ_VALU_MFMA_COEXEC_CYCLES / (clocks * 1024): MFMA busy while a VALU op issues",
           "#   valu_busy_pct  = 4 * SQ_ACTIVE_INST_VALU / (clocks * 1024)",
           "#   lds_*_pct      = SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE / (clocks * 256)",
           "#   valu_per_mfma  = SQ_INSTS_VALU / SQ_INSTS_MFMA",
           "#   clocks         = GRBM_GUI_ACTIVE / 8 XCDs (the dispatch's duration in GPU clocks)",
           "source_files=%s" % ",".join(sorted(args.sources.split(","))),
           "source_sha=%s" % source_digest(args.sources.split(","))]
    # an op with several kernels (the split backward's reduce) is keyed by
    # its longest kernel; the others by op/kernel
    clocks = {k: sum(per[k]["GRBM_GUI_ACTIVE"]) / max(len(per[k]["GRBM_GUI_ACTIVE"]), 1) for k in per}
    main_of = {}
    for k in per:
        op = names[k]
        if op and (op not in main_of or clocks[k] > clocks[main_of[op]]):
            main_of[op] = k
    for k in sorted(per, key=lambda k: (OP_ORDER.index(names[k]) if names[k] in OP_ORDER else 99, k)):
        c = {n: sum(v) / len(v) for n, v in per[k].items()}
        if not all(n in c for n in UTIL_COUNTERS):
            continue
        f = util_figures(c)
        op = names[k] or "-"
        if names[k] and main_of.get(names[k]) != k:
            op = "%s/%s" % (op, k.split("<")[0])
        for key, val in f.items():
            out.append("%s.%s=%.4g  # %s" % (op, key, val, k) if key == "mfma_busy_pct" else
                       "%s.%s=%.4g" % (op, key, val))
    out.append("")
    with open(args.out, "w") as fo:
        fo.write("\n".join(out))
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("out")
    a.add_argument("--cmd", required=True)
    a.add_argument("--bench-log", default=None,
                   help="stdout of the profiled bench.py run: its JSON line's per-op event "
                        "timings are listed beside the kernel trace")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("out")
    b.add_argument("--cmd", required=True)
    b.add_argument("--copy-mib", type=int, default=2048)
    b.add_argument("--sources", required=True,
                   help="comma-separated csrc/ files the profiled kernels are built from; the "
                        "summary is taken as stale once any of them changes")
    c = sub.add_parser("util")
    c.add_argument("out")
    c.add_argument("csv", nargs="+")
    c.add_argument("--cmd", required=True)
    c.add_argument("--sources", required=True)
    args = ap.parse_args(argv)
    if args.what == "stats":
        cmd_stats(args)
    elif args.what == "util":
        cmd_util(args)
    else:
        cmd_traffic(args)


if __name__ == "__main__":
    main()
