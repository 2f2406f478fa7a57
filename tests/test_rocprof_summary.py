"""The rocprofv3 summary helpers (host logic, no GPU): kernels map to ops,
and an op with a second, shorter kernel keeps its main kernel's figures."""
import argparse
import csv

from block_causal_transformer_amd import rocprof_summary as R


def test_kernels_map_to_ops():
    k = "void bca::(anonymous namespace)::attn_bwd_split_reduce_kernel<1>(bca::(anonymous namespace)::BwdParams, int)"
    assert R.op_of(k) == "time_bwd"
    assert R.op_of("attn_bwd_dkv_kernel<1, 1, true>(bca::BwdParams)") == "time_bwd"
    assert R.op_of("attn_bwd_split_reduce_kernel<0>(bca::BwdParams, int)") == "space_bwd"
    assert R.op_of("attn_fwd_kernel<1>(bca::FwdParams)") == "time_fwd"
    assert R.op_of("void bca::(anonymous namespace)::short_bwd_kernel<1, 16, 16>"
                   "(bca::(anonymous namespace)::ShortParams)") == "time_bwd"
    assert R.op_of("short_fwd_kernel<1, 16, 16>(bca::ShortParams)") == "time_fwd"
    assert R.op_of("short_fwd_kernel<0, 16, 16>(bca::ShortParams)") == "space_fwd"


def test_util_keeps_the_longest_kernel_of_an_op(tmp_path):
    path = tmp_path / "counters.csv"
    kernels = {"attn_bwd_dkv_kernel<1, 1, true>(bca::BwdParams)": 8.0e5,
               "attn_bwd_split_reduce_kernel<1>(bca::BwdParams, int)": 8.0e3}
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, clocks in kernels.items():
            for c in R.UTIL_COUNTERS:
                v = clocks * 8 if c == "GRBM_GUI_ACTIVE" else (clocks * 1024 * 0.2 if c == "SQ_VALU_MFMA_BUSY_CYCLES" else 1000.0)
                w.writerow({"Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})
    out = tmp_path / "util.txt"
    R.cmd_util(argparse.Namespace(csv=[str(path)], cmd="test", sources="attn_bwd.hip", out=str(out)))
    lines = dict(l.split("  #")[0].split("=", 1) for l in out.read_text().splitlines() if "=" in l and not l.startswith("#"))
    assert abs(float(lines["time_bwd.clocks"]) - 8.0e5) < 1
    assert abs(float(lines["time_bwd/attn_bwd_split_reduce_kernel.clocks"]) - 8.0e3) < 1
    assert abs(float(lines["time_bwd.mfma_busy_pct"]) - 20.0) < 1e-6


def test_stats_compares_shared_kernels_with_the_mean_of_their_configs(tmp_path):
    """Two configs on the same kernel: the trace's average is compared with
    the mean of the two configs' event times."""
    import json
    stats = tmp_path / "stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": "void bca::(anonymous namespace)::attn_fwd_kernel<0>(bca::(anonymous namespace)::FwdParams)",
                    "Calls": 4, "TotalDurationNs": 800000, "AverageNs": 200000, "Percentage": 100.0})
    log = tmp_path / "bench.log"
    log.write_text("noise\n" + json.dumps({"ms_per_step": 1.0, "ops": {"5a_space_fwd": {"ms": 0.25},
                                                                          "5b_space_fwd": {"ms": 0.15}}}) + "\n")
    out = tmp_path / "stats.md"
    R.cmd_stats(argparse.Namespace(csv=str(stats), out=str(out), cmd="test", bench_log=str(log)))
    text = out.read_text()
    assert "| space_fwd | 5a_space_fwd, 5b_space_fwd | 200.0 | 200.0 |" in text
    assert "| 5a_space_fwd | 250.0 | 200.0 |" in text
