"""bench.py host logic that needs no GPU: the one-GPU guard, the roofline
figures and the reading of committed counter summaries."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_roofline_bound_follows_the_ridge():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBPS * 1e9)  # FLOP per byte
    # above the ridge: MFMA-bound, achieved in TFLOP/s
    r = bench.roofline_of(2e12, 2e12 / (2 * ridge), 2.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1000.0) and r["frac"] == pytest.approx(0.4)
    # below: HBM-bound, achieved in GB/s
    r = bench.roofline_of(1e9, 1e9, 0.5)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(2000.0) and r["frac"] == pytest.approx(0.25)


def test_traffic_summary_is_used_only_for_the_sources_it_was_taken_on(tmp_path):
    files = ["gemm.hip", "bca_device.h"]
    good = tmp_path / "good.txt"
    good.write_text("# comment\nsource_files=%s\nsource_sha=%s\nout_proj.bytes=12345\n"
                    % (",".join(files), bench.source_digest(files)))
    assert bench.read_traffic("out_proj", str(good)) == 12345.0
    assert bench.read_traffic("qkv_proj", str(good)) is None
    stale = tmp_path / "stale.txt"
    stale.write_text("source_files=%s\nsource_sha=0000\nout_proj.bytes=1\n" % ",".join(files))
    assert bench.read_traffic("out_proj", str(stale)) is None
    assert bench.read_traffic("out_proj", str(tmp_path / "missing.txt")) is None
    # a file that names a source that no longer exists is stale
    gone = tmp_path / "gone.txt"
    gone.write_text("source_files=no_such.hip\nsource_sha=%s\nout_proj.bytes=1\n" % bench.source_digest(files))
    assert bench.read_traffic("out_proj", str(gone)) is None


def test_source_digest_ignores_comments(tmp_path, monkeypatch):
    # the counter summaries stay valid across comment edits, not code edits
    from block_causal_transformer_amd import rocprof_summary as R
    src = 'int f(int x) { return x / 2; } // half\n/* note */ const char* s = "//";\n'
    assert R.strip_comments(src) == 'int f(int x) { return x / 2; } const char* s = "//";'
    monkeypatch.setattr(R, "CSRC", str(tmp_path))
    (tmp_path / "k.hip").write_text(src)
    d0 = R.source_digest(["k.hip"])
    (tmp_path / "k.hip").write_text(src.replace("// half", "// one half").replace("note", "other"))
    assert R.source_digest(["k.hip"]) == d0
    (tmp_path / "k.hip").write_text(src.replace("x / 2", "x / 3"))
    assert R.source_digest(["k.hip"]) != d0


def test_spread_of_step_times():
    s = bench.spread([1.0] * 8 + [2.0, 9.0])
    assert s["ms_median"] == 1.0 and s["ms_p10"] == 1.0 and s["ms_p90"] == pytest.approx(2.7)


def test_profile_summary_maps_kernel_instances_to_ops():
    from block_causal_transformer_amd import rocprof_summary as R
    cases = {
        "void bca::(anonymous namespace)::attn_bwd_dkv_kernel<0, 3, true>(bca::(anonymous namespace)::BwdParams)": "space_bwd",
        "void bca::(anonymous namespace)::attn_bwd_dkv_kernel<1, 2, false>(bca::(anonymous namespace)::BwdParams)": "time_bwd",
        "void bca::(anonymous namespace)::attn_bwd_dq_kernel<1>(bca::(anonymous namespace)::BwdParams)": "time_bwd",
        "void bca::(anonymous namespace)::attn_fwd_kernel<2>(bca::(anonymous namespace)::FwdParams)": "time_decode",
        "void bca::(anonymous namespace)::gemm256_kernel<1, 6>(bca::(anonymous namespace)::GemmParams)": "out_proj",
        "void bca::(anonymous namespace)::gemm256_kernel<0, 8>(bca::(anonymous namespace)::GemmParams)": "qkv_proj",
        "void at::native::vectorized_elementwise_kernel<4, float>(int)": None,
    }
    for name, op in cases.items():
        assert R.op_of(name) == op, name


def test_committed_counter_summaries_match_the_kernel_sources():
    """The rocprofv3 summaries under profiles/ were taken on the kernels as
    they are: every figure the bench attaches to its roofline (HBM bytes of
    the step's ops, of the decode and of the projections; the MFMA
    utilisation of the step's kernels) is read, none is dropped as stale."""
    for op in ("space_fwd", "space_bwd", "time_fwd", "time_bwd"):
        assert bench.read_traffic(op) is not None, op
        assert bench.read_util(op) is not None, op
    assert bench.read_traffic("time_decode", bench.TRAFFIC_FILE_DECODE) is not None
    assert bench.read_traffic("out_proj", bench.TRAFFIC_FILE_PROJ) is not None
    assert bench.read_traffic("time_bwd", bench.TRAFFIC_FILE_LONG) is not None
