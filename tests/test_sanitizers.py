"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer builds (no GPU):

* the C ABI shim (validation, dispatch, error reporting) with the kernel
  launchers and its three HIP runtime calls replaced by recording stubs,
  driven through every entry point with valid, invalid and extreme sizes
  (tests/sanitize/abi_driver.cpp);
* the fp64 oracle, driven on small ragged shapes with closed-form checks
  (tests/sanitize/oracle_driver.c).

Both are built with g++/gcc (host code only, nothing for the GPU) with
-fsanitize=address,undefined and no recovery, so any out-of-bounds access,
leak or signed overflow fails the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-Wall"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env.pop("BCA_SYNC", None)
    env.pop("BCA_DEBUG_LDS_POISON", None)
    return env


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_abi_shim_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    _run(["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + os.path.join(ROOT, "include"),
          "-I" + os.path.join(ROOT, "block_causal_transformer_amd", "csrc"), "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
          os.path.join(ROOT, "block_causal_transformer_amd", "csrc", "bca_abi.cpp")], str(tmp_path))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=_env())
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-Wno-unknown-pragmas"] + SAN + ["-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "attn_oracle.c"), "-lm"], str(tmp_path))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=_env())
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
