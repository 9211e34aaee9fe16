"""The CPU oracle and libqb's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; no GPU code is built with them).

  * oracle/oracle.c with tests/sanitize/oracle_driver.c, which calls every
    oracle function on small ragged inputs (every code, dtype, block size and
    optimizer kind; quantile estimation with ragged chunks);
  * bit_optimizer_states_amd/csrc/qb_tables.cpp and qb_api.cpp (the exact
    table builder, and every entry point's argument checks and host
    arithmetic) with tests/sanitize/host_driver.cpp, linked against
    tests/sanitize/host_stubs.cpp in place of the HIP sources: every call
    must stop at a check or before any device work.
Both build with gcc/g++ -fsanitize=address,undefined -fno-sanitize-recover=all,
so any report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_address_and_undefined_behavior_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", *SAN, "-ffp-contract=off", os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe])
    out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "all calls returned 0" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="g++ or the ROCm headers not found")
def test_library_host_code_under_address_and_undefined_behavior_sanitizers(tmp_path):
    exe = str(tmp_path / "host_san")
    csrc = os.path.join(ROOT, "bit_optimizer_states_amd", "csrc")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include",
          f"-I{csrc}", os.path.join(csrc, "qb_tables.cpp"), os.path.join(csrc, "qb_api.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
          f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib", "-lamdhip64", "-o", exe], timeout=600)
    out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "every call returned the expected status" in out
