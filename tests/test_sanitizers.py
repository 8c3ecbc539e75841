"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

- The oracle (plain C) is built with both sanitizers and driven through every
  entry point on exactly sized buffers (tests/sanitize/oracle_driver.c).
- The C-ABI host layer (dsaidx_api.cpp) is built with g++ and both sanitizers
  against stub kernel launchers that record each launch: launch shapes, the
  argument checks (each rejection enqueues nothing), the status mapping of
  launch errors and the top-k workspace rules (tests/sanitize/host_driver.cpp).
Neither build involves GPU code."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ROCM_INCLUDE = "/opt/rocm/include"


def _sanitizers_work(tmp_path, cc):
    src = tmp_path / "probe.c"
    src.write_text("int main(void) { return 0; }\n")
    r = subprocess.run([cc] + SAN + [str(src), "-o", str(tmp_path / "probe")],
                       capture_output=True, text=True)
    return r.returncode == 0


def _run(exe, tmp_path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env, cwd=tmp_path)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc") or not _sanitizers_work(tmp_path, "gcc"):
        pytest.skip("gcc with AddressSanitizer is not available")
    exe = tmp_path / "oracle_driver"
    cmd = (["gcc", "-std=c99", "-ffp-contract=off", "-fopenmp"] + SAN +
           ["-I" + os.path.join(ROOT, "oracle"),
            os.path.join(ROOT, "oracle", "dsaidx_oracle.c"),
            os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", str(exe)])
    subprocess.run(cmd, check=True)
    _run(exe, tmp_path)


def test_host_layer_under_sanitizers(tmp_path):
    if not shutil.which("g++") or not _sanitizers_work(tmp_path, "g++"):
        pytest.skip("g++ with AddressSanitizer is not available")
    if not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("HIP headers are not available")
    exe = tmp_path / "host_driver"
    csrc = os.path.join(ROOT, "rope_fp8_quant_amd", "csrc")
    cmd = (["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__"] + SAN +
           ["-I" + ROCM_INCLUDE, "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
            os.path.join(csrc, "dsaidx_api.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", str(exe)])
    subprocess.run(cmd, check=True)
    _run(exe, tmp_path)
