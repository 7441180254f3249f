"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code.

* the CPU oracle (oracle/trellis_oracle.c) driven through every entry point
  by tests/sanitize/oracle_driver.c, built with gcc;
* the library's host side (validation, planning, workspace bookkeeping)
  driven through every C-ABI entry point by tests/sanitize/abi_driver.cpp,
  built with hipcc with the sanitizers on the host compilation only (device
  code is compiled as usual and never runs here: with no GPU present the
  in-domain calls must return TRELLIS_E_HIP).

Both run on the CPU; a sanitizer report makes the driver exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
         os.path.join(ROOT, "oracle", "trellis_oracle.c"), "-lm"])
    r = run([exe], env=SAN_ENV)
    assert "oracle driver ok" in r.stdout


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="checks the no-GPU error path; a GPU is present")
def test_library_host_side_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    env = dict(os.environ)
    env.pop("HIP_VISIBLE_DEVICES", None)
    run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined",
         "-I", os.path.join(ROOT, "include"), "-o", exe, os.path.join(HERE, "abi_driver.cpp"),
         os.path.join(ROOT, "trellis_coded_bit_prefill_amd", "csrc", "trellis.hip")], env=env)
    san = dict(SAN_ENV, HIP_VISIBLE_DEVICES="")  # no device even where one exists
    r = run([exe], env=san)
    assert "abi driver ok" in r.stdout
