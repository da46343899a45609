"""Sanitizer builds of the CPU-side code (no GPU): the fp64 oracle's C source and
the C ABI's host code, each compiled with AddressSanitizer and
UndefinedBehaviorSanitizer into a driver under tests/sanitize/ and run.

* oracle_driver.c runs every oracle entry point on ragged packed sequences (empty,
  one-token, sub-chunk-crossing lengths) with each flag, plus the beta = 0 closed
  form, under gcc's sanitizers.
* abi_driver.cpp runs every C entry point's argument checks (bad arguments must
  fail with their status; good ones must reach a stub launcher that records the
  call) and the prefill's workspace and window planning, with kda_api.hip's host
  code built by hipcc with the sanitizers on the host side only (the device side
  of that file holds nothing but the scratch array)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed for the oracle build")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", "-fopenmp",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(SAN_DIR, "oracle_driver.c"), "-o", exe, "-lm"])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "oracle sanitizer run ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is needed for the C ABI build")
def test_c_abi_host_code_under_address_and_undefined_sanitizers(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    inc = ["-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "gated_delta_rule_short_amd", "csrc")]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api.o", "driver.o", "abi_asan"))
    _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer"] + san
         + inc + ["-c", os.path.join(ROOT, "gated_delta_rule_short_amd", "csrc", "kda_api.hip"),
                  "-o", api_o])
    _run([HIPCC, "-x", "c++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
          "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"] + san + inc
         + ["-c", os.path.join(SAN_DIR, "abi_driver.cpp"), "-o", drv_o])
    _run([HIPCC, "--offload-arch=gfx950"] + san + [api_o, drv_o, "-o", exe])
    # the HIP runtime keeps allocations until exit: leaks are not reported
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert "C-ABI sanitizer run ok" in r.stdout
