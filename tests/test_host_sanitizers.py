"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU): the C ABI's validation
and planning layer (kda_abi.cpp, kda_plan.cpp, with stub launchers, tests/native/abi_host_check.cpp)
and the C oracle (oracle/kda_oracle.c, tests/native/oracle_check.c), each built with the host compiler
and run as its own process."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "gated_delta_rule_78_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd_build, exe):
    r = subprocess.run(cmd_build, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_abi_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    out = _run(["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                                             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                                             os.path.join(NATIVE, "abi_host_check.cpp"), os.path.join(CSRC, "kda_abi.cpp"),
                                             os.path.join(CSRC, "kda_plan.cpp"), "-o", exe], exe)
    assert "abi host check: ok" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    out = _run(["gcc", "-std=c11"] + SAN + ["-fopenmp", os.path.join(NATIVE, "oracle_check.c"),
                                            os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm", "-o", exe], exe)
    assert "oracle check: ok" in out
