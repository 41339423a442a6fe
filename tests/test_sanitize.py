"""Host-code sanitizer runs (no GPU): the CPU oracle and the C-ABI layer
built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++, host
code only) and driven through their functions on small inputs and on valid
and invalid argument lists.  The ABI layer is linked with host stand-ins for
the kernel launchers (tests/sanitize/abi_stubs.cpp), so its valid calls run
to the launch without a GPU.  Any sanitizer finding aborts the driver."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
ENV.pop("LD_PRELOAD", None)


def have(tool):
    return shutil.which(tool) is not None


def build_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-6000:]
    return r.stdout


@pytest.mark.skipif(not have("gcc"), reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = build_run(["gcc", "-std=c99", "-fopenmp", "-ffp-contract=off", *SAN,
                     os.path.join(ROOT, "oracle", "lca_oracle.c"),
                     os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe], exe)
    assert "oracle driver: ok" in out


@pytest.mark.skipif(not have("g++") or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
                    reason="g++ or the HIP runtime library not found")
def test_abi_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    out = build_run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN,
                     os.path.join(ROOT, "long_context_attention_13_amd", "csrc", "abi.cpp"),
                     os.path.join(ROOT, "tests", "sanitize", "abi_stubs.cpp"),
                     os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
                     "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], exe)
    assert "abi driver: ok" in out
