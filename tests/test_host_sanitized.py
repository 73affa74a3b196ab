"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* attn_api.cpp (the C ABI's argument checks, device check, parameter folding
  and dispatch) is compiled with g++ against stand-ins for the three HIP calls
  it makes and for the kernel launchers (tests/host/hip_stub.cpp); the driver
  tests/host/abi_host_check.cpp calls every entry point, with the stubbed
  device reporting gfx950 and then another architecture (gfx942), where every
  valid call must return ATTN_ERR_UNSUPPORTED and launch nothing.
* oracle/attn_oracle.c is compiled with gcc and driven through all its entry
  points by tests/host/oracle_host_check.c.

The two builds share nothing: the oracle and the library stay separate.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _build(tmp_path, compiler, sources, flags, name):
    exe = str(tmp_path / name)
    r = subprocess.run([compiler, *SAN, *flags, *sources, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def _run(cmd, env=None):
    e = dict(os.environ)
    e.update(env or {})
    # the environment is passed on unchanged; ASan is told not to insist on
    # being the first library loaded
    e["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    e["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run(cmd, capture_output=True, text=True, env=e, timeout=300)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_host_paths_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "fp8_bf16_causal_amd", "csrc")
    exe = _build(tmp_path, "g++",
                 [os.path.join(csrc, "attn_api.cpp"), os.path.join(HOST, "hip_stub.cpp"),
                  os.path.join(HOST, "abi_host_check.cpp")],
                 ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                  "-I", csrc], "abi_host_check")
    rc, out = _run([exe])
    assert rc == 0 and "gfx950: 0 failed" in out, out
    # the device check on another architecture (a fresh process: the library
    # caches the answer per device)
    rc, out = _run([exe, "other-arch"], env={"STUB_ARCH": "gfx942"})
    assert rc == 0 and "other-arch: 0 failed" in out, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = _build(tmp_path, "gcc",
                 [os.path.join(ROOT, "oracle", "attn_oracle.c"), os.path.join(HOST, "oracle_host_check.c")],
                 ["-std=c99", "-D_POSIX_C_SOURCE=200809L", "-ffp-contract=off", "-pthread", "-lm"], "oracle_host_check")
    rc, out = _run([exe])
    assert rc == 0 and "oracle: 0 failed" in out, out
