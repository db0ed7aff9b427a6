"""Host AddressSanitizer / UndefinedBehaviorSanitizer runs (no GPU):

* the fp64 oracle (oracle/oracle.c) built with gcc and driven over every entry
  point and every decoder code (tests/sanitize/oracle_driver.c);
* the C ABI's argument validation (dequant_gemv_amd/csrc/abi.hip, host code
  only) with the kernel launchers replaced by stubs, driven over every entry
  point's valid, invalid and largest-accepted arguments
  (tests/sanitize/abi_driver.cpp, launch_stubs.cpp).

Either binary exits non-zero on a wrong return code, and the sanitizers abort
it on the first out-of-bounds access, leak, overflow or other undefined
behaviour.  And: a valid call on a machine with no visible device returns
QGEMV_E_HIP instead of crashing."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)


def _check(r):
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-3000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    r = _run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", os.path.join(SAN, "oracle_driver.c"),
              os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe])
    assert r.returncode == 0, r.stderr[-3000:]
    _check(_run([exe]))


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    # host code only (--cuda-host-only); the sanitizers apply to the host pass
    r = _run([HIPCC, "--offload-arch=gfx950", "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all",
              "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "dequant_gemv_amd", "csrc"),
              os.path.join(ROOT, "dequant_gemv_amd", "csrc", "abi.hip"), os.path.join(SAN, "launch_stubs.cpp"),
              os.path.join(SAN, "abi_driver.cpp"), "-o", exe])
    assert r.returncode == 0, r.stderr[-3000:]
    _check(_run([exe]))


NO_DEVICE = r"""
import ctypes, sys
hip = ctypes.CDLL("libamdhip64.so")
n = ctypes.c_int(0)
rc = hip.hipGetDeviceCount(ctypes.byref(n))
if rc == 0 and n.value > 0:
    print("SKIP: a device is visible")
    sys.exit(0)
sys.path.insert(0, sys.argv[1])
from dequant_gemv_amd import qgemv
lib = qgemv.lib()
# aligned, distinct, never dereferenced: no device exists to run the kernel
code = lib.qgemv_q4k(0x100000, 0x200000, 0x300000, 16, 256, None)
print("RC", code, lib.qgemv_last_hip_error())
"""


def test_valid_call_without_a_device_returns_hip_error():
    if not os.path.exists(os.path.join(ROOT, "dequant_gemv_amd", "libqgemv.so")):
        pytest.skip("library not built")
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = _run([sys.executable, "-c", NO_DEVICE, ROOT], env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    if "SKIP" in r.stdout:
        pytest.skip("a device is visible; the call would launch")
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("RC")][-1]
    _, code, hip_err = line.split()
    assert int(code) == -4 and int(hip_err) != 0, r.stdout
