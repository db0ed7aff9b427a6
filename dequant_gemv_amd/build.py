"""Build libqgemv.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

The library embeds a build id: the SHA-256 of its sources and header, so a
measurement can check which code it ran (see ``qgemv_build_id``).
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqgemv.so")
ARCH = "gfx950"


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build_id(defines=(), flags=()) -> str:
    h = hashlib.sha256()
    for d in defines:
        h.update(("-D" + d).encode())
    for f in flags:
        h.update(f.encode())
    files = sources() + sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) + [os.path.join(INCLUDE, "qgemv.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False, out_path: str = LIB, defines=(), flags=()) -> str:
    """Compile every csrc/*.hip into one shared library.  `defines` (NAME=VALUE
    strings) override the kernels' tuning constants and `flags` add compiler
    options; both enter the build id."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = out_path + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # no packed-fp32 VALU forms anywhere in the device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-result",
           f"-DQGEMV_BUILD_ID=\"{build_id(defines, flags)}\"", *("-D" + d for d in defines), *flags,
           "-I", INCLUDE, "-I", CSRC, *sources(), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr)
    if verbose:
        print(r.stderr)
    os.replace(out, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
