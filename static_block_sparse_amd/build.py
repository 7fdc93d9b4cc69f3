"""Builds libradial.so in-tree with hipcc for gfx950.

    python -m static_block_sparse_amd.build      (from the repository root)

Every source is compiled on each call (the build is a few tens of seconds).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libradial.so")

SOURCES = ["mask.cpp", "capi.cpp", "attn_fwd.hip", "attn_bwd.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall"]
# packed fp32 instructions off for device code (a flag of the device pass;
# the host pass warns that it does not know it, which is harmless)
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, defines=(), out: str = LIB) -> str:
    """Compile every source and link libradial.so (or `out`); returns its path.
    `defines`: extra NAME=VALUE preprocessor definitions (tuning constants).
    `out` must name a ``.so`` file directly inside the package directory (the
    library and its temporary copy are never written anywhere else)."""
    out = os.path.abspath(out) if out else ""
    if not out.endswith(".so") or os.path.dirname(out) != PKG:
        raise ValueError(f"out must be a .so file in {PKG}, got {out!r}")
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    tmp = tempfile.mkdtemp(prefix="radial_build_")
    try:
        objs = []
        dflags = [f"-D{d}" for d in defines]
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            path = os.path.join(CSRC, src)
            if src.endswith(".hip"):
                cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, *dflags, "-c", path, "-o", obj]
            else:
                cmd = [HIPCC, *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
            msg = _run(cmd)
            if verbose and msg.strip():
                print(msg)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libradial.so")
        _run([HIPCC, *DEVICE, "-shared", "-fPIC", "-o", tmp_lib, *objs])
        shutil.copyfile(tmp_lib, out + ".tmp")
        os.replace(out + ".tmp", out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
