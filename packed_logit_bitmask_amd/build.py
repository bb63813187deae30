"""Compile the HIP library in-tree for gfx950.

``python -m packed_logit_bitmask_amd.build`` (or ``build()``) runs hipcc on
csrc/mi_bitmask.hip and writes libmi_bitmask.so next to this file.  The
device code is built for gfx950 only; hipcc cross-compiles without a GPU.
"""

from __future__ import annotations

import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCE = PKG / "csrc" / "mi_bitmask.hip"
HEADERS = [PKG / "csrc" / "apply_kernels.h", ROOT / "include" / "mi_bitmask.h"]
LIBRARY = PKG / "libmi_bitmask.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and pathlib.Path(cand).exists():
            return cand
    raise FileNotFoundError("hipcc not found (ROCm is required to build the library)")


def command(out: pathlib.Path) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-fvisibility=hidden",
        # no packed fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", str(ROOT / "include"), "-I", str(PKG / "csrc"),
        "-o", str(out), str(SOURCE),
    ]


def build(verbose: bool = False) -> pathlib.Path:
    tmp = LIBRARY.with_suffix(f".so.tmp{os.getpid()}")
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        tmp.unlink(missing_ok=True)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-4000:]}")
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
