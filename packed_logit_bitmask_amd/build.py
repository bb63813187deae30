"""Compile the HIP library in-tree for gfx950.

``python -m packed_logit_bitmask_amd.build`` (or ``build()``) compiles
csrc/host_apply.cpp (host-only C++, with x86 vector code) into an object
with the host C++ compiler, then runs hipcc on the .hip sources under csrc/
and links everything into libmi_bitmask.so next to this file.  The device code is built for
gfx950 only; hipcc cross-compiles without a GPU.
"""

from __future__ import annotations

import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCES = [PKG / "csrc" / "mi_bitmask.hip",   # device apply: shapes, launches, entry points
           PKG / "csrc" / "mi_sample.hip",    # fused apply + sampler entry point
           PKG / "csrc" / "mi_host.hip"]      # host-memory entry points and helpers
HOST_SOURCE = PKG / "csrc" / "host_apply.cpp"   # host-only C++: hipcc would give it a device pass
LIBRARY = PKG / "libmi_bitmask.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and pathlib.Path(cand).exists():
            return cand
    raise FileNotFoundError("hipcc not found (ROCm is required to build the library)")


def host_cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and pathlib.Path(cand).exists():
            return cand
    raise FileNotFoundError("no host C++ compiler (g++) found")


def host_command(obj: pathlib.Path) -> list:
    return [host_cxx(), "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-pthread",
            "-I", str(PKG / "csrc"), "-c", str(HOST_SOURCE), "-o", str(obj)]


def command(out: pathlib.Path, host_obj: pathlib.Path) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-fvisibility=hidden", "-pthread",
        # no packed fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", str(ROOT / "include"), "-I", str(PKG / "csrc"),
        # the object first: hipcc marks the .hip source with -x hip, which would carry over to later inputs
        "-o", str(out), str(host_obj), *map(str, SOURCES),
    ]


def _run(cmd: list, verbose: bool, what: str) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{what} failed ({res.returncode}):\n{res.stderr[-4000:]}")


def build(verbose: bool = False) -> pathlib.Path:
    tmp = LIBRARY.with_suffix(f".so.tmp{os.getpid()}")
    obj = LIBRARY.with_suffix(f".host{os.getpid()}.o")
    try:
        _run(host_command(obj), verbose, "host C++ compile")
        _run(command(tmp, obj), verbose, "hipcc")
        os.replace(tmp, LIBRARY)
    finally:
        tmp.unlink(missing_ok=True)
        obj.unlink(missing_ok=True)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
