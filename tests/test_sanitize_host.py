"""Host-side code under AddressSanitizer + UndefinedBehaviorSanitizer and ThreadSanitizer.

tests/sanitize_host.cpp compiles the library's host entry points and helpers
(argument checks, vocab rule, fill rounding), links the host apply loops
(AVX-512 and portable, with their thread split) and the oracle's C loop, and
drives every rejection, the fill conversion and applies checked against the
oracle.  It is built twice with the host compiler -- once with
-fsanitize=address,undefined, once with -fsanitize=thread -- and each build
runs with both host loops (MI_BITMASK_HOST_ISA=portable forces the portable
one).  Any sanitizer report fails the run.  A planted out-of-bounds read,
built with the same flags, must be caught: the check of the check.
"""

import os
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
CSRC = ROOT / "packed_logit_bitmask_amd" / "csrc"
ROCM_INCLUDE = pathlib.Path("/opt/rocm/include")

FLAGS = {
    "address,undefined": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
    "thread": ["-fsanitize=thread"],
}


def _need_tools():
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc / g++ not found")
    if not (ROCM_INCLUDE / "hip" / "hip_runtime_api.h").exists():
        pytest.skip("HIP headers not found")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return res.returncode, res.stdout, res.stderr


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    _need_tools()
    out = tmp_path_factory.mktemp("sanitize")
    exes = {}
    for name, flags in FLAGS.items():
        tag = name.replace(",", "_")
        obj = out / f"apply_loop_{tag}.o"
        rc, _, err = _run(["gcc", "-std=c99", "-g", "-O1", *flags, "-c", str(ROOT / "oracle" / "apply_loop.c"),
                           "-o", str(obj)])
        assert rc == 0, err[-3000:]
        exe = out / f"sanitize_host_{tag}"
        rc, _, err = _run(["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-pthread", *flags,
                           "-D__HIP_PLATFORM_AMD__", "-I", str(ROOT / "include"), "-I", str(CSRC),
                           "-I", str(ROCM_INCLUDE), str(ROOT / "tests" / "sanitize_host.cpp"),
                           str(CSRC / "host_apply.cpp"), str(obj), "-o", str(exe)])
        assert rc == 0, err[-3000:]
        exes[name] = exe
    return out, exes


@pytest.mark.parametrize("isa", ["default", "portable"])
@pytest.mark.parametrize("sanitizer", list(FLAGS))
def test_host_code_runs_clean(builds, sanitizer, isa):
    _, exes = builds
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", TSAN_OPTIONS="halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    if isa == "portable":
        env["MI_BITMASK_HOST_ISA"] = "portable"
    rc, out, err = _run([str(exes[sanitizer])], env=env, timeout=600)
    assert rc == 0 and "sanitized host checks: ok" in out, f"rc={rc}\n{out[-2000:]}\n{err[-4000:]}"
    assert "Sanitizer" not in err, err[-4000:]
    if isa == "portable":
        assert "host loop: portable" in out


def test_planted_overflow_is_caught(builds):
    out, _ = builds
    src = out / "planted.c"
    src.write_text("#include <stdlib.h>\nint main(void) { volatile int *p = malloc(4 * sizeof(int));\n"
                   "  int v = p[4]; free((void *)p); return v & 0; }\n")
    exe = out / "planted"
    rc, _, err = _run(["gcc", "-g", "-O0", *FLAGS["address,undefined"], str(src), "-o", str(exe)])
    assert rc == 0, err
    rc, _, err = _run([str(exe)], timeout=60)
    assert rc != 0 and "heap-buffer-overflow" in err
