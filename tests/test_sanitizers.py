"""Host builds under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

* tests/sanitize/plan_check.cpp drives the launch planning and argument checks of the GEMV
  calls (ultra_bit_weight_uint32_amd/csrc/plan.h: exact fast division, the workgroup unit
  ranges in both row-group modes, the default workgroup count, the group-width-4 chunking,
  staging and LDS sizes, the C-ABI argument and workspace checks) over random and edge shapes.
* tests/sanitize/oracle_check.c runs the CPU oracle (oracle/oracle.c) over random small shapes
  and checks its routes against each other.

Each is compiled with -fsanitize=address,undefined -fno-sanitize-recover=all, so any
out-of-bounds access, leak, signed overflow or other undefined behaviour fails the test.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _have(compiler):
    return shutil.which(compiler) is not None


def _build_and_run(tmp_path, cmd, exe):
    build = subprocess.run(cmd + ["-o", str(exe)], capture_output=True, text=True, timeout=300)
    if build.returncode != 0 and "fsanitize" in (build.stderr or "") and "unrecognized" in build.stderr:
        pytest.skip("compiler without sanitizer support")
    assert build.returncode == 0, build.stderr[-4000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=ENV)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.stdout[-2000:], run.stderr[-4000:])


@pytest.mark.skipif(not _have("g++"), reason="g++ not found")
def test_plan_under_sanitizers(tmp_path):
    src = os.path.join(HERE, "sanitize", "plan_check.cpp")
    _build_and_run(tmp_path, ["g++", "-std=c++17", "-Wall", "-Wextra"] + SAN + [src], tmp_path / "plan_check")


@pytest.mark.skipif(not _have("gcc"), reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    srcs = [os.path.join(HERE, "sanitize", "oracle_check.c"), os.path.join(ROOT, "oracle", "oracle.c")]
    _build_and_run(tmp_path, ["gcc", "-std=c11", "-fopenmp", "-Wall", "-Wextra"] + SAN + srcs + ["-lm"],
                   tmp_path / "oracle_check")
