"""Host-side sanitizer runs (CPU only).

The C-ABI layer (attention_fwd_02_amd/csrc/fa_api.cpp) is compiled by g++
alone against a simulated device (tests/host_sanitize/: a stand-in for the
few HIP runtime calls it makes, with host memory as device memory, and
launchers that read every input byte and write every output and workspace
byte the kernels would) and driven through every entry point of
include/fa.h; the oracle (oracle/oracle.c) is compiled with gcc and driven
over all rows, row subsets, key ranges and bad arguments.  Each runs under
AddressSanitizer + UndefinedBehaviorSanitizer, and the multi-threaded parts
under ThreadSanitizer; any report aborts the program and fails the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HS = os.path.join(ROOT, "tests", "host_sanitize")
ASAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
        "-fno-sanitize-recover=all"]
TSAN = ["-O1", "-g", "-fsanitize=thread"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc and g++")


def _build(out, compiler, flags, sources, extra=()):
    cmd = [compiler, *flags, *extra, "-o", out, *sources, "-pthread"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stderr[-3000:]}"
    return out


def _api_build(tmp, flags, name):
    return _build(os.path.join(tmp, name), "g++", ["-std=c++17", *flags],
                  [os.path.join(ROOT, "attention_fwd_02_amd", "csrc", "fa_api.cpp"),
                   os.path.join(HS, "sim_device.cpp"), os.path.join(HS, "driver_api.cpp")],
                  ["-I", os.path.join(HS, "include"), "-I", os.path.join(ROOT, "include"),
                   "-I", os.path.join(ROOT, "attention_fwd_02_amd", "csrc")])


def _oracle_build(tmp, flags, name):
    return _build(os.path.join(tmp, name), "gcc", ["-std=c11", *flags],
                  [os.path.join(ROOT, "oracle", "oracle.c"),
                   os.path.join(HS, "driver_oracle.c")], ["-lm"])


def _run(exe, *args):
    res = subprocess.run([exe, *args], capture_output=True, text=True, env=ENV, timeout=600)
    report = res.stderr[-4000:]
    assert res.returncode == 0, f"{os.path.basename(exe)} {' '.join(args)}: rc {res.returncode}\n{report}"
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer",
                   "ERROR: LeakSanitizer"):
        assert marker not in res.stderr, report
    assert "0 failures" in res.stdout, res.stdout


def test_abi_layer_under_asan_ubsan(tmp_path):
    _run(_api_build(str(tmp_path), ASAN, "api_asan"), "all")


def test_abi_layer_threads_under_tsan(tmp_path):
    _run(_api_build(str(tmp_path), TSAN, "api_tsan"), "threads")


def test_oracle_under_asan_ubsan(tmp_path):
    _run(_oracle_build(str(tmp_path), ASAN, "oracle_asan"))


def test_oracle_threads_under_tsan(tmp_path):
    _run(_oracle_build(str(tmp_path), TSAN, "oracle_tsan"))
