"""Build libfa.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m attention_fwd_02_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host compiler
pass warns that it does not know that feature, which is harmless.

The kernels' device assembly is generated alongside and scanned for accesses
to the registers of inline-assembly MFMAs that the compiler's hazard
recognizer cannot see (asm_check.py); any finding fails the build.
"""
from __future__ import annotations

import os
import subprocess
import sys
import threading

from attention_fwd_02_amd import asm_check

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["fa_kernels.hip", "fa_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def check_device_code() -> None:
    """Generate the kernels' gfx950 assembly and scan it; raise on findings."""
    asm = asm_check.device_asm(HIPCC, FLAGS, INCLUDE, os.path.join(CSRC, "fa_kernels.hip"))
    found = asm_check.scan(asm)
    if found:
        raise RuntimeError("inline-asm MFMA hazards in the generated code:\n  "
                           + "\n  ".join(found[:20]))
    found = asm_check.scan_divergent_copies(asm)
    if found:
        raise RuntimeError("register copies at the end of divergent regions:\n  "
                           + "\n  ".join(found[:20]))


def build_lib(verbose: bool = False) -> str:
    """Compile all sources into libfa.so (always recompiles) and check the
    device code of the kernels."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    check_err = []

    def _check():
        try:
            check_device_code()
        except Exception as e:  # reported after the library build
            check_err.append(e)

    checker = threading.Thread(target=_check)
    checker.start()
    res = subprocess.run(cmd, capture_output=True, text=True)
    checker.join()
    # drop the host pass's note about the unknown target feature
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip() != "1 warning generated.")
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if check_err:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise check_err[0]
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_lib(verbose=True))
