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


# sha256 of the kernels' generated gfx950 assembly, written next to libfa.so:
# it names the device code a measurement was taken on (the HBM traffic
# counters record it), unchanged by edits that do not change that code.
DEVICE_SHA = LIB + ".device-sha256"


def device_code_sha256(asm: str) -> str:
    """sha256 of the assembly without its compilation-unit id symbol (a name
    hipcc derives per compile, not code)."""
    import hashlib
    text = "\n".join(l for l in asm.splitlines() if "__hip_cuid_" not in l)
    return hashlib.sha256(text.encode()).hexdigest()


def check_device_code() -> str:
    """Generate the kernels' gfx950 assembly and scan it; raise on findings.
    Returns the assembly's sha256."""
    asm = asm_check.device_asm(HIPCC, FLAGS, INCLUDE, os.path.join(CSRC, "fa_kernels.hip"))
    found = asm_check.scan(asm)
    if found:
        raise RuntimeError("inline-asm MFMA hazards in the generated code:\n  "
                           + "\n  ".join(found[:20]))
    found = asm_check.scan_inline_dot(asm)
    if found:
        raise RuntimeError("inline-asm dot results read without their wait states:\n  "
                           + "\n  ".join(found[:20]))
    found = asm_check.scan_divergent_copies(asm)
    if found:
        raise RuntimeError("register copies at the end of divergent regions:\n  "
                           + "\n  ".join(found[:20]))
    return device_code_sha256(asm)


# Debug builds of the same sources with the LDS ring race checks on (see
# FA_LDS_CHECK in fa_kernels.hip): copies waited for at issue, or each copy's
# destination poisoned first.  Tests compare them bit for bit with libfa.so.
CHECK_VARIANTS = {"sync": 1, "poison": 2}


def check_lib_path(name: str) -> str:
    return os.path.join(HERE, f"libfa_check_{name}.so")


def build_check_variants(verbose: bool = False) -> list:
    """Compile every debug build in CHECK_VARIANTS (in parallel)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    procs = []
    for name, level in CHECK_VARIANTS.items():
        out = check_lib_path(name)
        cmd = [HIPCC, *FLAGS, f"-DFA_LDS_CHECK={level}", "-I", INCLUDE, "-o", out + ".tmp", *srcs]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    built = []
    for out, p in procs:
        _, err = p.communicate()
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed for {out} ({p.returncode}):\n{err[-4000:]}")
        os.replace(out + ".tmp", out)
        built.append(out)
    return built


CEIL_LIB = os.path.join(HERE, "libfa_ceilings.so")


def build_ceilings(verbose: bool = False) -> str:
    """Compile the ceiling loops (fa_ceilings.hip) into libfa_ceilings.so."""
    tmp = CEIL_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-o", tmp, os.path.join(CSRC, "fa_ceilings.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-4000:]}")
    os.replace(tmp, CEIL_LIB)
    return CEIL_LIB


def build_lib(verbose: bool = False) -> str:
    """Compile all sources into libfa.so (always recompiles) and check the
    device code of the kernels."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    check_err, sha = [], []

    def _check():
        try:
            sha.append(check_device_code())
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
    with open(DEVICE_SHA, "w") as f:
        f.write(sha[0] + "\n")
    return LIB


if __name__ == "__main__":
    print(build_lib(verbose=True))
    print(build_ceilings(verbose=True))
    print(build_check_variants(verbose=True))
