"""Fused attention forward for MI355X (gfx950): HIP kernels behind a C ABI.

The kernels and the C ABI live in ``csrc/`` and are built into ``libfa.so``
(``python -m attention_fwd_02_amd.build``); the ABI is declared in
``include/fa.h``.  ``attention_fwd_02_amd.ops`` is the ctypes binding with the
same names; importing it loads ``libfa.so`` and fails loudly if it is missing.
``attention_fwd_02_amd.inputs`` holds the seeded synthetic workloads.
"""

__all__ = ["ops", "inputs"]


def __getattr__(name):
    if name == "ops":
        from . import _binding as ops
        return ops
    if name == "inputs":
        from . import inputs
        return inputs
    raise AttributeError(name)
