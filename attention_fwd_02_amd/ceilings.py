"""ctypes binding of libfa_ceilings.so: same-machine ceilings (HBM read
bandwidth, MFMA rate and the clock it runs at, LDS read rate, VALU rate,
MFMA/VALU co-issue) that the attention kernels' rooflines are read against.
Raises when the library is not built; it is a measuring aid, not part of the
attention path."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa_ceilings.so")
EXPORTS = ("fa_ceil_hbm_read", "fa_ceil_mfma", "fa_ceil_coissue", "fa_ceil_lds",
           "fa_ceil_valu", "fa_ceil_last_error")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (attention_fwd_02_amd.build.build_ceilings)")
        lib = ctypes.CDLL(LIB_PATH)
        d = ctypes.POINTER(ctypes.c_double)
        lib.fa_ceil_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, d]
        lib.fa_ceil_mfma.argtypes = [ctypes.c_int, ctypes.c_int, d, d]
        lib.fa_ceil_coissue.argtypes = [ctypes.c_int, ctypes.c_int, d]
        lib.fa_ceil_lds.argtypes = [ctypes.c_int, ctypes.c_int, d]
        lib.fa_ceil_valu.argtypes = [ctypes.c_int, ctypes.c_int, d]
        for f in EXPORTS[:-1]:
            getattr(lib, f).restype = ctypes.c_int
        lib.fa_ceil_last_error.restype = ctypes.c_char_p
        lib.fa_ceil_last_error.argtypes = []
        _lib = lib
    return _lib


def _call(name, *args, n_out=1):
    lib = load()
    outs = [ctypes.c_double() for _ in range(n_out)]
    rc = getattr(lib, name)(*args, *[ctypes.byref(o) for o in outs])
    if rc != 0:
        raise RuntimeError(f"{name}: {lib.fa_ceil_last_error().decode()}")
    return [o.value for o in outs] if n_out > 1 else outs[0].value


def hbm_read_gbps(ptr: int, nbytes: int, reps: int = 10) -> float:
    return _call("fa_ceil_hbm_read", ctypes.c_void_p(ptr), ctypes.c_size_t(nbytes), reps)


def mfma(fp8: bool = False, iters: int = 50000):
    """(TFLOP/s, shader clock in MHz) of the whole chip's MFMA loop."""
    return tuple(_call("fa_ceil_mfma", int(fp8), iters, n_out=2))


def coissue_cycles(k_valu: int, iters: int = 20000) -> float:
    return _call("fa_ceil_coissue", k_valu, iters)


def lds_bytes_per_clk(transposing: bool = False, iters: int = 20000) -> float:
    return _call("fa_ceil_lds", int(transposing), iters)


def valu_cycles(exp: bool = False, iters: int = 20000) -> float:
    return _call("fa_ceil_valu", int(exp), iters)


def measure_all(torch, device="cuda:0") -> dict:
    """Every ceiling once, with the datasheet peaks they sit under."""
    buf = torch.empty(2 << 30, dtype=torch.uint8, device=device)
    torch.cuda.synchronize()
    hbm = hbm_read_gbps(buf.data_ptr(), buf.numel(), 10)
    del buf
    bf16_tf, bf16_mhz = mfma(False, 50000)
    fp8_tf, fp8_mhz = mfma(True, 50000)
    return {
        "hbm_read_GBps": round(hbm, 1),
        "mfma_bf16_TFLOPs": round(bf16_tf, 1), "mfma_bf16_clock_MHz": round(bf16_mhz, 1),
        "mfma_fp8_TFLOPs": round(fp8_tf, 1), "mfma_fp8_clock_MHz": round(fp8_mhz, 1),
        "lds_b128_bytes_per_clk_cu": round(lds_bytes_per_clk(False), 1),
        "lds_tr_b16_bytes_per_clk_cu": round(lds_bytes_per_clk(True), 1),
        "valu_fma_cycles_per_instr": round(valu_cycles(False), 2),
        "valu_exp_cycles_per_instr": round(valu_cycles(True), 2),
        "mfma32_cycles_with_k_fma": {str(k): round(coissue_cycles(k), 2) for k in (0, 4, 6, 8)},
        "mfma32_cycles_with_k_exp": {str(k): round(coissue_cycles(-k), 2) for k in (1, 2, 4)},
        "loops": ("HBM: 2 GiB streaming read x10, 16 B per lane, 8 workgroups per CU; MFMA: "
                  "one wave per SIMD, four independent 32x32 accumulators; LDS: 8 waves per "
                  "CU, conflict-free reads; VALU: one wave per SIMD, independent streams"),
    }
