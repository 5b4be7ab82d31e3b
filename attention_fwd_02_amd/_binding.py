"""ctypes binding of libfa.so: argument marshalling only.

Every function here has the name of the C entry point it calls (include/fa.h)
and does no arithmetic of its own: it checks that torch tensors have the
layout the library expects, passes their device pointers and sizes, and turns
a non-OK status into an exception.  If libfa.so is missing the import of this
module fails loudly: there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_NOMEM, FA_ERR_HIP = range(5)
FA_DTYPE_BF16, FA_DTYPE_F32 = 0, 1
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_INVALID_ARG", 2: "FA_ERR_UNSUPPORTED",
                3: "FA_ERR_NOMEM", 4: "FA_ERR_HIP"}

# every symbol include/fa.h declares
EXPORTS = ["fa_fwd", "fa_fwd_ex", "fa_fwd_noalloc", "fa_workspace_size", "fa_plan", "fa_fwd_paged",
           "fa_plan_paged", "fa_fwd_fp8", "fa_bwd", "fa_bwd_workspace_size", "fa_last_error",
           "fa_release_workspace", "fa_version"]


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class FaPlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("num_splits", ctypes.c_int),
                ("block_m", ctypes.c_int), ("block_n", ctypes.c_int),
                ("grid", ctypes.c_int), ("work_items", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t), ("waves", ctypes.c_int),
                ("rows_per_wave", ctypes.c_int)]


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m attention_fwd_02_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    c_int, c_float, c_void_p, c_size_t = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    fwd_args = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_void_p]
    lib.fa_fwd.argtypes = fwd_args
    lib.fa_fwd.restype = c_int
    lib.fa_fwd_ex.argtypes = fwd_args + [c_int, c_int, c_void_p, c_size_t]
    lib.fa_fwd_ex.restype = c_int
    lib.fa_fwd_noalloc.argtypes = fwd_args + [c_int, c_int]
    lib.fa_fwd_noalloc.restype = c_int
    lib.fa_workspace_size.argtypes = [c_int] * 7
    lib.fa_workspace_size.restype = c_size_t
    lib.fa_plan.argtypes = [c_int] * 8 + [ctypes.POINTER(FaPlanInfo)]
    lib.fa_plan.restype = c_int
    lib.fa_fwd_paged.argtypes = ([c_void_p] * 7 + [c_int] * 8 + [c_int, c_float, c_void_p,
                                                                c_int, c_int, c_void_p, c_size_t])
    lib.fa_fwd_paged.restype = c_int
    lib.fa_plan_paged.argtypes = [c_int] * 9 + [ctypes.POINTER(FaPlanInfo)]
    lib.fa_plan_paged.restype = c_int
    lib.fa_fwd_fp8.argtypes = ([c_void_p] * 5 + [c_int] * 7 + [c_float] * 4 +
                               [c_void_p, c_int])
    lib.fa_fwd_fp8.restype = c_int
    lib.fa_bwd.argtypes = [c_void_p] * 9 + [c_int] * 7 + [c_float, c_void_p, c_void_p, c_size_t]
    lib.fa_bwd.restype = c_int
    lib.fa_bwd_workspace_size.argtypes = [c_int] * 6
    lib.fa_bwd_workspace_size.restype = c_size_t
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_release_workspace.argtypes = []
    lib.fa_release_workspace.restype = c_int
    lib.fa_version.argtypes = []
    lib.fa_version.restype = c_int
    return lib


lib = _load()
_other_builds = {}


@contextlib.contextmanager
def using_library(path):
    """Inside the block, this module's functions call another build of the
    same library at `path` (the LDS race-check debug builds), then libfa.so
    again.  Not thread-safe; for tests."""
    global lib
    if path not in _other_builds:
        _other_builds[path] = _load(path)
    saved, lib = lib, _other_builds[path]
    try:
        yield
    finally:
        lib = saved


def _check(status: int):
    if status != FA_OK:
        raise FaError(status, (lib.fa_last_error() or b"").decode())


def fa_last_error() -> str:
    return (lib.fa_last_error() or b"").decode()


def fa_version() -> int:
    return lib.fa_version()


def fa_release_workspace() -> None:
    _check(lib.fa_release_workspace())


def fa_workspace_size(B, Hq, Hkv, Sq, Sk, D, num_splits=0) -> int:
    return int(lib.fa_workspace_size(B, Hq, Hkv, Sq, Sk, D, num_splits))


def fa_plan(B, Hq, Hkv, Sq, Sk, D, causal=False, num_splits=0) -> dict:
    info = FaPlanInfo()
    _check(lib.fa_plan(B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), num_splits, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in FaPlanInfo._fields_}


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _shapes(q, k, v, o, lse):
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or o.dim() != 4:
        raise ValueError("q, k, v, o must be 4-D: [B, S, H, D]")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    if tuple(k.shape) != (B, Sk, Hkv, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must both be [B, Sk, Hkv, D]")
    if tuple(o.shape) != (B, Sq, Hq, D):
        raise ValueError("o must be [B, Sq, Hq, D]")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [B, Hq, Sq] tensor")
    return B, Hq, Hkv, Sq, Sk, D


def fa_fwd(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """O (bf16) and LSE of q, k, v on the current (or given) HIP stream."""
    import torch
    if o.dtype != torch.bfloat16:
        raise TypeError("fa_fwd writes a bfloat16 o; use fa_fwd_ex for float32")
    B, Hq, Hkv, Sq, Sk, D = _shapes(q, k, v, o, lse)
    _check(lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                      lse.data_ptr() if lse is not None else None,
                      B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), float(scale),
                      _stream_handle(stream)))


def fa_fwd_ex(q, k, v, o, lse, causal: bool, scale: float, stream=None, num_splits: int = 0,
              workspace=None) -> None:
    """As fa_fwd; o may be bfloat16 or float32, num_splits forces the split path."""
    import torch
    if o.dtype == torch.bfloat16:
        odt = FA_DTYPE_BF16
    elif o.dtype == torch.float32:
        odt = FA_DTYPE_F32
    else:
        raise TypeError("o must be bfloat16 or float32")
    B, Hq, Hkv, Sq, Sk, D = _shapes(q, k, v, o, lse)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                         lse.data_ptr() if lse is not None else None,
                         B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), float(scale),
                         _stream_handle(stream), odt, int(num_splits), ws_ptr, ws_bytes))


def fa_fwd_noalloc(q, k, v, o, lse, causal: bool, scale: float, stream=None,
                   num_splits: int = 0) -> None:
    """As fa_fwd_ex, with the split partials in the library's static device
    array (the call allocates nothing)."""
    import torch
    if o.dtype == torch.bfloat16:
        odt = FA_DTYPE_BF16
    elif o.dtype == torch.float32:
        odt = FA_DTYPE_F32
    else:
        raise TypeError("o must be bfloat16 or float32")
    B, Hq, Hkv, Sq, Sk, D = _shapes(q, k, v, o, lse)
    _check(lib.fa_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr() if lse is not None else None,
                              B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), float(scale),
                              _stream_handle(stream), odt, int(num_splits)))


def fa_plan_paged(B, Hq, Hkv, Sq, D, num_pages, page_size, max_pages, num_splits=0) -> dict:
    info = FaPlanInfo()
    _check(lib.fa_plan_paged(B, Hq, Hkv, Sq, D, num_pages, page_size, max_pages, num_splits,
                             ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in FaPlanInfo._fields_}


def fa_fwd_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, causal: bool, scale: float,
                 stream=None, num_splits: int = 0, workspace=None) -> None:
    """Attention of q over a paged K/V cache; o bfloat16 or float32."""
    import torch
    if o.dtype == torch.bfloat16:
        odt = FA_DTYPE_BF16
    elif o.dtype == torch.float32:
        odt = FA_DTYPE_F32
    else:
        raise TypeError("o must be bfloat16 or float32")
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.dim() != 4 or o.dim() != 4:
        raise ValueError("q, o must be [B, Sq, Hq, D]; caches [num_pages, page_size, Hkv, D]")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("o", o),
                    ("block_table", block_table), ("seq_lens", seq_lens)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, Sq, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache must both be [num_pages, page_size, Hkv, D]")
    if tuple(o.shape) != (B, Sq, Hq, D):
        raise ValueError("o must be [B, Sq, Hq, D]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [B, Hq, Sq] tensor")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib.fa_fwd_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                            block_table.data_ptr(), seq_lens.data_ptr(), o.data_ptr(),
                            lse.data_ptr() if lse is not None else None,
                            B, Hq, Hkv, Sq, D, num_pages, page_size, block_table.shape[1],
                            int(bool(causal)), float(scale), _stream_handle(stream), odt,
                            int(num_splits), ws_ptr, ws_bytes))


def fa_fwd_fp8(q, k, v, o, lse, causal: bool, scale: float, q_descale: float, k_descale: float,
               v_descale: float, stream=None) -> None:
    """Attention on float8_e4m3fn q, k, v with per-tensor descales; o bf16 or f32."""
    import torch
    if o.dtype == torch.bfloat16:
        odt = FA_DTYPE_BF16
    elif o.dtype == torch.float32:
        odt = FA_DTYPE_F32
    else:
        raise TypeError("o must be bfloat16 or float32")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or o.dim() != 4:
        raise ValueError("q, k, v, o must be 4-D: [B, S, H, D]")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.float8_e4m3fn:
            raise TypeError(f"{name} must be float8_e4m3fn")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    if tuple(k.shape) != (B, Sk, Hkv, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must both be [B, Sk, Hkv, D]")
    if tuple(o.shape) != (B, Sq, Hq, D):
        raise ValueError("o must be [B, Sq, Hq, D]")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [B, Hq, Sq] tensor")
    _check(lib.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          lse.data_ptr() if lse is not None else None,
                          B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), float(scale),
                          float(q_descale), float(k_descale), float(v_descale),
                          _stream_handle(stream), odt))


def fa_bwd_workspace_size(B, Hq, Hkv, Sq, Sk, D) -> int:
    return int(lib.fa_bwd_workspace_size(B, Hq, Hkv, Sq, Sk, D))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, causal: bool, scale: float, stream=None,
           workspace=None) -> None:
    """dq, dk, dv (bf16) of the attention forward that produced o and lse."""
    import torch
    B, Hq, Hkv, Sq, Sk, D = _shapes(q, k, v, o, lse)
    for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor")
    if tuple(dout.shape) != tuple(q.shape) or tuple(dq.shape) != tuple(q.shape):
        raise ValueError("dout and dq must be [B, Sq, Hq, D]")
    if tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(k.shape):
        raise ValueError("dk and dv must be [B, Sk, Hkv, D]")
    if o.dtype != torch.bfloat16:
        raise TypeError("o must be bfloat16")
    if lse is None:
        raise ValueError("the backward needs the forward's lse")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), float(scale),
                      _stream_handle(stream), ws_ptr, ws_bytes))
