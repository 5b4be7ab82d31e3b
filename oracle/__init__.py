"""Double-precision CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the library under
``attention_fwd_02_amd`` never does, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, libm ``exp``/``log``,
pthreads over rows); this module only loads it with ctypes and marshals numpy
arrays.  ``oracle.c`` documents which passage of the pages each step follows
and every reading taken where the pages are silent.

Parity status: pinned.  ``tests/test_oracle.py`` checks it against a 40-digit
``decimal`` brute force, a torch fp64 library evaluation of the same
definition, closed forms worked out by hand, invariants and layout probes;
``tests/test_oracle_mutants.py`` shows that planted slips fail those pins.
``attn_fwd_paged`` (paged K/V cache, one length per sequence) gathers each
sequence's keys in plain numpy and hands them to the same definition; its
gather is pinned by hand-placed page contents with closed-form answers in
``tests/test_oracle.py`` and by planted slips in the mutant tests.
``attn_fwd_fp8`` (OCP FP8 E4M3 inputs with per-tensor descales) decodes the
codes with its own table, written from the format's definition and pinned
code by code against it and against torch's float8_e4m3fn, then applies the
same definition; planted decode and descale slips must fail its pins.
``attn_bwd`` (dQ, dK, dV) is the gradient of the definition written out in
numpy fp64; it is pinned against torch's fp64 autograd of the forward
definition, central finite differences and closed forms, and five planted
slips must fail those pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    lib.oracle_attn_fwd.restype = ctypes.c_int
    lib.oracle_attn_fwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_allowed_pairs.restype = ctypes.c_int64
    lib.oracle_allowed_pairs.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    return lib


def _bits(x) -> np.ndarray:
    """bf16 data as a contiguous uint16 numpy array (accepts torch or numpy)."""
    if hasattr(x, "detach"):  # torch tensor
        import torch
        t = x.detach()
        if t.device.type != "cpu":
            t = t.cpu()
        if t.dtype != torch.bfloat16:
            raise TypeError(f"oracle expects bfloat16 inputs, got {t.dtype}")
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint16:
        raise TypeError("numpy inputs must be raw bf16 bits (uint16)")
    return a


def default_threads() -> int:
    """The host cores this process may run on: its CPU affinity set, capped
    by a cgroup CPU quota when one is set (a container's share of a larger
    host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, -(-int(quota) // int(period))))
    except (OSError, ValueError):
        pass
    return max(1, n)


def attn_fwd(q, k, v, causal: bool, scale: float, *, rows=None,
             key_range=None, nthreads: int | None = None, _lib_override=None):
    """Run the oracle.

    q: [B, Sq, Hq, D] bf16; k, v: [B, Sk, Hkv, D] bf16.
    rows: None for every row, else an int64 array [n, 3] of (b, hq, i).
    key_range: None for all keys, else (begin, end).
    Returns (o, lse) as float64 numpy arrays: o [B,Sq,Hq,D] / lse [B,Hq,Sq],
    or o [n, D] / lse [n] when rows is given.
    """
    lib = _lib_override if _lib_override is not None else _load()
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    if qb.ndim != 4 or kb.ndim != 4 or vb.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, S, H, D]")
    B, Sq, Hq, D = qb.shape
    Bk, Sk, Hkv, Dk = kb.shape
    if (Bk, Dk) != (B, D) or vb.shape != kb.shape:
        raise ValueError("shape mismatch between q, k, v")
    kr = (0, Sk) if key_range is None else (int(key_range[0]), int(key_range[1]))
    if rows is None:
        o = np.empty((B, Sq, Hq, D), dtype=np.float64)
        lse = np.empty((B, Hq, Sq), dtype=np.float64)
        rows_p, n_rows = None, 0
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        n_rows = r.shape[0]
        o = np.empty((n_rows, D), dtype=np.float64)
        lse = np.empty((n_rows,), dtype=np.float64)
        rows_p = r.ctypes.data
    nt = default_threads() if nthreads is None else int(nthreads)
    rc = lib.oracle_attn_fwd(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data,
                             B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), float(scale),
                             kr[0], kr[1], rows_p, n_rows, o.ctypes.data, lse.ctypes.data, nt)
    if rc != 0:
        raise RuntimeError(f"oracle_attn_fwd failed with code {rc}")
    return o, lse


def allowed_pairs(Sq: int, Sk: int, causal: bool) -> int:
    """Allowed (query, key) pairs of one head: the unit of algorithmic work."""
    return int(_load().oracle_allowed_pairs(Sq, Sk, int(bool(causal))))


def gather_pages(cache: np.ndarray, table_row: np.ndarray, n: int) -> np.ndarray:
    """Rows 0..n-1 of one sequence out of a paged cache [pages, page_size, H, D]:
    logical key j is slot j % page_size of page table_row[j // page_size]."""
    page_size = cache.shape[1]
    j = np.arange(n)
    return cache[table_row[j // page_size], j % page_size]


def attn_fwd_paged(q, k_cache, v_cache, block_table, seq_lens, causal: bool, scale: float, *,
                   nthreads: int | None = None, _lib_override=None):
    """The oracle over a paged K/V cache with one length per sequence.

    The pages name paged K/V only as a way of loading K and V ("SM80 内核实现对比",
    section 7.3, the PagedKV row of the scenario table: both kernels fetch it with
    cp.async).  Layout and meaning are this project's reading: k_cache and
    v_cache are [num_pages, page_size, Hkv, D] bf16; block_table [B, max_pages]
    maps sequence b's logical page p to a cache page; seq_lens[b] = Sk_b keys.
    Sequence b is then exactly the contiguous problem over its first Sk_b keys
    (causal: key j allowed for query i iff j <= i + Sk_b - Sq); Sk_b = 0 gives
    O = 0 and LSE = -inf, as for any row without an allowed key.

    q: [B, Sq, Hq, D] bf16.  Returns (o [B,Sq,Hq,D], lse [B,Hq,Sq]) float64.
    """
    qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
    table = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                       dtype=np.int64)
    lens = np.asarray(seq_lens.cpu() if hasattr(seq_lens, "cpu") else seq_lens, dtype=np.int64)
    B, Sq, Hq, D = qb.shape
    o = np.zeros((B, Sq, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq, Sq), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        kc = gather_pages(kb, table[b], n)[None]
        vc = gather_pages(vb, table[b], n)[None]
        ob, lb = attn_fwd(qb[b:b + 1], np.ascontiguousarray(kc), np.ascontiguousarray(vc),
                          causal, scale, nthreads=nthreads, _lib_override=_lib_override)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def fp8_e4m3_value(code: int) -> float:
    """Value of one OCP FP8 E4M3 code ("fn" variant: no infinities).

    Bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa; exponent
    field 0 is subnormal (m / 8 * 2^-6); S.1111.111 is NaN, so the largest
    finite magnitude is 1.75 * 2^8 = 448."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_FP8_TABLE = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)


def fp8_values(x) -> np.ndarray:
    """float64 values of an array of FP8 E4M3 codes (uint8 numpy, or a torch
    float8_e4m3fn / uint8 tensor)."""
    if hasattr(x, "detach"):
        import torch
        t = x.detach().cpu()
        if t.dtype != torch.uint8:
            t = t.view(torch.uint8)
        x = t.numpy()
    return _FP8_TABLE[np.asarray(x, dtype=np.uint8)]


def attn_fwd_fp8(q8, k8, v8, causal: bool, scale: float, q_descale: float, k_descale: float,
                 v_descale: float, *, rows=None, nthreads: int | None = None,
                 _lib_override=None):
    """The oracle for FP8 E4M3 inputs with per-tensor descale factors.

    The pages name FP8 only as a capability of the SM90 kernel ("SM80 内核实现对比",
    section 7.3, the FP8 row of the scenario table); the convention is this
    project's reading, the usual per-tensor one: the real inputs are
    q_descale * q8, k_descale * k8, v_descale * v8, and the attention is the
    plain definition on them.  Every E4M3 value is exact in bfloat16 (3
    mantissa bits, exponents 2^-9 .. 2^8), so the codes are handed to the fp64
    definition as bf16 and the descales are folded in: scores use
    scale * q_descale * k_descale (rounded once to float32, the oracle's scale
    argument), and O is multiplied by v_descale.  LSE is unaffected by v.
    """
    import torch

    def as_bf16(x):
        vals = fp8_values(x)
        t = torch.from_numpy(vals.astype(np.float32))      # exact: E4M3 fits in fp32
        b = t.to(torch.bfloat16)                            # exact: E4M3 fits in bf16
        assert torch.equal(b.to(torch.float32), t), "an FP8 value is not exact in bf16"
        return b

    o, lse = attn_fwd(as_bf16(q8), as_bf16(k8), as_bf16(v8), causal,
                      float(scale) * float(q_descale) * float(k_descale), rows=rows,
                      nthreads=nthreads, _lib_override=_lib_override)
    return o * float(v_descale), lse


def attn_bwd(q, k, v, do, causal: bool, scale: float):
    """Gradients of the attention forward, in fp64, straight from its definition.

    The pages list the backward pass only by the title of a page that is not
    reproduced ("SM80 内核实现对比", navigation), so this follows the
    mathematics of O = softmax(scale * Q K^T [+ causal mask]) V alone.  For one
    (b, query head) with allowed-key mask, P = softmax(scale * Q K^T) row by
    row, and for the upstream gradient dO:
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(dP * P))            (softmax Jacobian, per row)
        dQ = scale * dS K,   dK = scale * dS^T Q
    Query heads sharing a KV head (hq / (Hq / Hkv)) add their dK and dV.
    Rows with no allowed key have P = 0 and contribute nothing.  Plain numpy
    matrix products on float64 values of the bf16 inputs.

    q, do: [B, Sq, Hq, D]; k, v: [B, Sk, Hkv, D] (bf16 torch tensors or raw
    bf16 bits).  Returns (dq, dk, dv) float64 in the same layouts.
    """
    def f64(x):
        bits = _bits(x).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)

    Q, K, V, dO = f64(q), f64(k), f64(v), f64(do)
    B, Sq, Hq, D = Q.shape
    Sk, Hkv = K.shape[1], K.shape[2]
    group = Hq // Hkv
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    allowed = (j <= i + (Sk - Sq)) if causal else np.ones((Sq, Sk), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            s = scale * (Q[b, :, h, :] @ K[b, :, g, :].T)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            live = np.isfinite(m)
            e = np.where(allowed, np.exp(s - np.where(live, m, 0.0)), 0.0)
            l = e.sum(axis=1, keepdims=True)
            p = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)
            dV[b, :, g, :] += p.T @ dO[b, :, h, :]
            dp = dO[b, :, h, :] @ V[b, :, g, :].T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dQ[b, :, h, :] = scale * (ds @ K[b, :, g, :])
            dK[b, :, g, :] += scale * (ds.T @ Q[b, :, h, :])
    return dQ, dK, dV
