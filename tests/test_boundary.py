"""C-ABI boundary on the CPU: the library loads, exports every symbol its
header declares, and rejects each class of bad argument before any HIP call.
No test here launches a kernel."""
from __future__ import annotations

import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def b():
    from attention_fwd_02_amd import _binding
    return _binding


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports(b):
    assert declared_functions() == sorted(b.EXPORTS)


def test_library_exports_every_declared_symbol(b):
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)", out))
    for name in declared_functions():
        assert name in exported, f"{name} declared in fa.h but not exported"
        assert hasattr(b.lib, name)


def test_ceilings_library_exports_its_header():
    """The measuring loops' library (libfa_ceilings.so) loads and exports
    every function include/fa_ceilings.h declares."""
    from attention_fwd_02_amd import ceilings
    names = declared_functions(os.path.join(ROOT, "include", "fa_ceilings.h"))
    assert names == sorted(ceilings.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", ceilings.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)", out))
    lib = ceilings.load()
    for name in names:
        assert name in exported and hasattr(lib, name)


def test_version(b):
    assert b.fa_version() == 100


P = 0x10000  # a 16-byte aligned fake device address; never dereferenced


def call(b, q=P, k=P, v=P, o=P, lse=None, B=1, Hq=1, Hkv=1, Sq=128, Sk=128, D=64,
         causal=0, scale=0.125, o_dtype=0, num_splits=0, ws=None, ws_bytes=0):
    st = b.lib.fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, scale, None, o_dtype,
                         num_splits, ws, ws_bytes)
    return st, b.fa_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=0), 1), (dict(Hq=0), 1), (dict(Hkv=0), 1), (dict(Sq=0), 1), (dict(Sk=0), 1),
    (dict(B=-3), 1), (dict(D=0), 1),
    (dict(Hq=6, Hkv=4), 1),
    (dict(scale=math.inf), 1), (dict(scale=-math.inf), 1), (dict(scale=math.nan), 1),
    (dict(causal=2), 1), (dict(o_dtype=7), 1), (dict(num_splits=-1), 1),
    (dict(D=96), 2), (dict(D=512), 2), (dict(D=32), 2),
    (dict(q=P + 2), 2), (dict(k=P + 8), 2), (dict(v=P + 4), 2), (dict(o=P + 2), 2),
    (dict(lse=P + 4), 2), (dict(ws=P + 8, ws_bytes=1 << 20, num_splits=2, Sq=1), 2),
    # split path limited to 32 query rows per KV head
    (dict(num_splits=4, Sq=33), 2), (dict(num_splits=2, Sq=9, Hq=4, Hkv=1), 2),
])
def test_bad_arguments_rejected_before_any_hip_call(b, kw, status):
    st, msg = call(b, **kw)
    assert st == status, (st, msg)
    assert msg, "a non-OK status must leave a message"


def test_fa_fwd_checks_too(b):
    st = b.lib.fa_fwd(P, P, None, P, None, 1, 1, 1, 4, 4, 64, 0, 0.1, None)
    assert st == 1 and "NULL" in b.fa_last_error()


def test_valid_call_without_device_reports_hip_error(b):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present: this test never launches on fake pointers")
    st, msg = call(b)
    assert st == 4 and msg


def test_workspace_size_and_plan_host_arithmetic(b):
    # decode shape: a 3-stage ring of 2 x 8 KiB tiles (48 KiB of LDS) leaves 3
    # single-wave workgroups per CU, so 256 (b, g) pairs x 3 splits fill a
    # 256-CU part once; partials [splits][B][Hq][Sq][D+1] fp32
    assert b.fa_workspace_size(32, 32, 8, 1, 8192, 128, 0) == 3 * 32 * 32 * 1 * 129 * 4
    assert b.fa_workspace_size(32, 32, 8, 1, 8192, 128, 16) == 16 * 32 * 32 * 129 * 4
    assert b.fa_workspace_size(32, 32, 8, 1, 8192, 128, 1) == 0
    assert b.fa_workspace_size(4, 16, 16, 4096, 4096, 128, 0) == 0   # prefill path
    assert b.fa_workspace_size(0, 16, 16, 4096, 4096, 128, 0) == 0   # invalid sizes
    # head dim 128: the pipelined kernel, 8 waves x 32 rows, 32-key tiles
    # (separate 3-stage K and V rings, 48 KiB), two waves per SIMD: one
    # workgroup per CU
    p = b.fa_plan(16, 16, 16, 1024, 1024, 128, True, 0)
    assert p["path"] == 0 and p["block_m"] == 256 and p["block_n"] == 32
    assert p["waves"] == 8 and p["rows_per_wave"] == 32
    assert p["work_items"] == 16 * 16 * 4 and p["grid"] == 256
    for causal, S in ((False, 4096), (True, 4096), (True, 16384)):
        p = b.fa_plan(1, 32, 8, S, S, 128, causal, 0)
        assert p["block_m"] == 256 and p["block_n"] == 32 and p["grid"] == 256
        assert p["waves"] == 8 and p["rows_per_wave"] == 32
    # head dim 64, short causal rows: 8 waves x 32 rows, 64-key tiles
    p = b.fa_plan(16, 16, 16, 1024, 1024, 64, True, 0)
    assert p["block_m"] == 256 and p["block_n"] == 64 and p["waves"] == 8
    # head dim 64, non-causal and causal from 2048 rows: 4 waves x 64 rows
    for causal, S in ((False, 4096), (True, 4096)):
        p = b.fa_plan(1, 32, 8, S, S, 64, causal, 0)
        assert p["block_m"] == 256 and p["block_n"] == 64 and p["grid"] == 256
        assert p["waves"] == 4 and p["rows_per_wave"] == 64
    # too few 256-row items to cover the CUs: 4-wave workgroups, 32-key tiles
    p = b.fa_plan(4, 8, 8, 1024, 1024, 64, True, 0)
    assert p["block_m"] == 128 and p["block_n"] == 32 and p["work_items"] == 4 * 8 * 8
    assert p["grid"] == 4 * 8 * 8 and p["waves"] == 4
    # ... and too few 128-row items as well: 2-wave workgroups (64 rows)
    p = b.fa_plan(2, 8, 8, 1024, 1024, 64, True, 0)
    assert p["block_m"] == 64 and p["block_n"] == 32 and p["work_items"] == 2 * 8 * 16
    assert p["grid"] == 2 * 8 * 16 and p["waves"] == 2
    p = b.fa_plan(32, 32, 8, 1, 8192, 128, False, 0)
    assert p["path"] == 1 and p["num_splits"] == 3 and p["grid"] == 32 * 8 * 3
    # splits clamp to one per 32-key tile, and forced splits are honoured
    assert b.fa_plan(1, 4, 1, 1, 100, 64, False, 64)["num_splits"] == 4
    assert b.fa_plan(1, 4, 1, 1, 1000, 64, False, 3)["num_splits"] == 3
    with pytest.raises(b.FaError) as e:
        b.fa_plan(1, 64, 1, 1, 100, 64, False, 2)
    assert e.value.status == 2


def test_plan_tile_overrides(b, monkeypatch):
    """FA_PREFILL_BN / _NW / _NR pick a compiled tile configuration; anything
    not compiled falls back to the planner's own choice."""
    # 64 rows per wave (two 32-row column blocks), 4 waves: 256-row blocks
    monkeypatch.setenv("FA_PREFILL_BN", "64")
    monkeypatch.setenv("FA_PREFILL_NW", "4")
    monkeypatch.setenv("FA_PREFILL_NR", "2")
    p = b.fa_plan(1, 32, 8, 16384, 16384, 128, False, 0)
    assert p["block_m"] == 256 and p["block_n"] == 64 and p["work_items"] == 32 * 64
    assert p["grid"] == 256          # one wave per SIMD: one workgroup per CU
    # the wide kernel needs two key blocks per tile: 32-key tiles are not
    # compiled, and the default (the pipelined 32-key kernel) applies again
    monkeypatch.setenv("FA_PREFILL_BN", "32")
    p = b.fa_plan(4, 16, 16, 4096, 4096, 128, True, 0)
    assert p["block_m"] == 256 and p["block_n"] == 32 and p["waves"] == 8
    monkeypatch.setenv("FA_PREFILL_NR", "1")
    monkeypatch.setenv("FA_PREFILL_NW", "8")
    p = b.fa_plan(4, 16, 16, 4096, 4096, 128, True, 0)
    assert p["block_m"] == 256 and p["block_n"] == 32


def test_plan_pipelined_kernel_switch(b, monkeypatch):
    """FA_PREFILL_PIPE: 0 turns the pipelined head-dim-128 kernel off (the
    64-row kernel takes long rows again), 2 forces it where the planner would
    give the shape to the small-problem configurations."""
    monkeypatch.setenv("FA_PREFILL_PIPE", "0")
    p = b.fa_plan(4, 16, 16, 4096, 4096, 128, True, 0)
    assert p["block_n"] == 64 and p["waves"] == 4 and p["rows_per_wave"] == 64
    monkeypatch.setenv("FA_PREFILL_PIPE", "2")
    p = b.fa_plan(2, 8, 8, 1024, 1024, 128, True, 0)
    assert p["block_m"] == 256 and p["block_n"] == 32 and p["waves"] == 8
    assert p["work_items"] == 2 * 8 * 4 and p["grid"] == 2 * 8 * 4
    # head dim 64 has no pipelined kernel: the planner's own choice
    p = b.fa_plan(2, 8, 8, 1024, 1024, 64, True, 0)
    assert p["block_m"] == 64 and p["waves"] == 2
    monkeypatch.delenv("FA_PREFILL_PIPE")
    p = b.fa_plan(2, 8, 8, 1024, 1024, 128, True, 0)
    assert p["block_n"] == 32 and p["waves"] == 2   # 64-row items: too few for the CUs


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "attention_fwd_02_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f
                assert "oracle.c" not in text and "liboracle" not in text, f


def call_paged(b, q=P, kc=P, vc=P, table=P, lens=P, o=P, lse=None, B=2, Hq=8, Hkv=2, Sq=1, D=128,
               num_pages=64, page_size=16, max_pages=32, causal=0, scale=0.125, o_dtype=0,
               num_splits=0, ws=None, ws_bytes=0):
    st = b.lib.fa_fwd_paged(q, kc, vc, table, lens, o, lse, B, Hq, Hkv, Sq, D, num_pages,
                            page_size, max_pages, causal, scale, None, o_dtype, num_splits, ws,
                            ws_bytes)
    return st, b.fa_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kc=None), 1), (dict(vc=None), 1), (dict(table=None), 1),
    (dict(lens=None), 1), (dict(o=None), 1),
    (dict(B=0), 1), (dict(num_pages=0), 1), (dict(max_pages=0), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(page_size=24), 1), (dict(page_size=8), 1), (dict(page_size=0), 1),
    (dict(scale=math.nan), 1), (dict(causal=3), 1), (dict(o_dtype=5), 1),
    (dict(num_splits=-2), 1),
    (dict(D=96), 2), (dict(Sq=9), 2), (dict(Hq=64, Hkv=1), 2),
    (dict(q=P + 2), 2), (dict(kc=P + 8), 2), (dict(table=P + 2), 2), (dict(lens=P + 1), 2),
    (dict(page_size=1 << 20, Hkv=8), 2),           # one page over 2 GiB
])
def test_paged_bad_arguments_rejected_before_any_hip_call(b, kw, status):
    st, msg = call_paged(b, **kw)
    assert st == status, (st, msg)
    assert msg


def test_head_dim_256_decode_plans(b, monkeypatch):
    # D = 256: separate K and V rings of 3 + 2 32-key tiles (80 KiB of LDS)
    # leave two single-wave workgroups per CU, so the 256 (b, g) pairs of the
    # decode workload take 2 splits (a 256-CU part filled once)
    p = b.fa_plan(32, 32, 8, 1, 8192, 256, False, 0)
    assert p["path"] == 1 and p["num_splits"] == 2 and p["grid"] == 32 * 8 * 2
    assert p["workspace_bytes"] == 2 * 32 * 32 * 257 * 4
    assert b.fa_workspace_size(32, 32, 8, 1, 8192, 256, 0) == 2 * 32 * 32 * 257 * 4
    # the paged kernel uses the same rings (at least 2 splits; here the
    # 256-page bound per split, 512 16-key pages, asks for one more) when
    # its keys are cut into equal splits
    monkeypatch.setenv("FA_PAGED_BALANCED", "0")
    q = b.fa_plan_paged(32, 32, 8, 1, 256, 16384, 16, 512, 0)
    assert q["path"] == 2 and q["num_splits"] == 3
    q = b.fa_plan_paged(32, 32, 8, 1, 256, 16384, 64, 128, 0)
    assert q["num_splits"] == 2 and q["grid"] == 32 * 8 * 2


def test_paged_plan_host_arithmetic(b, monkeypatch):
    monkeypatch.setenv("FA_PAGED_BALANCED", "0")
    # equal splits: the paged decode workload: 256 (b, g) pairs x 3 splits, like the
    # contiguous decode; partials [splits][B][Hq][Sq][D+1] fp32
    p = b.fa_plan_paged(32, 32, 8, 1, 128, 16384, 16, 512, 0)
    assert p["path"] == 2 and p["num_splits"] == 3 and p["grid"] == 32 * 8 * 3
    assert p["workspace_bytes"] == 3 * 32 * 32 * 129 * 4
    # capacity 16384 keys in 16-key pages: one split may span at most 256
    # pages, so at least 5 splits (3277 -> 3296 keys = 206 + 1 pages)
    p = b.fa_plan_paged(32, 32, 8, 1, 128, 32768, 16, 1024, 0)
    assert p["num_splits"] == 5
    assert b.fa_plan_paged(1, 8, 2, 1, 128, 1024, 16, 256, 1)["num_splits"] == 2
    # bigger pages lift the bound; forced counts are honoured
    assert b.fa_plan_paged(1, 8, 2, 1, 128, 1024, 256, 64, 1)["num_splits"] == 1
    assert b.fa_plan_paged(1, 8, 2, 1, 128, 1024, 256, 64, 7)["num_splits"] == 7
    assert b.fa_plan_paged(1, 8, 2, 1, 128, 1024, 16, 2, 64)["num_splits"] == 1


def test_workspace_size_matches_the_plan_before_any_call(b):
    # a pure size query (no call made yet in this process on a device) plans
    # for the same compute-unit count as the call itself, so the two agree
    for shape in ((32, 32, 8, 1, 8192, 128, 0), (2, 8, 2, 1, 3000, 128, 6), (4, 16, 4, 2, 700, 64, 0)):
        B, Hq, Hkv, Sq, Sk, D, ns = shape
        plan = b.fa_plan(B, Hq, Hkv, Sq, Sk, D, 0, ns)
        assert b.fa_workspace_size(B, Hq, Hkv, Sq, Sk, D, ns) == plan["workspace_bytes"] > 0


def range_count(lens, Hkv, slots, range_cap, len_min, len_max, cap):
    """The length-balanced ranges for these lengths, by the rule the paged
    kernels apply on the device, restated as a linear search: L is the
    shortest multiple of 32 in [len_min, len_max] whose range count fits
    slots / Hkv, else len_max.  Returns (L, count)."""
    lens = [min(max(x, 0), cap) for x in lens]
    count = lambda L: sum(-(-x // L) for x in lens)  # noqa: E731
    for L in range(len_min, len_max + 1, 32):
        if count(L) <= max(1, slots // Hkv):
            return L, count(L)
    return len_max, count(len_max)


def test_balanced_paged_plan_host_arithmetic(b):
    # automatic cut: length-balanced ranges; 768 resident slots (3 decode
    # waves per CU x 256 CUs), ranges of at most 254 16-key pages (4064 keys)
    # and at least 128 keys; range_cap = max(slots / Hkv, B * ceil(cap / 4064))
    p = b.fa_plan_paged(32, 32, 8, 1, 128, 16384, 16, 512, 0)       # capacity 8192
    assert p["path"] == 2 and p["num_splits"] == 0
    assert p["grid"] == p["work_items"] == 96 * 8
    assert p["workspace_bytes"] == 96 * 32 * 1 * 129 * 4 + 2 * 32 * 4
    p = b.fa_plan_paged(32, 32, 8, 1, 128, 16384, 16, 1024, 0)      # capacity 16384
    assert p["grid"] == 160 * 8
    p = b.fa_plan_paged(32, 32, 8, 1, 256, 16384, 16, 512, 0)       # D = 256: 512 slots
    assert p["grid"] == 96 * 8
    # a forced split count keeps the equal splits, and so do more than 256
    # sequences (the kernels keep the lengths in four registers of 64 lanes)
    assert b.fa_plan_paged(32, 32, 8, 1, 128, 16384, 16, 512, 3)["num_splits"] == 3
    assert b.fa_plan_paged(257, 32, 8, 1, 128, 16384, 16, 512, 0)["num_splits"] >= 1


@pytest.mark.parametrize("B,Hkv,ps,max_pages", [(32, 8, 16, 512), (32, 8, 16, 1024), (3, 2, 16, 20),
                                                (7, 1, 256, 64), (256, 8, 16, 4096), (1, 8, 64, 4)])
def test_balanced_ranges_never_exceed_the_capacity(b, B, Hkv, ps, max_pages):
    # for any lengths the range count stays within range_cap (grid and
    # workspace), every range spans at most 256 pages, and the lengths of
    # the bench's two paged workloads give one range per resident slot or so
    import random
    p = b.fa_plan_paged(B, 8 * Hkv, Hkv, 1, 128, 1 << 16, ps, max_pages, 0)
    cap, slots = max_pages * ps, 768
    range_cap = p["grid"] // Hkv
    len_min, len_max = 128, max(128, (255 * ps) // 32 * 32)
    assert (len_max + ps - 1) // ps + 1 <= 256
    rng = random.Random(B * 131 + max_pages)
    draws = [[cap] * B, [0] * B, [1] * B, [cap] + [0] * (B - 1), [cap - 1] * B]
    draws += [[rng.randint(0, cap) for _ in range(B)] for _ in range(50)]
    for lens in draws:
        L, n = range_count(lens, Hkv, slots, range_cap, len_min, len_max, cap)
        assert n <= range_cap, (lens[:4], L, n, range_cap)
        assert len_min <= L <= len_max and L % 32 == 0
    if (B, Hkv, ps, max_pages) == (32, 8, 16, 512):
        L, n = range_count([8192] * 32, Hkv, slots, range_cap, len_min, len_max, cap)
        assert (L, n * Hkv) == (2752, 768)          # the equal-length workload: one round
