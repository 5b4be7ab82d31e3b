"""The allocation-free entry point fa_fwd_noalloc, through the C ABI: on the
split-key path its output equals fa_fwd_ex's bit for bit (the same kernels,
the partials in the library's static device array instead of a workspace),
and both match the oracle.  Two calls in a row, the second with a smaller
problem, so that the second reuses the array the first left filled."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from attention_fwd_02_amd.inputs import random_qkv
from tests.helpers import check, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from attention_fwd_02_amd import _binding
    return _binding


@pytest.fixture(scope="module")
def oracle():
    import oracle as o
    o._load()
    return o


def outputs(q, out):
    B, Sq, Hq, D = q.shape
    o = torch.empty((B, Sq, Hq, D), dtype=torch.float32 if out == "f32" else torch.bfloat16,
                    device=DEV)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    return o, lse


# B, Hq, Hkv, Sq, Sk, D, causal, num_splits, out
CASES = [
    (32, 32, 8, 1, 8192, 128, False, 0, "bf16"),   # the decode workload's shape: 3 splits
    (4, 8, 2, 2, 3000, 64, True, 7, "f32"),       # smaller, more splits, causal offset
]


def test_noalloc_matches_fa_fwd_ex_on_two_calls(ops, oracle):
    for B, Hq, Hkv, Sq, Sk, D, causal, ns, out in CASES:
        q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, seed=B + Sk)
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
        scale = 1.0 / math.sqrt(D)
        o1, l1 = outputs(q, out)
        o2, l2 = outputs(q, out)
        ops.fa_fwd_noalloc(qd, kd, vd, o1, l1, causal, scale, num_splits=ns)
        ops.fa_fwd_ex(qd, kd, vd, o2, l2, causal, scale, num_splits=ns)
        torch.cuda.synchronize()
        plan = ops.fa_plan(B, Hq, Hkv, Sq, Sk, D, causal, ns)
        assert plan["path"] == 1 and plan["workspace_bytes"] > 0
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        o_ref, l_ref = oracle.attn_fwd(q, k, v, causal, scale)
        check(to64(o1), to64(l1), o_ref, l_ref, out, f"noalloc {B, Hq, Hkv, Sq, Sk, D}")


def test_noalloc_prefill_and_limits(ops, oracle):
    # the prefill path uses no scratch at all
    q, k, v = random_qkv(1, 4, 2, 300, 300, 128, seed=3)
    o, lse = outputs(q, "bf16")
    ops.fa_fwd_noalloc(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, True, 0.088)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_fwd(q, k, v, True, 0.088)
    check(to64(o), to64(lse), o_ref, l_ref, "bf16", "noalloc prefill")
    # a split plan beyond the 16 MiB array is refused before any launch (the
    # sizes are checked on the host: the fake, never dereferenced pointers
    # are not touched)
    B, Hq, Hkv, Sq, Sk, D = 64, 64, 16, 1, 65536, 128
    need = ops.fa_workspace_size(B, Hq, Hkv, Sq, Sk, D, 64)
    assert need > (16 << 20)
    P = 0x10000
    st = ops.lib.fa_fwd_noalloc(P, P, P, P, None, B, Hq, Hkv, Sq, Sk, D, 0, 0.1, None,
                                ops.FA_DTYPE_BF16, 64)
    assert st == ops.FA_ERR_UNSUPPORTED and "static" in ops.fa_last_error()
