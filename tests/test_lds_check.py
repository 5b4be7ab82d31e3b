"""The LDS-ring race checks: debug builds of the same sources compared bit for
bit with the product library on shapes that cover every kernel with a ring.

libfa_check_sync.so waits for every HBM -> LDS copy right after issuing it, so
each ring stage is ready long before the product build's own wait and barrier
make it so; libfa_check_poison.so writes NaN into each copy's destination just
before the copy.  A stage read before its copy has landed, or overwritten
while a wave still reads it ("理解 H100：从硬件数据路径到 Nsight Compute 瓶颈分析",
section 6: ready before read, reusable before overwrite), would change the
result of one build and not the other.  Every kernel here is deterministic (no
atomics, fixed reduction order), so any difference in any bit fails.
"""
from __future__ import annotations

import math
import os

import pytest
import torch

from attention_fwd_02_amd import _binding as fa
from attention_fwd_02_amd import build as fa_build
from attention_fwd_02_amd.inputs import PagedWorkload, make_paged_inputs, random_fp8, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dense(B, Hq, Hkv, Sq, Sk, D, causal, o_f32=False, splits=0, seed=5):
    q, k, v = (t.to(DEV) for t in random_qkv(B, Hq, Hkv, Sq, Sk, D, seed=seed))
    scale = 1.0 / math.sqrt(D)

    def run():
        o = torch.full((B, Sq, Hq, D), float("nan"), device=DEV,
                       dtype=torch.float32 if o_f32 else torch.bfloat16)
        lse = torch.full((B, Hq, Sq), float("nan"), device=DEV)
        fa.fa_fwd_ex(q, k, v, o, lse, causal, scale, num_splits=splits)
        torch.cuda.synchronize()
        return [o, lse]
    return run


def _paged():
    w = PagedWorkload("check", B=4, Hq=8, Hkv=2, Sq=1, max_len=1500, page_size=16, D=128)
    q, kc, vc, table, lens = (t.to(DEV) for t in make_paged_inputs(w, lens=[1500, 0, 37, 900]))

    def run():
        o = torch.full((4, 1, 8, 128), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = torch.full((4, 8, 1), float("nan"), device=DEV)
        fa.fa_fwd_paged(q, kc, vc, table, lens, o, lse, False, w.scale)
        torch.cuda.synchronize()
        return [o, lse]
    return run


def _fp8(causal):
    q, k, v, dq, dk, dv = random_fp8(2, 4, 2, 700, 700, 128, seed=21)
    q, k, v = (t.to(DEV) for t in (q, k, v))

    def run():
        o = torch.full((2, 700, 4, 128), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = torch.full((2, 4, 700), float("nan"), device=DEV)
        fa.fa_fwd_fp8(q, k, v, o, lse, causal, 1.0 / math.sqrt(128), dq, dk, dv)
        torch.cuda.synchronize()
        return [o, lse]
    return run


def _bwd():
    B, Hq, Hkv, S, D = 1, 4, 2, 600, 128
    q, k, v = (t.to(DEV) for t in random_qkv(B, Hq, Hkv, S, S, D, seed=23))
    do = torch.randn((B, S, Hq, D), generator=torch.Generator().manual_seed(24)).to(
        torch.bfloat16).to(DEV)
    scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), device=DEV)
    fa.fa_fwd(q, k, v, o, lse, True, scale)
    torch.cuda.synchronize()

    def run():
        dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, True, scale)
        torch.cuda.synchronize()
        return [dq, dk, dv]
    return run


# name -> (planner overrides, inputs + call)
CASES = {
    "prefill_rows32_causal": ({}, lambda: _dense(2, 4, 4, 700, 700, 128, True)),
    "prefill_rows32_d64_gqa": ({}, lambda: _dense(1, 8, 2, 333, 517, 64, False, o_f32=True)),
    "prefill_rows64_causal": ({"FA_PREFILL_BN": "64", "FA_PREFILL_NW": "4", "FA_PREFILL_NR": "2"},
                              lambda: _dense(1, 4, 4, 1100, 1300, 128, True)),
    "prefill_rows64_noncausal": ({"FA_PREFILL_BN": "64", "FA_PREFILL_NW": "4",
                                  "FA_PREFILL_NR": "2"},
                                 lambda: _dense(1, 8, 2, 1200, 1200, 128, False)),
    "prefill_bn32_w8": ({"FA_PREFILL_BN": "32", "FA_PREFILL_NW": "8", "FA_PREFILL_NR": "1"},
                        lambda: _dense(2, 3, 3, 513, 513, 128, True)),
    "prefill_bn32_w2": ({"FA_PREFILL_BN": "32", "FA_PREFILL_NW": "2", "FA_PREFILL_NR": "1"},
                        lambda: _dense(1, 4, 2, 300, 333, 64, True)),
    "prefill_pingpong_ring4": ({"FA_PREFILL_PP": "4"},
                               lambda: _dense(1, 4, 4, 1100, 1300, 128, True)),
    "prefill_pingpong_ring5": ({"FA_PREFILL_PP": "5"},
                               lambda: _dense(1, 8, 2, 1200, 1200, 128, False)),
    "prefill_d256": ({}, lambda: _dense(1, 4, 4, 600, 600, 256, True)),
    # the 8-wave pipelined kernel (six-stage rings, a barrier every second
    # step): forced on a causal ragged shape (waves past their last block,
    # odd and even step counts) and a non-causal GQA one with an odd count,
    # and chosen by the planner at a shape whose 256-row items fill the CUs
    "prefill_pipe8_causal": ({"FA_PREFILL_PIPE": "2"},
                             lambda: _dense(2, 4, 4, 700, 700, 128, True)),
    "prefill_pipe8_gqa": ({"FA_PREFILL_PIPE": "2"},
                          lambda: _dense(1, 8, 2, 1200, 1100, 128, False)),
    "prefill_pipe8_default": ({}, lambda: _dense(4, 16, 16, 1024, 1024, 128, True)),
    "decode_split": ({}, lambda: _dense(4, 8, 2, 1, 3000, 128, False, splits=3)),
    "decode_split_d256": ({}, lambda: _dense(4, 8, 2, 1, 3000, 256, False, splits=2)),
    "decode_paged_ragged": ({}, _paged),
    "fp8_prefill_causal": ({}, lambda: _fp8(True)),
    "fp8_prefill_unpipelined": ({"FA_FP8_PIPE": "0"}, lambda: _fp8(True)),
    "backward": ({}, _bwd),
}


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.fixture
def env_vars():
    saved = {}

    def set_(vars_):
        for k, val in vars_.items():
            saved.setdefault(k, os.environ.get(k))
            os.environ[k] = val

    yield set_
    for k, val in saved.items():
        if val is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = val


@pytest.mark.parametrize("variant", sorted(fa_build.CHECK_VARIANTS))
@pytest.mark.parametrize("case", list(CASES))
def test_race_check_build_is_bitwise_equal(variant, case, env_vars):
    path = fa_build.check_lib_path(variant)
    assert os.path.exists(path), f"{path} is not built"
    env, make = CASES[case]
    env_vars(env)
    print(f"[lds-check] {variant} {case}", flush=True)
    run = make()
    ref = run()
    with fa.using_library(path):
        got = run()
    for i, (a, b) in enumerate(zip(ref, got)):
        nan = int(torch.isnan(b.float()).sum())
        diff = int((_bits(a) != _bits(b)).sum())
        assert diff == 0, (f"{variant} build differs from libfa.so in output {i}: "
                           f"{diff} of {a.numel()} elements ({nan} NaN in the debug build)")
    # the product build's own run is finite where the oracle says so: a second
    # product run must repeat it bit for bit as well
    again = run()
    for a, b in zip(ref, again):
        assert torch.equal(_bits(a), _bits(b))
