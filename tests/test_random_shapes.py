"""Seeded random shapes against the oracle, element by element.

The hand-picked shapes of test_parity.py and test_paged.py aim at known
edges; these draw the shape, head grouping, head dim, causality, scale,
output type, split count and prefill configuration at random (fixed seeds,
so a failure names a reproducible case) to catch combinations nobody listed.
Sizes stay small enough for the fp64 oracle to finish in well under a
second each.  Tolerances are those of tests/helpers.py.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest
import torch

from attention_fwd_02_amd.inputs import PagedWorkload, make_paged_inputs, random_qkv
from tests.helpers import check, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CONFIG_VARS = ("FA_PREFILL_BN", "FA_PREFILL_NW", "FA_PREFILL_NR")
# even seeds without a forced configuration force the pipelined kernel at
# D = 128 (the planner gives small shapes to the others)
PIPE_VAR = "FA_PREFILL_PIPE"
CONFIGS = [None, ("64", "4", "2"), ("32", "8", "1"), ("64", "4", "1")]


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


@pytest.fixture
def clean_env():
    saved = {k: os.environ.get(k) for k in CONFIG_VARS + (PIPE_VAR,)}
    yield
    for k, val in saved.items():
        if val is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = val


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dense_case(seed):
    r = np.random.default_rng(1000 + seed)
    D = int(r.choice([64, 128, 256]))
    Hkv = int(r.choice([1, 2, 4]))
    group = int(r.choice([1, 2, 3, 4, 8]))
    B = int(r.integers(1, 4))
    Sq = int(r.integers(1, 5)) if r.random() < 0.3 else int(r.integers(1, 700))
    Sk = int(r.integers(1, 1500))
    causal = bool(r.random() < 0.5)
    out = "f32" if r.random() < 0.3 else "bf16"
    scale = float(r.choice([1.0 / math.sqrt(D), -0.2, 0.7, 0.0]))
    # keep the fp64 oracle fast
    while B * Hkv * group * Sq * Sk * D > 6e8 and Sk > 1:
        Sk = max(1, Sk // 2)
        Sq = max(1, Sq // 2)
    split_ok = Sq * group <= 32
    ns = int(r.choice([0, 0, 1, 3, 7])) if split_ok else 0
    cfg = CONFIGS[int(r.integers(len(CONFIGS)))]
    return dict(B=B, Hq=Hkv * group, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, causal=causal, out=out,
                scale=scale, ns=ns, cfg=cfg)


def paged_case(seed):
    r = np.random.default_rng(2000 + seed)
    D = int(r.choice([64, 128, 256]))
    Hkv = int(r.choice([1, 2, 4]))
    group = int(r.choice([1, 2, 4, 8]))
    Sq = int(r.integers(1, 5))
    while Sq * group > 32:
        Sq -= 1
    B = int(r.integers(1, 5))
    ps = int(r.choice([16, 32, 64, 128, 256]))
    max_len = int(r.integers(1, 2000))
    lens = [int(r.integers(0, max_len + 1)) for _ in range(B)]
    causal = bool(r.random() < 0.5)
    out = "f32" if r.random() < 0.3 else "bf16"
    ns = int(r.choice([0, 0, 1, 2, 5]))
    return dict(B=B, Hq=Hkv * group, Hkv=Hkv, Sq=Sq, D=D, ps=ps, max_len=max_len, lens=lens,
                causal=causal, out=out, ns=ns)


@pytest.mark.parametrize("seed", range(60))
def test_random_dense(ops, oracle, clean_env, seed):
    c = dense_case(seed)
    say(f"[random] dense seed {seed}: {c}")
    for k in CONFIG_VARS + (PIPE_VAR,):
        os.environ.pop(k, None)
    if c["cfg"] is not None:
        for k, val in zip(CONFIG_VARS, c["cfg"]):
            os.environ[k] = val
    elif seed % 2 == 0:
        os.environ[PIPE_VAR] = "2"
    q, k, v = random_qkv(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sk"], c["D"], seed=seed)
    o = torch.empty((c["B"], c["Sq"], c["Hq"], c["D"]),
                    dtype=torch.float32 if c["out"] == "f32" else torch.bfloat16, device=DEV)
    lse = torch.empty((c["B"], c["Hq"], c["Sq"]), dtype=torch.float32, device=DEV)
    ops.fa_fwd_ex(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, c["causal"], c["scale"],
                  num_splits=c["ns"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, c["causal"], c["scale"])
    check(to64(o), to64(lse), o_ref, lse_ref, c["out"], f"dense seed {seed}")


@pytest.mark.parametrize("seed", range(40))
def test_random_paged(ops, oracle, seed):
    c = paged_case(seed)
    say(f"[random] paged seed {seed}: {c}")
    w = PagedWorkload(name="random", B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], Sq=c["Sq"],
                      max_len=c["max_len"], page_size=c["ps"], D=c["D"], causal=c["causal"],
                      o_dtype=c["out"], seed=seed)
    q, kc, vc, table, lens = make_paged_inputs(w, lens=c["lens"])
    o = torch.empty((c["B"], c["Sq"], c["Hq"], c["D"]),
                    dtype=torch.float32 if c["out"] == "f32" else torch.bfloat16, device=DEV)
    lse = torch.empty((c["B"], c["Hq"], c["Sq"]), dtype=torch.float32, device=DEV)
    ops.fa_fwd_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV), lens.to(DEV), o, lse,
                     c["causal"], w.scale, num_splits=c["ns"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd_paged(q, kc, vc, table, lens, c["causal"], w.scale)
    check(to64(o), to64(lse), o_ref, lse_ref, c["out"], f"paged seed {seed}")
