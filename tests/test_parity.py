"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small and ragged shapes are compared element by element on every output;
the five full-size workloads run in the launch configuration the benchmark
times and are compared on every row (the long GQA workload: every row of two
heads and every 64th row of the others).
Tolerances and the -inf rule are in tests/helpers.py.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest
import torch

from attention_fwd_02_amd.inputs import HEADDIM_WORKLOADS, WORKLOADS, make_inputs, random_qkv
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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(ops, q, k, v, causal, scale, out="bf16", num_splits=0, with_lse=True, stream=None,
            workspace=None):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    B, Sq, Hq, D = q.shape
    o = torch.empty((B, Sq, Hq, D), dtype=torch.float32 if out == "f32" else torch.bfloat16,
                    device=DEV)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV) if with_lse else None
    ops.fa_fwd_ex(qd, kd, vd, o, lse, causal, scale, stream=stream, num_splits=num_splits,
                  workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


def full_check(ops, oracle, q, k, v, causal, scale, out="bf16", num_splits=0, label=""):
    o, lse = run_gpu(ops, q, k, v, causal, scale, out=out, num_splits=num_splits)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale)
    return check(to64(o), to64(lse), o_ref, lse_ref, out, label)


# ---------------------------------------------------------------------------
# element-by-element on small, ragged and edge shapes
# ---------------------------------------------------------------------------
SHAPES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, out
    (1, 1, 1, 128, 128, 64, False, "f32"),
    (1, 1, 1, 128, 128, 64, True, "bf16"),
    (2, 3, 3, 77, 77, 64, True, "bf16"),          # one ragged block
    (1, 2, 1, 200, 333, 128, False, "bf16"),      # ragged Sq and Sk, MQA
    (1, 2, 1, 200, 333, 128, True, "f32"),        # causal with Sk > Sq
    (1, 2, 2, 300, 100, 64, True, "bf16"),        # Sq > Sk: leading rows see no key
    (1, 8, 2, 129, 257, 128, False, "bf16"),      # GQA, one row past a block
    (2, 4, 4, 513, 513, 128, True, "bf16"),       # several blocks + tail
    (1, 2, 2, 640, 640, 64, True, "f32"),         # several tiles of 128 keys
    (1, 64, 1, 1, 300, 128, False, "bf16"),       # Sq = 1 but 64 rows per KV head: prefill path
    (1, 1, 1, 1, 1, 64, False, "bf16"),           # one query, one key
    (1, 1, 1, 5, 1, 128, True, "f32"),            # one key, causal: only the last row sees it
    # head dim 256: 4 waves x 32 rows, 32-key tiles
    (1, 2, 2, 128, 128, 256, False, "f32"),
    (2, 4, 2, 200, 333, 256, True, "bf16"),       # ragged, GQA, causal with Sk > Sq
    (1, 2, 2, 300, 100, 256, True, "f32"),        # Sq > Sk: leading rows see no key
    (1, 2, 1, 513, 513, 256, True, "bf16"),       # several items + tail
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_shapes_elementwise(ops, oracle, shape):
    B, Hq, Hkv, Sq, Sk, D, causal, out = shape
    say(f"[parity] shape {shape}")
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, seed=Sq * 31 + Sk + D)
    full_check(ops, oracle, q, k, v, causal, 1.0 / math.sqrt(D), out=out, label=str(shape))


# The other compiled prefill configurations, forced through the planner's
# override variables: 64 rows per wave (one wave per SIMD, software-pipelined
# block loop), 32-key tiles with 8 waves, 64-key tiles with 4 waves; and the
# pipelined kernel forced at D = 128 on shapes the planner would give others.
CONFIGS = {
    "rows64_bn64_w4": {"FA_PREFILL_BN": "64", "FA_PREFILL_NW": "4", "FA_PREFILL_NR": "2"},
    "bn32_w8": {"FA_PREFILL_BN": "32", "FA_PREFILL_NW": "8", "FA_PREFILL_NR": "1"},
    "bn64_w4": {"FA_PREFILL_BN": "64", "FA_PREFILL_NW": "4", "FA_PREFILL_NR": "1"},
    "bn32_w2": {"FA_PREFILL_BN": "32", "FA_PREFILL_NW": "2", "FA_PREFILL_NR": "1"},
    # the pipelined 32-key kernel (the default at D = 128 when 256-row items
    # cover the CUs) on every shape
    "pipe_forced": {"FA_PREFILL_PIPE": "2"},
    # ping-pong kernel (8 waves, alternating MFMA and softmax phases), 4- and 5-tile rings
    "pingpong_ring4": {"FA_PREFILL_PP": "4"},
    "pingpong_ring5": {"FA_PREFILL_PP": "5"},
}
CONFIG_SHAPES = [
    (1, 1, 1, 128, 128, 64, True, "bf16"),
    (1, 1, 1, 64, 64, 128, True, "f32"),          # one diagonal tile: every row's LSE
    (2, 3, 3, 77, 77, 64, True, "bf16"),
    (1, 2, 1, 200, 333, 128, True, "f32"),
    (1, 2, 2, 300, 100, 64, True, "bf16"),
    (1, 8, 2, 129, 257, 128, False, "bf16"),
    (2, 4, 4, 513, 513, 128, True, "bf16"),
    (1, 2, 2, 1200, 1200, 128, False, "f32"),     # tiles of the fast body
    (1, 2, 2, 1100, 1300, 128, True, "bf16"),     # fast tiles, diagonal and tail
    (1, 1, 1, 5, 1, 128, True, "f32"),
]


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


@pytest.mark.parametrize("shape", CONFIG_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("cfg", list(CONFIGS))
def test_prefill_configs_elementwise(ops, oracle, env_vars, cfg, shape):
    B, Hq, Hkv, Sq, Sk, D, causal, out = shape
    env_vars(CONFIGS[cfg])
    say(f"[parity] config {cfg} shape {shape}")
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, seed=Sq * 17 + Sk + D)
    full_check(ops, oracle, q, k, v, causal, 1.0 / math.sqrt(D), out=out,
               label=f"{cfg} {shape}")


@pytest.mark.parametrize("scale", [-0.3, 2.5])
def test_rows64_config_scales_and_overflow_redo(ops, oracle, env_vars, scale):
    # large |scale| and hot rows make P pass the block-sum bound, which redoes
    # the block against its exact row max
    env_vars(CONFIGS["rows64_bn64_w4"])
    q, k, v = random_qkv(1, 4, 2, 700, 900, 128, seed=29)
    q[:, ::7] *= 8.0
    full_check(ops, oracle, q, k, v, True, scale, out="f32", label=f"rows64 scale={scale}")


def test_rows64_overflow_redo_in_diagonal_tile(ops, oracle, env_vars):
    # keys from 512 on are 6x larger: the rows 512..575 first meet them in
    # their diagonal tile (keys 512..575), so that tile's masked fast body
    # redoes its blocks, and the keys it masks are the largest ones
    env_vars(CONFIGS["rows64_bn64_w4"])
    q, k, v = random_qkv(1, 2, 1, 640, 640, 128, seed=31)
    k[:, 512:] *= 6.0
    full_check(ops, oracle, q, k, v, True, 0.5, out="f32", label="redo in the diagonal tile")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
def test_d256_scales_and_overflow_redo(ops, oracle, scale):
    # head dim 256 (the pipelined 32-row kernel): hot rows and a large |scale|
    # make P pass the block-sum bound, which redoes the block against its
    # exact row max; scale 0 runs as a zero Q with c = 1
    q, k, v = random_qkv(1, 4, 2, 700, 900, 256, seed=37)
    q[:, ::7] *= 8.0
    full_check(ops, oracle, q, k, v, True, scale, out="f32", label=f"d256 scale={scale}")


def test_d256_overflow_redo_in_diagonal_block(ops, oracle):
    # keys from 512 on are 6x larger: rows 512.. first meet them in their
    # diagonal block, which is masked and redone
    q, k, v = random_qkv(1, 2, 1, 640, 640, 256, seed=41)
    k[:, 512:] *= 6.0
    full_check(ops, oracle, q, k, v, True, 0.5, out="f32", label="d256 redo in the diagonal block")


def test_item_order_does_not_change_results(ops, env_vars):
    # head-major and rank-major walks run the same per-item arithmetic
    q, k, v = random_qkv(2, 8, 8, 1000, 1000, 128, seed=30)
    outs = []
    for hm in ("0", "1"):
        env_vars({"FA_HEAD_MAJOR": hm})
        outs.append(run_gpu(ops, q, k, v, True, 0.088))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


DECODE_SHAPES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, num_splits
    (2, 8, 2, 1, 1000, 128, False, 0),
    (2, 8, 2, 1, 1000, 128, False, 1),
    (2, 8, 2, 1, 1000, 128, False, 7),
    (1, 4, 1, 1, 8192, 64, False, 0),
    (3, 8, 2, 3, 517, 128, True, 0),      # 12 (row, head) columns, causal decode
    (1, 32, 4, 4, 300, 128, True, 5),     # 32 columns: the largest the split path serves
    (2, 1, 1, 1, 33, 64, False, 2),       # last split holds one key
    (1, 2, 2, 7, 5, 64, True, 2),         # Sq > Sk on the split path: empty rows
    (2, 8, 2, 1, 1000, 256, False, 0),    # head dim 256: one tile per trip
    (1, 32, 4, 4, 300, 256, True, 5),
    (2, 4, 4, 1, 65, 256, False, 3),
]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_shapes_elementwise(ops, oracle, shape):
    B, Hq, Hkv, Sq, Sk, D, causal, ns = shape
    say(f"[parity] decode shape {shape}")
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, seed=Sk + 7 * Sq)
    plan = ops.fa_plan(B, Hq, Hkv, Sq, Sk, D, causal, ns)
    assert plan["path"] == 1
    full_check(ops, oracle, q, k, v, causal, 1.0 / math.sqrt(D), num_splits=ns, label=str(shape))


@pytest.mark.parametrize("scale", [-0.125, 0.0, 2.5])
@pytest.mark.parametrize("causal", [False, True])
def test_scale_sign_and_zero(ops, oracle, scale, causal):
    say(f"[parity] scale {scale} causal {causal}")
    q, k, v = random_qkv(1, 2, 2, 150, 150, 64, seed=21)
    full_check(ops, oracle, q, k, v, causal, scale, out="f32", label=f"scale={scale}")
    qd, kd, vd = random_qkv(2, 8, 2, 1, 700, 128, seed=22)
    full_check(ops, oracle, qd, kd, vd, causal, scale, out="f32", label=f"decode scale={scale}")


def test_lse_optional(ops, oracle):
    q, k, v = random_qkv(1, 2, 2, 100, 100, 128, seed=23)
    o, lse = run_gpu(ops, q, k, v, True, 0.088, with_lse=False)
    o_ref, _ = oracle.attn_fwd(q, k, v, True, 0.088)
    check(to64(o), None, o_ref, None, "bf16", "no lse")
    o, lse = run_gpu(ops, *random_qkv(2, 4, 1, 1, 900, 64, seed=24), False, 0.125,
                     with_lse=False, num_splits=3)
    assert lse is None


def split_rounding_bound(q, k, v, scale, o_ref):
    """Per-(row, dim) bound on how far one split count's O may sit from the
    exact O.  Each split rounds P_j = exp2(c s_j - c m_s) to bf16 against its
    own reference max, a relative error |delta_j| <= 2^-9 (round to nearest
    even, 8 significant bits), and O is normalised by the sum of the same
    rounded values, so O - O_exact = sum_j w_j delta_j (v_j - O_exact) /
    (1 + sum_j w_j delta_j) with w the exact softmax weights:
    |dO_d| <= 2^-9 sum_j w_j |v_jd - O_d| / (1 - 2^-9).  The LSE comes from the
    unrounded fp32 sums: only fp32 and the merge's exp/log move it."""
    qf = q.float().numpy().astype(np.float64)
    kf = k.float().numpy().astype(np.float64)
    vf = v.float().numpy().astype(np.float64)
    B, Sq, Hq, D = qf.shape
    group = Hq // kf.shape[2]
    tol = np.zeros((B, Sq, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Sq):
                s = (kf[b, :, g, :] @ qf[b, i, h, :]) * scale
                w = np.exp(s - s.max())
                w /= w.sum()
                dev = np.abs(vf[b, :, g, :] - o_ref[b, i, h][None, :])
                tol[b, i, h] = 2.0 ** -9 * (w[:, None] * dev).sum(0) / (1 - 2.0 ** -9)
    return tol


def test_split_invariance(ops, oracle):
    # Splitting the keys changes only rounding: every split count's O lies
    # within split_rounding_bound of the exact O, so two split counts differ
    # by at most twice that (plus 1e-5 for fp32 accumulation and the merge).
    # The LSE uses the exact fp32 row sums: 2e-5 covers fp32 and __expf/__logf.
    q, k, v = random_qkv(4, 16, 4, 1, 4096, 128, seed=25)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, False, 0.088)
    tol = 2 * split_rounding_bound(q, k, v, 0.088, o_ref) + 1e-5
    outs = []
    for ns in (1, 2, 4, 8, 16, 32):
        o, lse = run_gpu(ops, q, k, v, False, 0.088, out="f32", num_splits=ns)
        outs.append((ns, to64(o), to64(lse)))
    for ns, o, lse in outs[1:]:
        err = np.abs(o - outs[0][1])
        assert (err <= tol).all(), (ns, float((err / tol).max()))
        assert np.abs(lse - outs[0][2]).max() <= 2e-5, ns
        say(f"[parity] splits {ns}: max |dO| / bound = {(err / tol).max():.3f}, "
            f"max |dLSE| = {np.abs(lse - outs[0][2]).max():.2e}")


def test_repeat_launches_bitwise_equal(ops):
    for shape, ns in (((2, 8, 8, 300, 300, 128), 0), ((8, 32, 8, 1, 2048, 128), 0)):
        q, k, v = random_qkv(*shape, seed=26)
        causal = shape[3] > 1
        o1, l1 = run_gpu(ops, q, k, v, causal, 0.1, num_splits=ns)
        o2, l2 = run_gpu(ops, q, k, v, causal, 0.1, num_splits=ns)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_caller_workspace_and_stream(ops):
    q, k, v = random_qkv(2, 8, 2, 1, 3000, 128, seed=27)
    ref_o, ref_l = run_gpu(ops, q, k, v, False, 0.088, num_splits=6)
    nbytes = ops.fa_workspace_size(2, 8, 2, 1, 3000, 128, 6)
    assert nbytes > 0
    ws = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, l = run_gpu(ops, q, k, v, False, 0.088, num_splits=6, stream=s, workspace=ws)
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    # a too-small caller workspace is rejected
    small = torch.empty(16, dtype=torch.float32, device=DEV)
    with pytest.raises(ops.FaError) as e:
        run_gpu(ops, q, k, v, False, 0.088, num_splits=6, workspace=small)
    assert e.value.status == ops.FA_ERR_INVALID_ARG


def test_workspace_size_queried_first_in_a_fresh_process():
    # fa_workspace_size as the very first call of a process must already
    # size the workspace for this device's compute units: a caller workspace
    # of exactly that size is then accepted by the call
    code = """
import sys, torch
sys.path.insert(0, %r)
from attention_fwd_02_amd import _binding as fa
n = fa.fa_workspace_size(32, 32, 8, 1, 8192, 128, 0)
q = torch.randn(32, 1, 32, 128, device='cuda').to(torch.bfloat16)
k = torch.randn(32, 8192, 8, 128, device='cuda').to(torch.bfloat16)
o = torch.empty_like(q)
ws = torch.empty(n // 4, dtype=torch.float32, device='cuda')
fa.fa_fwd_ex(q, k, k, o, None, False, 0.088, workspace=ws)
torch.cuda.synchronize()
plan = fa.fa_plan(32, 32, 8, 1, 8192, 128, 0, 0)
assert plan['workspace_bytes'] == n, (plan, n)
print('ok', n, plan['num_splits'])
""" % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))),)
    import subprocess
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]


def test_forced_allocation_failure_reports_nomem(ops):
    q, k, v = random_qkv(1, 4, 1, 1, 500, 64, seed=28)
    os.environ["FA_TEST_FAIL_ALLOC"] = "1"
    try:
        with pytest.raises(ops.FaError) as e:
            run_gpu(ops, q, k, v, False, 0.125, num_splits=4)
        assert e.value.status == ops.FA_ERR_NOMEM
    finally:
        del os.environ["FA_TEST_FAIL_ALLOC"]
    run_gpu(ops, q, k, v, False, 0.125, num_splits=4)   # works again


# ---------------------------------------------------------------------------
# the five full-size workloads, in the benchmark's launch configuration
# ---------------------------------------------------------------------------
def sample_rows(w, q, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    edge_i = sorted({0, 1, 31, 32, 63, 64, 127, 128, w.Sq // 2, w.Sq - 2, w.Sq - 1} &
                    set(range(w.Sq)))
    for b in {0, w.B - 1}:
        for h in {0, w.Hq - 1, w.Hq // 2}:
            for i in edge_i:
                rows.add((b, h, i))
    for _ in range(n_random):
        rows.add((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.Sq))))
    if w.hot_row_frac > 0:
        hot = (q.float().abs().amax(dim=-1) > 6.0).nonzero().tolist()   # [b, i, h]
        for b, i, h in hot[:: max(1, len(hot) // 64)][:64]:
            rows.add((b, h, i))
    return np.array(sorted(rows), dtype=np.int64)


def subset_rows(w, q):
    """Rows of a full-size workload compared with the oracle: every row when
    the oracle finishes them in seconds (up to about 4e11 flops), else every
    row of the first and last head plus every 64th row of the others, plus
    the edge, random and hot rows of sample_rows."""
    if w.flops() <= 4e11:
        return None   # every row
    rows = {tuple(r) for r in sample_rows(w, q, 160, seed=w.seed)}
    for b in range(w.B):
        for h in range(w.Hq):
            step = 1 if h in (0, w.Hq - 1) else 64
            for i in range(0, w.Sq, step):
                rows.add((b, h, i))
    return np.array(sorted(rows), dtype=np.int64)


def compare_rows(o, lse, o_ref, lse_ref, rows, out_dtype, label):
    og, lg = to64(o), to64(lse)
    if rows is None:
        return check(og, lg, o_ref, lse_ref, out_dtype, label)
    o_s = og[rows[:, 0], rows[:, 2], rows[:, 1]]
    l_s = lg[rows[:, 0], rows[:, 1], rows[:, 2]]
    return check(o_s, l_s, o_ref, lse_ref, out_dtype, label)


@pytest.mark.parametrize("name", list(WORKLOADS) + list(HEADDIM_WORKLOADS))
def test_full_size_workloads(ops, oracle, name):
    w = WORKLOADS[name] if name in WORKLOADS else HEADDIM_WORKLOADS[name]
    say(f"[parity] full-size workload {name}")
    q, k, v = make_inputs(w)
    o, lse = run_gpu(ops, q, k, v, w.causal, w.scale, out=w.o_dtype)
    rows = subset_rows(w, q)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.causal, w.scale, rows=rows)
    eo, el = compare_rows(o, lse, o_ref, lse_ref, rows, w.o_dtype, name)
    n = w.B * w.Hq * w.Sq if rows is None else len(rows)
    say(f"[parity] {name}: {n} rows, max|dO|={eo:.2e} max|dLSE|={el:.2e}")
    assert np.isfinite(to64(lse)).all() or w.causal  # no -inf rows in these workloads
    assert not torch.isnan(o).any()


@pytest.mark.parametrize("name", ["causal_b4_h16_s4096_d128", "gqa_b1_hq32_hkv8_s16384_d128"])
def test_full_size_rows64_config_sampled(ops, oracle, env_vars, name):
    # the 64-rows-per-wave kernel at full size, on sampled rows
    env_vars(CONFIGS["rows64_bn64_w4"])
    w = WORKLOADS[name]
    say(f"[parity] full-size workload {name}, 64 rows per wave")
    q, k, v = make_inputs(w)
    o, lse = run_gpu(ops, q, k, v, w.causal, w.scale, out=w.o_dtype)
    rows = sample_rows(w, q, 96, seed=w.seed + 1)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.causal, w.scale, rows=rows)
    og, lg = to64(o), to64(lse)
    o_s = np.stack([og[b, i, h] for b, h, i in rows])
    l_s = np.array([lg[b, h, i] for b, h, i in rows])
    check(o_s, l_s, o_ref, lse_ref, w.o_dtype, name + " rows64")


@pytest.mark.parametrize("ring", ["4", "5"])
def test_full_size_pingpong_every_row(ops, oracle, env_vars, ring):
    # the ping-pong kernel on every row of the causal S=4096 workload, fp32 O
    # at the plain 1e-2 bound: several items per workgroup, every ring stage
    # reused many times, hot rows
    env_vars({"FA_PREFILL_PP": ring})
    w = WORKLOADS["causal_b4_h16_s4096_d128"]
    q, k, v = make_inputs(w)
    o, lse = run_gpu(ops, q, k, v, w.causal, w.scale, out="f32")
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.causal, w.scale)
    eo, el = check(to64(o), to64(lse), o_ref, lse_ref, "f32", f"ping-pong ring {ring}")
    say(f"[parity] ping-pong ring {ring}, all rows: max|dO|={eo:.2e} max|dLSE|={el:.2e}")


def test_compute_bound_workload_float32_output_strict(ops, oracle):
    # float32 O on every row of the causal S=4096 workload: the plain 1e-2
    # bound, with no allowance for the output format's rounding
    w = WORKLOADS["causal_b4_h16_s4096_d128"]
    q, k, v = make_inputs(w)
    o, lse = run_gpu(ops, q, k, v, w.causal, w.scale, out="f32")
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.causal, w.scale)
    eo, el = check(to64(o), to64(lse), o_ref, lse_ref, "f32", "f32 output, every row")
    say(f"[parity] causal S=4096 fp32 O, all {w.B * w.Hq * w.Sq} rows: "
        f"max|dO|={eo:.2e} max|dLSE|={el:.2e}")
