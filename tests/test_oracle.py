"""Pins for the fp64 oracle (CPU only).

The oracle is the plain definition softmax(scale * Q K^T [+ causal mask]) V plus
the row log-sum-exp.  Nothing here re-calls the oracle's own code to check it:
each test compares it with something else that fixes the answer --

  * a 40-digit ``decimal`` brute force on tiny inputs;
  * torch's float64 ``softmax`` / ``logsumexp`` (a library evaluation of the
    same definition) on medium shapes;
  * closed forms worked out by hand: one key, two keys, uniform scores,
    causal first row, constant V;
  * invariants: key permutation, GQA == MHA with repeated KV heads, key
    partition + log-sum-exp merge, sign of the scale;
  * layout probes whose answer is known from where each value was placed.

Each is chosen so that a plausible slip (a dropped term, the causal offset on
the wrong side, the GQA head map hq % Hkv instead of hq // group, q and k
swapped, a transposed layout) fails at least one of them.
"""
from __future__ import annotations

import decimal
import math

import numpy as np
import pytest
import torch

from attention_fwd_02_amd.inputs import random_qkv

pytestmark = []


def bf16(x) -> torch.Tensor:
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


# ----------------------------------------------------------------------------
# brute force in 40-digit decimal arithmetic
# ----------------------------------------------------------------------------
def decimal_reference(q, k, v, causal, scale, key_range=None):
    ctx = decimal.Context(prec=40)
    qf = q.float().numpy().astype(np.float64)
    kf = k.float().numpy().astype(np.float64)
    vf = v.float().numpy().astype(np.float64)
    B, Sq, Hq, D = qf.shape
    _, Sk, Hkv, _ = kf.shape
    group = Hq // Hkv
    sc = decimal.Decimal(float(np.float32(scale)))
    lo, hi = (0, Sk) if key_range is None else key_range
    o = np.zeros((B, Sq, Hq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Sq):
                keys = [j for j in range(lo, hi) if (not causal) or j <= i + Sk - Sq]
                if not keys:
                    lse[b, h, i] = -math.inf
                    continue
                s = {}
                for j in keys:
                    acc = decimal.Decimal(0)
                    for d in range(D):
                        acc = ctx.add(acc, ctx.multiply(decimal.Decimal(qf[b, i, h, d]),
                                                        decimal.Decimal(kf[b, j, g, d])))
                    s[j] = ctx.multiply(sc, acc)
                m = max(s.values())
                w = {j: ctx.exp(ctx.subtract(s[j], m)) for j in keys}
                l_sum = decimal.Decimal(0)
                for j in keys:
                    l_sum = ctx.add(l_sum, w[j])
                for d in range(D):
                    acc = decimal.Decimal(0)
                    for j in keys:
                        acc = ctx.add(acc, ctx.multiply(w[j], decimal.Decimal(vf[b, j, g, d])))
                    o[b, i, h, d] = float(ctx.divide(acc, l_sum))
                lse[b, h, i] = float(ctx.add(m, ctx.ln(l_sum)))
    return o, lse


BRUTE_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, scale, key_range
    (1, 1, 1, 4, 4, 4, False, 0.5, None),
    (1, 1, 1, 5, 5, 8, True, 0.35355339, None),
    (2, 4, 2, 3, 7, 4, True, 0.5, None),        # GQA, Sq < Sk causal
    (1, 2, 1, 7, 3, 4, True, 0.5, None),        # Sq > Sk causal: empty rows
    (1, 2, 2, 4, 6, 8, False, -0.7, None),      # negative scale
    (1, 3, 1, 4, 8, 4, False, 0.25, (2, 6)),    # key sub-range, MQA
    (1, 2, 1, 6, 6, 4, True, 0.5, (1, 5)),      # key sub-range with causal
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_oracle_matches_decimal_bruteforce(oracle_mod, case):
    B, Hq, Hkv, Sq, Sk, D, causal, scale, kr = case
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, seed=11 + Sq * 7 + D)
    o, lse = oracle_mod.attn_fwd(q, k, v, causal, scale, key_range=kr)
    o_ref, lse_ref = decimal_reference(q, k, v, causal, scale, key_range=kr)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(lse[~fin] == -np.inf)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# library evaluation of the same definition (torch, float64, CPU)
# ----------------------------------------------------------------------------
def torch_reference(q, k, v, causal, scale):
    qd, kd, vd = (t.double() for t in (q, k, v))
    B, Sq, Hq, D = qd.shape
    Sk, Hkv = kd.shape[1], kd.shape[2]
    kd = kd.repeat_interleave(Hq // Hkv, dim=2)
    vd = vd.repeat_interleave(Hq // Hkv, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", qd, kd) * float(np.float32(scale))
    if causal:
        i = torch.arange(Sq).view(-1, 1)
        j = torch.arange(Sk).view(1, -1)
        s = s.masked_fill(j > i + (Sk - Sq), -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,bjhd->bihd", p, vd)
    return o.numpy(), lse.numpy()


@pytest.mark.parametrize("shape", [
    (1, 2, 2, 128, 128, 64, False),
    (2, 4, 2, 96, 160, 64, True),
    (1, 8, 2, 200, 200, 128, True),
    (1, 4, 1, 1, 300, 128, False),
    (1, 2, 2, 257, 129, 64, False),
])
def test_oracle_matches_torch_float64(oracle_mod, shape):
    B, Hq, Hkv, Sq, Sk, D, causal = shape
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, seed=Sq + Sk)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle_mod.attn_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = torch_reference(q, k, v, causal, scale)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-10)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def test_single_key_gives_that_value_row(oracle_mod):
    # one key: the softmax weight is exactly 1, O = v0, LSE = s0
    q = bf16([[[[1.0, 2.0, 0.0, -1.0]]]])
    k = bf16([[[[0.5, 0.25, 3.0, 2.0]]]])
    v = bf16([[[[7.0, -3.0, 0.125, 1.5]]]])
    o, lse = oracle_mod.attn_fwd(q, k, v, False, 0.5)
    s0 = 0.5 * (0.5 + 0.5 + 0.0 - 2.0)
    assert lse[0, 0, 0] == pytest.approx(s0, abs=1e-15)
    np.testing.assert_array_equal(o[0, 0, 0], [7.0, -3.0, 0.125, 1.5])


def test_two_keys_closed_form(oracle_mod):
    # q = e0, k0 = 2 e0, k1 = -e0, scale 0.5: scores s0 = 1, s1 = -0.5
    q = bf16([[[[1.0, 0.0]]]])
    k = bf16([[[[2.0, 0.0]], [[-1.0, 0.0]]]])
    v = bf16([[[[1.0, 2.0]], [[3.0, -1.0]]]])
    o, lse = oracle_mod.attn_fwd(q, k, v, False, 0.5)
    s0, s1 = 1.0, -0.5
    want_lse = math.log(math.exp(s0) + math.exp(s1))
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))  # logistic of the score gap
    p1 = 1.0 - p0
    assert lse[0, 0, 0] == pytest.approx(want_lse, abs=1e-14)
    np.testing.assert_allclose(o[0, 0, 0], [p0 * 1 + p1 * 3, p0 * 2 - p1 * 1], atol=1e-14)


@pytest.mark.parametrize("Sq,Sk", [(3, 5), (5, 3), (6, 6), (1, 9)])
def test_uniform_scores_lse_is_log_count_and_o_is_prefix_mean(oracle_mod, Sq, Sk):
    # scale = 0 makes every allowed score 0: LSE = ln(#allowed), O = mean of allowed V
    q, k, v = random_qkv(1, 2, 1, Sq, Sk, 8, seed=5)
    o, lse = oracle_mod.attn_fwd(q, k, v, True, 0.0)
    vf = v.double().numpy()
    for h in range(2):
        for i in range(Sq):
            n = min(max(i + Sk - Sq + 1, 0), Sk)
            if n == 0:
                assert lse[0, h, i] == -math.inf
                assert np.all(o[0, i, h] == 0.0)
            else:
                assert lse[0, h, i] == pytest.approx(math.log(n), abs=1e-14)
                np.testing.assert_allclose(o[0, i, h], vf[0, :n, 0].mean(axis=0), atol=1e-14)


def test_zero_q_is_uniform_too(oracle_mod):
    q, k, v = random_qkv(1, 1, 1, 4, 10, 8, seed=9)
    q = torch.zeros_like(q)
    o, lse = oracle_mod.attn_fwd(q, k, v, False, 0.125)
    assert np.allclose(lse, math.log(10), atol=1e-14)
    np.testing.assert_allclose(o[0, :, 0], np.broadcast_to(v.double().numpy()[0, :, 0].mean(0), (4, 8)),
                               atol=1e-14)


def test_causal_first_row_is_v0(oracle_mod):
    q, k, v = random_qkv(2, 4, 2, 16, 16, 64, seed=3)
    scale = 0.125
    o, lse = oracle_mod.attn_fwd(q, k, v, True, scale)
    qd, kd, vd = (t.double().numpy() for t in (q, k, v))
    for b in range(2):
        for h in range(4):
            g = h // 2
            np.testing.assert_array_equal(o[b, 0, h], vd[b, 0, g])
            s00 = float(np.float32(scale)) * float(qd[b, 0, h] @ kd[b, 0, g])
            assert lse[b, h, 0] == pytest.approx(s00, abs=1e-12)


def test_causal_last_row_sees_every_key(oracle_mod):
    q, k, v = random_qkv(1, 2, 2, 24, 24, 64, seed=4)
    oc, lc = oracle_mod.attn_fwd(q, k, v, True, 0.125)
    on, ln_ = oracle_mod.attn_fwd(q, k, v, False, 0.125)
    np.testing.assert_allclose(oc[:, -1], on[:, -1], atol=1e-14)
    np.testing.assert_allclose(lc[:, :, -1], ln_[:, :, -1], atol=1e-14)
    # and an interior row differs (the mask is not a no-op)
    assert not np.allclose(oc[:, 5], on[:, 5])


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_o(oracle_mod, causal):
    q, k, _ = random_qkv(1, 2, 1, 12, 12, 64, seed=6)
    v = torch.full((1, 12, 1, 64), 1.75, dtype=torch.bfloat16)
    o, _ = oracle_mod.attn_fwd(q, k, v, causal, 0.3)
    np.testing.assert_allclose(o, 1.75, atol=1e-14)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def test_key_permutation_invariance(oracle_mod):
    q, k, v = random_qkv(2, 2, 2, 20, 33, 64, seed=7)
    perm = torch.randperm(33, generator=torch.Generator().manual_seed(1))
    o1, l1 = oracle_mod.attn_fwd(q, k, v, False, 0.125)
    o2, l2 = oracle_mod.attn_fwd(q, k[:, perm].contiguous(), v[:, perm].contiguous(), False, 0.125)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads(oracle_mod):
    q, k, v = random_qkv(2, 8, 2, 10, 14, 64, seed=8)
    o1, l1 = oracle_mod.attn_fwd(q, k, v, True, 0.125)
    k4 = k.repeat_interleave(4, dim=2).contiguous()
    v4 = v.repeat_interleave(4, dim=2).contiguous()
    o2, l2 = oracle_mod.attn_fwd(q, k4, v4, True, 0.125)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_negative_scale_equals_negated_query(oracle_mod):
    q, k, v = random_qkv(1, 2, 2, 9, 9, 64, seed=10)
    o1, l1 = oracle_mod.attn_fwd(q, k, v, True, -0.2)
    o2, l2 = oracle_mod.attn_fwd(-q, k, v, True, 0.2)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def lse_merge(parts):
    """Combine per-partition (O_s, LSE_s) into the whole: the merge the split
    decode path performs, written out in float64."""
    lses = np.stack([p[1] for p in parts])            # [S, ...]
    M = np.max(lses, axis=0)
    Msafe = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Msafe), 0.0)
    wsum = w.sum(axis=0)
    lse = np.where(wsum > 0, Msafe + np.log(np.where(wsum > 0, wsum, 1.0)), -np.inf)
    o = sum(wi[..., None] * p[0] for wi, p in zip(w, parts))
    o = np.where(wsum[..., None] > 0, o / np.where(wsum > 0, wsum, 1.0)[..., None], 0.0)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_key_partition_merge_equals_whole(oracle_mod, causal):
    B, Hq, Hkv, Sq, Sk, D = 1, 4, 2, 6, 50, 64
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, seed=12)
    o, lse = oracle_mod.attn_fwd(q, k, v, causal, 0.125)
    rng = np.random.default_rng(0)
    cuts = sorted(rng.choice(np.arange(1, Sk), size=4, replace=False).tolist())
    bounds = [0] + cuts + [Sk]
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        po, pl = oracle_mod.attn_fwd(q, k, v, causal, 0.125, key_range=(a, b))
        # rows are (b, i, h, d) for o and (b, h, i) for lse: bring o to (b, h, i, d)
        parts.append((po.transpose(0, 2, 1, 3), pl))
    mo, ml = lse_merge(parts)
    np.testing.assert_allclose(mo.transpose(0, 2, 1, 3), o, atol=1e-13)
    np.testing.assert_allclose(ml, lse, atol=1e-13)


# ----------------------------------------------------------------------------
# layout probes
# ----------------------------------------------------------------------------
def test_layout_of_v_o_and_lse(oracle_mod):
    # scale 0 and non-causal: O[b,i,hq,:] = mean_j V[b,j,g,:]; V encodes its own position
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 2, 3, 5, 4
    v = torch.zeros((B, Sk, Hkv, D))
    for b in range(B):
        for j in range(Sk):
            for g in range(Hkv):
                for d in range(D):
                    v[b, j, g, d] = 64 * b + 16 * g + d + (j - 2)   # mean over j adds 0
    v = v.to(torch.bfloat16)
    q = torch.zeros((B, Sq, Hq, D), dtype=torch.bfloat16)
    k = torch.zeros((B, Sk, Hkv, D), dtype=torch.bfloat16)
    o, lse = oracle_mod.attn_fwd(q, k, v, False, 0.0)
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                g = h // 2
                np.testing.assert_allclose(o[b, i, h], [64 * b + 16 * g + d for d in range(D)],
                                           atol=1e-12)
    assert np.allclose(lse, math.log(Sk))


def test_layout_of_q_and_k(oracle_mod):
    # one query row (b=1, i=2, hq=3) aligned with one key (b=1, j=4, g=1); all
    # other scores are 0.  With a large scale that row picks V[1,4,1] exactly.
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 2, 3, 6, 8
    q = torch.zeros((B, Sq, Hq, D))
    k = torch.zeros((B, Sk, Hkv, D))
    q[1, 2, 3, 5] = 1.0
    k[1, 4, 1, 5] = 1.0
    v = torch.arange(B * Sk * Hkv * D, dtype=torch.float32).reshape(B, Sk, Hkv, D)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    o, lse = oracle_mod.attn_fwd(q, k, v, False, 200.0)
    vd = v.double().numpy()
    np.testing.assert_allclose(o[1, 2, 3], vd[1, 4, 1], rtol=1e-12)
    assert lse[1, 3, 2] == pytest.approx(200.0, abs=1e-9)
    # the same query slot in other heads / batches sees only zero scores
    assert lse[0, 3, 2] == pytest.approx(math.log(Sk), abs=1e-14)
    assert lse[1, 2, 2] == pytest.approx(math.log(Sk), abs=1e-14)


def test_row_subset_matches_full(oracle_mod):
    q, k, v = random_qkv(2, 4, 2, 33, 40, 64, seed=13)
    o, lse = oracle_mod.attn_fwd(q, k, v, True, 0.125)
    rows = np.array([[0, 0, 0], [1, 3, 32], [0, 2, 17], [1, 1, 5]], dtype=np.int64)
    ro, rl = oracle_mod.attn_fwd(q, k, v, True, 0.125, rows=rows)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(ro[n], o[b, i, h])
        assert rl[n] == lse[b, h, i]


def test_allowed_pairs_count(oracle_mod):
    assert oracle_mod.allowed_pairs(4096, 4096, True) == 4096 * 4097 // 2
    assert oracle_mod.allowed_pairs(3, 5, True) == 3 + 4 + 5
    assert oracle_mod.allowed_pairs(5, 3, True) == 0 + 0 + 1 + 2 + 3
    assert oracle_mod.allowed_pairs(7, 9, False) == 63


# ----------------------------------------------------------------------------
# paged K/V cache: the gather, pinned by where each value was placed
# ----------------------------------------------------------------------------
# 4 pages of 2 slots; the value of every element of page p, slot s is
# 1 + 10 p + s (exact in bf16).  Sequence 0 has 3 keys: page 3 (slots 0, 1),
# then page 1 (slot 0) -> values 31, 32, 11.  Sequence 1 has 1 key: page 0
# slot 0 -> 1.  Sequence 2 has 5 keys: pages 2, 0, 3 -> 21, 22, 1, 2, 31.
PAGED_TABLE = np.array([[3, 1, -1], [0, 2, -1], [2, 0, 3]], dtype=np.int32)
PAGED_LENS = np.array([3, 1, 5], dtype=np.int32)


def paged_ids_cache(Hkv=1, D=4):
    ids = 1.0 + 10.0 * np.arange(4)[:, None] + np.arange(2)[None, :]
    return bf16(np.broadcast_to(ids[:, :, None, None], (4, 2, Hkv, D)).copy())


def test_paged_uniform_scores_average_the_sequences_own_rows(oracle_mod):
    # K = 0: every allowed key scores 0, so O is the mean of the sequence's V
    # rows and LSE = ln(count)
    v = paged_ids_cache()
    k = bf16(np.zeros((4, 2, 1, 4)))
    q = bf16(np.random.default_rng(0).standard_normal((3, 1, 2, 4)))
    o, lse = oracle_mod.attn_fwd_paged(q, k, v, PAGED_TABLE, PAGED_LENS, False, 0.5)
    expect = [74.0 / 3.0, 1.0, 77.0 / 5.0]
    for b in range(3):
        np.testing.assert_allclose(o[b], np.full((1, 2, 4), expect[b]), rtol=1e-13)
        np.testing.assert_allclose(lse[b], np.full((2, 1), math.log(PAGED_LENS[b])),
                                   rtol=0, atol=1e-13)


def test_paged_dominant_key_picks_its_slot(oracle_mod):
    # q = e0; K rows -1 in dim 0 except logical key 2 of sequence 0 (page 1,
    # slot 0) and logical key 3 of sequence 2 (page 0, slot 1), which are +1.
    # With scale 30 the others weigh e^-60: O is that key's V row (11, 2).
    v = paged_ids_cache()
    k = np.zeros((4, 2, 1, 4), dtype=np.float32)
    k[:, :, 0, 0] = -1.0
    k[1, 0, 0, 0] = 1.0
    k[0, 1, 0, 0] = 1.0
    q = np.zeros((3, 1, 1, 4), dtype=np.float32)
    q[:, 0, 0, 0] = 1.0
    lens = np.array([3, 1, 5], dtype=np.int32)
    o, lse = oracle_mod.attn_fwd_paged(bf16(q), bf16(k), v, PAGED_TABLE, lens, False, 30.0)
    assert o[0, 0, 0, 0] == pytest.approx(11.0, abs=1e-20)
    assert o[2, 0, 0, 0] == pytest.approx(2.0, abs=1e-20)
    # sequence 1 (one key, page 0 slot 0 with -1): the single row itself
    assert o[1, 0, 0, 0] == 1.0 and lse[1, 0, 0] == pytest.approx(-30.0, abs=1e-13)
    # sequence 0: one key at +30, two at -30
    assert lse[0, 0, 0] == pytest.approx(30.0 + math.log1p(2 * math.exp(-60.0)), abs=1e-13)


def test_paged_causal_offset_is_per_sequence(oracle_mod):
    # Sq = 2, causal: row i of sequence b sees keys j <= i + len_b - 2.
    # Sequence 2 (5 keys): row 0 -> first 4 keys (21, 22, 1, 2), row 1 -> all 5.
    # Sequence 1 (1 key): row 0 sees none (O = 0, LSE = -inf), row 1 key 0.
    v = paged_ids_cache()
    k = bf16(np.zeros((4, 2, 1, 4)))
    q = bf16(np.ones((3, 2, 1, 4)))
    o, lse = oracle_mod.attn_fwd_paged(q, k, v, PAGED_TABLE, PAGED_LENS, True, 0.5)
    assert o[2, 0, 0, 0] == pytest.approx(46.0 / 4.0, rel=1e-13)
    assert o[2, 1, 0, 0] == pytest.approx(77.0 / 5.0, rel=1e-13)
    assert lse[2, 0, 0] == pytest.approx(math.log(4), abs=1e-13)
    assert np.all(o[1, 0] == 0.0) and lse[1, 0, 0] == -math.inf
    assert o[1, 1, 0, 0] == 1.0 and lse[1, 0, 1] == 0.0
    # sequence 0 (3 keys): row 0 -> 31, 32; row 1 -> 31, 32, 11
    assert o[0, 0, 0, 0] == pytest.approx(31.5, rel=1e-13)
    assert o[0, 1, 0, 0] == pytest.approx(74.0 / 3.0, rel=1e-13)


def test_paged_empty_sequence(oracle_mod):
    v = paged_ids_cache()
    q = bf16(np.ones((3, 1, 2, 4)))
    lens = np.array([3, 0, 5], dtype=np.int32)
    o, lse = oracle_mod.attn_fwd_paged(q, v, v, PAGED_TABLE, lens, False, 0.5)
    assert np.all(o[1] == 0.0) and np.all(lse[1] == -math.inf)
    assert np.isfinite(lse[0]).all() and np.isfinite(lse[2]).all()


def test_paged_identity_table_equals_contiguous(oracle_mod):
    # pages laid out in order, every sequence full: the contiguous problem
    B, Hq, Hkv, S, D, ps = 2, 4, 2, 24, 8, 4
    q, k, v = random_qkv(B, Hq, Hkv, 3, S, D, seed=21)
    table = np.arange(B * S // ps, dtype=np.int32).reshape(B, S // ps)
    kc = k.reshape(B * S // ps, ps, Hkv, D)
    vc = v.reshape(B * S // ps, ps, Hkv, D)
    lens = np.full(B, S, dtype=np.int32)
    for causal in (False, True):
        o1, l1 = oracle_mod.attn_fwd_paged(q, kc, vc, table, lens, causal, 0.3)
        o2, l2 = oracle_mod.attn_fwd(q, k, v, causal, 0.3)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_paged_page_permutation_invariance(oracle_mod):
    # moving pages around the cache and remapping the table changes nothing
    rng = np.random.default_rng(3)
    q = bf16(rng.standard_normal((3, 1, 2, 8)))
    k = bf16(rng.standard_normal((4, 2, 1, 8)))
    v = bf16(rng.standard_normal((4, 2, 1, 8)))
    o1, l1 = oracle_mod.attn_fwd_paged(q, k, v, PAGED_TABLE, PAGED_LENS, False, 0.4)
    perm = np.array([2, 0, 3, 1])                 # page p moves to slot perm[p]
    inv = np.argsort(perm)
    table2 = np.where(PAGED_TABLE >= 0, perm[np.maximum(PAGED_TABLE, 0)], -1).astype(np.int32)
    o2, l2 = oracle_mod.attn_fwd_paged(q, k[inv], v[inv], table2, PAGED_LENS, False, 0.4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ----------------------------------------------------------------------------
# FP8 E4M3 inputs: the decode of every code and the descale convention
# ----------------------------------------------------------------------------
def test_fp8_decode_matches_the_format_and_torch(oracle_mod):
    # hand-worked codes of the OCP E4M3 format
    expect = {0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
              0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0,
              0x30: 0.5, 0x3C: 1.5}
    for code, val in expect.items():
        assert oracle_mod.fp8_e4m3_value(code) == val, hex(code)
    assert math.isnan(oracle_mod.fp8_e4m3_value(0x7F))
    assert math.isnan(oracle_mod.fp8_e4m3_value(0xFF))
    # and every code against torch's float8_e4m3fn
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().double().numpy()
    got = oracle_mod.fp8_values(codes.numpy())
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(ref[~np.isnan(ref)], got[~np.isnan(got)])


def test_fp8_uniform_scores_average_descaled_v(oracle_mod):
    # K = 0: O is the mean of the (descaled) V rows, LSE = ln(Sk)
    Sk = 6
    q8 = torch.full((1, 2, 1, 4), 3.0).to(torch.float8_e4m3fn)
    k8 = torch.zeros((1, Sk, 1, 4)).to(torch.float8_e4m3fn)
    vals = torch.tensor([1.0, 2.0, 3.0, 4.0, 6.0, 8.0])
    v8 = vals.view(1, Sk, 1, 1).expand(1, Sk, 1, 4).contiguous().to(torch.float8_e4m3fn)
    o, lse = oracle_mod.attn_fwd_fp8(q8, k8, v8, False, 0.5, 0.25, 3.0, 0.125)
    assert np.allclose(o, 24.0 / 6.0 * 0.125, rtol=0, atol=1e-15)
    assert np.allclose(lse, math.log(Sk), rtol=0, atol=1e-14)


def test_fp8_descales_enter_scores_and_output(oracle_mod):
    # two keys: s_j = scale*dq*dk*(q.k_j); weights by hand
    q8 = torch.tensor([[[[2.0, 0.0]]]]).to(torch.float8_e4m3fn)          # [1,1,1,2]
    k8 = torch.tensor([[[[1.0, 0.0]], [[0.0, 1.0]]]]).to(torch.float8_e4m3fn)  # [1,2,1,2]
    v8 = torch.tensor([[[[4.0, 0.0]], [[0.0, 8.0]]]]).to(torch.float8_e4m3fn)
    scale, dq, dk, dv = 0.5, 1.5, 0.75, 0.25
    s0 = scale * dq * dk * 2.0
    w0 = math.exp(s0) / (math.exp(s0) + 1.0)
    o, lse = oracle_mod.attn_fwd_fp8(q8, k8, v8, False, scale, dq, dk, dv)
    # the oracle rounds scale*dq*dk to float32 once
    assert o[0, 0, 0, 0] == pytest.approx(dv * 4.0 * w0, rel=1e-6)
    assert o[0, 0, 0, 1] == pytest.approx(dv * 8.0 * (1.0 - w0), rel=1e-6)
    assert lse[0, 0, 0] == pytest.approx(math.log(math.exp(s0) + 1.0), rel=1e-6)


def test_fp8_equals_bf16_oracle_on_exact_values(oracle_mod):
    # descales of 1: the FP8 oracle is the bf16 oracle on the same values
    q8, k8, v8, *_ = (t for t in (torch.randn(1, 5, 2, 8), torch.randn(1, 7, 2, 8),
                                  torch.randn(1, 7, 2, 8)))
    q8, k8, v8 = (t.to(torch.float8_e4m3fn) for t in (q8, k8, v8))
    o1, l1 = oracle_mod.attn_fwd_fp8(q8, k8, v8, True, 0.3, 1.0, 1.0, 1.0)
    o2, l2 = oracle_mod.attn_fwd(q8.float().to(torch.bfloat16), k8.float().to(torch.bfloat16),
                                 v8.float().to(torch.bfloat16), True, 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ----------------------------------------------------------------------------
# backward: against torch autograd (fp64), finite differences, closed forms
# ----------------------------------------------------------------------------
def torch_grads(q, k, v, do, causal, scale):
    """fp64 autograd of softmax(scale Q K^T [mask]) V: a different evaluation
    of the same gradients (no hand-written backward formula)."""
    Q, K, V, dO = (t.double().clone().requires_grad_(i < 3) for i, t in enumerate((q, k, v, do)))
    B, Sq, Hq, D = Q.shape
    Sk, Hkv = K.shape[1], K.shape[2]
    Ke = K.repeat_interleave(Hq // Hkv, dim=2)
    Ve = V.repeat_interleave(Hq // Hkv, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", Q, Ke) * scale
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        s = s.masked_fill(~(j <= i + Sk - Sq), float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)
    o = torch.einsum("bhij,bjhd->bihd", p, Ve)
    (o * dO).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("shape", [(1, 2, 2, 5, 7, 8, False), (2, 4, 2, 6, 6, 4, True),
                                   (1, 3, 1, 7, 4, 8, True)])
def test_bwd_matches_torch_autograd(oracle_mod, shape):
    B, Hq, Hkv, Sq, Sk, D, causal = shape
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, seed=51)
    do = bf16(torch.randn(B, Sq, Hq, D, generator=torch.Generator().manual_seed(52)))
    got = oracle_mod.attn_bwd(q, k, v, do, causal, 0.4)
    ref = torch_grads(q.float(), k.float(), v.float(), do.float(), causal, 0.4)
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12, err_msg=name)


def test_bwd_matches_finite_differences(oracle_mod):
    # L = sum(O * dO); central differences of the fp64 forward definition
    q, k, v = random_qkv(1, 2, 1, 4, 5, 4, seed=53)
    do = bf16(torch.randn(1, 4, 2, 4, generator=torch.Generator().manual_seed(54)))
    dq, dk, dv = oracle_mod.attn_bwd(q, k, v, do, True, 0.7)
    Q, K, V, dO = (t.double().numpy() for t in (q.float(), k.float(), v.float(), do.float()))

    def loss(Q, K, V):
        total = 0.0
        for h in range(2):
            s = 0.7 * Q[0, :, h] @ K[0, :, 0].T
            s = np.where(np.arange(5)[None, :] <= np.arange(4)[:, None] + 1, s, -np.inf)
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            total += ((p @ V[0, :, 0]) * dO[0, :, h]).sum()
        return total

    eps = 1e-6
    for X, G in ((Q, dq), (K, dk), (V, dv)):
        for idx in [(0, 0, 0, 0), (0, 2, 0, 3), (0, 3, X.shape[2] - 1, 1)]:
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = [Xp if Y is X else Y for Y in (Q, K, V)]
            args_m = [Xm if Y is X else Y for Y in (Q, K, V)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert G[idx] == pytest.approx(fd, abs=1e-7), idx


def test_bwd_single_key_closed_form(oracle_mod):
    # one key: P = 1, so dV = sum over queries of dO, and dQ = dK = 0
    q, k, v = random_qkv(1, 2, 1, 3, 1, 4, seed=55)
    do = bf16(torch.randn(1, 3, 2, 4, generator=torch.Generator().manual_seed(56)))
    dq, dk, dv = oracle_mod.attn_bwd(q, k, v, do, False, 0.5)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    np.testing.assert_allclose(dv[0, 0, 0], do.double().numpy()[0].sum(axis=(0, 1)), rtol=1e-15)


def test_bwd_uniform_scores_dv_is_column_mean(oracle_mod):
    # K = 0: P = 1/Sk for every allowed key; dV_j = sum over queries of dO / Sk
    q, _, v = random_qkv(1, 1, 1, 3, 4, 4, seed=57)
    k = bf16(np.zeros((1, 4, 1, 4)))
    do = bf16(torch.randn(1, 3, 1, 4, generator=torch.Generator().manual_seed(58)))
    _, _, dv = oracle_mod.attn_bwd(q, k, v, do, False, 0.5)
    expect = do.double().numpy()[0, :, 0, :].sum(axis=0) / 4.0
    for j in range(4):
        np.testing.assert_allclose(dv[0, j, 0], expect, rtol=1e-14)
