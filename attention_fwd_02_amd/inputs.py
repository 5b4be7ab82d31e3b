"""Seeded synthetic inputs for the attention forward pass.

This module only draws numbers and names workloads; it holds none of the
attention arithmetic.  Both the GPU path's tests and the oracle consume what it
returns, so neither side generates its own inputs.

Recipe (the same on every machine, CPU generator only):
  * ``torch.Generator('cpu').manual_seed(seed)``;
  * q, k, v drawn in that order with ``torch.randn`` in float32, multiplied by
    ``std``, then cast to bfloat16 (round to nearest even);
  * ``hot_row_frac > 0``: a Bernoulli(hot_row_frac) mask over the (b, i, hq)
    query rows, drawn after v from the same generator with ``torch.rand``;
    selected rows are multiplied by ``hot_row_mult`` in float32 before the cast
    (8 is a power of two, so the bf16 values are exactly 8x the plain draw).

Paged K/V caches (``PagedWorkload``), same generator:
  * sequence lengths: every sequence ``max_len`` keys ("equal"), or
    ``torch.randint(1, max_len + 1)`` per sequence ("ragged", mean about
    max_len / 2);
  * each sequence takes ceil(len / page_size) pages; the cache holds exactly
    those pages, handed out in the order of ``torch.randperm`` (a fragmented
    pool: a sequence's pages are scattered over the cache); unused block-table
    entries are -1;
  * then q, k_cache, v_cache with ``torch.randn`` as above.

FP8 inputs (``make_fp8_inputs``): q, k, v drawn as above in float32 (times
``std``, hot rows included), then quantized per tensor to OCP FP8 E4M3:
descale = amax / 448 (a power of two is not forced), codes = the float32
values divided by descale, converted with torch's round-to-nearest-even
``float8_e4m3fn`` cast.  The real inputs are descale * codes.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    o_dtype: str = "bf16"          # "bf16" or "f32"
    std: float = 1.0
    hot_row_frac: float = 0.0
    hot_row_mult: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def allowed_pairs(self) -> int:
        """Allowed (query, key) pairs over all (b, hq)."""
        if not self.causal:
            per_head = self.Sq * self.Sk
        else:
            per_head = 0
            off = self.Sk - self.Sq
            # rows i with i + off + 1 keys (clamped to [0, Sk])
            for i in range(self.Sq):
                per_head += min(max(i + off + 1, 0), self.Sk)
        return per_head * self.B * self.Hq

    def flops(self) -> int:
        """Algorithmic FLOPs: 4*D per allowed pair (2*D for QK^T, 2*D for PV)."""
        return 4 * self.D * self.allowed_pairs()

    def hbm_bytes(self) -> int:
        """Algorithmic bytes: Q, K, V read once, O and LSE written once."""
        q = self.B * self.Sq * self.Hq * self.D * 2
        kv = 2 * self.B * self.Sk * self.Hkv * self.D * 2
        o = self.B * self.Sq * self.Hq * self.D * (4 if self.o_dtype == "f32" else 2)
        lse = self.B * self.Hq * self.Sq * 4
        return q + kv + o + lse


# The five workloads of the benchmark suite, named by what they are.
WORKLOADS = {
    w.name: w for w in [
        Workload("single_head_s128_d64", B=1, Hq=1, Hkv=1, Sq=128, Sk=128, D=64,
                 causal=False, o_dtype="f32", seed=0),
        Workload("causal_b2_h8_s1024_d64", B=2, Hq=8, Hkv=8, Sq=1024, Sk=1024, D=64,
                 causal=True, seed=1),
        Workload("causal_b4_h16_s4096_d128", B=4, Hq=16, Hkv=16, Sq=4096, Sk=4096, D=128,
                 causal=True, hot_row_frac=0.01, hot_row_mult=8.0, seed=2),
        Workload("decode_b32_hq32_hkv8_sk8192_d128", B=32, Hq=32, Hkv=8, Sq=1, Sk=8192,
                 D=128, causal=False, seed=3),
        Workload("gqa_b1_hq32_hkv8_s16384_d128", B=1, Hq=32, Hkv=8, Sq=16384, Sk=16384,
                 D=128, causal=False, std=0.5, seed=4),
    ]
}


# Head dim 256 (the head-dim variants beyond the five): a causal prefill with
# the causal workload's sequence length and the decode workload's shape.
HEADDIM_WORKLOADS = {
    w.name: w for w in [
        Workload("causal_b2_h16_s4096_d256", B=2, Hq=16, Hkv=16, Sq=4096, Sk=4096, D=256,
                 causal=True, seed=7),
        Workload("decode_b32_hq32_hkv8_sk8192_d256", B=32, Hq=32, Hkv=8, Sq=1, Sk=8192,
                 D=256, causal=False, seed=8),
    ]
}


def make_inputs(w: Workload, seed: int | None = None, device: str = "cpu"):
    """Return (q, k, v) bf16 tensors: q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D]."""
    g = torch.Generator("cpu")
    g.manual_seed(w.seed if seed is None else seed)
    q = torch.randn((w.B, w.Sq, w.Hq, w.D), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Sk, w.Hkv, w.D), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Sk, w.Hkv, w.D), generator=g, dtype=torch.float32)
    if w.std != 1.0:
        q.mul_(w.std)
        k.mul_(w.std)
        v.mul_(w.std)
    if w.hot_row_frac > 0.0:
        hot = torch.rand((w.B, w.Sq, w.Hq), generator=g) < w.hot_row_frac
        q = torch.where(hot.unsqueeze(-1), q * w.hot_row_mult, q)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    if device != "cpu":
        q, k, v = (t.to(device) for t in (q, k, v))
    return q, k, v


def random_qkv(B, Hq, Hkv, Sq, Sk, D, seed, std=1.0, device="cpu"):
    """Ad-hoc shapes for tests: same recipe, no hot rows."""
    w = Workload("adhoc", B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, causal=False,
                 std=std, seed=seed)
    return make_inputs(w, device=device)


@dataclasses.dataclass(frozen=True)
class PagedWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    max_len: int
    page_size: int
    D: int
    lengths: str = "equal"         # "equal" or "ragged"
    causal: bool = False
    o_dtype: str = "bf16"
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def max_pages(self) -> int:
        return (self.max_len + self.page_size - 1) // self.page_size

    def hbm_bytes(self, seq_lens) -> int:
        """Algorithmic bytes: every sequence's K and V rows, Q, the block-table
        entries of its pages and its length read once; O and LSE written once."""
        lens = [int(x) for x in seq_lens]
        kv = 2 * sum(lens) * self.Hkv * self.D * 2
        q = self.B * self.Sq * self.Hq * self.D * 2
        o = self.B * self.Sq * self.Hq * self.D * (4 if self.o_dtype == "f32" else 2)
        lse = self.B * self.Hq * self.Sq * 4
        table = 4 * sum((n + self.page_size - 1) // self.page_size for n in lens) + 4 * self.B
        return kv + q + o + lse + table


PAGED_WORKLOADS = {
    w.name: w for w in [
        # the decode workload's shape (B=32, Hq=32, Hkv=8, 8192 keys, D=128)
        # with its K/V in 16-key pages scattered over the cache
        PagedWorkload("paged_decode_b32_hq32_hkv8_len8192_ps16_d128", B=32, Hq=32, Hkv=8,
                      Sq=1, max_len=8192, page_size=16, D=128, seed=5),
        # the same with lengths drawn from [1, 16384] (mean about 8192)
        PagedWorkload("paged_decode_b32_hq32_hkv8_ragged16384_ps16_d128", B=32, Hq=32, Hkv=8,
                      Sq=1, max_len=16384, page_size=16, D=128, lengths="ragged", seed=6),
    ]
}


def make_paged_inputs(w: PagedWorkload, seed: int | None = None, device: str = "cpu",
                      lens=None):
    """Return (q, k_cache, v_cache, block_table, seq_lens).

    q [B,Sq,Hq,D] bf16; caches [num_pages, page_size, Hkv, D] bf16;
    block_table [B, max_pages] int32; seq_lens [B] int32.  ``lens`` (a list)
    replaces the drawn lengths (edge cases in tests)."""
    g = torch.Generator("cpu")
    g.manual_seed(w.seed if seed is None else seed)
    if lens is not None:
        seq = torch.tensor(lens, dtype=torch.int64)
    elif w.lengths == "equal":
        seq = torch.full((w.B,), w.max_len, dtype=torch.int64)
    else:
        seq = torch.randint(1, w.max_len + 1, (w.B,), generator=g, dtype=torch.int64)
    npages = (seq + w.page_size - 1) // w.page_size
    total = int(npages.sum())
    perm = torch.randperm(max(total, 1), generator=g)
    table = torch.full((w.B, w.max_pages), -1, dtype=torch.int32)
    at = 0
    for b in range(w.B):
        n = int(npages[b])
        table[b, :n] = perm[at:at + n].to(torch.int32)
        at += n
    q = torch.randn((w.B, w.Sq, w.Hq, w.D), generator=g, dtype=torch.float32)
    kc = torch.randn((max(total, 1), w.page_size, w.Hkv, w.D), generator=g, dtype=torch.float32)
    vc = torch.randn((max(total, 1), w.page_size, w.Hkv, w.D), generator=g, dtype=torch.float32)
    q, kc, vc = (t.to(torch.bfloat16) for t in (q, kc, vc))
    seq = seq.to(torch.int32)
    if device != "cpu":
        q, kc, vc, table, seq = (t.to(device) for t in (q, kc, vc, table, seq))
    return q, kc, vc, table, seq


# FP8 E4M3 inputs: the causal benchmark workload's shape.
FP8_WORKLOADS = {
    w.name: w for w in [
        Workload("causal_b4_h16_s4096_d128_fp8", B=4, Hq=16, Hkv=16, Sq=4096, Sk=4096, D=128,
                 causal=True, hot_row_frac=0.01, hot_row_mult=8.0, seed=9),
    ]
}


def make_fp8_inputs(w: Workload, seed: int | None = None, device: str = "cpu"):
    """Return (q8, k8, v8, q_descale, k_descale, v_descale): float8_e4m3fn
    tensors of the usual shapes and per-tensor float descale factors."""
    g = torch.Generator("cpu")
    g.manual_seed(w.seed if seed is None else seed)
    q = torch.randn((w.B, w.Sq, w.Hq, w.D), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Sk, w.Hkv, w.D), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Sk, w.Hkv, w.D), generator=g, dtype=torch.float32)
    if w.std != 1.0:
        q.mul_(w.std)
        k.mul_(w.std)
        v.mul_(w.std)
    if w.hot_row_frac > 0.0:
        hot = torch.rand((w.B, w.Sq, w.Hq), generator=g) < w.hot_row_frac
        q = torch.where(hot.unsqueeze(-1), q * w.hot_row_mult, q)
    out = []
    scales = []
    for t in (q, k, v):
        descale = float(t.abs().max()) / 448.0
        out.append((t / descale).to(torch.float8_e4m3fn))
        scales.append(descale)
    if device != "cpu":
        out = [t.to(device) for t in out]
    return (*out, *scales)


def random_fp8(B, Hq, Hkv, Sq, Sk, D, seed, std=1.0, device="cpu"):
    """Ad-hoc FP8 shapes for tests: same recipe, no hot rows."""
    w = Workload("adhoc", B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, causal=False, std=std,
                 seed=seed)
    return make_fp8_inputs(w, device=device)
