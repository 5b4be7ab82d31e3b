"""Every entry point can be captured into a HIP graph and replayed.

A serving loop replays one captured graph per step instead of launching each
kernel.  The library makes no allocation, memset or synchronisation inside a
call once its device state exists and the caller passes the workspace, so the
calls record as plain kernel nodes.  One graph holds a causal prefill, a
split-key decode with its merge, a paged decode, the FP8 prefill and the
backward.  It is replayed three times; before each replay the inputs are
refilled eagerly with new values, and after it every output must equal,
bit for bit, what the same calls produce eagerly on those inputs (each
kernel's reduction order is fixed by its launch configuration).
"""
from __future__ import annotations

import math
import sys

import pytest
import torch

from attention_fwd_02_amd.inputs import make_paged_inputs, PagedWorkload, random_fp8, random_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from attention_fwd_02_amd import _binding
    return _binding


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Calls:
    """Inputs, outputs and workspaces of the five calls; run() issues them
    on the current stream."""

    def __init__(self, ops):
        self.ops = ops
        # causal prefill, ragged (several items and a tail)
        self.pq, self.pk, self.pv = (t.to(DEV) for t in random_qkv(2, 8, 2, 1100, 1100, 128, seed=1))
        self.po = torch.empty_like(self.pq)
        self.pl = torch.empty((2, 8, 1100), dtype=torch.float32, device=DEV)
        # split-key decode, 8 splits, caller workspace
        self.dq, self.dk, self.dv = (t.to(DEV) for t in random_qkv(4, 16, 4, 1, 5000, 128, seed=2))
        self.do = torch.empty_like(self.dq)
        self.dl = torch.empty((4, 16, 1), dtype=torch.float32, device=DEV)
        self.dws = torch.empty(ops.fa_workspace_size(4, 16, 4, 1, 5000, 128, 8), dtype=torch.uint8,
                               device=DEV)
        # paged decode, caller workspace
        self.pw = PagedWorkload(name="graph", B=3, Hq=8, Hkv=2, Sq=1, max_len=700, page_size=16,
                                D=128)
        q, kc, vc, table, lens = (t.to(DEV) for t in make_paged_inputs(self.pw, lens=[700, 333, 1]))
        self.gq, self.gk, self.gv, self.gt, self.gs = q, kc, vc, table, lens
        self.go = torch.empty_like(q)
        self.gl = torch.empty((3, 8, 1), dtype=torch.float32, device=DEV)
        plan = ops.fa_plan_paged(3, 8, 2, 1, 128, kc.shape[0], 16, table.shape[1])
        self.gws = torch.empty(max(1, plan["workspace_bytes"]), dtype=torch.uint8, device=DEV)
        # FP8 prefill
        q8, k8, v8, d1, d2, d3 = random_fp8(1, 4, 2, 600, 600, 128, seed=3)
        self.fq, self.fk, self.fv = q8.to(DEV), k8.to(DEV), v8.to(DEV)
        self.fd = (d1, d2, d3)
        self.fo = torch.empty((1, 600, 4, 128), dtype=torch.bfloat16, device=DEV)
        self.fl = torch.empty((1, 4, 600), dtype=torch.float32, device=DEV)
        # backward of a causal forward, caller workspace
        self.bq, self.bk, self.bv = (t.to(DEV) for t in random_qkv(1, 4, 2, 300, 300, 128, seed=4))
        self.bo = torch.empty_like(self.bq)
        self.bl = torch.empty((1, 4, 300), dtype=torch.float32, device=DEV)
        self.bdo = torch.randn(self.bq.shape, generator=torch.Generator().manual_seed(5)).to(
            torch.bfloat16).to(DEV)
        self.bdq, self.bdk, self.bdv = (torch.empty_like(t) for t in (self.bq, self.bk, self.bv))
        self.bws = torch.empty(ops.fa_bwd_workspace_size(1, 4, 2, 300, 300, 128),
                               dtype=torch.uint8, device=DEV)
        self.inputs = [self.pq, self.pk, self.pv, self.dq, self.dk, self.dv, self.gq, self.gk,
                       self.gv, self.bq, self.bk, self.bv, self.bdo]
        self.outputs = [self.po, self.pl, self.do, self.dl, self.go, self.gl, self.fo, self.fl,
                        self.bo, self.bl, self.bdq, self.bdk, self.bdv]

    def run(self):
        ops = self.ops
        ops.fa_fwd(self.pq, self.pk, self.pv, self.po, self.pl, True, 1 / math.sqrt(128))
        ops.fa_fwd_ex(self.dq, self.dk, self.dv, self.do, self.dl, False, 0.08, num_splits=8,
                      workspace=self.dws)
        ops.fa_fwd_paged(self.gq, self.gk, self.gv, self.gt, self.gs, self.go, self.gl, False,
                         0.09, workspace=self.gws)
        ops.fa_fwd_fp8(self.fq, self.fk, self.fv, self.fo, self.fl, True, 0.1, *self.fd)
        ops.fa_fwd(self.bq, self.bk, self.bv, self.bo, self.bl, True, 0.12)
        ops.fa_bwd(self.bq, self.bk, self.bv, self.bo, self.bdo, self.bl, self.bdq, self.bdk,
                   self.bdv, True, 0.12, workspace=self.bws)

    def refill(self, seed):
        g = torch.Generator(DEV).manual_seed(seed)
        for t in self.inputs:
            t.copy_(torch.randn(t.shape, generator=g, device=DEV).to(t.dtype))
        r = torch.randint(0, 256, self.fq.shape, generator=g, device=DEV, dtype=torch.int32)
        # E4M3 bytes without the NaN codes (0x7f, 0xff)
        self.fq.copy_(torch.where((r & 0x7f) == 0x7f, r - 1, r).to(torch.uint8).view(
            self.fq.dtype))


def test_graph_replays_match_eager(ops):
    c = Calls(ops)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        c.run()   # the library's device state exists before the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.run()
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"[graph] replay {rep}")
        c.refill(100 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in c.outputs]
        for t in c.outputs:
            t.fill_(float("nan"))
        c.run()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, c.outputs)):
            assert not torch.isnan(a.float()).any(), f"replay {rep}: output {i} has NaN"
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                f"replay {rep}: output {i} differs from the eager call"
