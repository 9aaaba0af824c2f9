"""The library's launches under HIP graph capture (torch.cuda.CUDAGraph).

A caller may capture a whole step of the path into a graph.  The entry points allocate
nothing, set no memory and never synchronise, so a captured step must replay exactly
like eager calls: every replay here is checked bitwise against the same calls made
eagerly on a twin copy of the state, with fresh inputs copied in, eager work and
synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity_util import host, say

pytestmark = pytest.mark.gpu


def same(a, b, what):
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), what


class Step:
    """Compensate-quantize over 4 segments, dequant-reduce of 4 peers with the fused Adam
    step, Top-k, and sparse aggregation: one state, updated in place by each call."""

    def __init__(self, loco, n, chunk=4096, k=82):
        d = "cuda"
        self.loco, self.n, self.chunk, self.k = loco, n, chunk, k
        part = n // 4
        self.part = part
        self.g = torch.zeros(n, dtype=torch.bfloat16, device=d)
        self.e = torch.zeros(n, device=d)
        self.codes = [torch.zeros(loco.code_bytes(part, 4), dtype=torch.uint8, device=d) for _ in range(4)]
        self.am = [torch.zeros(loco.num_blocks(part, 256), device=d) for _ in range(4)]
        self.th = torch.zeros(part, device=d)
        self.m = torch.zeros(part, device=d)
        self.v = torch.zeros(part, device=d)
        self.tb = torch.zeros(part, dtype=torch.bfloat16, device=d)
        chunks = -(-n // chunk)
        self.tg = torch.zeros(n, device=d)
        self.te = torch.zeros(n, device=d)
        self.idx = torch.zeros(chunks * k, dtype=torch.int16, device=d)
        self.tc = torch.zeros(chunks * loco.code_bytes(k, 2), dtype=torch.uint8, device=d)
        self.ta = torch.zeros(chunks, device=d)
        self.sout = torch.zeros(n, device=d)

    def run(self):
        L, p = self.loco, self.part
        segs = [(self.g[i * p:(i + 1) * p], self.e[i * p:(i + 1) * p], self.codes[i], self.am[i]) for i in range(4)]
        L.loco_compensate_quantize(segs, bits=4, block=256, beta=0.9)
        L.loco_dequant_reduce_adam(list(zip(self.codes, self.am)), p, bits=4, block=256, out_scale=0.25,
                                   param=self.th, m=self.m, v=self.v, lr=1e-3, beta1=0.1, beta2=0.01, delta=1e-8,
                                   param_bf16=self.tb)
        L.loco_topk_quantize(self.tg, self.te, chunk=self.chunk, k=self.k, idx=self.idx, codes=self.tc,
                             absmax=self.ta, bits=2, ef_decay=1.0)
        L.loco_sparse_aggregate([(self.idx, self.tc, self.ta)] * 3, self.n, chunk=self.chunk, k=self.k,
                                out=self.sout, out_scale=1.0 / 3.0)

    def feed(self, step):
        self.g.copy_(W.shard7b_grad(step, n=self.n, device="cuda", chain="graph"))
        self.tg.copy_(W.sparseloco_grad(step, n=self.n, device="cuda"))

    def tensors(self):
        return ([self.e, self.th, self.m, self.v, self.tb, self.te, self.idx, self.tc, self.ta, self.sout] +
                self.codes + self.am)


def test_graph_replays_match_eager(gpu_lib):
    n = 4096 * 64 + 4 * 1000  # the last Top-k chunk is short; partitions end mid-block
    say(f"graph capture of a step, n={n}")
    cap, eag = Step(gpu_lib, n), Step(gpu_lib, n)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cap.run()  # warm-up outside the capture, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    eag.run()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        cap.run()
    torch.cuda.synchronize()
    for rep in range(4):
        cap.feed(rep)
        eag.feed(rep)
        torch.cuda.synchronize()
        graph.replay()
        eag.run()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(cap.tensors(), eag.tensors())):
            same(a, b, f"replay {rep}, tensor {i}")
        assert float(host(cap.ta).max()) > 0.0  # the replay really ran on the new inputs
        # eager work of the program's own between replays
        cap.sout.mul_(1.0)
        torch.cuda.synchronize()
    say("  4 replays bitwise equal to eager calls")
