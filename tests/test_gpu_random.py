"""Seeded random configurations through every entry point, against the CPU oracle, and
concurrent calls on several streams.

Each case draws its own sizes, segment counts, element types, code widths, blocks,
chunks, k and hyper-parameters from a fixed seed, so odd combinations the structured
tests do not list are covered too; the bar is the same (bit-exact codes, indices and
scales; errors and outputs within 1e-6 relative or 1 bf16 ulp).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import (assert_bf16_close, assert_bytes_equal, assert_f32_close, bf16_bits, host, say,
                         step_per_elem)

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}
ORA = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8}


def oracle_form(t, dt):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else t.numpy()


@pytest.mark.parametrize("case", range(12))
def test_cq_random(gpu_lib, case):
    rng = np.random.default_rng(1000 + case)
    nseg = int(rng.integers(1, 40))
    sizes = [int(x) for x in rng.integers(0, 20_000, nseg)]
    gd = str(rng.choice(["f32", "bf16"]))
    ed = str(rng.choice(["f32", "bf16", "i8"]))
    bits = int(rng.choice([2, 4, 8]))
    fixed = float(rng.choice([0.0, 0.0, 2.0 ** 17]))
    block = int(rng.choice([64, 128, 256, 512]))
    beta = float(rng.choice([0.0, 0.5, 0.9, 0.99, 1.0]))
    s_e = float(rng.choice([2.0 ** 16, 2.0 ** 18, 123456.0])) if ed == "i8" else 0.0
    say(f"cq random {case}: {nseg} segs, {gd}/{ed}, bits {bits}, B {block}, beta {beta}, fixed {fixed}, s_e {s_e}")
    segs, ora_e = [], []
    for n in sizes:
        segs.append((torch.empty(n, dtype=TD[gd], device="cuda"), torch.zeros(n, dtype=TD[ed], device="cuda"),
                     torch.empty(gpu_lib.code_bytes(n, bits), dtype=torch.uint8, device="cuda"),
                     None if fixed else torch.empty(gpu_lib.num_blocks(n, block), device="cuda")))
        ora_e.append(np.zeros(n, ORA[ed]))
    for step in range(3):
        reset = bool(rng.random() < 0.3)
        for i, (g, _, _, _) in enumerate(segs):
            x = W.shard7b_grad(step, n=max(1, g.numel()), chain=f"rnd{case}-{i}")[:g.numel()].float()
            x = x * (1e-2 if fixed else 1.0)
            g.copy_(x.to(TD[gd]).cuda())
        gpu_lib.loco_compensate_quantize_ex(segs, bits=bits, block=block, beta=beta, fixed_scale=fixed,
                                            err_scale=s_e, reset_error=reset)
        torch.cuda.synchronize()
        for i, (g, e, c, a) in enumerate(segs):
            n = g.numel()
            ref = oracle.compensate_quantize(oracle_form(g, gd), ora_e[i], bits=bits, block=block, beta=beta,
                                             fixed_scale=fixed, grad_dtype=gd, err_dtype=ed, err_scale=s_e,
                                             reset=reset)
            t = f"case {case} step {step} seg {i} n={n}"
            assert_bytes_equal(host(c), ref["codes"], f"{t} codes")
            if a is not None:
                assert_bytes_equal(host(a).view(np.uint32), ref["absmax"].view(np.uint32), f"{t} absmax")
            if ed == "i8":
                assert_bytes_equal(host(e), ref["e_new"], f"{t} error")
            elif ed == "bf16":
                assert_bf16_close(bf16_bits(e), ref["e_new"], f"{t} error")
            else:
                floor = step_per_elem(ref["absmax"], bits, block, n) if a is not None else np.full(n, 1 / fixed)
                assert_f32_close(host(e), ref["e_new"], floor, f"{t} error")
            ora_e[i] = ref["e_new"]


@pytest.mark.parametrize("case", range(8))
def test_dr_random(gpu_lib, case):
    rng = np.random.default_rng(2000 + case)
    n = int(rng.integers(1, 300_000))
    npeers = int(rng.integers(1, 20))
    bits = int(rng.choice([2, 4, 8]))
    block = int(rng.choice([64, 128, 256, 512]))
    fixed = float(rng.choice([0.0, 0.0, 2.0 ** 19]))
    od = str(rng.choice(["f32", "bf16"]))
    scale = float(rng.choice([1.0 / npeers, 0.3, 1.0]))
    say(f"dr random {case}: n={n}, {npeers} peers, bits {bits}, B {block}, fixed {fixed}, out {od}")
    pays = [W.random_payload(n, bits, block, key=("rnd", case, p)) for p in range(npeers)]
    out = torch.empty(n, dtype=TD[od], device="cuda")
    gpu_lib.loco_dequant_reduce([(c.cuda(), None if fixed else a.cuda()) for c, a in pays], n, bits=bits,
                                block=block, out=out, out_scale=scale, fixed_scale=fixed)
    torch.cuda.synchronize()
    want = oracle.dequant_reduce([(host(c), None if fixed else host(a)) for c, a in pays], n, bits=bits,
                                 block=block, out_scale=scale, out_dtype=od, fixed_scale=fixed)
    if od == "bf16":
        assert_bf16_close(bf16_bits(out), want, f"case {case}")
    else:
        assert_f32_close(host(out), want, np.zeros(n), f"case {case}")


@pytest.mark.parametrize("case", range(8))
def test_tk_sa_random(gpu_lib, case):
    """Top-k on a random shape, then the sparse aggregation of its payload with others."""
    rng = np.random.default_rng(3000 + case)
    chunk = int(rng.choice([256, 512, 1024, 2048, 4096]))
    n = int(rng.integers(1, 12 * chunk))
    k = int(rng.integers(1, chunk + 1))
    bits = int(rng.choice([2, 4, 8]))
    decay = float(rng.choice([1.0, 0.9, 0.0]))
    say(f"tk+sa random {case}: n={n}, chunk {chunk}, k {k}, bits {bits}, decay {decay}")
    chunks = -(-n // chunk)
    nb = gpu_lib.code_bytes(k, bits)
    g = W.sparseloco_grad(case, n=n)
    e0 = (torch.randn(n, generator=torch.Generator().manual_seed(case)) * 1e-4).float()
    e = e0.cuda()
    idx = torch.empty(chunks * k, dtype=torch.int16, device="cuda")
    codes = torch.empty(chunks * nb, dtype=torch.uint8, device="cuda")
    am = torch.empty(chunks, device="cuda")
    gpu_lib.loco_topk_quantize(g.cuda(), e, chunk=chunk, k=k, idx=idx, codes=codes, absmax=am, bits=bits,
                               ef_decay=decay)
    torch.cuda.synchronize()
    ref = oracle.topk_quantize(g.numpy(), e0.numpy(), chunk=chunk, k=k, bits=bits, decay=decay)
    assert_bytes_equal(host(idx).view(np.uint16), ref["idx"], f"case {case} idx")
    assert_bytes_equal(host(codes), ref["codes"], f"case {case} codes")
    assert_bytes_equal(host(am).view(np.uint32), ref["absmax"].view(np.uint32), f"case {case} absmax")
    assert_f32_close(host(e), ref["e_new"], np.repeat(ref["absmax"], chunk)[:n].astype(np.float64), f"case {case} e")
    # aggregate the oracle's payload with generated ones (no GPU output feeds the oracle)
    others = [W.random_sparse_payload(n, chunk, k, bits, key=("rnd", case, p)) for p in range(3)]
    mine = (torch.from_numpy(ref["idx"].view(np.int16).copy()), torch.from_numpy(ref["codes"].copy()),
            torch.from_numpy(ref["absmax"].copy()))
    peers = [others[0], mine, others[1], others[2]]
    od = str(rng.choice(["f32", "bf16"]))
    out = torch.empty(n, dtype=TD[od], device="cuda")
    gpu_lib.loco_sparse_aggregate([tuple(x.cuda() for x in pp) for pp in peers], n, chunk=chunk, k=k, bits=bits,
                                  out=out, out_scale=0.25)
    torch.cuda.synchronize()
    want = oracle.sparse_aggregate([(host(ix).view(np.uint16), host(c), host(a)) for ix, c, a in peers], n,
                                   chunk=chunk, k=k, bits=bits, out_scale=0.25, out_dtype=od)
    if od == "bf16":
        assert_bf16_close(bf16_bits(out), want, f"case {case} aggregate")
    else:
        assert_f32_close(host(out), want, np.zeros(n), f"case {case} aggregate")


def test_concurrent_streams(gpu_lib):
    """Four streams each run compensate-quantize and dequant-reduce on their own buffers at
    the same time; every result equals the same calls made one after another."""
    n, P = 2_000_003, 4
    streams = [torch.cuda.Stream() for _ in range(P)]
    gs = [W.shard7b_grad(0, n=n, device="cuda", chain=f"conc{i}") for i in range(P)]

    def make():
        es = [torch.zeros(n, device="cuda") for _ in range(P)]
        cs = [torch.empty(gpu_lib.code_bytes(n, 4), dtype=torch.uint8, device="cuda") for _ in range(P)]
        ams = [torch.empty(gpu_lib.num_blocks(n, 256), device="cuda") for _ in range(P)]
        outs = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
        return es, cs, ams, outs

    def run(bufs, use_streams):
        es, cs, ams, outs = bufs
        cur = torch.cuda.current_stream()
        for i in range(P):
            st = streams[i] if use_streams else cur
            st.wait_stream(cur)
            with torch.cuda.stream(st):
                for _ in range(3):
                    gpu_lib.loco_compensate_quantize([(gs[i], es[i], cs[i], ams[i])], bits=4, block=256, beta=0.9)
                    gpu_lib.loco_dequant_reduce([(cs[i], ams[i])] * 3, n, bits=4, block=256, out=outs[i],
                                                out_scale=1.0 / 3.0)
        for st in streams:
            cur.wait_stream(st)
        torch.cuda.synchronize()

    say("concurrent streams")
    a, b = make(), make()
    run(a, True)
    run(b, False)
    for i in range(P):
        for x, y in zip(a, b):
            assert torch.equal(x[i].view(torch.uint8), y[i].view(torch.uint8)), i
