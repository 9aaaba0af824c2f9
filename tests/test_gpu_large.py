"""Parity past 2^31 elements in one segment, payload or tensor.

Every kernel indexes elements with 64-bit integers; these launches put element indices
(not only byte offsets) beyond 2^31 and end in a ragged block or chunk.  The GPU
processes the whole tensors; the oracle checks sampled runs of whole blocks (whole
chunks for Top-k and sparse aggregation): the first, the ones on both sides of element
2^31, the last (ragged) one, and a few random ones.  Inputs come from the seeded
generators on the GPU and are read back for the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import assert_bf16_close, assert_bytes_equal, assert_f32_close, bf16_bits, host, say, step_per_elem

pytestmark = pytest.mark.gpu

BIG = 1 << 31


def sample_units(nunits, unit, rng, count=6, run=2):
    """Sorted, disjoint runs [u0, u1) of `run` units: the first, those around element
    2^31, the last, and `count` random ones."""
    edge = BIG // unit
    starts = {0, edge - run, edge, nunits - run} | set(int(x) for x in rng.integers(0, nunits - run, count))
    out, last = [], -1
    for s in sorted(starts):
        s = max(s, last)
        e = min(nunits, s + run)
        if e > s:
            out.append((s, e))
            last = e
    return out


@pytest.mark.parametrize("ed", ["f32", "i8"])
def test_cq_past_2p31(gpu_lib, ed):
    """One segment of 2^31 + 3*2^20 + 77 bf16 elements (4-bit, block 256), 2 steps."""
    n, bits, block = BIG + 3 * (1 << 20) + 77, 4, 256
    s_e = 2.0 ** 17 if ed == "i8" else 0.0
    rng = np.random.default_rng(31)
    nb = gpu_lib.num_blocks(n, block)
    ranges = sample_units(nb, block, rng)
    e = torch.zeros(n, dtype=torch.float32 if ed == "f32" else torch.int8, device="cuda")
    codes = torch.empty(gpu_lib.code_bytes(n, bits), dtype=torch.uint8, device="cuda")
    absmax = torch.empty(nb, dtype=torch.float32, device="cuda")
    ora_e = {b0: np.zeros(min(b1 * block, n) - b0 * block, np.float32 if ed == "f32" else np.int8)
             for b0, b1 in ranges}
    for step in range(2):
        say(f"cq past 2^31 ({ed} error): step {step}, n={n:,}")
        g = W.shard7b_grad(step, n=n, device="cuda", chain=f"big-{ed}")
        gpu_lib.loco_compensate_quantize_ex([(g, e, codes, absmax)], bits=bits, block=block, beta=0.9, err_scale=s_e)
        torch.cuda.synchronize()
        for b0, b1 in ranges:
            lo, hi = b0 * block, min(b1 * block, n)
            gb = bf16_bits(g[lo:hi])
            ref = oracle.compensate_quantize(gb, ora_e[b0], bits=bits, block=block, beta=0.9, grad_dtype="bf16",
                                             err_dtype=ed, err_scale=s_e)
            t = f"step {step} blocks {b0}:{b1} (elements {lo:,}..{hi:,})"
            assert_bytes_equal(host(codes[lo * bits // 8:(hi * bits + 7) // 8]), ref["codes"], f"{t} codes")
            assert_bytes_equal(host(absmax[b0:b1]).view(np.uint32), ref["absmax"].view(np.uint32), f"{t} absmax")
            if ed == "i8":
                assert_bytes_equal(host(e[lo:hi]), ref["e_new"], f"{t} 8-bit error")
            else:
                assert_f32_close(host(e[lo:hi]), ref["e_new"], step_per_elem(ref["absmax"], bits, block, hi - lo),
                                 f"{t} error")
            ora_e[b0] = ref["e_new"]
        del g
    say(f"  {len(ranges)} block runs checked over 2 steps")


def test_dequant_reduce_past_2p31(gpu_lib):
    """2 peer payloads of 2^31 + 2^20 + 5 elements (4-bit, block 256) into bf16 x 1/2."""
    n, bits, block, P = BIG + (1 << 20) + 5, 4, 256, 2
    say(f"dr past 2^31: n={n:,}, generating {P} payloads")
    pays = [W.random_payload(n, bits, block, key=("big", p), device="cuda") for p in range(P)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    gpu_lib.loco_dequant_reduce(pays, n, bits=bits, block=block, out=out, out_scale=0.5)
    torch.cuda.synchronize()
    rng = np.random.default_rng(32)
    ranges = sample_units(-(-n // block), block, rng)
    for b0, b1 in ranges:
        lo, hi = b0 * block, min(b1 * block, n)
        sl = [(host(c[lo * bits // 8:(hi * bits + 7) // 8]), host(a[b0:b1])) for c, a in pays]
        want = oracle.dequant_reduce(sl, hi - lo, bits=bits, block=block, out_scale=0.5, out_dtype="bf16")
        assert_bf16_close(bf16_bits(out[lo:hi]), want, f"dr blocks {b0}:{b1}")
    say(f"  {len(ranges)} block runs checked")


def test_topk_past_2p31(gpu_lib):
    """2^31 + 3*4096 + 100 fp32 elements, chunk 4096, k = 82, 2-bit, decay 1, 2 steps (the
    last chunk is short and goes through the tail kernel)."""
    n, C, k, bits = BIG + 3 * 4096 + 100, 4096, 82, 2
    chunks = -(-n // C)
    nb = gpu_lib.code_bytes(k, bits)
    e = torch.zeros(n, device="cuda")
    idx = torch.empty(chunks * k, dtype=torch.int16, device="cuda")
    codes = torch.empty(chunks * nb, dtype=torch.uint8, device="cuda")
    am = torch.empty(chunks, device="cuda")
    rng = np.random.default_rng(33)
    ranges = sample_units(chunks, C, rng, run=1)
    ora_e = {c0: np.zeros(min((c0 + 1) * C, n) - c0 * C, np.float32) for c0, _ in ranges}
    for step in range(2):
        say(f"top-k past 2^31: step {step}, n={n:,}")
        g = W.sparseloco_grad(step, n=n, device="cuda")
        gpu_lib.loco_topk_quantize(g, e, chunk=C, k=k, idx=idx, codes=codes, absmax=am, bits=bits, ef_decay=1.0)
        torch.cuda.synchronize()
        for c, _ in ranges:
            lo, hi = c * C, min((c + 1) * C, n)
            ref = oracle.topk_quantize(host(g[lo:hi]), ora_e[c], chunk=C, k=k, bits=bits, decay=1.0)
            t = f"step {step} chunk {c} (elements {lo:,}..{hi:,})"
            assert_bytes_equal(host(idx[c * k:(c + 1) * k]).view(np.uint16), ref["idx"], f"{t} idx")
            assert_bytes_equal(host(codes[c * nb:(c + 1) * nb]), ref["codes"], f"{t} codes")
            assert_bytes_equal(host(am[c:c + 1]).view(np.uint32), ref["absmax"].view(np.uint32), f"{t} absmax")
            assert_f32_close(host(e[lo:hi]), ref["e_new"], np.full(hi - lo, float(ref["absmax"][0])), f"{t} error")
            ora_e[c] = ref["e_new"]
        del g
    say(f"  {len(ranges)} chunks checked over 2 steps")


def test_topk_more_chunks_than_one_launch(gpu_lib):
    """2^20 + 3 whole chunks of 256 and a short one (n = 2^28 + 818): the whole chunks take
    two launches of at most 2^20 workgroups; the chunks on both sides of the launch
    boundary, the first and the short last one are checked, over 2 steps."""
    C, k, bits = 256, 5, 2
    n = (1 << 20) * C + 3 * C + 50
    chunks = -(-n // C)
    nb = gpu_lib.code_bytes(k, bits)
    e = torch.zeros(n, device="cuda")
    idx = torch.empty(chunks * k, dtype=torch.int16, device="cuda")
    codes = torch.empty(chunks * nb, dtype=torch.uint8, device="cuda")
    am = torch.empty(chunks, device="cuda")
    check = [0, (1 << 20) - 1, 1 << 20, (1 << 20) + 1, chunks - 2, chunks - 1]
    ora_e = {c: np.zeros(min((c + 1) * C, n) - c * C, np.float32) for c in check}
    for step in range(2):
        say(f"top-k over two launches: step {step}, n={n:,}, {chunks:,} chunks of {C}")
        g = W.sparseloco_grad(step, n=n, device="cuda")
        gpu_lib.loco_topk_quantize(g, e, chunk=C, k=k, idx=idx, codes=codes, absmax=am, bits=bits, ef_decay=1.0)
        torch.cuda.synchronize()
        for c in check:
            lo, hi = c * C, min((c + 1) * C, n)
            ref = oracle.topk_quantize(host(g[lo:hi]), ora_e[c], chunk=C, k=k, bits=bits, decay=1.0)
            t = f"step {step} chunk {c} (elements {lo:,}..{hi:,})"
            assert_bytes_equal(host(idx[c * k:(c + 1) * k]).view(np.uint16), ref["idx"], f"{t} idx")
            assert_bytes_equal(host(codes[c * nb:(c + 1) * nb]), ref["codes"], f"{t} codes")
            assert_bytes_equal(host(am[c:c + 1]).view(np.uint32), ref["absmax"].view(np.uint32), f"{t} absmax")
            assert_f32_close(host(e[lo:hi]), ref["e_new"], np.full(hi - lo, float(ref["absmax"][0])), f"{t} error")
            ora_e[c] = ref["e_new"]
        del g
    say(f"  {len(check)} chunks checked over 2 steps")


def test_sparse_aggregate_past_2p31(gpu_lib):
    """2 peers' Top-k payloads of 2^31 + 4096 + 33 elements (chunk 4096, k = 82, 2-bit) into
    fp32 x 1/2: chunks past 2^31, the short last chunk, and (fp32 output) launches of at
    most 128 MB of payload, each after its pre-read (two here)."""
    n, C, k, bits, P = BIG + 4096 + 33, 4096, 82, 2, 2
    cb = gpu_lib.code_bytes(k, bits)
    say(f"sparse aggregate past 2^31: n={n:,}, generating {P} payloads")
    pays = [W.random_sparse_payload(n, C, k, bits, key=("big", p), device="cuda") for p in range(P)]
    out = torch.empty(n, device="cuda")
    gpu_lib.loco_sparse_aggregate(pays, n, chunk=C, k=k, bits=bits, out=out, out_scale=0.5)
    torch.cuda.synchronize()
    chunks = -(-n // C)
    rng = np.random.default_rng(34)
    ranges = sample_units(chunks, C, rng, run=1)
    for c, _ in ranges:
        lo, hi = c * C, min((c + 1) * C, n)
        sl = [(host(ix[c * k:(c + 1) * k]).view(np.uint16), host(cd[c * cb:(c + 1) * cb]), host(a[c:c + 1]))
              for ix, cd, a in pays]
        want = oracle.sparse_aggregate(sl, hi - lo, chunk=C, k=k, bits=bits, out_scale=0.5)
        assert_f32_close(host(out[lo:hi]), want, np.zeros(hi - lo), f"sparse aggregate chunk {c}")
    say(f"  {len(ranges)} chunks checked")
