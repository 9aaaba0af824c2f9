"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

The GPU processes the whole tensors; the oracle follows its own free-running chain on
sampled runs of whole scale blocks (whole chunks for Top-k), which are independent of the
rest.  Samples always include the first and the (ragged) last block of every segment.
Inputs are generated on the GPU by the seeded generators and read back for the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import assert_bf16_close, assert_bytes_equal, assert_f32_close, bf16_bits, host, say, step_per_elem

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}
ORA_E = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8}


def block_ranges(nblocks, rng, count=24, run=3):
    starts = {0, max(0, nblocks - run)}
    starts |= set(int(x) for x in rng.integers(0, max(1, nblocks - run), count))
    out, last = [], -1
    for s in sorted(starts):
        s = max(s, last)
        e = min(nblocks, s + run)
        if e > s:
            out.append((s, e))
            last = e
    return out


def storage(t, dt):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else t.numpy()


def fullsize_cq(loco, sizes, gd, ed, bits, block, beta, steps, gen, tag, seed=0, err_scale=0.0, reset_every=0):
    dev = "cuda"
    rng = np.random.default_rng(seed)
    e = [torch.zeros(n, dtype=TD[ed], device=dev) for n in sizes]
    codes = [torch.empty(loco.code_bytes(n, bits), dtype=torch.uint8, device=dev) for n in sizes]
    absmax = [torch.empty(loco.num_blocks(n, block), dtype=torch.float32, device=dev) for n in sizes]
    ranges = [block_ranges(loco.num_blocks(n, block), rng) for n in sizes]
    ora_e = {}
    for s, n in enumerate(sizes):
        for b0, b1 in ranges[s]:
            m = min(b1 * block, n) - b0 * block
            ora_e[(s, b0)] = np.zeros(m, ORA_E[ed])
    checked = 0
    bitwise = True
    for step in range(steps):
        say(f"{tag}: step {step}: generating and launching ({sum(sizes):,} elements, {len(sizes)} segments)")
        gs = gen(step)
        assert [g.numel() for g in gs] == list(sizes)
        reset = reset_every > 0 and (step + 1) % reset_every == 0
        if ed == "i8" or reset_every:
            loco.loco_compensate_quantize_ex(list(zip(gs, e, codes, absmax)), bits=bits, block=block, beta=beta,
                                             err_scale=err_scale, reset_error=reset)
        else:
            loco.loco_compensate_quantize(list(zip(gs, e, codes, absmax)), bits=bits, block=block, beta=beta)
        torch.cuda.synchronize()
        for s, n in enumerate(sizes):
            for b0, b1 in ranges[s]:
                lo, hi = b0 * block, min(b1 * block, n)
                ref = oracle.compensate_quantize(storage(gs[s][lo:hi], gd), ora_e[(s, b0)], bits=bits, block=block,
                                                 beta=beta, grad_dtype=gd, err_dtype=ed, err_scale=err_scale,
                                                 reset=reset)
                t = f"{tag} step {step} seg {s} blocks {b0}:{b1}"
                assert_bytes_equal(host(codes[s][lo * bits // 8:(hi * bits + 7) // 8]), ref["codes"], f"{t} codes")
                assert_bytes_equal(host(absmax[s][b0:b1]).view(np.uint32), ref["absmax"].view(np.uint32),
                                   f"{t} absmax")
                if ed == "i8":
                    assert_bytes_equal(host(e[s][lo:hi]), ref["e_new"], f"{t} 8-bit error")
                elif ed == "f32":
                    bitwise &= assert_f32_close(host(e[s][lo:hi]), ref["e_new"],
                                                step_per_elem(ref["absmax"], bits, block, hi - lo), f"{t} error")
                else:
                    bitwise &= assert_bf16_close(bf16_bits(e[s][lo:hi]), ref["e_new"], f"{t} error")
                ora_e[(s, b0)] = ref["e_new"]
                checked += hi - lo
        del gs
    say(f"{tag}: {checked:,} sampled element-steps checked; error buffer bitwise equal: {bitwise}")


@pytest.mark.parametrize("bits,steps", [(4, 3), (8, 3)])
def test_fullsize_7b_shard(gpu_lib, bits, steps):
    """842,000,000 bf16 as 8 partitions of 105,250,000, fp32 error, block 256 (bench's launch)."""
    part, P = W.SHARD7B_PART, W.SHARD7B_PEERS

    def gen(step):
        g = W.shard7b_grad(step, n=W.SHARD7B_N, device="cuda", chain=f"full{bits}")
        return [g[i * part:(i + 1) * part] for i in range(P)]
    fullsize_cq(gpu_lib, [part] * P, "bf16", "f32", bits, 256, 0.9, steps, gen, f"7b-shard {bits}-bit")


def test_fullsize_7b_shard_i8_error(gpu_lib):
    """The 7B shard with the paper's 8-bit error (s_e = 2^17) reset every T_c = 3 steps, 4 steps."""
    part, P = W.SHARD7B_PART, W.SHARD7B_PEERS

    def gen(step):
        g = W.shard7b_grad(step, n=W.SHARD7B_N, device="cuda", chain="full-i8")
        return [g[i * part:(i + 1) * part] for i in range(P)]
    fullsize_cq(gpu_lib, [part] * P, "bf16", "i8", 4, 256, 0.9, 4, gen, "7b-shard 4-bit, 8-bit error",
                seed=8, err_scale=2.0 ** 17, reset_every=3)


def test_fullsize_llama_layer(gpu_lib):
    """One LLaMA-7B layer's 7 gradients (202,375,168 bf16), fp32 error, 4-bit, block 128, 5 steps."""
    sizes = [r * c for _, r, c in W.llama_layer_shapes()]
    fullsize_cq(gpu_lib, sizes, "bf16", "f32", 4, 128, 0.9, 5,
                lambda s: W.llama_layer_grads(s, device="cuda"), "llama layer")


def test_fullsize_moe(gpu_lib):
    """8 experts x 3 matrices (1,409,286,144 bf16, 30% zero rows), bf16 error, 4-bit, block 128, 3 steps."""
    sizes = [r * c for _, _, r, c in W.moe_shapes()]
    fullsize_cq(gpu_lib, sizes, "bf16", "bf16", 4, 128, 0.9, 3,
                lambda s: W.moe_grads(s, device="cuda"), "moe", seed=4)


def test_fullsize_dequant_reduce_7b(gpu_lib):
    """8 peer payloads of 105,250,000 (4-bit, block 256) into bf16 x 1/8, as bench launches it."""
    n, P, bits, block = W.SHARD7B_PART, W.SHARD7B_PEERS, 4, 256
    say("dr full: generating 8 payloads")
    pays = [W.random_payload(n, bits, block, key=("full", p), device="cuda") for p in range(P)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    gpu_lib.loco_dequant_reduce(pays, n, bits=bits, block=block, out=out, out_scale=1.0 / P)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    for b0, b1 in block_ranges(-(-n // block), rng, count=64):
        lo, hi = b0 * block, min(b1 * block, n)
        sl = [(host(c[lo * bits // 8:(hi * bits + 7) // 8]), host(a[b0:b1])) for c, a in pays]
        want = oracle.dequant_reduce(sl, hi - lo, bits=bits, block=block, out_scale=1.0 / P, out_dtype="bf16")
        assert_bf16_close(bf16_bits(out[lo:hi]), want, f"dr full blocks {b0}:{b1}")


def test_fullsize_sparseloco(gpu_lib):
    """2^28 fp32, chunk 4096, k = 82, 2-bit, decay 1, 5 steps; sampled chunks follow the oracle."""
    n, C, k, bits = W.SPARSE_N, 4096, 82, 2
    chunks = n // C
    dev = "cuda"
    e = torch.zeros(n, device=dev)
    idx = torch.empty(chunks * k, dtype=torch.int16, device=dev)
    codes = torch.empty(chunks * gpu_lib.code_bytes(k, bits), dtype=torch.uint8, device=dev)
    am = torch.empty(chunks, device=dev)
    rng = np.random.default_rng(5)
    sample = sorted({0, chunks - 1} | set(int(x) for x in rng.integers(0, chunks, 48)))
    ora_e = {c: np.zeros(C, np.float32) for c in sample}
    nb = gpu_lib.code_bytes(k, bits)
    for step in range(5):
        say(f"sparseloco full: step {step}")
        g = W.sparseloco_grad(step, n=n, device=dev)
        gpu_lib.loco_topk_quantize(g, e, chunk=C, k=k, idx=idx, codes=codes, absmax=am, bits=bits, ef_decay=1.0)
        torch.cuda.synchronize()
        for c in sample:
            lo, hi = c * C, (c + 1) * C
            ref = oracle.topk_quantize(host(g[lo:hi]), ora_e[c], chunk=C, k=k, bits=bits, decay=1.0)
            t = f"sparseloco step {step} chunk {c}"
            assert_bytes_equal(host(idx[c * k:(c + 1) * k]).view(np.uint16), ref["idx"], f"{t} idx")
            assert_bytes_equal(host(codes[c * nb:(c + 1) * nb]), ref["codes"], f"{t} codes")
            assert_bytes_equal(host(am[c:c + 1]).view(np.uint32), ref["absmax"].view(np.uint32), f"{t} absmax")
            assert_f32_close(host(e[lo:hi]), ref["e_new"], np.full(C, float(ref["absmax"][0])), f"{t} error")
            ora_e[c] = ref["e_new"]
        del g


def test_fullsize_sparse_aggregate(gpu_lib):
    """8 peers' Top-k payloads of 2^28 (chunk 4096, k = 82, 2-bit) into fp32 x 1/8, as bench
    launches it; sampled chunks against the oracle."""
    n, C, k, bits, P = W.SPARSE_N, 4096, 82, 2, 8
    cb = gpu_lib.code_bytes(k, bits)
    say("sparse aggregate full: generating 8 payloads")
    pays = [W.random_sparse_payload(n, C, k, bits, key=("full", p), device="cuda") for p in range(P)]
    out = torch.empty(n, device="cuda")
    gpu_lib.loco_sparse_aggregate(pays, n, chunk=C, k=k, bits=bits, out=out, out_scale=1.0 / P)
    torch.cuda.synchronize()
    chunks = n // C
    rng = np.random.default_rng(11)
    sample = sorted({0, chunks - 1} | set(int(x) for x in rng.integers(0, chunks, 64)))
    for c in sample:
        sl = [(host(ix[c * k:(c + 1) * k]).view(np.uint16), host(cd[c * cb:(c + 1) * cb]), host(a[c:c + 1]))
              for ix, cd, a in pays]
        want = oracle.sparse_aggregate(sl, C, chunk=C, k=k, bits=bits, out_scale=1.0 / P)
        assert_f32_close(host(out[c * C:(c + 1) * C]), want, np.zeros(C), f"sparse aggregate chunk {c}")
    say(f"sparse aggregate full: {len(sample)} chunks checked")


def test_fullsize_dequant_reduce_adam_7b(gpu_lib):
    """8 peer payloads of 105,250,000 (4-bit, block 256) averaged and fed to one Adam step on
    fp32 weights and moments with a bf16 weight copy, as bench launches it; 2 steps on
    sampled blocks."""
    n, P, bits, block = W.SHARD7B_PART, W.SHARD7B_PEERS, 4, 256
    hp = dict(lr=1e-4, beta1=0.1, beta2=0.01, delta=1e-8)
    th = (torch.randn(n, device="cuda") * 0.02).contiguous()
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    tb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(9)
    ranges = block_ranges(-(-n // block), rng, count=48)
    ora = {}
    for b0, b1 in ranges:
        lo, hi = b0 * block, min(b1 * block, n)
        ora[b0] = (host(th[lo:hi]).copy(), np.zeros(hi - lo, np.float32), np.zeros(hi - lo, np.float32))
    for step in range(2):
        say(f"dra full: step {step}, generating 8 payloads")
        pays = [W.random_payload(n, bits, block, key=("dra-full", step, p), device="cuda") for p in range(P)]
        gpu_lib.loco_dequant_reduce_adam(pays, n, bits=bits, block=block, out_scale=1.0 / P, param=th, m=m, v=v,
                                         param_bf16=tb, **hp)
        torch.cuda.synchronize()
        for b0, b1 in ranges:
            lo, hi = b0 * block, min(b1 * block, n)
            sl = [(host(c[lo * bits // 8:(hi * bits + 7) // 8]), host(a[b0:b1])) for c, a in pays]
            o_th, o_m, o_v = ora[b0]
            ref = oracle.dequant_reduce_adam(sl, hi - lo, bits=bits, block=block, out_scale=1.0 / P, theta=o_th,
                                             m=o_m, v=o_v, **hp)
            z = np.zeros(hi - lo)
            t = f"dra full step {step} blocks {b0}:{b1}"
            assert_f32_close(host(m[lo:hi]), ref["m"], z, f"{t} m")
            assert_f32_close(host(v[lo:hi]), ref["v"], z, f"{t} v")
            assert_f32_close(host(th[lo:hi]), ref["theta"], z, f"{t} theta")
            assert_bf16_close(bf16_bits(tb[lo:hi]), ref["theta_bf16"], f"{t} theta bf16")
            ora[b0] = (ref["theta"], ref["m"], ref["v"])
        del pays
    say(f"dra full: {len(ranges)} block runs checked")
