"""Parity at the workloads' full sizes, in the launch configuration bench.py times, on
every element of every step.

The GPU processes the whole tensors.  The oracle, unchanged, follows its own free-running
chain over the whole arrays: it runs in spawned worker processes over slabs of whole scale
blocks (whole chunks for Top-k and the sparse aggregation), which are independent of one
another, with the arrays shared through /dev/shm (tests/fullsize_pool.py).  Inputs are
generated on the GPU by the seeded generators and copied out for the oracle.  Before each
launch the outputs are filled with sentinels (NaN scales and outputs, a code byte that
alternates between steps), so a tile the kernel never writes cannot pass.  Each test logs
"N of N elements checked" per step.
"""
import numpy as np
import pytest
import torch

import fullsize_pool as FP
import workloads as W
from parity_util import say

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}
SLAB = 1 << 21       # elements per oracle task (a multiple of every block size)
TK_SLAB_CHUNKS = 256  # chunks per Top-k / sparse-aggregation task


def to_shared(dst, t):
    """Copy a device tensor's bytes into a shared array of the same element size."""
    src = t.detach().contiguous().view(-1)
    d = torch.from_numpy(dst)
    if src.dtype != d.dtype:
        src = src.view(d.dtype)
    d.copy_(src)


def code_sentinel(step):
    return 0xA5 if step % 2 == 0 else 0x5A


def check(pool, fn, tasks, total, tag):
    n, bad, bitwise = FP.run(pool, fn, tasks)
    assert not bad, f"{tag}:\n" + "\n".join(bad)
    assert n == total, f"{tag}: {n} of {total} elements checked"
    say(f"{tag}: {n:,} of {total:,} elements checked against the oracle; floats bitwise equal: {bitwise}")


def fullsize_cq(loco, pool, sizes, gd, ed, bits, block, beta, steps, gen, tag, err_scale=0.0, reset_every=0):
    dev = "cuda"
    total = sum(sizes)
    offs, coffs, boffs = FP.cq_layout(sizes, bits, block)
    cbytes = [loco.code_bytes(n, bits) for n in sizes]
    nblk = [loco.num_blocks(n, block) for n in sizes]
    assert cbytes == np.diff(coffs).tolist() and nblk == np.diff(boffs).tolist()
    S = FP.SharedArrays()
    try:
        g_sh = S.new("g", total, gd)
        S.new("e_ora", total, ed)
        e_sh = S.new("e_gpu", total, ed)
        c_sh = S.new("codes", coffs[-1], "u8")
        a_sh = S.new("absmax", boffs[-1], "f32")
        e = torch.zeros(total, dtype=TD[ed], device=dev)
        codes = [torch.empty(c, dtype=torch.uint8, device=dev) for c in cbytes]
        absmax = [torch.empty(b, dtype=torch.float32, device=dev) for b in nblk]
        for step in range(steps):
            say(f"{tag}: step {step}: generating and launching ({total:,} elements, {len(sizes)} segments)")
            gs = gen(step)
            assert [g.numel() for g in gs] == list(sizes)
            for s, g in enumerate(gs):
                to_shared(g_sh[offs[s]:offs[s + 1]], g)
                codes[s].fill_(code_sentinel(step))
                absmax[s].view(torch.int32).fill_(-1)  # NaN
            reset = reset_every > 0 and (step + 1) % reset_every == 0
            segs = [(gs[s], e[offs[s]:offs[s + 1]], codes[s], absmax[s]) for s in range(len(sizes))]
            if ed == "i8" or reset_every:
                loco.loco_compensate_quantize_ex(segs, bits=bits, block=block, beta=beta, err_scale=err_scale,
                                                 reset_error=reset)
            else:
                loco.loco_compensate_quantize(segs, bits=bits, block=block, beta=beta)
            torch.cuda.synchronize()
            to_shared(e_sh, e)
            for s in range(len(sizes)):
                to_shared(c_sh[coffs[s]:coffs[s + 1]], codes[s])
                to_shared(a_sh[boffs[s]:boffs[s + 1]], absmax[s])
            assert not np.isnan(np.asarray(a_sh)).any(), f"{tag} step {step}: an absmax was never written"
            del gs, segs
            tasks = FP.cq_tasks(S, sizes, SLAB, bits=bits, block=block, beta=beta, gd=gd, ed=ed,
                                err_scale=err_scale, reset=reset, tag=f"{tag} step {step}")
            check(pool, FP.cq_task, tasks, total, f"{tag} step {step}")
    finally:
        S.close()


@pytest.mark.parametrize("bits,steps", [(4, 3), (8, 3)])
def test_fullsize_7b_shard(gpu_lib, oracle_pool, bits, steps):
    """842,000,000 bf16 as 8 partitions of 105,250,000, fp32 error, block 256 (bench's launch)."""
    part, P = W.SHARD7B_PART, W.SHARD7B_PEERS

    def gen(step):
        g = W.shard7b_grad(step, n=W.SHARD7B_N, device="cuda", chain=f"full{bits}")
        return [g[i * part:(i + 1) * part] for i in range(P)]
    fullsize_cq(gpu_lib, oracle_pool, [part] * P, "bf16", "f32", bits, 256, 0.9, steps, gen, f"7b-shard {bits}-bit")


def test_fullsize_7b_shard_i8_error(gpu_lib, oracle_pool):
    """The 7B shard with the paper's 8-bit error (s_e = 2^17) reset every T_c = 3 steps, 4 steps."""
    part, P = W.SHARD7B_PART, W.SHARD7B_PEERS

    def gen(step):
        g = W.shard7b_grad(step, n=W.SHARD7B_N, device="cuda", chain="full-i8")
        return [g[i * part:(i + 1) * part] for i in range(P)]
    fullsize_cq(gpu_lib, oracle_pool, [part] * P, "bf16", "i8", 4, 256, 0.9, 4, gen, "7b-shard 4-bit, 8-bit error",
                err_scale=2.0 ** 17, reset_every=3)


def test_fullsize_llama_layer(gpu_lib, oracle_pool):
    """One LLaMA-7B layer's 7 gradients (202,375,168 bf16), fp32 error, 4-bit, block 128, 5 steps."""
    sizes = [r * c for _, r, c in W.llama_layer_shapes()]
    fullsize_cq(gpu_lib, oracle_pool, sizes, "bf16", "f32", 4, 128, 0.9, 5,
                lambda s: W.llama_layer_grads(s, device="cuda"), "llama layer")


def test_fullsize_moe(gpu_lib, oracle_pool):
    """8 experts x 3 matrices (1,409,286,144 bf16, 30% zero rows), bf16 error, 4-bit, block 128, 3 steps."""
    sizes = [r * c for _, _, r, c in W.moe_shapes()]
    fullsize_cq(gpu_lib, oracle_pool, sizes, "bf16", "bf16", 4, 128, 0.9, 3,
                lambda s: W.moe_grads(s, device="cuda"), "moe")


def shared_payloads(S, loco, pays, n, bits, block):
    """The peers' codes and absmax, concatenated in shared arrays; returns their offsets."""
    cb, nb = loco.code_bytes(n, bits), loco.num_blocks(n, block)
    c_sh = S.new("codes", cb * len(pays), "u8")
    a_sh = S.new("absmax", nb * len(pays), "f32")
    for p, (c, a) in enumerate(pays):
        to_shared(c_sh[p * cb:(p + 1) * cb], c)
        to_shared(a_sh[p * nb:(p + 1) * nb], a)
    return [p * cb for p in range(len(pays))], [p * nb for p in range(len(pays))]


def test_fullsize_dequant_reduce_7b(gpu_lib, oracle_pool):
    """8 peer payloads of 105,250,000 (4-bit, block 256) into bf16 x 1/8, as bench launches it."""
    n, P, bits, block = W.SHARD7B_PART, W.SHARD7B_PEERS, 4, 256
    say("dr full: generating 8 payloads")
    pays = [W.random_payload(n, bits, block, key=("full", p), device="cuda") for p in range(P)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    out.view(torch.int16).fill_(-1)  # NaN
    gpu_lib.loco_dequant_reduce(pays, n, bits=bits, block=block, out=out, out_scale=1.0 / P)
    torch.cuda.synchronize()
    S = FP.SharedArrays()
    try:
        coffs, boffs = shared_payloads(S, gpu_lib, pays, n, bits, block)
        to_shared(S.new("out", n, "bf16"), out)
        base = dict(codes=S.spec("codes"), absmax=S.spec("absmax"), coffs=coffs, boffs=boffs, out=S.spec("out"),
                    bits=bits, block=block, out_scale=1.0 / P, out_dtype="bf16", tag="dr full")
        tasks = [dict(base, lo=lo, hi=min(lo + SLAB, n)) for lo in range(0, n, SLAB)]
        check(oracle_pool, FP.dr_task, tasks, n, "dequant-reduce 8 x 105,250,000 -> bf16")
    finally:
        S.close()


def test_fullsize_dequant_reduce_adam_7b(gpu_lib, oracle_pool):
    """8 peer payloads of 105,250,000 (4-bit, block 256) averaged and fed to one Adam step on
    fp32 weights and moments with a bf16 weight copy, as bench launches it; 2 steps, the
    oracle keeping its own weights and moments."""
    n, P, bits, block = W.SHARD7B_PART, W.SHARD7B_PEERS, 4, 256
    hp = dict(lr=1e-4, beta1=0.1, beta2=0.01, delta=1e-8)
    th = (torch.randn(n, device="cuda") * 0.02).contiguous()
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    tb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    S = FP.SharedArrays()
    try:
        to_shared(S.new("theta_ora", n, "f32"), th)
        S.new("m_ora", n, "f32")
        S.new("v_ora", n, "f32")
        outs = {k: S.new(f"{k}_gpu", n, "f32") for k in ("theta", "m", "v")}
        tb_sh = S.new("tb_gpu", n, "bf16")
        for step in range(2):
            say(f"dra full: step {step}, generating 8 payloads")
            pays = [W.random_payload(n, bits, block, key=("dra-full", step, p), device="cuda") for p in range(P)]
            tb.view(torch.int16).fill_(-1)
            gpu_lib.loco_dequant_reduce_adam(pays, n, bits=bits, block=block, out_scale=1.0 / P, param=th, m=m, v=v,
                                             param_bf16=tb, **hp)
            torch.cuda.synchronize()
            for k, t in (("theta", th), ("m", m), ("v", v)):
                to_shared(outs[k], t)
            to_shared(tb_sh, tb)
            coffs, boffs = shared_payloads(S, gpu_lib, pays, n, bits, block)
            del pays
            base = dict(codes=S.spec("codes"), absmax=S.spec("absmax"), coffs=coffs, boffs=boffs, bits=bits,
                        block=block, out_scale=1.0 / P, adam=hp, tag=f"dra full step {step}",
                        **{f"{k}_ora": S.spec(f"{k}_ora") for k in ("theta", "m", "v")},
                        **{f"{k}_gpu": S.spec(f"{k}_gpu") for k in ("theta", "m", "v")}, tb_gpu=S.spec("tb_gpu"))
            tasks = [dict(base, lo=lo, hi=min(lo + SLAB, n)) for lo in range(0, n, SLAB)]
            check(oracle_pool, FP.dr_task, tasks, n, f"dequant-reduce + Adam step {step}")
    finally:
        S.close()


def test_fullsize_sparseloco(gpu_lib, oracle_pool):
    """2^28 fp32, chunk 4096, k = 82, 2-bit, decay 1, 5 steps; every chunk follows the oracle."""
    n, C, k, bits = W.SPARSE_N, 4096, 82, 2
    chunks = n // C
    nb = gpu_lib.code_bytes(k, bits)
    dev = "cuda"
    e = torch.zeros(n, device=dev)
    idx = torch.empty(chunks * k, dtype=torch.int16, device=dev)
    codes = torch.empty(chunks * nb, dtype=torch.uint8, device=dev)
    am = torch.empty(chunks, device=dev)
    S = FP.SharedArrays()
    try:
        g_sh = S.new("g", n, "f32")
        S.new("e_ora", n, "f32")
        e_sh = S.new("e_gpu", n, "f32")
        i_sh = S.new("idx", chunks * k, "u16")
        c_sh = S.new("codes", chunks * nb, "u8")
        a_sh = S.new("absmax", chunks, "f32")
        for step in range(5):
            say(f"sparseloco full: step {step}")
            g = W.sparseloco_grad(step, n=n, device=dev)
            to_shared(g_sh, g)
            idx.fill_(0x5A5A)
            codes.fill_(code_sentinel(step))
            am.view(torch.int32).fill_(-1)
            gpu_lib.loco_topk_quantize(g, e, chunk=C, k=k, idx=idx, codes=codes, absmax=am, bits=bits, ef_decay=1.0)
            torch.cuda.synchronize()
            del g
            for dst, t in ((e_sh, e), (i_sh, idx), (c_sh, codes), (a_sh, am)):
                to_shared(dst, t)
            base = dict(g=S.spec("g"), e_ora=S.spec("e_ora"), e_gpu=S.spec("e_gpu"), idx=S.spec("idx"),
                        codes=S.spec("codes"), absmax=S.spec("absmax"), n=n, chunk=C, k=k, bits=bits, decay=1.0,
                        tag=f"sparseloco step {step}")
            tasks = [dict(base, c0=c0, c1=min(c0 + TK_SLAB_CHUNKS, chunks)) for c0 in range(0, chunks, TK_SLAB_CHUNKS)]
            check(oracle_pool, FP.tk_task, tasks, n, f"sparseloco top-k step {step}")
    finally:
        S.close()


def test_fullsize_sparse_aggregate(gpu_lib, oracle_pool):
    """8 peers' Top-k payloads of 2^28 (chunk 4096, k = 82, 2-bit) into fp32 x 1/8, as bench
    launches it; every chunk against the oracle."""
    n, C, k, bits, P = W.SPARSE_N, 4096, 82, 2, 8
    chunks = n // C
    nb = gpu_lib.code_bytes(k, bits)
    say("sparse aggregate full: generating 8 payloads")
    pays = [W.random_sparse_payload(n, C, k, bits, key=("full", p), device="cuda") for p in range(P)]
    out = torch.empty(n, device="cuda")
    out.view(torch.int32).fill_(-1)
    gpu_lib.loco_sparse_aggregate(pays, n, chunk=C, k=k, bits=bits, out=out, out_scale=1.0 / P)
    torch.cuda.synchronize()
    S = FP.SharedArrays()
    try:
        i_sh = S.new("idx", P * chunks * k, "u16")
        c_sh = S.new("codes", P * chunks * nb, "u8")
        a_sh = S.new("absmax", P * chunks, "f32")
        for p, (ix, c, a) in enumerate(pays):
            to_shared(i_sh[p * chunks * k:(p + 1) * chunks * k], ix)
            to_shared(c_sh[p * chunks * nb:(p + 1) * chunks * nb], c)
            to_shared(a_sh[p * chunks:(p + 1) * chunks], a)
        to_shared(S.new("out", n, "f32"), out)
        base = dict(idx=S.spec("idx"), codes=S.spec("codes"), absmax=S.spec("absmax"), out=S.spec("out"),
                    ioffs=[p * chunks * k for p in range(P)], coffs=[p * chunks * nb for p in range(P)],
                    aoffs=[p * chunks for p in range(P)], n=n, chunk=C, k=k, bits=bits, out_scale=1.0 / P,
                    tag="sparse aggregate")
        tasks = [dict(base, c0=c0, c1=min(c0 + TK_SLAB_CHUNKS, chunks)) for c0 in range(0, chunks, TK_SLAB_CHUNKS)]
        check(oracle_pool, FP.sa_task, tasks, n, "sparse aggregation 8 x 2^28 -> fp32")
    finally:
        S.close()
