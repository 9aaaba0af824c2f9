"""GPU parity of loco_compensate_quantize against the CPU oracle.

Every case runs a free-running chain: the GPU keeps its error buffer, the oracle keeps
its own, both start from zero and see the same seeded gradients.  Codes and absmax must
be bit-exact; the error buffer within 1e-6 relative (floor 1e-6 * step) in fp32 or
1 ulp in bf16 (bitwise equality is expected and reported).  Every output buffer has
canaries on both sides.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import (Guarded, assert_bf16_close, assert_bytes_equal, assert_f32_close, bf16_bits, host,
                         say, step_per_elem)

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}
EDGE_SIZES = [1, 0, 7, 8, 9, 511, 512, 513, 1023, 1024, 1025, 4099, 65536 + 17]


def grads(step, n, gd, key, scale=None):
    if gd == "bf16":
        x = W.shard7b_grad(step, n=n, chain=key)
    else:
        x = W.tiny_grad(step, n=n, stream=key)
    if scale is not None:
        x = (x.float() * scale).to(TD[gd])
    return x


def storage(t, dt):
    """CPU tensor -> the oracle's storage form (float32, int8, or uint16 bf16 patterns)."""
    if dt == "bf16":
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


ORA_E = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8}


def run_chain(loco, sizes, gd, ed, bits, block, beta, steps, fixed=0.0, gen=None, key="cq", err_scale=0.0,
              reset_every=0):
    """reset_every = T_c > 0 resets the error on steps T_c - 1, 2 T_c - 1, ... (Eqn. (7));
    an int8 error ('i8') has the scale err_scale.  Both go through the _ex entry point."""
    segs = []
    for n in sizes:
        g = Guarded(n, TD[gd])
        e = Guarded(n, TD[ed], init=torch.zeros(n, dtype=TD[ed]))
        c = Guarded(loco.code_bytes(n, bits), torch.uint8)
        a = None if fixed else Guarded(loco.num_blocks(n, block), torch.float32)
        segs.append((g, e, c, a))
    e_ora = [np.zeros(n, ORA_E[ed]) for n in sizes]
    use_ex = ed == "i8" or reset_every > 0
    bitwise = True
    total = sum(sizes)
    for step in range(steps):
        gall = gen(step, total) if gen else grads(step, total, gd, f"{key}-{bits}-{block}")
        off = 0
        for (g, _, _, _), n in zip(segs, sizes):
            g.t.copy_(gall[off:off + n])
            off += n
        reset = reset_every > 0 and (step + 1) % reset_every == 0
        args = [(g.t, e.t, c.t, None if a is None else a.t) for g, e, c, a in segs]
        if use_ex:
            loco.loco_compensate_quantize_ex(args, bits=bits, block=block, beta=beta, fixed_scale=fixed,
                                             err_scale=err_scale, reset_error=reset)
        else:
            loco.loco_compensate_quantize(args, bits=bits, block=block, beta=beta, fixed_scale=fixed)
        torch.cuda.synchronize()
        off = 0
        for i, ((g, e, c, a), n) in enumerate(zip(segs, sizes)):
            gn = storage(gall[off:off + n], gd)
            off += n
            ref = oracle.compensate_quantize(gn, e_ora[i], bits=bits, block=block, beta=beta,
                                             fixed_scale=fixed, grad_dtype=gd, err_dtype=ed,
                                             err_scale=err_scale, reset=reset)
            tag = f"step {step} segment {i} (n={n})"
            assert_bytes_equal(host(c.t), ref["codes"], f"{tag} codes")
            if a is not None:
                assert_bytes_equal(host(a.t).view(np.uint32), ref["absmax"].view(np.uint32), f"{tag} absmax")
            if ed == "i8":
                # the 8-bit codes are integer decisions taken in fp32 on both sides: bit-exact
                assert_bytes_equal(host(e.t), ref["e_new"], f"{tag} 8-bit error")
            elif ed == "f32":
                floor = (step_per_elem(ref["absmax"], bits, block, n) if a is not None
                         else np.full(n, 1.0 / fixed))
                bitwise &= assert_f32_close(host(e.t), ref["e_new"], floor, f"{tag} error")
            else:
                bitwise &= assert_bf16_close(bf16_bits(e.t), ref["e_new"], f"{tag} error")
            e_ora[i] = ref["e_new"]
            for b, nm in zip((g, e, c, a), ("grad", "err", "codes", "absmax")):
                if b is not None:
                    b.check(f"{tag} {nm}")
    return bitwise


def test_cq_tiny_workload(gpu_lib):
    """1,048,576 fp32 ~ N(0, 1e-3), fp32 error, 4-bit, block 128, beta 0.9, 10 steps."""
    say("cq tiny: n=1048576 f32/f32 4-bit B=128 beta=0.9 x10")
    bw = run_chain(gpu_lib, [W.TINY_N], "f32", "f32", 4, 128, 0.9, 10,
                   gen=lambda s, n: W.tiny_grad(s, n=n))
    say("  error buffer bitwise equal:", bw)


@pytest.mark.parametrize("gd", ["f32", "bf16"])
@pytest.mark.parametrize("ed", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("block", [64, 128, 256, 512])
def test_cq_matrix(gpu_lib, gd, ed, bits, block):
    """Every dtype pair, code width and block size on ragged multi-segment calls."""
    say(f"cq matrix {gd}/{ed} bits={bits} B={block} sizes={EDGE_SIZES}")
    run_chain(gpu_lib, EDGE_SIZES, gd, ed, bits, block, 0.9, 2, key="matrix")


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0, 0.99])
def test_cq_beta(gpu_lib, beta):
    say(f"cq beta={beta}")
    run_chain(gpu_lib, [4096 + 5, 300_001], "bf16", "f32", 4, 128, beta, 3, key=f"beta{beta}")


@pytest.mark.parametrize("gd", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("s", [2.0 ** 19, 2.0 ** 17])
def test_cq_fixed_scale(gpu_lib, gd, bits, s):
    """Eqn. (1) with the paper's global scale; bf16 inputs near 1e-5 hit exact .5 ties
    and the clamp at both ends."""
    say(f"cq fixed scale s={s} {gd} bits={bits}")
    run_chain(gpu_lib, [1, 1000, 70_001], gd, "f32", bits, 128, 0.9, 3, fixed=s,
              gen=lambda st, n: grads(st, n, gd, "fixed", scale=1e-2))


def test_cq_zero_blocks(gpu_lib):
    """All-zero blocks and rows keep zero codes, zero absmax and a zero error."""
    def gen(step, n):
        x = grads(step, n, "bf16", "zeros").float()
        x[128:1024] = 0
        x[5000:9000] = 0
        x[-300:] = 0
        return x.to(torch.bfloat16)
    say("cq zero blocks")
    run_chain(gpu_lib, [20_000, 333], "bf16", "bf16", 4, 128, 0.9, 3, gen=gen)


def test_cq_many_segments(gpu_lib):
    """75 segments in one call: more than one launch's segment table."""
    rng = np.random.default_rng(75)
    sizes = [int(x) for x in rng.integers(0, 3000, 75)]
    say(f"cq 75 segments, total {sum(sizes)}")
    run_chain(gpu_lib, sizes, "bf16", "f32", 4, 64, 0.9, 2, key="many")


def test_cq_llama_layer_scaled(gpu_lib):
    """The LLaMA-7B layer recipe with rows / 64: 7 bf16 tensors, fp32 error, 4-bit, B=128."""
    shapes = W.llama_layer_shapes(64)
    sizes = [r * c for _, r, c in shapes]
    say(f"cq llama layer /64: {sizes}")
    run_chain(gpu_lib, sizes, "bf16", "f32", 4, 128, 0.9, 5,
              gen=lambda s, n: torch.cat(W.llama_layer_grads(s, div=64)))


def test_cq_moe_scaled(gpu_lib):
    """The MoE recipe with rows / 256: 24 bf16 matrices with 30% zero rows, bf16 error."""
    shapes = W.moe_shapes(256)
    sizes = [r * c for _, _, r, c in shapes]
    say(f"cq moe /256: {len(sizes)} segments")
    run_chain(gpu_lib, sizes, "bf16", "bf16", 4, 128, 0.9, 3,
              gen=lambda s, n: torch.cat(W.moe_grads(s, div=256)))


@pytest.mark.parametrize("bits", [4, 8])
def test_cq_shard_scaled(gpu_lib, bits):
    """The 7B-shard recipe at 1/1024 size, split into 8 partitions, B=256."""
    n = W.SHARD7B_N // 1024
    part = -(-n // 8)
    sizes = [part] * 7 + [n - 7 * part]
    say(f"cq shard /1024 bits={bits} sizes={sizes}")
    run_chain(gpu_lib, sizes, "bf16", "f32", bits, 256, 0.9, 3,
              gen=lambda s, m: W.shard7b_grad(s, n=m, chain=f"small{bits}"))


def test_cq_deterministic_and_stream(gpu_lib):
    """Two identical calls give identical bytes, also on a non-default stream."""
    n = 200_003
    g = W.shard7b_grad(0, n=n).cuda()
    outs = []
    for use_stream in (False, True):
        e = torch.full((n,), 1e-4, dtype=torch.float32, device="cuda")
        c = torch.empty(gpu_lib.code_bytes(n, 4), dtype=torch.uint8, device="cuda")
        a = torch.empty(gpu_lib.num_blocks(n, 256), dtype=torch.float32, device="cuda")
        st = torch.cuda.Stream() if use_stream else None
        if st is not None:
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                gpu_lib.loco_compensate_quantize([(g, e, c, a)], bits=4, block=256, beta=0.9)
            st.synchronize()
        else:
            gpu_lib.loco_compensate_quantize([(g, e, c, a)], bits=4, block=256, beta=0.9)
        torch.cuda.synchronize()
        outs.append((host(c), host(a), host(e)))
    for x, y in zip(outs[0], outs[1]):
        assert np.array_equal(x, y)


# -- the paper's 8-bit error and its periodic reset (LoCo Sec. 3.2, Eqn. (7)) ---------------

ES = {"f32": 4, "bf16": 2, "i8": 1}


@pytest.mark.parametrize("gd,ed", [("bf16", "f32"), ("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"),
                                   ("bf16", "i8")])
@pytest.mark.parametrize("block", [64, 256])
def test_cq_segments_inside_lines(gpu_lib, gd, ed, block):
    """Segments that are views into one flat gradient and one flat error, as an FSDP
    rank's partitions are, starting at every 16-byte-aligned offset within a 128-byte line
    that the element sizes allow.  A wave tile's first and last line of a stream then also
    hold a neighbouring tile's elements, and the kernel loads the lanes in those lines
    with another cache policy; the results must be the oracle's all the same (3-step
    chain, 4-bit, several tiles per segment)."""
    g16 = max(16 // ES[gd], 16 // ES[ed])  # elements per 16 bytes of the sparser stream
    sizes = [g16 * (597 + k) for k in range(16)]
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]]).tolist()
    total = sum(sizes)
    say(f"cq segments inside lines: {gd}/{ed} B={block}, 16 segments of {sizes[0]}..{sizes[-1]}")
    gflat = torch.empty(total, dtype=TD[gd], device="cuda")
    eflat = torch.zeros(total, dtype=TD[ed], device="cuda")
    # every start offset within a line that 16-byte alignment allows is present
    for flat, es in ((gflat, ES[gd]), (eflat, ES[ed])):
        got = {(flat.data_ptr() + o * es) % 128 for o in starts}
        assert got == set(range(0, 128, g16 * es)), (got, es)
    codes = [Guarded(gpu_lib.code_bytes(n, 4), torch.uint8) for n in sizes]
    absmax = [Guarded(gpu_lib.num_blocks(n, block), torch.float32) for n in sizes]
    e_ora = [np.zeros(n, ORA_E[ed]) for n in sizes]
    s_e = 2.0 ** 17 if ed == "i8" else 0.0
    bitwise = True
    for step in range(3):
        gall = grads(step, total, gd, f"inline-{gd}-{ed}-{block}")
        gflat.copy_(gall.to("cuda"))
        segs = [(gflat[o:o + n], eflat[o:o + n], c.t, a.t) for o, n, c, a in zip(starts, sizes, codes, absmax)]
        gpu_lib.loco_compensate_quantize_ex(segs, bits=4, block=block, beta=0.9, err_scale=s_e)
        torch.cuda.synchronize()
        for i, (o, n) in enumerate(zip(starts, sizes)):
            ref = oracle.compensate_quantize(storage(gall[o:o + n], gd), e_ora[i], bits=4, block=block, beta=0.9,
                                             grad_dtype=gd, err_dtype=ed, err_scale=s_e)
            tag = f"step {step} segment {i} (start {o}, n={n})"
            assert_bytes_equal(host(codes[i].t), ref["codes"], f"{tag} codes")
            assert_bytes_equal(host(absmax[i].t).view(np.uint32), ref["absmax"].view(np.uint32), f"{tag} absmax")
            e_seg = eflat[o:o + n]
            if ed == "i8":
                assert_bytes_equal(host(e_seg), ref["e_new"], f"{tag} 8-bit error")
            elif ed == "f32":
                bitwise &= assert_f32_close(host(e_seg), ref["e_new"], step_per_elem(ref["absmax"], 4, block, n),
                                            f"{tag} error")
            else:
                bitwise &= assert_bf16_close(bf16_bits(e_seg), ref["e_new"], f"{tag} error")
            e_ora[i] = ref["e_new"]
            codes[i].check(f"{tag} codes")
            absmax[i].check(f"{tag} absmax")
    say("  error buffer bitwise equal:", bitwise)


@pytest.mark.parametrize("s_e", [2.0 ** 18, 300_000.0])
def test_cq_i8_error_tiny(gpu_lib, s_e):
    """The tiny workload with the error in 8 bits (s_e a power of two, and not), reset
    every T_c = 5 steps, 12 steps."""
    say(f"cq i8 error tiny: s_e={s_e} T_c=5 x12")
    run_chain(gpu_lib, [W.TINY_N], "f32", "i8", 4, 128, 0.9, 12, gen=lambda s, n: W.tiny_grad(s, n=n),
              err_scale=s_e, reset_every=5)


@pytest.mark.parametrize("gd", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("block", [64, 512])
def test_cq_i8_matrix(gpu_lib, gd, bits, block):
    """8-bit error with every code width on the ragged multi-segment sizes."""
    say(f"cq i8 matrix {gd} bits={bits} B={block}")
    run_chain(gpu_lib, EDGE_SIZES, gd, "i8", bits, block, 0.9, 3, key="i8matrix", err_scale=2.0 ** 18)


@pytest.mark.parametrize("s_e", [2.0 ** 22, 5.0e6])
def test_cq_i8_error_clamps(gpu_lib, s_e):
    """A scale too large for the error's range: many codes clamp at -128 and 127."""
    say(f"cq i8 clamping s_e={s_e}")
    run_chain(gpu_lib, [70_001, 513], "bf16", "i8", 4, 256, 0.9, 4, key="i8clamp", err_scale=s_e)


def test_cq_i8_fixed_scale(gpu_lib):
    """Eqn. (1) with a global scale and the error in 8 bits: the paper's own configuration."""
    say("cq i8 + fixed scale")
    run_chain(gpu_lib, [1000, 70_001], "bf16", "i8", 4, 128, 0.9, 4, fixed=2.0 ** 19,
              gen=lambda st, n: grads(st, n, "bf16", "i8fixed", scale=1e-2), err_scale=2.0 ** 21)


@pytest.mark.parametrize("ed", ["f32", "bf16"])
def test_cq_reset_float_error(gpu_lib, ed):
    """The reset of Eqn. (7) on a float error: reset on every other step."""
    say(f"cq reset every 2 steps, {ed} error")
    run_chain(gpu_lib, EDGE_SIZES, "bf16", ed, 4, 128, 0.9, 5, key="reset", reset_every=2)


def test_cq_i8_llama_layer_scaled(gpu_lib):
    """The LLaMA-7B layer recipe with rows / 64, 8-bit error, T_c = 4."""
    shapes = W.llama_layer_shapes(64)
    sizes = [r * c for _, r, c in shapes]
    say(f"cq i8 llama layer /64: {sizes}")
    run_chain(gpu_lib, sizes, "bf16", "i8", 4, 128, 0.9, 6,
              gen=lambda s, n: torch.cat(W.llama_layer_grads(s, div=64)), err_scale=2.0 ** 18, reset_every=4)


@pytest.mark.parametrize("ed", ["f32", "bf16", "i8"])
def test_cq_teacher_forced(gpu_lib, ed):
    """Teacher-forced chain: before every step the GPU's error buffer is overwritten with
    the oracle's, so each step is compared from the same state (no compounding)."""
    n, bits, block, s_e = 300_007, 4, 128, 2.0 ** 17
    say(f"cq teacher-forced, {ed} error")
    g = Guarded(n, torch.bfloat16)
    e = Guarded(n, TD[ed], init=torch.zeros(n, dtype=TD[ed]))
    c = Guarded(gpu_lib.code_bytes(n, bits), torch.uint8)
    a = Guarded(gpu_lib.num_blocks(n, block), torch.float32)
    e_ora = np.zeros(n, ORA_E[ed])
    for step in range(4):
        x = grads(step, n, "bf16", "teacher")
        g.t.copy_(x)
        if ed == "bf16":
            e.t.copy_(torch.from_numpy(e_ora.view(np.int16)).view(torch.bfloat16))
        else:
            e.t.copy_(torch.from_numpy(e_ora))
        gpu_lib.loco_compensate_quantize_ex([(g.t, e.t, c.t, a.t)], bits=bits, block=block, beta=0.9,
                                            err_scale=s_e if ed == "i8" else 0.0)
        torch.cuda.synchronize()
        ref = oracle.compensate_quantize(storage(x, "bf16"), e_ora, bits=bits, block=block, beta=0.9,
                                         grad_dtype="bf16", err_dtype=ed, err_scale=s_e if ed == "i8" else 0.0)
        tag = f"teacher-forced step {step}"
        assert_bytes_equal(host(c.t), ref["codes"], f"{tag} codes")
        assert_bytes_equal(host(a.t).view(np.uint32), ref["absmax"].view(np.uint32), f"{tag} absmax")
        if ed == "i8":
            assert_bytes_equal(host(e.t), ref["e_new"], f"{tag} error")
        elif ed == "bf16":
            assert_bf16_close(bf16_bits(e.t), ref["e_new"], f"{tag} error")
        else:
            assert_f32_close(host(e.t), ref["e_new"], step_per_elem(ref["absmax"], bits, block, n), f"{tag} error")
        # the next step starts from a perturbed oracle state, not from the GPU's
        e_ora = ref["e_new"].copy()
        if ed == "f32":
            e_ora[::7] = np.float32(1e-4)
        for b, nm in ((g, "grad"), (e, "err"), (c, "codes"), (a, "absmax")):
            b.check(f"{tag} {nm}")


def test_cq_segments_share_a_gradient(gpu_lib):
    """Gradients are only read, so segments may overlap in them: two segments on the same
    gradient tensor (and a third on an overlapping slice of it) each give the oracle's
    result for their own range."""
    n = 100_000 + 37
    g = W.shard7b_grad(0, n=n, device="cuda", chain="shared")
    views = [(0, n), (0, n), (4096, n)]  # the third starts at a block-aligned offset
    outs = []
    for lo, hi in views:
        m = hi - lo
        outs.append((torch.zeros(m, device="cuda"),
                     torch.empty(gpu_lib.code_bytes(m, 4), dtype=torch.uint8, device="cuda"),
                     torch.empty(gpu_lib.num_blocks(m, 256), device="cuda")))
    say("cq segments sharing one gradient")
    gpu_lib.loco_compensate_quantize([(g[lo:hi], e, c, a) for (lo, hi), (e, c, a) in zip(views, outs)],
                                     bits=4, block=256, beta=0.9)
    torch.cuda.synchronize()
    for (lo, hi), (e, c, a) in zip(views, outs):
        ref = oracle.compensate_quantize(bf16_bits(g[lo:hi]), np.zeros(hi - lo, np.float32), bits=4, block=256,
                                         beta=0.9, grad_dtype="bf16")
        t = f"segment on [{lo}, {hi})"
        assert_bytes_equal(host(c), ref["codes"], f"{t} codes")
        assert_bytes_equal(host(a).view(np.uint32), ref["absmax"].view(np.uint32), f"{t} absmax")
        assert_f32_close(host(e), ref["e_new"], np.zeros(hi - lo), f"{t} error")
