"""The full-size parity machinery on the CPU (no GPU): slabs cover every element of every
segment exactly once, the oracle's state is carried between steps, and a difference
anywhere is reported.  The "device" outputs here are the oracle's own whole-segment
results written into the shared arrays, so a correct checker reports nothing until a
byte is changed."""
import multiprocessing
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest

import fullsize_pool as FP
import oracle


@pytest.fixture(scope="module")
def pool():
    with ProcessPoolExecutor(2, mp_context=multiprocessing.get_context("spawn")) as p:
        yield p


def _grad(rng, n, gd):
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    return oracle.bf16_rne(x) if gd == "bf16" else x


@pytest.mark.parametrize("gd,ed,bits", [("bf16", "f32", 4), ("f32", "bf16", 8), ("bf16", "i8", 2)])
def test_cq_slabs(pool, gd, ed, bits):
    rng = np.random.default_rng(bits)
    sizes, block, slab = [5000, 3 * 4096 + 7, 64, 1], 64, 1024
    kw = dict(bits=bits, block=block, beta=0.9, gd=gd, ed=ed, err_scale=2.0 ** 17 if ed == "i8" else 0.0)
    offs, coffs, boffs = FP.cq_layout(sizes, bits, block)
    S = FP.SharedArrays()
    try:
        g_sh = S.new("g", offs[-1], gd)
        S.new("e_ora", offs[-1], ed)
        e_sh = S.new("e_gpu", offs[-1], ed)
        c_sh = S.new("codes", coffs[-1], "u8")
        a_sh = S.new("absmax", boffs[-1], "f32")
        view = (lambda a: a.view(np.uint16)) if gd == "bf16" else (lambda a: a)
        eview = (lambda a: a.view(np.uint16)) if ed == "bf16" else (lambda a: a)
        e_ref = [np.zeros(n, {"f32": np.float32, "bf16": np.uint16, "i8": np.int8}[ed]) for n in sizes]
        for step in range(2):
            for s, n in enumerate(sizes):
                g = _grad(rng, n, gd)
                view(g_sh)[offs[s]:offs[s + 1]] = g
                r = oracle.compensate_quantize(g, e_ref[s], bits=bits, block=block, beta=0.9, grad_dtype=gd,
                                               err_dtype=ed, err_scale=kw["err_scale"])
                eview(e_sh)[offs[s]:offs[s + 1]] = r["e_new"]
                c_sh[coffs[s]:coffs[s + 1]] = r["codes"]
                a_sh[boffs[s]:boffs[s + 1]] = r["absmax"]
                e_ref[s] = r["e_new"]
            for a in (g_sh, e_sh, c_sh, a_sh):
                a.flush()
            e_prev = np.array(np.memmap(S.spec("e_ora")[0], dtype=FP.FILE_DTYPE[ed], mode="r", shape=(offs[-1],)))
            tasks = FP.cq_tasks(S, sizes, slab, reset=False, tag=f"step {step}", **kw)
            n, bad, _ = FP.run(pool, FP.cq_task, tasks)
            assert not bad and n == sum(sizes), bad
        # the oracle's carried state equals the whole-segment chain
        e_state = np.memmap(S.spec("e_ora")[0], dtype=FP.FILE_DTYPE[ed], mode="r", shape=(offs[-1],))
        assert np.array_equal(eview(e_state), np.concatenate(e_ref))
        # one changed code byte in segment 1 and one changed error element in segment 0
        c_sh[coffs[1] + 777] ^= 0x10
        eview(e_sh)[3] += 3 if ed != "f32" else 0
        if ed == "f32":
            e_sh[3] = e_sh[3] * np.float32(1.5) + np.float32(1e-3)
        for a in (c_sh, e_sh):
            a.flush()
        # re-run the last step from the oracle's state before it: only the planted slabs differ
        rw = np.memmap(S.spec("e_ora")[0], dtype=FP.FILE_DTYPE[ed], mode="r+", shape=(offs[-1],))
        rw[:] = e_prev
        rw.flush()
        tasks = FP.cq_tasks(S, sizes, slab, reset=False, tag="planted", **kw)
        _, bad, _ = FP.run(pool, FP.cq_task, tasks)
        assert len(bad) == 2, bad
        lo = (777 * 8 // bits) // slab * slab
        assert any(f"segment 1 elements {lo}:{lo + slab} codes: 1 of" in b for b in bad), bad
        assert any("segment 0 elements 0:1024" in b and "error" in b for b in bad), bad
    finally:
        S.close()


def test_dr_slabs(pool):
    rng = np.random.default_rng(7)
    n, bits, block, P = 10_000 + 37, 4, 64, 3
    pays = [(rng.integers(0, 256, (n * bits + 7) // 8).astype(np.uint8),
             (rng.random(-(-n // block)) * 1e-2).astype(np.float32)) for _ in range(P)]
    want = oracle.dequant_reduce(pays, n, bits=bits, block=block, out_scale=1 / 3, out_dtype="bf16")
    S = FP.SharedArrays()
    try:
        cb, nb = (n * bits + 7) // 8, -(-n // block)
        c_sh, a_sh = S.new("codes", P * cb, "u8"), S.new("absmax", P * nb, "f32")
        for p, (c, a) in enumerate(pays):
            c_sh[p * cb:(p + 1) * cb] = c
            a_sh[p * nb:(p + 1) * nb] = a
        out = S.new("out", n, "bf16")
        out.view(np.uint16)[:] = want
        for a in (c_sh, a_sh, out):
            a.flush()
        base = dict(codes=S.spec("codes"), absmax=S.spec("absmax"), coffs=[p * cb for p in range(P)],
                    boffs=[p * nb for p in range(P)], out=S.spec("out"), bits=bits, block=block, out_scale=1 / 3,
                    out_dtype="bf16", tag="dr")
        tasks = [dict(base, lo=lo, hi=min(lo + 1024, n)) for lo in range(0, n, 1024)]
        got, bad, bw = FP.run(pool, FP.dr_task, tasks)
        assert got == n and not bad and bw
        out.view(np.uint16)[n - 1] += 2  # two ulps off at the ragged end
        out.flush()
        _, bad, _ = FP.run(pool, FP.dr_task, tasks)
        assert len(bad) == 1 and f"{(n - 1) // 1024 * 1024}:{n}" in bad[0], bad
    finally:
        S.close()
