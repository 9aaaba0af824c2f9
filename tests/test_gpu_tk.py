"""GPU parity of loco_topk_quantize (SparseLoCo-style mode) against the CPU oracle.

Indices, codes and absmax must be bit-exact; the error buffer within 1e-6 relative
(bitwise expected).  Inputs cover the workload's law (Gaussian with exact-tie outliers),
heavy ties, all-zero chunks, k = 1 and k = chunk, ragged tails and a layout built to push
the kernel off its fast candidate path.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import Guarded, assert_bytes_equal, assert_f32_close, host, say

pytestmark = pytest.mark.gpu


def run_tk_chain(loco, n, chunk, k, bits, decay, steps, gen, tag=""):
    chunks = -(-n // chunk)
    nb = loco.code_bytes(k, bits)
    g = Guarded(n, torch.float32)
    e = Guarded(n, torch.float32, init=torch.zeros(n))
    idx = Guarded(chunks * k, torch.int16)
    codes = Guarded(chunks * nb, torch.uint8)
    am = Guarded(chunks, torch.float32)
    e_ora = np.zeros(n, np.float32)
    bw = True
    for step in range(steps):
        x = gen(step, n)
        g.t.copy_(x)
        loco.loco_topk_quantize(g.t, e.t, chunk=chunk, k=k, idx=idx.t, codes=codes.t, absmax=am.t, bits=bits,
                                ef_decay=decay)
        torch.cuda.synchronize()
        ref = oracle.topk_quantize(x.numpy(), e_ora, chunk=chunk, k=k, bits=bits, decay=decay)
        t = f"{tag} step {step}"
        assert_bytes_equal(host(idx.t).view(np.uint16), ref["idx"], f"{t} idx")
        assert_bytes_equal(host(codes.t), ref["codes"], f"{t} codes")
        assert_bytes_equal(host(am.t).view(np.uint32), ref["absmax"].view(np.uint32), f"{t} absmax")
        bw &= assert_f32_close(host(e.t), ref["e_new"], np.repeat(ref["absmax"], chunk)[:n].astype(np.float64),
                               f"{t} error")
        e_ora = ref["e_new"]
        for b, nm in ((g, "grad"), (e, "err"), (idx, "idx"), (codes, "codes"), (am, "absmax")):
            b.check(f"{t} {nm}")
    return bw


def sparse_gen(step, n):
    return W.sparseloco_grad(step, n=n)


def test_tk_workload_scaled(gpu_lib):
    """The SparseLoCo workload's law on 40 chunks of 4096 (+ a ragged one), k = 82, 2-bit,
    decay 1, 5 steps."""
    say("tk workload scaled: n=40*4096+1234 C=4096 k=82 2-bit x5")
    assert run_tk_chain(gpu_lib, 40 * 4096 + 1234, 4096, 82, 2, 1.0, 5, sparse_gen, "workload")


@pytest.mark.parametrize("chunk", [256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("decay", [1.0, 0.5])
def test_tk_matrix(gpu_lib, chunk, bits, decay):
    for k in sorted({1, 3, min(82, chunk), chunk // 2 + 1, chunk}):
        n = 5 * chunk + chunk // 3 + 1
        say(f"tk matrix C={chunk} bits={bits} decay={decay} k={k} n={n}")
        run_tk_chain(gpu_lib, n, chunk, k, bits, decay, 2, sparse_gen, f"C{chunk} k{k}")


def ties_gen(step, n):
    rng = np.random.default_rng(1000 + step)
    vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0], np.float32)
    return torch.from_numpy(rng.choice(vals, n).astype(np.float32) * np.float32(1e-3))


@pytest.mark.parametrize("k", [1, 5, 82, 128, 129, 600, 4096])
def test_tk_heavy_ties(gpu_lib, k):
    """Seven distinct magnitudes: thousands of equal keys; ties go to the lower index."""
    say(f"tk heavy ties k={k}")
    run_tk_chain(gpu_lib, 3 * 4096 + 77, 4096, k, 2, 1.0, 3, ties_gen, f"ties k{k}")


def test_tk_zero_chunks(gpu_lib):
    """All-zero chunks keep the first k indices, zero codes, zero absmax."""
    def gen(step, n):
        x = W.sparseloco_grad(step, n=n)
        x[:4096] = 0
        x[2 * 4096 + 100:] = 0
        return x
    say("tk zero chunks")
    run_tk_chain(gpu_lib, 3 * 4096 + 500, 4096, 82, 2, 1.0, 3, gen, "zeros")


# Host model of the kernel's routing at chunk 4096 (256 threads, thread t holding the 16
# elements q*1024 + 4t + r): the lower bound L is the largest key with only bits 30..19 set
# that at least k per-thread maxima reach; the keys >= L are the candidates, and the fast
# path takes a chunk when they fit the 512-slot list.
TK_CAP = 512


def fast_path_candidates(h_chunk, k):
    key = np.abs(np.asarray(h_chunk, np.float32)).view(np.uint32)
    per_thread = key.reshape(4, 256, 4).transpose(1, 0, 2).reshape(256, 16).max(axis=1)
    L = 0
    for bit in range(30, 18, -1):
        cand = L | (1 << bit)
        if np.count_nonzero(per_thread >= cand) >= k:
            L = cand
    return int(np.count_nonzero(key >= L))


def test_tk_fallback_layout(gpu_lib):
    """Large values only in lanes 0..9 of every 64-element row: per-thread maxima give a
    low bound, more keys than the 512-slot candidate list reach it, and the kernel takes
    its exhaustive path (asserted on the host model of its routing)."""
    def gen(step, n):
        x = W.sparseloco_grad(step, n=n)
        i = torch.arange(n)
        big = (i % 64) < 10
        x[big] = x[big] * 50 + torch.sign(x[big]) * 0.05
        return x
    x = gen(0, 6 * 4096).numpy()  # step 0: e = 0, so h = g
    assert min(fast_path_candidates(x[c * 4096:(c + 1) * 4096], 82) for c in range(6)) > TK_CAP
    say("tk fallback layout")
    run_tk_chain(gpu_lib, 6 * 4096, 4096, 82, 2, 1.0, 3, gen, "fallback")


def fast_ties_gen(step, n):
    """Per 4096-element chunk: 40 elements at exactly +-0.1 and 200 at exactly +-0.05, each
    in a different thread's 16 elements (240 random threads of 256), the rest N(0, 1e-3)."""
    rng = np.random.default_rng([4242, step])
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    for c in range(n // 4096):
        threads = rng.permutation(256)[:240]
        q = rng.integers(0, 4, 240)
        r = rng.integers(0, 4, 240)
        pos = c * 4096 + q * 1024 + 4 * threads + r
        sgn = np.where(rng.random(240) < 0.5, -1.0, 1.0).astype(np.float32)
        x[pos[:40]] = np.float32(0.1) * sgn[:40]
        x[pos[40:]] = np.float32(0.05) * sgn[40:]
    return torch.from_numpy(x)


@pytest.mark.parametrize("k", [41, 82, 150])
def test_tk_fast_path_ties(gpu_lib, k):
    """Many equal magnitudes at the threshold on the fast path: k - 40 of the 200 ties at
    0.05 are kept, the lower indices first.  The host model of the kernel's routing shows
    every chunk on the fast path (at most 512 candidates) with the kept ties ending past
    the first 64-slot candidate group in some chunk.  Decay 0.5 keeps the leftover ties'
    error (0.025) below the next step's bound."""
    n, C = 8 * 4096, 4096
    e = np.zeros(n, np.float32)
    crossed = False
    for step in range(2):
        x = fast_ties_gen(step, n).numpy()
        h = x + np.float32(0.5) * e
        for c in range(n // C):
            hc = h[c * C:(c + 1) * C]
            assert fast_path_candidates(hc, k) <= TK_CAP, (step, c)
            key = np.abs(hc).view(np.uint32)
            cand = np.flatnonzero(key >= np.abs(np.float32(0.05)).view(np.uint32))
            kept = oracle.topk_order_select(key, k)
            crossed |= int(np.searchsorted(cand, kept.max())) >= 64
        e = oracle.topk_quantize(x, e, chunk=C, k=k, bits=2, decay=0.5)["e_new"]
    assert crossed
    say(f"tk fast-path ties k={k}")
    run_tk_chain(gpu_lib, n, C, k, 2, 0.5, 2, fast_ties_gen, f"fast ties k{k}")


def test_tk_small_tail_only(gpu_lib):
    """n smaller than one chunk, and k larger than the ragged chunk."""
    for n in (1, 5, 63, 64, 65, 300):
        say(f"tk small n={n}")
        run_tk_chain(gpu_lib, n, 256, 100, 2, 1.0, 2, sparse_gen, f"small n{n}")


def test_tk_teacher_forced(gpu_lib):
    """Teacher-forced: each step starts from the oracle's error (perturbed), not the GPU's."""
    n, C, k = 9 * 4096 + 333, 4096, 82
    chunks = -(-n // C)
    g = Guarded(n, torch.float32)
    e = Guarded(n, torch.float32)
    idx = Guarded(chunks * k, torch.int16)
    codes = Guarded(chunks * gpu_lib.code_bytes(k, 2), torch.uint8)
    am = Guarded(chunks, torch.float32)
    e_ora = np.zeros(n, np.float32)
    for step in range(4):
        x = W.sparseloco_grad(step, n=n)
        g.t.copy_(x)
        e.t.copy_(torch.from_numpy(e_ora))
        gpu_lib.loco_topk_quantize(g.t, e.t, chunk=C, k=k, idx=idx.t, codes=codes.t, absmax=am.t, bits=2,
                                   ef_decay=0.9)
        torch.cuda.synchronize()
        ref = oracle.topk_quantize(x.numpy(), e_ora, chunk=C, k=k, bits=2, decay=0.9)
        t = f"tk teacher-forced step {step}"
        assert_bytes_equal(host(idx.t).view(np.uint16), ref["idx"], f"{t} idx")
        assert_bytes_equal(host(codes.t), ref["codes"], f"{t} codes")
        assert_bytes_equal(host(am.t).view(np.uint32), ref["absmax"].view(np.uint32), f"{t} absmax")
        assert_f32_close(host(e.t), ref["e_new"], np.repeat(ref["absmax"], C)[:n].astype(np.float64), f"{t} error")
        e_ora = ref["e_new"].copy()
        e_ora[::11] *= np.float32(0.5)
