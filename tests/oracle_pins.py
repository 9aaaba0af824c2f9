"""Checks that pin the CPU oracle to facts outside itself.

Each pin_* function takes the oracle module and raises AssertionError when the
oracle disagrees with what the pages, the mathematics or an independent library
routine fix.  They are plain functions so that the mutation test can run them
against an oracle with a planted mistake.
"""

import numpy as np
import torch

import golden_io

F32 = np.float32


def _rng(seed):
    return np.random.default_rng(seed)


def _h_blocks(x, block):
    nb = -(-x.size // block)
    pad = np.zeros(nb * block, x.dtype)
    pad[: x.size] = x
    return pad.reshape(nb, block)


# -- P-1: error feedback with e = 0 and an identity compressor reproduces g -------------------

def pin_identity_compressor(O):
    rng = _rng(1)
    n = 1000
    e = np.zeros(n, F32)
    for _ in range(5):
        g = (rng.standard_normal(n) * 1e-3).astype(F32)
        out = O.compensate_quantize(g, e, bits=4, block=128, beta=0.9,
                                    compressor=lambda h: (h.copy(), {}))
        assert np.array_equal(out["d"].view(np.uint32), g.view(np.uint32)), "transmitted != g"
        assert not np.any(out["e_new"]), "error left non-zero"
        e = out["e_new"]


# -- P-2: beta = 0 is plain error feedback, e' = h - d bitwise (Eqn. (4)) --------------------

def pin_beta_zero_is_efc(O):
    rng = _rng(2)
    n = 3000
    g = (rng.standard_normal(n) * 1e-3).astype(F32)
    e = (rng.standard_normal(n) * 1e-4).astype(F32)
    out = O.compensate_quantize(g, e, bits=4, block=128, beta=0.0)
    h = g + e
    assert np.array_equal(out["e_new"], h - out["d"])


# -- P-3: per-element quantisation error bound step/2 -------------------------------------------

def pin_quantisation_bound(O):
    rng = _rng(3)
    for bits, block in ((4, 128), (8, 256), (4, 64), (2, 128)):
        n = 5 * block + 37
        g = (rng.standard_t(3, n) * 1e-3).astype(F32)
        e = (rng.standard_normal(n) * 1e-4).astype(F32)
        out = O.compensate_quantize(g, e, bits=bits, block=block, beta=0.5)
        h = g + e
        hb = _h_blocks(h, block)
        absmax = np.abs(hb).max(axis=1)
        assert np.array_equal(out["absmax"], absmax), "absmax is not the block max |h|"
        qmax = (1 << (bits - 1)) - 1
        q = out["q"]
        assert q.min() >= -qmax - 1 and q.max() <= qmax
        step = (absmax.astype(np.float64) / qmax)
        bound = np.repeat(step, block)[:n] * (0.5 + 4 * qmax * 2.0 ** -24)
        r = np.abs(h.astype(np.float64) - out["d"].astype(np.float64))
        assert np.all(r <= bound), "|h - d| exceeds step/2"


# -- P-4: the moving-average error stays bounded over a 1000-step random walk --------------------

def pin_random_walk_bounded(O):
    rng = _rng(4)
    n, block, beta = 2048, 128, 0.9
    g = (rng.standard_normal(n) * 1e-3).astype(F32)
    e = np.zeros(n, F32)
    run_bound = np.zeros(n)
    worst = 0.0
    for _ in range(1000):
        g = (g + rng.standard_normal(n) * 1e-4).astype(F32)
        out = O.compensate_quantize(g, e, bits=4, block=block, beta=beta)
        h = g + e
        step = np.abs(_h_blocks(h, block)).max(axis=1).astype(np.float64) / 7
        run_bound = np.maximum(run_bound, np.repeat(step, block)[:n] / 2)
        e = out["e_new"]
        ratio = np.abs(e.astype(np.float64)) / np.maximum(run_bound, 1e-30)
        worst = max(worst, float(ratio.max()))
    assert worst <= 1 + 1e-5, f"|e| exceeded the running max of step/2 (ratio {worst})"


# -- P-5: telescoping identity of Eqn. (5), the non-accumulation of Eqn. (6) ----------------------

def pin_telescoping(O):
    """sum_i (g_i - d_i) = (e_K - e_0) / (1 - beta) in real arithmetic (float64 twin)."""
    rng = _rng(5)
    n, beta, K = 4096, 0.9, 50
    e = np.zeros(n, np.float64)
    e0 = e.copy()
    acc = np.zeros(n, np.float64)
    gabs = 0.0
    for _ in range(K):
        g = (rng.standard_t(3, n) * 1e-3).astype(F32).astype(np.float64)
        out = O.compensate_quantize(g, e, bits=4, block=128, beta=beta,
                                    grad_dtype="f64", err_dtype="f64", ftype=np.float64)
        acc += g - out["d"]
        gabs += np.abs(g).max()
        e = out["e_new"]
    rhs = (e - e0) / (1 - beta)
    assert np.max(np.abs(acc - rhs)) <= 1e-11 * gabs, "error accumulates: telescoping broken"
    # and in float32 the same chain stays within the accumulated rounding
    rng = _rng(5)
    e = np.zeros(n, F32)
    acc = np.zeros(n, np.float64)
    for _ in range(K):
        g = (rng.standard_t(3, n) * 1e-3).astype(F32)
        out = O.compensate_quantize(g, e, bits=4, block=128, beta=beta)
        acc += g.astype(np.float64) - out["d"].astype(np.float64)
        e = out["e_new"]
    rhs = e.astype(np.float64) / (1 - beta)
    assert np.max(np.abs(acc - rhs)) <= 1e-5 * gabs


# -- P-6: the fixed-scale compressor of Eqn. (1) on hand-worked values ----------------------------

def pin_fixed_scale_golden(O):
    s = 2.0 ** 19
    for bits, m, expect in golden_io.rounding_cases():
        h = np.array([m * 2.0 ** -19], F32)
        q, step = O.fixed_scale_quantize(h, bits, s)
        assert int(q[0]) == expect, f"Round_{bits}({m}) -> {int(q[0])}, want {expect}"
        assert step == F32(2.0 ** -19)


# -- P-7: PyTorch's own quantiser (the page names it as the one used) ------------------------------

def pin_torch_quantiser(O):
    rng = _rng(7)
    block = 256
    nb = 80
    n = nb * block
    h = (rng.standard_t(3, n) * 1e-3).astype(F32)
    # half of the blocks sit one ulp off the rounding boundaries (k + 1/2) * step, where
    # multiplying by fl(1/step) and dividing by step give different codes
    for b in range(nb // 2, nb):
        a = F32(rng.uniform(1e-4, 1e-2))
        step = a / F32(127)
        k = rng.integers(-126, 126, block - 1).astype(F32)
        v = ((k + F32(0.5)) * step).astype(F32)
        v = np.nextafter(v, np.where(rng.random(block - 1) < 0.5, -np.inf, np.inf).astype(F32))
        h[b * block] = a
        h[b * block + 1:(b + 1) * block] = v
    # 8 bits against torch.quantize_per_channel(qint8) with one scale per block
    out = O.compensate_quantize(h, np.zeros(n, F32), bits=8, block=block, beta=0.9)
    step = O.block_steps(out["absmax"], 8)
    tq = torch.quantize_per_channel(torch.from_numpy(h.reshape(nb, block)),
                                    torch.from_numpy(step.astype(np.float64)),
                                    torch.zeros(nb, dtype=torch.int64), 0, torch.qint8)
    assert np.array_equal(tq.int_repr().numpy().reshape(-1).astype(np.int64), out["q"])
    # 4 bits, one block at a time, against quint4x2 (offset-8 nibbles, element 2j low)
    out4 = O.compensate_quantize(h, np.zeros(n, F32), bits=4, block=block, beta=0.9)
    step4 = O.block_steps(out4["absmax"], 4)
    for b in range(nb):
        t = torch.quantize_per_tensor(torch.from_numpy(h[b * block:(b + 1) * block]),
                                      float(step4[b]), 8, torch.quint4x2)
        ours = out4["codes"][b * block // 2:(b + 1) * block // 2]
        assert np.array_equal(t.int_repr().numpy() ^ 0x88, ours), f"4-bit block {b} differs"


# -- P-8: Top-k by brute force on tiny inputs with many ties --------------------------------------

def _brute_topk(key, k):
    n = key.size
    sel = []
    for i in range(n):
        better = sum(1 for j in range(n) if key[j] > key[i] or (key[j] == key[i] and j < i))
        if better < k:
            sel.append(i)
    return np.array(sel, dtype=np.int64)


def pin_topk_brute_force(O):
    rng = _rng(8)
    for trial in range(200):
        n = int(rng.integers(1, 65))
        k = int(rng.integers(1, n + 1))
        key = rng.integers(0, 6, n).astype(np.uint32)  # few distinct values: many ties
        got = O.topk_order_select(key, k)
        assert np.array_equal(got, _brute_topk(key, k)), (n, k, key)
    for trial in range(30):
        chunk = int(rng.choice([4, 8, 16]))
        n = int(rng.integers(1, 4 * chunk))
        k = int(rng.integers(1, chunk + 1))
        g = rng.choice(np.array([0, 0.5, -0.5, 1, -1, 2], F32), n).astype(F32)
        out = O.topk_quantize(g, np.zeros(n, F32), chunk=chunk, k=k)
        for c in range(-(-n // chunk)):
            hc = g[c * chunk:(c + 1) * chunk]
            keff = min(k, hc.size)
            want = _brute_topk(np.abs(hc).view(np.uint32), keff)
            idx = out["idx"][c * k:(c + 1) * k]
            assert np.array_equal(idx[:keff].astype(np.int64), want)
            assert np.all(idx[keff:] == 0xFFFF)
            mask = np.zeros(hc.size, bool)
            mask[want] = True
            assert np.array_equal(out["e_new"][c * chunk:c * chunk + hc.size][~mask], hc[~mask])


# -- P-9: payload byte layout and round trip --------------------------------------------------------

def pin_pack_layout(O):
    for bits, codes, want in golden_io.pack_cases():
        got = O.pack_codes(np.array(codes), bits)
        assert bytes(got.tobytes()) == want, (bits, codes, got.tobytes().hex(), want.hex())
        back = O.unpack_codes(got, bits, len(codes))
        assert list(back) == codes
    rng = _rng(9)
    for bits in (2, 4, 8):
        for n in (1, 2, 3, 7, 64, 1001):
            q = rng.integers(-(1 << (bits - 1)), 1 << (bits - 1), n)
            assert np.array_equal(O.unpack_codes(O.pack_codes(q, bits), bits, n), q)


# -- hand-worked compensate-quantize, dequant-reduce and Top-k steps ---------------------------

def pin_cq_worked(O):
    for c in golden_io.cq_cases():
        out = O.compensate_quantize(c["g"], c["e"], bits=c["bits"], block=c["block"], beta=c["beta"],
                                    err_dtype=c["err_dtype"], err_scale=c["err_scale"], reset=c["reset"])
        assert np.array_equal(out["absmax"], c["absmax"]), ("absmax", out["absmax"], c["absmax"])
        assert out["codes"].tobytes() == c["codes"], ("codes", out["codes"].tobytes().hex())
        assert np.array_equal(out["e_new"], c["e_new"]), ("e_new", out["e_new"], c["e_new"])


def pin_dr_worked(O):
    c = golden_io.dr_case()
    out = O.dequant_reduce(c["peers"], c["n"], bits=c["bits"], block=c["block"],
                           out_scale=c["out_scale"])
    assert np.array_equal(out, c["out"]), (out, c["out"])


def pin_topk_worked(O):
    for c in golden_io.topk_cases():
        out = O.topk_quantize(c["g"], c["e"], chunk=c["chunk"], k=c["k"], decay=c["decay"])
        assert np.array_equal(out["idx"], c["idx"]), ("idx", out["idx"], c["idx"])
        assert out["codes"].tobytes() == c["codes"], ("codes", out["codes"].tobytes().hex())
        assert np.array_equal(out["absmax"], c["absmax"])
        assert np.array_equal(out["e_new"], c["e_new"]), ("e_new", out["e_new"], c["e_new"])


# -- P-10: dequant-reduce special cases and the high-precision average -----------------------------

def pin_dequant_reduce(O):
    rng = _rng(10)
    n, block = 3 * 256 + 100, 256
    outs = []
    for p in range(5):
        g = (rng.standard_t(3, n) * 1e-3).astype(F32)
        outs.append(O.compensate_quantize(g, np.zeros(n, F32), bits=4, block=block, beta=0.9))
    pay = [(o["codes"], o["absmax"]) for o in outs]
    # one peer, scale 1: exactly that peer's decompressed value
    one = O.dequant_reduce(pay[:1], n, bits=4, block=block, out_scale=1.0)
    assert np.array_equal(one, outs[0]["d"])
    # two identical peers averaged: exact
    two = O.dequant_reduce([pay[1], pay[1]], n, bits=4, block=block, out_scale=0.5)
    assert np.array_equal(two, outs[1]["d"])
    # five peers: the float64 average of the decompressed values, within fp32 rounding
    got = O.dequant_reduce(pay, n, bits=4, block=block, out_scale=F32(1) / F32(5))
    ds = np.stack([o["d"].astype(np.float64) for o in outs])
    want = ds.sum(0) / 5
    bound = 2.0 ** -23 * (len(outs) + 1) * np.abs(ds).sum(0) / 5 + 1e-45
    assert np.all(np.abs(got.astype(np.float64) - want) <= bound)
    # bf16 output is the RNE of the fp32 output
    gotb = O.dequant_reduce(pay, n, bits=4, block=block, out_scale=F32(1) / F32(5), out_dtype="bf16")
    tb = torch.from_numpy(got).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gotb, tb)


def pin_dequant_huge_scales(O):
    """Eqn. (8) at the top of the fp32 range: d = q * step stays the exact product as long
    as it is representable (a decoder that forms it as (q + 8) * step - 8 * step
    overflows), and a sum that leaves the range is infinite.  4-bit, blocks of 4, absmax
    7 * 2^124 so that step = 2^124 exactly."""
    step = 2.0 ** 124
    am = np.array([7 * step], F32)
    pos7 = np.array([0x77, 0x77], np.uint8)    # four codes +7
    neg8 = np.array([0x88, 0x88], np.uint8)    # four codes -8
    mixed = np.array([0x07, 0x8f], np.uint8)   # codes 7, 0, -1, -8
    got = O.dequant_reduce([(pos7, am), (neg8, am)], 4, bits=4, block=4, out_scale=0.5)
    assert np.array_equal(got, np.full(4, -step / 2, F32))          # (7 - 8) * 2^124 / 2
    got = O.dequant_reduce([(mixed, am)], 4, bits=4, block=4, out_scale=1.0)
    assert np.array_equal(got, np.array([7 * step, 0, -step, -8 * step], F32))
    with np.errstate(over="ignore"):
        got = O.dequant_reduce([(pos7, am)] * 3, 4, bits=4, block=4, out_scale=1.0)
    assert np.all(np.isposinf(got))                                  # 21 * 2^124 > 2^128
    # the largest block scale: 7 * fl(FLT_MAX / 7) is finite
    fmax = np.array([np.finfo(F32).max], F32)
    got = O.dequant_reduce([(pos7, fmax)], 4, bits=4, block=4, out_scale=1.0)
    assert np.all(np.isfinite(got)) and np.all(got == F32(7) * (fmax[0] / F32(7)))


def pin_dequant_reduce_peer_order(O):
    """Eqn. (8) sums the peers' decompressed values in peer order, rounding after each add:
    with d = 1, 2^-24, -1 (4-bit codes 1, 1, -1 at steps 1, 2^-24, 1) the fp32 sum is
    (1 + 2^-24) - 1 = 0, since 1 + 2^-24 is a tie that rounds to 1; in the reverse order it
    would be (-1 + 2^-24) + 1 = 2^-24."""
    one = np.array([0x01], np.uint8)          # codes +1, 0
    neg = np.array([0x0F], np.uint8)          # codes -1, 0
    p0 = (one, np.array([7.0], F32))          # step 1
    p1 = (one, np.array([7 * 2.0 ** -24], F32))  # step 2^-24
    p2 = (neg, np.array([7.0], F32))          # step 1
    got = O.dequant_reduce([p0, p1, p2], 2, bits=4, block=2, out_scale=1.0)
    assert np.array_equal(got.view(np.uint32), np.zeros(2, F32).view(np.uint32)), got
    got = O.dequant_reduce([p2, p1, p0], 2, bits=4, block=2, out_scale=1.0)
    assert np.array_equal(got, np.array([2.0 ** -24, 0.0], F32)), got


# -- P-11: all-zero blocks ---------------------------------------------------------------------

def pin_zero_blocks(O):
    rng = _rng(11)
    block = 128
    g = (rng.standard_normal(6 * block) * 1e-3).astype(F32)
    g[block:3 * block] = 0
    g[5 * block:] = 0
    e = np.zeros_like(g)
    for _ in range(3):
        out = O.compensate_quantize(g, e, bits=4, block=block, beta=0.9)
        for b in (1, 2, 5):
            assert out["absmax"][b] == 0
            assert not np.any(out["q"][b * block:(b + 1) * block])
            assert not np.any(out["e_new"][b * block:(b + 1) * block])
        e = out["e_new"]


# -- P-12: bf16 rounding equals torch's conversion ---------------------------------------------

def pin_bf16_rne(O):
    rng = _rng(12)
    x = (rng.standard_normal(100000) * rng.choice([1e-6, 1e-3, 1.0, 1e3], 100000)).astype(F32)
    u = x.view(np.uint32).copy()
    u[:2000] = (u[:2000] & 0xFFFF0000) | 0x8000  # exact ties, both parities of the kept bit
    u[2000:4000] = (u[2000:4000] & 0xFFFF0000) | 0x7FFF
    u[4000:6000] = (u[4000:6000] & 0xFFFF0000) | 0x8001
    x = u.view(F32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_rne(x), want)
    assert np.array_equal(O.bf16_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


# -- SparseLoCo error feedback: transmitted + final error telescopes to the gradient sum ------------

def pin_topk_error_feedback(O):
    """decay = 1: sum_k transmitted_k = sum_k g_k - e_K (float64 twin, exact up to rounding)."""
    rng = _rng(13)
    n, chunk, k, K = 4 * 256 + 50, 256, 6, 20
    e = np.zeros(n)
    sent = np.zeros(n)
    gsum = np.zeros(n)
    for _ in range(K):
        g = (rng.standard_normal(n) * 1e-3).astype(F32).astype(np.float64)
        out = O.topk_quantize(g, e, chunk=chunk, k=k, decay=1.0, ftype=np.float64)
        sent += out["h"] - out["e_new"]
        gsum += g
        e = out["e_new"]
        # kept values carry at most half a step of error; the rest are untouched
        for c in range(-(-n // chunk)):
            lo = c * chunk
            hc = out["h"][lo:lo + chunk]
            idx = out["idx"][c * k:(c + 1) * k]
            idx = idx[idx != 0xFFFF].astype(np.int64)
            am = out["absmax"][c]
            assert am == np.abs(hc).max()
            assert np.all(np.abs(out["e_new"][lo + idx]) <= am / 2 * (1 + 1e-12))
            # exactly k entries move: the others equal h
            mask = np.ones(hc.size, bool)
            mask[idx] = False
            assert np.array_equal(out["e_new"][lo:lo + chunk][mask], hc[mask])
    assert np.max(np.abs(sent - (gsum - e))) <= 1e-12 * K


# -- the paper's 8-bit error (LoCo Sec. 3.2, Eqn. (7)) ------------------------------------------

def pin_i8_error_accounting(O):
    """With the error stored as e8 (value E = e8/s_e), g_k - d_k = (E_k - delta_k - E_{k-1}) /
    (1 - beta), delta_k = E_k - e~_k the 8-bit rounding of the new error; so the sum over K
    steps is (E_K - E_0)/(1 - beta) within K / (2 s_e (1 - beta)) when nothing clips
    (float64 twin)."""
    rng = _rng(21)
    n, beta, K, s_e = 4096, 0.9, 40, 2.0 ** 18
    e8 = np.zeros(n, np.int8)
    acc = np.zeros(n)
    for _ in range(K):
        g = (rng.standard_normal(n) * 1e-3).astype(F32).astype(np.float64)
        out = O.compensate_quantize(g, e8, bits=4, block=128, beta=beta, grad_dtype="f64",
                                    err_dtype="i8", err_scale=s_e, ftype=np.float64)
        acc += g - out["d"]
        e8 = out["e_new"]
        assert e8.max() < 127 and e8.min() > -128, "clipped: the bound below needs no clipping"
    E_K = e8.astype(np.float64) / s_e
    slack = K / (2 * s_e * (1 - beta)) * (1 + 1e-9)
    dev = np.abs(acc - E_K / (1 - beta))
    assert np.all(dev <= slack), (dev.max(), slack)
    assert dev.max() > slack * 1e-3  # the 8-bit rounding is really there


def pin_i8_equals_float_when_exact(O):
    """When every new error is a multiple of 1/s_e inside the 8-bit range, storing it as
    e8 loses nothing: the chain equals the fp32-error chain bitwise.  Built with a fixed
    scale s = 4, beta = 1/2 and g on the grid 1/64, so e~ lies on the grid 1/128."""
    rng = _rng(22)
    n, s_e = 3000, 128.0
    e_f = np.zeros(n, F32)
    e8 = np.zeros(n, np.int8)
    for _ in range(12):
        g = (rng.integers(-20, 21, n) / 64.0).astype(F32)
        a = O.compensate_quantize(g, e_f, bits=4, block=64, beta=0.5, fixed_scale=4.0)
        b = O.compensate_quantize(g, e8, bits=4, block=64, beta=0.5, fixed_scale=4.0,
                                  err_dtype="i8", err_scale=s_e)
        assert np.array_equal(a["codes"], b["codes"])
        assert np.array_equal(a["d"], b["d"])
        assert np.all(np.abs(a["e_new"] * s_e) <= 127)
        assert np.array_equal(a["e_new"], b["e_new"].astype(F32) / F32(s_e))
        e_f, e8 = a["e_new"], b["e_new"]


def pin_reset(O):
    """The periodic reset of Eqn. (7): the step's codes are unchanged, its stored error is
    zero, and the next step starts from e = 0."""
    rng = _rng(23)
    n = 2000
    for ed, e0 in (("f32", (rng.standard_normal(n) * 1e-4).astype(F32)),
                   ("i8", rng.integers(-100, 100, n).astype(np.int8))):
        kw = dict(bits=4, block=128, beta=0.9, err_dtype=ed, err_scale=2.0 ** 17)
        g = (rng.standard_normal(n) * 1e-3).astype(F32)
        a = O.compensate_quantize(g, e0, **kw)
        b = O.compensate_quantize(g, e0, reset=True, **kw)
        assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["absmax"], b["absmax"])
        assert not np.any(b["e_new"])
        c = O.compensate_quantize(g, b["e_new"], **kw)
        d0 = O.compensate_quantize(g, np.zeros_like(e0), **kw)
        assert np.array_equal(c["codes"], d0["codes"])


def pin_i8_compressor_vs_torch(O):
    """The error's compressor Round_8(s_e * e~) equals PyTorch's qint8 quantiser with scale
    1/s_e (a power of two, so its reciprocal is s_e exactly), ties and clamps included."""
    rng = _rng(24)
    for s_e in (2.0 ** 10, 2.0 ** 17, 2.0 ** 21):
        x = (rng.standard_normal(20000) * 60 / s_e).astype(F32)
        x[:200] = (rng.integers(-140, 140, 200) + 0.5).astype(F32) / F32(s_e)  # exact ties, clamps
        want = torch.quantize_per_tensor(torch.from_numpy(x), 1.0 / s_e, 0, torch.qint8).int_repr().numpy()
        assert np.array_equal(O.error_compress(x, s_e), want)
        assert np.array_equal(O.error_decompress(want, s_e), want.astype(F32) / F32(s_e))


# -- scalar twins: the same steps element by element, in fp32 scalars, on tiny inputs ------------

def _decode(codes, j, bits):
    """Code j of a packed array by the layout rule (little end first, two's complement)."""
    bit = j * bits
    raw = (int(codes[bit // 8]) >> (bit % 8)) & ((1 << bits) - 1)
    return raw - (1 << bits) if raw >= (1 << (bits - 1)) else raw


def _cq_twin(g, e, bits, block, beta):
    qmax = (1 << (bits - 1)) - 1
    n = len(g)
    b, om = F32(beta), F32(1) - F32(beta)
    h = [F32(F32(g[i]) + F32(e[i])) for i in range(n)]
    q, absmax, e_new = [0] * n, [], [F32(0)] * n
    for b0 in range(0, n, block):
        idx = range(b0, min(n, b0 + block))
        am = F32(0)
        for i in idx:
            am = max(am, F32(abs(h[i])))
        step = F32(am / F32(qmax)) if am != 0 else F32(0)
        inv = F32(F32(1) / step) if am != 0 else F32(0)
        absmax.append(am)
        for i in idx:
            q[i] = int(min(max(np.rint(F32(h[i] * inv)), -qmax - 1), qmax))
            d = F32(F32(q[i]) * step)
            r = F32(h[i] - d)
            e_new[i] = F32(F32(b * F32(e[i])) + F32(om * r))
    packed = [0] * (-(-n * bits // 8))
    for i, c in enumerate(q):
        packed[i * bits // 8] |= (c & ((1 << bits) - 1)) << (i * bits % 8)
    return bytes(packed), np.array(absmax, F32), np.array(e_new, F32)


def pin_cq_scalar_twin(O):
    """compensate_quantize against an element-by-element fp32 scalar twin that packs by the
    layout rule: bit-exact codes, absmax and error, for every code width, ragged blocks."""
    rng = _rng(50)
    for bits in (2, 4, 8):
        for n, block, beta in ((37, 8, 0.9), (64, 16, 0.5), (13, 4, 0.0), (29, 64, 1.0)):
            g = (rng.standard_normal(n) * 1e-3).astype(F32)
            e = (rng.standard_normal(n) * 1e-4).astype(F32)
            g[rng.random(n) < 0.1] = 0
            codes, am, en = _cq_twin(g, e, bits, block, beta)
            out = O.compensate_quantize(g, e, bits=bits, block=block, beta=beta)
            assert out["codes"].tobytes() == codes, (bits, n, block)
            assert np.array_equal(out["absmax"].view(np.uint32), am.view(np.uint32))
            assert np.array_equal(out["e_new"].view(np.uint32), en.view(np.uint32)), (bits, n, block, beta)


def pin_dr_scalar_twin(O):
    """dequant_reduce against an element-by-element fp32 scalar twin decoding the bytes by
    the layout rule, peers added in order."""
    rng = _rng(51)
    for bits in (2, 4, 8):
        qmax = (1 << (bits - 1)) - 1
        n, block, npeers, scale = 45, 8, 3, 1.0 / 3.0
        peers = [(rng.integers(0, 256, -(-n * bits // 8)).astype(np.uint8),
                  (rng.random(-(-n // block)) * 1e-2).astype(F32)) for _ in range(npeers)]
        peers[1][1][2] = 0
        want = []
        for i in range(n):
            acc = F32(0)
            for codes, am in peers:
                a = F32(am[i // block])
                step = F32(a / F32(qmax)) if a != 0 else F32(0)
                acc = F32(acc + F32(F32(_decode(codes, i, bits)) * step))
            want.append(F32(acc * F32(scale)))
        got = O.dequant_reduce(peers, n, bits=bits, block=block, out_scale=scale)
        assert np.array_equal(got.view(np.uint32), np.array(want, F32).view(np.uint32)), bits


# -- SparseLoCo sparse aggregation (SparseLoCo summary; LoCo Sec. 3.3, Eqn. (8)) -----------------

def pin_sa_worked(O):
    c = golden_io.sa_case()
    out = O.sparse_aggregate(c["peers"], c["n"], chunk=c["chunk"], k=c["k"], bits=c["bits"],
                             out_scale=c["out_scale"])
    assert np.array_equal(out, c["out"]), (out, c["out"])


def _sparse_payload(rng, n, chunk, k, bits, ordered=False):
    """A random valid sparse payload: distinct in-chunk indices (unused slots 0xFFFF),
    random code bytes, random positive fp32 scales (some chunks zero)."""
    nch = -(-n // chunk)
    cb = -(-k * bits // 8)
    idx = np.full((nch, k), 0xFFFF, np.uint16)
    for c in range(nch):
        L = min(chunk, n - c * chunk)
        m = min(k, L) - int(rng.integers(0, 2))  # sometimes one slot fewer than possible
        sel = rng.permutation(L)[:max(m, 0)]
        idx[c, :sel.size] = np.sort(sel) if ordered else sel
    codes = rng.integers(0, 256, nch * cb).astype(np.uint8)
    absmax = (rng.random(nch) * 2.0 ** rng.integers(-12, 3, nch)).astype(F32)
    absmax[rng.random(nch) < 0.1] = 0
    return idx.reshape(-1), codes, absmax


def _sa_brute(peers, n, chunk, k, bits, out_scale):
    """Element by element from the definition and the packing layout, in fp32 scalars."""
    qmax = (1 << (bits - 1)) - 1
    cb = -(-k * bits // 8)
    acc = [F32(0)] * n
    for idx, codes, absmax in peers:
        for c in range(-(-n // chunk)):
            L = min(chunk, n - c * chunk)
            a = F32(absmax[c])
            step = F32(a / F32(qmax)) if a != 0 else F32(0)
            for j in range(k):
                i = int(idx[c * k + j])
                if i >= L:
                    continue
                bit = j * bits
                raw = (int(codes[c * cb + bit // 8]) >> (bit % 8)) & ((1 << bits) - 1)
                q = raw - (1 << bits) if raw >= (1 << (bits - 1)) else raw
                acc[c * chunk + i] = F32(acc[c * chunk + i] + F32(F32(q) * step))
    return np.array([F32(v * F32(out_scale)) for v in acc], F32)


def pin_sa_brute_force(O):
    """Tiny random cases with overlapping indices across peers, ragged last chunks, k*bits
    not a whole number of bytes, unused slots and zero chunks, against the element-by-
    element definition; bf16 output against torch's RNE conversion."""
    rng = _rng(30)
    for n, chunk, k, bits, npeers in ((29, 8, 3, 2, 3), (50, 16, 9, 4, 4), (37, 8, 6, 8, 5),
                                      (64, 32, 13, 2, 2), (5, 8, 4, 4, 3)):
        peers = [_sparse_payload(rng, n, chunk, k, bits) for _ in range(npeers)]
        scale = 1.0 / 3.0
        want = _sa_brute(peers, n, chunk, k, bits, scale)
        got = O.sparse_aggregate(peers, n, chunk=chunk, k=k, bits=bits, out_scale=scale)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (n, chunk, k, bits, got, want)
        gb = O.sparse_aggregate(peers, n, chunk=chunk, k=k, bits=bits, out_scale=scale, out_dtype="bf16")
        tb = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(gb, tb)


def pin_sa_dense_equivalent(O):
    """With every slot used (k = chunk) the sparse aggregation is the dense dequant-reduce
    of the same codes with one scale block per chunk, whatever order the slots take."""
    rng = _rng(31)
    for bits in (2, 4, 8):
        chunk, n, npeers = 16, 16 * 5 + 7, 3
        qmax = (1 << (bits - 1)) - 1
        dense, sparse = [], []
        for _ in range(npeers):
            q = rng.integers(-qmax - 1, qmax + 1, n)
            absmax = (rng.random(-(-n // chunk)) * 1e-2).astype(F32)
            idx = np.full((len(absmax), chunk), 0xFFFF, np.uint16)
            rows = []
            for c in range(len(absmax)):
                L = min(chunk, n - c * chunk)
                perm = rng.permutation(L)
                idx[c, :L] = perm
                qc = np.zeros(chunk, np.int64)
                qc[:L] = q[c * chunk + perm]
                rows.append(O.pack_codes(qc, bits))
            dense.append((O.pack_codes(q, bits), absmax))
            sparse.append((idx.reshape(-1), np.concatenate(rows), absmax))
        for od in ("f32", "bf16"):
            a = O.sparse_aggregate(sparse, n, chunk=chunk, k=chunk, bits=bits, out_scale=1 / 3, out_dtype=od)
            b = O.dequant_reduce(dense, n, bits=bits, block=chunk, out_scale=1 / 3, out_dtype=od)
            assert np.array_equal(a, b), (bits, od)


def pin_sa_transmits_topk(O):
    """One peer, scale 1: the aggregation of a Top-k payload is exactly what that step
    transmitted, h - e' on the kept elements (Sterbenz: h - d is exact there) and 0
    elsewhere, so transmitted + new error = h."""
    rng = _rng(32)
    for bits in (2, 4, 8):
        n, chunk, k = 64 * 7 + 19, 64, 5
        g = (rng.standard_normal(n) * 1e-3).astype(F32)
        e = (rng.standard_normal(n) * 1e-4).astype(F32)
        r = O.topk_quantize(g, e, chunk=chunk, k=k, bits=bits, decay=0.9)
        out = O.sparse_aggregate([(r["idx"], r["codes"], r["absmax"])], n, chunk=chunk, k=k, bits=bits,
                                 out_scale=1.0)
        kept = np.zeros(n, bool)
        ix = r["idx"].reshape(-1, k).astype(np.int64)
        for c in range(ix.shape[0]):
            kept[c * chunk + ix[c][ix[c] != 0xFFFF]] = True
        assert kept.sum() == sum(min(k, n - c * chunk) for c in range(ix.shape[0]))
        sent = r["h"] - r["e_new"]
        assert np.array_equal(out[kept].view(np.uint32), sent[kept].view(np.uint32))
        assert not np.any(out[~kept])


# -- LoCo-Adam on the synchronised gradient (LoCo Sec. 4, Eqn. (9)) --------------------------------

def pin_adam_worked(O):
    c = golden_io.adam_case()
    th, m, v = O.adam_step(c["theta"], c["m"], c["v"], c["g"], lr=c["lr"], beta1=c["beta1"], beta2=c["beta2"],
                           delta=c["delta"])
    assert np.array_equal(m, c["m_new"]), (m, c["m_new"])
    assert np.array_equal(v, c["v_new"]), (v, c["v_new"])
    assert np.array_equal(th, c["theta_new"]), (th, c["theta_new"])
    tb = torch.from_numpy(th).to(torch.bfloat16).float().numpy()
    assert np.array_equal(tb, th)  # the worked weights are exact in bf16 too


def pin_adam_closed_form(O):
    """A constant gradient from m_0 = v_0 = 0: m_k = (1 - (1 - b1)^k) g and
    v_k = (1 - (1 - b2)^k) g^2, so theta_K = theta_0 - lr * sum_k m_k / sqrt(v_k + delta)
    (float64 twin, to rounding)."""
    rng = _rng(40)
    n, K, lr, b1, b2, delta = 500, 30, 1e-3, 0.1, 0.02, 1e-8
    g = rng.standard_normal(n) * 1e-3
    th0 = rng.standard_normal(n)
    th, m, v = th0.copy(), np.zeros(n), np.zeros(n)
    want = th0.copy()
    for k in range(1, K + 1):
        th, m, v = O.adam_step(th, m, v, g, lr=lr, beta1=b1, beta2=b2, delta=delta, ftype=np.float64)
        mk = (1 - (1 - b1) ** k) * g
        vk = (1 - (1 - b2) ** k) * g * g
        assert np.allclose(m, mk, rtol=1e-12, atol=0) and np.allclose(v, vk, rtol=1e-12, atol=0)
        want = want - lr * mk / np.sqrt(vk + delta)
    assert np.allclose(th, want, rtol=1e-12, atol=1e-15)


def pin_adam_limits(O):
    """beta1 = beta2 = 1 with a tiny delta is sign descent: theta moves by lr * sign(g) to a
    few ulp; lr = 0 leaves theta bitwise; a zero gradient only decays m and v."""
    rng = _rng(41)
    n = 4000
    g = (rng.standard_normal(n) * 10.0 ** rng.integers(-6, 1, n)).astype(F32)
    th = rng.standard_normal(n).astype(F32)
    m = rng.standard_normal(n).astype(F32)
    v = (rng.random(n) * 1e-4).astype(F32)
    t1, m1, v1 = O.adam_step(th, m, v, g, lr=2.0 ** -10, beta1=1.0, beta2=1.0, delta=2.0 ** -120)
    assert np.array_equal(m1, g) and np.array_equal(v1, g * g)
    step = (th.astype(np.float64) - t1.astype(np.float64)) / 2.0 ** -10
    slack = 8 * np.spacing(np.abs(th)).astype(np.float64) / 2.0 ** -10 + 4 * 2.0 ** -23
    assert np.all(np.abs(step - np.sign(g)) <= slack)
    t2, _, _ = O.adam_step(th, m, v, g, lr=0.0, beta1=0.1, beta2=0.01, delta=1e-8)
    assert np.array_equal(t2, th)
    _, m3, v3 = O.adam_step(th, m, v, np.zeros(n, F32), lr=1e-3, beta1=0.1, beta2=0.01, delta=1e-8)
    assert np.array_equal(m3, (F32(1) - F32(0.1)) * m) and np.array_equal(v3, (F32(1) - F32(0.01)) * v)


def pin_dra_worked(O):
    """Eqn. (8) feeding Eqn. (9) on a hand-worked case whose average is exact in fp32 but
    not in bf16: the gradient of the step is the fp32 average (never rounded to bf16), the
    step uses the average (out_scale applied before it), and the weight copy is rounded to
    nearest even."""
    c = golden_io.dra_case()
    r = O.dequant_reduce_adam(c["peers"], c["n"], bits=c["bits"], block=c["block"], out_scale=c["out_scale"],
                              theta=c["theta"], m=c["m"], v=c["v"], lr=c["lr"], beta1=c["beta1"],
                              beta2=c["beta2"], delta=c["delta"])
    for key, want in (("g", "g"), ("m", "m_new"), ("v", "v_new"), ("theta", "theta_new")):
        assert np.array_equal(np.asarray(r[key], F32).view(np.uint32), c[want].view(np.uint32)), (key, r[key], c[want])
    tb = np.asarray(r["theta_bf16"], np.uint16).astype(np.uint32) << np.uint32(16)
    assert np.array_equal(tb.view(np.float32), c["theta_bf16"]), (tb.view(np.float32), c["theta_bf16"])


# -- blocks too small for a finite reciprocal (absmax below ~qmax * 2^-128) ------------------------

# IEEE binary32 overflow under round to nearest: a real result of magnitude at least
# 2^128 - 2^103 (the largest finite value plus half its ulp) rounds to infinity.
_F32_OVERFLOW = 2.0 ** 128 - 2.0 ** 103


def _tiny_blocks(rng, block, qmax, nblocks):
    """Blocks of subnormal / near-subnormal values: half with absmax far below the
    reciprocal's overflow (1/(absmax/qmax) >= 4 * 2^128), half with a subnormal step
    in [2^-127, 1.7 * 2^-127) whose reciprocal is finite; some exact zeros inside every
    block, one all-zero block."""
    out, kind = [], []
    for b in range(nblocks):
        if b == nblocks - 1:
            out.append(np.zeros(block, F32))
            kind.append("zero")
            continue
        over = b % 2 == 0
        # target absmax: qmax * 2^-131 .. qmax * 2^-130 (overflowing) or
        # qmax * 2^-127 .. qmax * 1.7 * 2^-127 (a subnormal step, finite reciprocal)
        if over:
            hi = qmax * 2.0 ** -130 * (0.5 + 0.5 * rng.random())
        else:
            hi = qmax * 2.0 ** -127 * (1.0 + 0.7 * rng.random())
        x = (rng.random(block) * 2 - 1) * hi
        x[rng.random(block) < 0.2] = 0.0
        x[int(rng.integers(0, block))] = hi if rng.random() < 0.5 else -hi
        x = x.astype(F32)
        if over:
            x[0] = F32(2.0 ** -149)  # the smallest subnormal
        out.append(x)
        kind.append("over" if over else "finite")
    return np.concatenate(out), kind


def pin_tiny_scales(O):
    """Blocks whose reciprocal 1/step overflows fp32 are sent as zero codes and, with
    beta = 0 (Eqn. (4)), leave the new error equal to h exactly; blocks just above that
    range (a subnormal step with a finite reciprocal) are still quantised within the
    rounding bound, with the largest element at +-qmax; exact zeros code to 0; nothing is
    NaN or infinite."""
    rng = _rng(60)
    for bits, block in ((4, 64), (8, 128), (2, 64)):
        qmax = (1 << (bits - 1)) - 1
        g, kind = _tiny_blocks(rng, block, qmax, 9)
        out = O.compensate_quantize(g, np.zeros(g.size, F32), bits=bits, block=block, beta=0.0)
        assert np.all(np.isfinite(out["e_new"])) and np.all(np.isfinite(out["d"]))
        q = out["q"]
        assert q.min() >= -qmax - 1 and q.max() <= qmax
        for b, kd in enumerate(kind):
            sl = slice(b * block, (b + 1) * block)
            hb, qb = g[sl].astype(np.float64), q[sl]
            am = float(out["absmax"][b])
            assert am == np.abs(hb).max()
            if kd in ("zero", "over"):
                if kd == "over":
                    assert 1.0 / (am / qmax) >= 4 * _F32_OVERFLOW  # far inside the overflow range
                assert not np.any(qb), (bits, b, kd)
                assert np.array_equal(out["e_new"][sl].view(np.uint32), g[sl].view(np.uint32)), (bits, b)
            else:
                assert 1.0 / (am / qmax) <= 2.0 ** 127  # comfortably finite
                # step = fl(am / qmax) is subnormal (>= 2^-127): its relative rounding is
                # at most 2^-23; with the roundings of 1/step, h * inv and q * step
                # (half a subnormal ulp, 2^-150, or 2^-24 relative) the bound below holds
                step = am / qmax
                assert step < 2.0 ** -126
                bound = step * (0.5 + qmax * 2.0 ** -20) + 2.0 ** -149
                r = np.abs(hb - out["d"][sl].astype(np.float64))
                assert np.all(r <= bound), (bits, b, r.max(), bound)
                assert np.abs(qb).max() == qmax, (bits, b)
            zeros = hb == 0
            assert not np.any(qb[zeros]) and not np.any(out["e_new"][sl][zeros])


def pin_topk_tiny_scales(O):
    """Top-k on chunks of tiny values: a chunk whose kept absmax is too small for a finite
    1/step keeps the right indices, sends zero codes and feeds every value back whole
    (e' = h everywhere); a chunk with a subnormal but invertible step quantises its largest
    kept value to +-qmax."""
    rng = _rng(61)
    for bits in (2, 4):
        qmax = (1 << (bits - 1)) - 1
        chunk, k = 64, 5
        g, kind = _tiny_blocks(rng, chunk, qmax, 5)
        r = O.topk_quantize(g, np.zeros(g.size, F32), chunk=chunk, k=k, bits=bits, decay=1.0)
        assert np.all(np.isfinite(r["e_new"]))
        q = O.unpack_codes(r["codes"], bits, r["codes"].size * 8 // bits).reshape(len(kind), -1)[:, :k]
        for c, kd in enumerate(kind):
            sl = slice(c * chunk, (c + 1) * chunk)
            key = np.abs(g[sl]).view(np.uint32)
            assert np.array_equal(r["idx"][c * k:(c + 1) * k], _brute_topk(key, k).astype(np.uint16))
            if kd in ("zero", "over"):
                assert not np.any(q[c]), (bits, c)
                assert np.array_equal(r["e_new"][sl].view(np.uint32), g[sl].view(np.uint32))
            else:
                assert np.abs(q[c]).max() == qmax, (bits, c, q[c])


ALL_PINS = [
    pin_identity_compressor, pin_beta_zero_is_efc, pin_quantisation_bound,
    pin_random_walk_bounded, pin_telescoping, pin_fixed_scale_golden, pin_torch_quantiser,
    pin_topk_brute_force, pin_pack_layout, pin_cq_worked, pin_dr_worked, pin_topk_worked,
    pin_dequant_reduce, pin_zero_blocks, pin_bf16_rne, pin_topk_error_feedback,
    pin_i8_error_accounting, pin_i8_equals_float_when_exact, pin_reset, pin_i8_compressor_vs_torch,
    pin_sa_worked, pin_sa_brute_force, pin_sa_dense_equivalent, pin_sa_transmits_topk,
    pin_adam_worked, pin_adam_closed_form, pin_adam_limits, pin_cq_scalar_twin, pin_dr_scalar_twin,
    pin_dra_worked, pin_tiny_scales, pin_topk_tiny_scales, pin_dequant_huge_scales,
    pin_dequant_reduce_peer_order,
]
