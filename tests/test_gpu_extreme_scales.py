"""GPU parity of dequant-reduce, the fused Adam step and the sparse aggregation at extreme
block scales (LoCo Sec. 3.3, Eqn. (8); Sec. 4, Eqn. (9); SparseLoCo's aggregation).

The kernels' fast decoder forms fl(q * step) as one fma against the offset
-2^(b-1) * step (and, at 4 and 8 bits, a step scaled by 2^24), which would overflow for a
step of 2^100 or more; a tile holding such a step (or an infinite or NaN one) is redone
element-wise as q * step.  The payloads here interleave regions of ordinary blocks
(absmax log-uniform in [1e-5, 1e-2], some zero) with regions of extreme ones: absmax at and
just below qmax * 2^100, log-uniform in [2^95, 2^128), FLT_MAX, subnormal, zero, inf and
NaN, so that one launch takes both paths.  Payload codes are random bytes (any byte is a
valid payload).  Every output is compared bitwise with the oracle, except that where the
oracle's value is a NaN the GPU's must be a NaN (of any payload).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import Guarded, bf16_bits, host, say

pytestmark = pytest.mark.gpu

F32_MAX = float(np.finfo(np.float32).max)


def extreme_absmax(nb, bits, seed, region=16):
    """Per-block absmax: blocks in every third run of `region` blocks are extreme, the rest
    ordinary."""
    qmax = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(seed)
    a = np.exp(rng.uniform(np.log(1e-5), np.log(1e-2), nb)).astype(np.float32)
    a[rng.random(nb) < 0.1] = 0.0
    thr = np.float32(qmax * 2.0 ** 100)
    below = np.nextafter(thr, np.float32(0))
    kinds = [thr, below, np.float32(F32_MAX), np.float32(0.0), np.float32(1e-42), np.float32(np.inf),
             np.float32(np.nan)]
    for b in range(nb):
        if (b // region) % 3 != 0:
            continue
        r = rng.random()
        if r < 0.5:
            a[b] = np.float32(np.exp(rng.uniform(np.log(2.0 ** 95), np.log(F32_MAX))))
        elif r < 0.75:
            a[b] = kinds[rng.integers(0, 3)]
        elif r < 0.95:
            a[b] = kinds[rng.integers(3, 5)]
        else:
            a[b] = kinds[rng.integers(5, 7)]
    return a


def assert_f32_nan_aware(got, want, what):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    wn = np.isnan(want)
    if not np.array_equal(np.isnan(got), wn):
        i = int(np.argmax(np.isnan(got) != wn))
        raise AssertionError(f"{what}: NaN positions differ; first at {i}: got {got[i]!r} want {want[i]!r}")
    g, w = got[~wn].view(np.uint32), want[~wn].view(np.uint32)
    if not np.array_equal(g, w):
        i = int(np.flatnonzero(g != w)[0])
        raise AssertionError(f"{what}: {int(np.sum(g != w))} values differ; first (of the non-NaN) at {i}: "
                             f"got {got[~wn][i]!r} want {want[~wn][i]!r}")


def bf16_isnan(u):
    u = np.asarray(u, np.uint16)
    return ((u & 0x7F80) == 0x7F80) & ((u & 0x007F) != 0)


def assert_bf16_nan_aware(got, want, what):
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    wn = bf16_isnan(want)
    if not np.array_equal(bf16_isnan(got), wn):
        raise AssertionError(f"{what}: NaN positions differ")
    if not np.array_equal(got[~wn], want[~wn]):
        raise AssertionError(f"{what}: {int(np.sum(got[~wn] != want[~wn]))} values differ")


def extreme_payloads(n, bits, block, npeers, key):
    nb = -(-n // block)
    out = []
    for p in range(npeers):
        codes, _ = W.random_payload(n, bits, block, key=("extreme", key, p))
        a = extreme_absmax(nb, bits, W.seed_of("extreme-absmax", key, p, n, bits, block) % 2 ** 32)
        out.append((codes, torch.from_numpy(a)))
    return out


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("block", [64, 256])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("npeers", [3, 8])
def test_dr_extreme_scales(gpu_lib, bits, block, out_dtype, npeers):
    for n in (2049, 100_003):
        say(f"dr extreme scales bits={bits} B={block} out={out_dtype} peers={npeers} n={n}")
        pays = extreme_payloads(n, bits, block, npeers, (bits, block, out_dtype, npeers, n))
        dev = [(Guarded(c.numel(), torch.uint8, init=c), Guarded(a.numel(), torch.float32, init=a)) for c, a in pays]
        out = Guarded(n, torch.float32 if out_dtype == "f32" else torch.bfloat16)
        gpu_lib.loco_dequant_reduce([(c.t, a.t) for c, a in dev], n, bits=bits, block=block, out=out.t,
                                    out_scale=1.0 / npeers)
        torch.cuda.synchronize()
        with np.errstate(over="ignore", invalid="ignore"):
            want = oracle.dequant_reduce([(c.numpy(), a.numpy()) for c, a in pays], n, bits=bits, block=block,
                                         out_scale=1.0 / npeers, out_dtype=out_dtype)
        out.check("out")
        tag = f"n={n} bits={bits} B={block} peers={npeers}"
        if out_dtype == "f32":
            assert_f32_nan_aware(host(out.t), want, tag)
        else:
            assert_bf16_nan_aware(bf16_bits(out.t), want, tag)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("fixed", [2.0 ** -99, 2.0 ** -110, 1e-40])
def test_dr_fixed_scale_extreme(gpu_lib, bits, fixed):
    """The paper's fixed scale s at the edges: step = fl(1/s) just below 2^100 (fast
    decoder), at 2^110 (element-wise) and infinite (s subnormal)."""
    n = 70_001
    say(f"dr fixed extreme bits={bits} s={fixed}")
    pays = [(W.random_payload(n, bits, 64, key=("fxe", p))[0], None) for p in range(4)]
    out = Guarded(n, torch.float32)
    gpu_lib.loco_dequant_reduce([(c.cuda(), None) for c, _ in pays], n, bits=bits, block=64, out=out.t,
                                out_scale=0.25, fixed_scale=fixed)
    torch.cuda.synchronize()
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        want = oracle.dequant_reduce([(c.numpy(), None) for c, _ in pays], n, bits=bits, block=64,
                                     out_scale=0.25, fixed_scale=fixed)
    out.check("out")
    assert_f32_nan_aware(host(out.t), want, f"fixed s={fixed} bits={bits}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("block", [64, 256])
def test_dra_extreme_scales(gpu_lib, bits, block):
    """Two fused Adam steps on payloads with extreme scales; weights, moments and the bf16
    copy bitwise (NaN-aware)."""
    n, npeers = 65536 + 300, 8
    rng = np.random.default_rng(W.seed_of("dra-extreme", bits, block) % 2 ** 32)
    theta0 = rng.standard_normal(n).astype(np.float32) * 0.02
    th = Guarded(n, torch.float32, init=torch.from_numpy(theta0))
    m = Guarded(n, torch.float32, init=torch.zeros(n))
    v = Guarded(n, torch.float32, init=torch.zeros(n))
    tb = Guarded(n, torch.bfloat16)
    o_th, o_m, o_v = theta0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    hp = dict(lr=1e-4, beta1=0.1, beta2=0.01, delta=1e-8)
    for s in range(2):
        say(f"dra extreme scales bits={bits} B={block} step {s}")
        pays = extreme_payloads(n, bits, block, npeers, ("dra", bits, block, s))
        gpu_lib.loco_dequant_reduce_adam([(c.cuda(), a.cuda()) for c, a in pays], n, bits=bits, block=block,
                                         out_scale=1.0 / npeers, param=th.t, m=m.t, v=v.t, param_bf16=tb.t, **hp)
        torch.cuda.synchronize()
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            ref = oracle.dequant_reduce_adam([(c.numpy(), a.numpy()) for c, a in pays], n, bits=bits, block=block,
                                             out_scale=1.0 / npeers, theta=o_th, m=o_m, v=o_v, **hp)
        tag = f"step {s} bits={bits} B={block}"
        assert_f32_nan_aware(host(m.t), ref["m"], f"{tag} m")
        assert_f32_nan_aware(host(v.t), ref["v"], f"{tag} v")
        assert_f32_nan_aware(host(th.t), ref["theta"], f"{tag} theta")
        assert_bf16_nan_aware(bf16_bits(tb.t), ref["theta_bf16"], f"{tag} theta bf16")
        for b, nm in ((th, "theta"), (m, "m"), (v, "v"), (tb, "theta bf16")):
            b.check(f"{tag} {nm}")
        o_th, o_m, o_v = ref["theta"], ref["m"], ref["v"]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("od", ["f32", "bf16"])
def test_sa_extreme_scales(gpu_lib, bits, od):
    """Sparse aggregation (SparseLoCo) of 8 peers whose chunk scales mix ordinary and extreme
    values (the same mix as above, per chunk): fp32 output through the pre-read and the
    general kernel, bf16 output through the streaming kernel; bitwise, NaN-aware."""
    n, chunk, k, npeers = 300 * 1024 + 77, 1024, 41, 8
    nch = -(-n // chunk)
    say(f"sparse aggregation extreme scales bits={bits} out={od}")
    pays = []
    for p in range(npeers):
        ix, c, _ = W.random_sparse_payload(n, chunk, k, bits, key=("extreme-sa", bits, od, p))
        a = extreme_absmax(nch, bits, W.seed_of("extreme-sa-absmax", bits, od, p) % 2 ** 32, region=8)
        pays.append((ix, c, torch.from_numpy(a)))
    out = Guarded(n, torch.float32 if od == "f32" else torch.bfloat16)
    gpu_lib.loco_sparse_aggregate([(ix.cuda(), c.cuda(), a.cuda()) for ix, c, a in pays], n, chunk=chunk, k=k,
                                  bits=bits, out=out.t, out_scale=1.0 / npeers)
    torch.cuda.synchronize()
    with np.errstate(over="ignore", invalid="ignore"):
        want = oracle.sparse_aggregate([(ix.numpy().view(np.uint16), c.numpy(), a.numpy()) for ix, c, a in pays], n,
                                       chunk=chunk, k=k, bits=bits, out_scale=1.0 / npeers, out_dtype=od)
    out.check("out")
    if od == "f32":
        assert_f32_nan_aware(host(out.t), want, f"bits={bits}")
    else:
        assert_bf16_nan_aware(bf16_bits(out.t), want, f"bits={bits}")


@pytest.mark.parametrize("adam", [False, True])
def test_extreme_scale_in_a_late_peer_group(gpu_lib, adam):
    """40 peers: the steps of a tile are computed for one group of peers at a time (16 peers
    per group for the bf16 shard, 32 for the fused Adam step), so a tile whose only extreme
    scales sit in the last group has accumulated the earlier groups when it switches to the
    element-wise path; that path must start the tile over."""
    n, bits, block, npeers = 50_000 + 123, 4, 256, 40
    nb = -(-n // block)
    say(f"extreme scale in the last peer group ({'fused Adam' if adam else 'bf16 out'})")
    pays = []
    for p in range(npeers):
        codes, a = W.random_payload(n, bits, block, key=("late-group", adam, p))
        if p >= 32:
            a = torch.from_numpy(extreme_absmax(nb, bits, W.seed_of("late-group-absmax", adam, p) % 2 ** 32,
                                                region=4))
        pays.append((codes, a))
    hp = dict(lr=1e-4, beta1=0.1, beta2=0.01, delta=1e-8)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        if adam:
            rng = np.random.default_rng(5)
            theta0 = rng.standard_normal(n).astype(np.float32) * 0.02
            th = Guarded(n, torch.float32, init=torch.from_numpy(theta0))
            m = Guarded(n, torch.float32, init=torch.zeros(n))
            v = Guarded(n, torch.float32, init=torch.zeros(n))
            gpu_lib.loco_dequant_reduce_adam([(c.cuda(), a.cuda()) for c, a in pays], n, bits=bits, block=block,
                                             out_scale=1.0 / npeers, param=th.t, m=m.t, v=v.t, **hp)
            torch.cuda.synchronize()
            ref = oracle.dequant_reduce_adam([(c.numpy(), a.numpy()) for c, a in pays], n, bits=bits, block=block,
                                             out_scale=1.0 / npeers, theta=theta0, m=np.zeros(n, np.float32),
                                             v=np.zeros(n, np.float32), **hp)
            assert_f32_nan_aware(host(m.t), ref["m"], "m")
            assert_f32_nan_aware(host(v.t), ref["v"], "v")
            assert_f32_nan_aware(host(th.t), ref["theta"], "theta")
            for b, nm in ((th, "theta"), (m, "m"), (v, "v")):
                b.check(nm)
        else:
            out = Guarded(n, torch.bfloat16)
            gpu_lib.loco_dequant_reduce([(c.cuda(), a.cuda()) for c, a in pays], n, bits=bits, block=block,
                                        out=out.t, out_scale=1.0 / npeers)
            torch.cuda.synchronize()
            want = oracle.dequant_reduce([(c.numpy(), a.numpy()) for c, a in pays], n, bits=bits, block=block,
                                         out_scale=1.0 / npeers, out_dtype="bf16")
            out.check("out")
            assert_bf16_nan_aware(bf16_bits(out.t), want, "out")
