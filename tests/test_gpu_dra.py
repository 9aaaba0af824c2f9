"""GPU parity of loco_dequant_reduce_adam (LoCo Eqn. (8) fused with the Eqn. (9) step)
against the CPU oracle.

Each case runs a chain of steps: the GPU keeps its weights and moments, the oracle its
own; every step gets fresh seeded payloads.  Weights and moments must be within 1e-6
relative (fp32) and the bf16 copy within 1 ulp; bitwise equality is expected, since both
sides take the same IEEE operations in the same order.  Every buffer has canaries.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import Guarded, assert_bf16_close, assert_f32_close, bf16_bits, host, say

pytestmark = pytest.mark.gpu


def run_chain(loco, n, npeers, bits, block, steps, *, lr=1e-4, beta1=0.1, beta2=0.01, delta=1e-8,
              fixed=0.0, with_bf16=True, key="dra"):
    rng = np.random.default_rng(W.seed_of("dra-theta", n, npeers, bits, block, key) % 2 ** 32)
    theta0 = rng.standard_normal(n).astype(np.float32) * 0.02
    th = Guarded(n, torch.float32, init=torch.from_numpy(theta0))
    m = Guarded(n, torch.float32, init=torch.zeros(n))
    v = Guarded(n, torch.float32, init=torch.zeros(n))
    tb = Guarded(n, torch.bfloat16) if with_bf16 else None
    o_th, o_m, o_v = theta0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    bitwise = True
    for s in range(steps):
        pays = [W.random_payload(n, bits, block, key=(key, s, p)) for p in range(npeers)]
        dev = [(c.cuda(), None if fixed else a.cuda()) for c, a in pays]
        loco.loco_dequant_reduce_adam(dev, n, bits=bits, block=block, out_scale=1.0 / npeers, param=th.t, m=m.t,
                                      v=v.t, lr=lr, beta1=beta1, beta2=beta2, delta=delta,
                                      param_bf16=None if tb is None else tb.t, fixed_scale=fixed)
        torch.cuda.synchronize()
        ref = oracle.dequant_reduce_adam([(host(c), None if fixed else host(a)) for c, a in pays], n, bits=bits,
                                         block=block, out_scale=1.0 / npeers, theta=o_th, m=o_m, v=o_v, lr=lr,
                                         beta1=beta1, beta2=beta2, delta=delta, fixed_scale=fixed)
        tag = f"step {s} n={n} peers={npeers} bits={bits} B={block} fixed={fixed}"
        z = np.zeros(n)
        bitwise &= assert_f32_close(host(m.t), ref["m"], z, f"{tag} m")
        bitwise &= assert_f32_close(host(v.t), ref["v"], z, f"{tag} v")
        bitwise &= assert_f32_close(host(th.t), ref["theta"], z, f"{tag} theta")
        if tb is not None:
            bitwise &= assert_bf16_close(bf16_bits(tb.t), ref["theta_bf16"], f"{tag} theta bf16")
        for b, nm in ((th, "theta"), (m, "m"), (v, "v"), (tb, "theta bf16")):
            if b is not None:
                b.check(f"{tag} {nm}")
        o_th, o_m, o_v = ref["theta"], ref["m"], ref["v"]
    assert bitwise, "not bitwise equal"


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("block", [64, 256, 512])
def test_dra_matrix(gpu_lib, bits, block):
    """Every code width and a range of blocks on ragged sizes (whole tiles and tails)."""
    for n in (1, 511, 512, 513, 4096 + 77, 65536 + 300):
        say(f"dra bits={bits} B={block} n={n}")
        run_chain(gpu_lib, n, 3, bits, block, 3, with_bf16=(n % 2 == 1))


@pytest.mark.parametrize("beta2", [0.001, 0.05])
def test_dra_page_hyperparameters(gpu_lib, beta2):
    """The page's typical beta1 = 0.1 and beta2 in [0.001, 0.05], 6 steps, 8 peers."""
    say(f"dra beta2={beta2}")
    run_chain(gpu_lib, 300_001, 8, 4, 128, 6, lr=3e-4, beta1=0.1, beta2=beta2, delta=1e-8, key=f"page{beta2}")


@pytest.mark.parametrize("npeers", [1, 9, 128])
def test_dra_peers(gpu_lib, npeers):
    say(f"dra peers={npeers}")
    run_chain(gpu_lib, 20_000 + 13, npeers, 4, 256, 2, key=f"peers{npeers}")


def test_dra_fixed_scale(gpu_lib):
    say("dra fixed scale")
    run_chain(gpu_lib, 70_001, 4, 4, 128, 3, fixed=2.0 ** 19, key="fixed")


def test_dra_limits(gpu_lib):
    """beta1 = beta2 = 1 (m = g, v = g^2), lr = 0, and a large delta."""
    say("dra limits")
    run_chain(gpu_lib, 10_000, 2, 4, 64, 2, beta1=1.0, beta2=1.0, delta=2.0 ** -100, key="sign")
    run_chain(gpu_lib, 10_000, 2, 4, 64, 2, lr=0.0, key="lr0")
    run_chain(gpu_lib, 10_000, 2, 4, 64, 2, delta=1.0, beta1=0.0, beta2=0.0, key="frozen")


def test_dra_matches_unfused_reduce(gpu_lib):
    """The fused step sees exactly the fp32 gradient that loco_dequant_reduce writes."""
    n, P = 100_003, 5
    pays = [tuple(x.cuda() for x in W.random_payload(n, 4, 256, key=("unf", p))) for p in range(P)]
    g = torch.empty(n, device="cuda")
    gpu_lib.loco_dequant_reduce(pays, n, bits=4, block=256, out=g, out_scale=1.0 / P)
    th = torch.zeros(n, device="cuda")
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    # beta1 = 1, lr = 0: m becomes the gradient itself
    gpu_lib.loco_dequant_reduce_adam(pays, n, bits=4, block=256, out_scale=1.0 / P, param=th, m=m, v=v, lr=0.0,
                                     beta1=1.0, beta2=1.0, delta=1.0)
    torch.cuda.synchronize()
    assert np.array_equal(host(m).view(np.uint32), host(g).view(np.uint32))
