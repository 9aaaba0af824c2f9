"""GPU parity of loco_dequant_reduce against the CPU oracle.

Payloads are either the oracle's own compensate-quantize output or uniformly random
bytes from the seeded generator (any bytes are a valid payload), never GPU output.
The reduced output must match within 1e-6 relative in fp32 (bitwise expected) or 1 ulp
in bf16.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import Guarded, assert_bf16_close, assert_f32_close, bf16_bits, host, say

pytestmark = pytest.mark.gpu

SIZES = [1, 31, 32, 33, 2047, 2048, 2049, 100_003]


def run_dr(loco, payloads, n, bits, block, out_dtype, out_scale, fixed=0.0):
    dev_pay = []
    for c, a in payloads:
        gc = Guarded(c.numel(), torch.uint8, init=c)
        ga = None if a is None else Guarded(a.numel(), torch.float32, init=a)
        dev_pay.append((gc, ga))
    out = Guarded(n, torch.float32 if out_dtype == "f32" else torch.bfloat16)
    loco.loco_dequant_reduce([(c.t, None if a is None else a.t) for c, a in dev_pay], n, bits=bits, block=block,
                             out=out.t, out_scale=out_scale, fixed_scale=fixed)
    torch.cuda.synchronize()
    want = oracle.dequant_reduce([(c.numpy(), None if a is None else a.numpy()) for c, a in payloads], n,
                                 bits=bits, block=block, out_scale=out_scale, out_dtype=out_dtype,
                                 fixed_scale=fixed)
    out.check("out")
    for c, a in dev_pay:
        c.check("codes")
        if a is not None:
            a.check("absmax")
    if out_dtype == "f32":
        # floor: the largest single contribution's step times the scale
        return assert_f32_close(host(out.t), want, np.full(n, 1e-30), "out")
    return assert_bf16_close(bf16_bits(out.t), want, "out")


def test_dr_tiny_workload(gpu_lib):
    """4 peers of 1,048,576 elements quantised by the oracle (4-bit, B=128), fp32 out, x1/4."""
    n, bits, block = W.TINY_N, 4, 128
    pay = []
    for g in W.tiny_peer_grads(4, n=n):
        r = oracle.compensate_quantize(g.numpy(), np.zeros(n, np.float32), bits=bits, block=block, beta=0.9)
        pay.append((torch.from_numpy(r["codes"]), torch.from_numpy(r["absmax"])))
    say("dr tiny: 4 peers x 1048576, f32 out")
    assert run_dr(gpu_lib, pay, n, bits, block, "f32", 0.25)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("block", [64, 128, 256, 512])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("npeers", [1, 3, 8])
def test_dr_matrix(gpu_lib, bits, block, out_dtype, npeers):
    say(f"dr matrix bits={bits} B={block} out={out_dtype} peers={npeers}")
    for n in SIZES:
        pay = [W.random_payload(n, bits, block, key=(p, "m")) for p in range(npeers)]
        run_dr(gpu_lib, pay, n, bits, block, out_dtype, 1.0 / npeers)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_dr_fixed_scale(gpu_lib, bits):
    say(f"dr fixed scale bits={bits}")
    for n in (1, 2049, 70_001):
        pay = [(W.random_payload(n, bits, 64, key=(p, "fx"))[0], None) for p in range(4)]
        run_dr(gpu_lib, pay, n, bits, 64, "f32", 0.25, fixed=2.0 ** 19)


def test_dr_max_peers(gpu_lib):
    n = 5000
    say("dr 128 peers")
    pay = [W.random_payload(n, 4, 256, key=(p, "max")) for p in range(gpu_lib.LOCO_MAX_PEERS)]
    run_dr(gpu_lib, pay, n, 4, 256, "bf16", 1.0 / 128)


def test_dr_shard_scaled(gpu_lib):
    """The 7B-shard reduce at 1/64 size: 8 peers, 4-bit, B=256, bf16 out, x1/8, with the
    payloads made by the oracle from Student-t partitions."""
    n = W.SHARD7B_PART // 64
    pay = []
    for g in W.shard7b_peer_grads(8, n=n):
        gn = g.view(torch.int16).numpy().view(np.uint16)
        r = oracle.compensate_quantize(gn, np.zeros(n, np.float32), bits=4, block=256, beta=0.9,
                                       grad_dtype="bf16")
        pay.append((torch.from_numpy(r["codes"]), torch.from_numpy(r["absmax"])))
    say(f"dr shard /64: 8 x {n}, bf16 out")
    assert run_dr(gpu_lib, pay, n, 4, 256, "bf16", 0.125)
