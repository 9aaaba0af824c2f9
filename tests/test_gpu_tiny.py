"""GPU parity on blocks too small for a finite reciprocal (LoCo Sec. 3.1, Eqn. (1)), and
on blocks near the top of the fp32 range.

A block whose absmax is below about qmax * 2^-128 has a step whose reciprocal overflows
fp32; both sides then take inv = 0, send zero codes and keep the block's values in the
error.  Blocks whose step is subnormal but invertible are quantised as usual.  The inputs
mix such blocks (absmax log-uniform in [1e-45, 4e-37], exact zeros inside), all-zero
blocks and ordinary N(0, 1e-3) blocks, for every gradient and error type, the 8-bit
error, every code width, and the Top-k mode.  Codes, absmax and the 8-bit error are
bit-exact; fp32 and bf16 errors within the usual bar (bitwise expected).
"""
import numpy as np
import pytest
import torch

from parity_util import say
from test_gpu_cq import TD, run_chain
from test_gpu_tk import run_tk_chain

pytestmark = pytest.mark.gpu


def tiny_values(step, n, block, seed):
    """Per block of `block` elements: 70% tiny (absmax log-uniform in [1e-45, 4e-37]),
    10% all zero, 20% N(0, 1e-3); 20% exact zeros inside the tiny blocks."""
    rng = np.random.default_rng([seed, step])
    nb = -(-n // block)
    kind = rng.random(nb)
    amp = np.exp(rng.uniform(np.log(1e-45), np.log(4e-37), nb))
    x = np.empty(nb * block, np.float64)
    for b in range(nb):
        sl = slice(b * block, (b + 1) * block)
        if kind[b] < 0.7:
            v = rng.uniform(-1, 1, block) * amp[b]
            v[rng.random(block) < 0.2] = 0.0
            x[sl] = v
        elif kind[b] < 0.8:
            x[sl] = 0.0
        else:
            x[sl] = rng.standard_normal(block) * 1e-3
    return torch.from_numpy(x[:n].astype(np.float32))


@pytest.mark.parametrize("gd", ["f32", "bf16"])
@pytest.mark.parametrize("ed", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("block", [64, 256])
def test_cq_tiny_blocks(gpu_lib, gd, ed, bits, block):
    sizes = [block * 37 + 5, 3 * 512 + 64]
    say(f"cq tiny blocks {gd}/{ed} bits={bits} B={block} sizes={sizes}")
    gen = lambda step, n: tiny_values(step, n, block, seed=bits * 1000 + block).to(TD[gd])  # noqa: E731
    run_chain(gpu_lib, sizes, gd, ed, bits, block, 0.9, 3, gen=gen,
              err_scale=2.0 ** 17 if ed == "i8" else 0.0)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_tk_tiny_chunks(gpu_lib, bits):
    """Top-k chunks of tiny values: zero codes where the chunk's reciprocal overflows,
    the error keeps every value; invertible subnormal steps quantise."""
    say(f"tk tiny chunks bits={bits}")
    run_tk_chain(gpu_lib, 20 * 1024 + 300, 1024, 41, bits, 1.0, 3,
                 lambda step, n: tiny_values(step, n, 1024, seed=77 + bits), f"tiny b{bits}")


def huge_values(step, n, block, seed):
    """Per block of `block` elements: 60% of magnitude log-uniform in [1e30, 3e38] (values
    uniform in +-that, below FLT_MAX / 1.2 so that h = g + e stays finite), 10% all zero,
    30% N(0, 1e-3)."""
    rng = np.random.default_rng([seed, step])
    nb = -(-n // block)
    kind = rng.random(nb)
    amp = np.exp(rng.uniform(np.log(1e30), np.log(2.8e38), nb))
    x = np.empty(nb * block, np.float64)
    for b in range(nb):
        sl = slice(b * block, (b + 1) * block)
        if kind[b] < 0.6:
            x[sl] = rng.uniform(-1, 1, block) * amp[b]
        elif kind[b] < 0.7:
            x[sl] = 0.0
        else:
            x[sl] = rng.standard_normal(block) * 1e-3
    return torch.from_numpy(x[:n].astype(np.float32))


@pytest.mark.filterwarnings("ignore:overflow encountered in multiply:RuntimeWarning")
@pytest.mark.parametrize("gd", ["f32", "bf16"])
@pytest.mark.parametrize("ed", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_cq_huge_blocks(gpu_lib, gd, ed, bits):
    """Block scales up to ~2.8e38: steps, (subnormal) reciprocals, codes and the error update
    stay the oracle's.  The 8-bit error's e * s_e overflows to inf there and clamps to 127
    on both sides (the oracle's overflow warning is expected)."""
    block = 128
    sizes = [block * 37 + 5, 3 * 512 + 64]
    say(f"cq huge blocks {gd}/{ed} bits={bits}")
    gen = lambda step, n: huge_values(step, n, block, seed=bits * 100 + 7).to(TD[gd])  # noqa: E731
    run_chain(gpu_lib, sizes, gd, ed, bits, block, 0.9, 3, gen=gen, err_scale=2.0 ** 17 if ed == "i8" else 0.0)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_tk_huge_chunks(gpu_lib, bits):
    """Top-k chunks whose selected values reach ~2.8e38: the chunk step, its (subnormal)
    reciprocal, the codes and the error feedback stay the oracle's."""
    say(f"tk huge chunks bits={bits}")
    run_tk_chain(gpu_lib, 20 * 1024 + 300, 1024, 41, bits, 1.0, 3,
                 lambda step, n: huge_values(step, n, 1024, seed=91 + bits), f"huge b{bits}")
