"""Seeded synthetic gradients shaped like the LoCo / SparseLoCo workloads.

Shared by the tests, the benchmark and the smoke check.  This module only draws
random numbers and lays them out; it holds none of the compression arithmetic.

Every tensor is drawn in slices of 2^24 elements, each from its own torch
generator seeded by a stable hash of (workload, step, tensor, slice), so a given
(device, key) always gives the same bytes.  bf16 tensors are rounded from fp32 by
torch's own conversion.

Workloads (sizes are the full ones; every function takes smaller sizes too):
  tiny        one flat fp32 gradient of 1,048,576 elements ~ N(0, 1e-3)
  llama_layer the 7 weight gradients of one LLaMA-7B layer (q, k, v, o 4096x4096;
              gate, up 11008x4096; down 4096x11008) in bf16, Student-t(3) times a
              per-tensor log-uniform factor in [1e-5, 1e-2]
  shard7b     one rank's flat 842,000,000-element bf16 shard, 1e-3 * Student-t(3);
              peer partitions of 105,250,000 elements from the same law
  moe         8 experts x (w1, w3: 14336x4096; w2: 4096x14336) bf16; per matrix 30% of
              the rows are zero (fixed across steps), the rest N(0, sigma_x) with one
              log-uniform sigma_x in [1e-5, 1e-3] per expert
  sparseloco  flat fp32 N(0, 1e-3) with each element replaced, with probability 1e-3,
              by exactly +-0.1 (100 sigma) with a random sign
"""

from __future__ import annotations

import hashlib
import math

import torch

SLICE = 1 << 24

LLAMA_LAYER = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
               ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
MOE_EXPERT = [("w1", 14336, 4096), ("w3", 14336, 4096), ("w2", 4096, 14336)]
SHARD7B_N = 842_000_000
SHARD7B_PEERS = 8
SHARD7B_PART = 105_250_000
TINY_N = 1 << 20
SPARSE_N = 1 << 28


def seed_of(*key) -> int:
    """Stable 63-bit seed from a key tuple."""
    h = hashlib.sha256(repr(key).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*key))
    return g


def _fill(n, device, key, draw):
    """Allocate fp32[n] and fill it slice by slice with draw(m, generator)."""
    out = torch.empty(n, dtype=torch.float32, device=device)
    for s, lo in enumerate(range(0, n, SLICE)):
        m = min(SLICE, n - lo)
        out[lo:lo + m] = draw(m, _gen(device, *key, s))
    return out


def _normal(m, g, device):
    return torch.randn(m, generator=g, device=device, dtype=torch.float32)


def _student_t3(m, g, device):
    """Student-t with 3 degrees of freedom: z0 / sqrt((z1^2 + z2^2 + z3^2) / 3)."""
    z = torch.randn(4, m, generator=g, device=device, dtype=torch.float32)
    chi = (z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0
    return z[0] / torch.sqrt(chi)


def _log_uniform(lo, hi, *key) -> float:
    g = _gen("cpu", *key)
    u = torch.rand(1, generator=g, dtype=torch.float64).item()
    return math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))


# -- tiny ---------------------------------------------------------------------

def tiny_grad(step, n=TINY_N, device="cpu", stream="grad"):
    """fp32 N(0, 1e-3); `stream` separates the rank's gradient from peer draws."""
    return _fill(n, device, ("tiny", stream, step), lambda m, g: _normal(m, g, device) * 1e-3)


def tiny_peer_grads(npeers=4, n=TINY_N, device="cpu"):
    return [tiny_grad(0, n, device, stream=f"peer{p}") for p in range(npeers)]


# -- LLaMA-7B layer -------------------------------------------------------------

def llama_layer_shapes(div=1):
    """(name, rows, cols); div > 1 shrinks the rows for small parity runs."""
    return [(nm, max(1, r // div), c) for nm, r, c in LLAMA_LAYER]


def llama_layer_grads(step, div=1, device="cpu"):
    out = []
    for t, (nm, r, c) in enumerate(llama_layer_shapes(div)):
        scale = _log_uniform(1e-5, 1e-2, "llama", "scale", nm)
        x = _fill(r * c, device, ("llama", nm, step, div),
                  lambda m, g: _student_t3(m, g, device) * scale)
        out.append(x.to(torch.bfloat16))
    return out


# -- 7B FSDP shard --------------------------------------------------------------

def shard7b_grad(step, n=SHARD7B_N, device="cpu", chain="cq4"):
    x = _fill(n, device, ("shard7b", chain, step, n),
              lambda m, g: _student_t3(m, g, device) * 1e-3)
    return x.to(torch.bfloat16)


def shard7b_peer_grads(npeers=SHARD7B_PEERS, n=SHARD7B_PART, device="cpu"):
    return [shard7b_grad(0, n, device, chain=f"peer{p}") for p in range(npeers)]


# -- MoE experts ----------------------------------------------------------------

def moe_shapes(div=1, experts=8):
    return [(f"e{x}.{nm}", x, max(1, r // div), c)
            for x in range(experts) for nm, r, c in MOE_EXPERT]


def moe_zero_rows(name, rows):
    """The round(0.3 * rows) rows of a matrix that stay zero at every step."""
    nz = int(round(0.3 * rows))
    perm = torch.randperm(rows, generator=_gen("cpu", "moe", "zero", name, rows))
    mask = torch.zeros(rows, dtype=torch.bool)
    mask[perm[:nz]] = True
    return mask


def moe_grads(step, div=1, experts=8, device="cpu"):
    out = []
    for name, x, r, c in moe_shapes(div, experts):
        sigma = _log_uniform(1e-5, 1e-3, "moe", "sigma", x)
        v = _fill(r * c, device, ("moe", name, step, div),
                  lambda m, g: _normal(m, g, device) * sigma).view(r, c)
        v[moe_zero_rows(name, r).to(device)] = 0.0
        out.append(v.reshape(-1).to(torch.bfloat16))
    return out


# -- payloads as the dequant-reduce input ---------------------------------------

def random_payload(n, bits, block, key, device="cpu", zero_frac=0.1):
    """Uniformly random code bytes (padding bits included) and positive absmax values
    (log-uniform in [1e-5, 1e-2], a fraction of them exactly zero)."""
    nbytes = (n * bits + 7) // 8
    g = _gen(device, "payload", key, n, bits, block)
    codes = torch.randint(0, 256, (nbytes,), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    nb = -(-n // block)
    u = torch.rand(nb, generator=g, device=device, dtype=torch.float32)
    absmax = torch.exp(math.log(1e-5) + u * (math.log(1e-2) - math.log(1e-5)))
    z = torch.rand(nb, generator=g, device=device) < zero_frac
    absmax[z] = 0.0
    return codes, absmax


def random_sparse_payload(n, chunk, k, bits, key, device="cpu", zero_frac=0.1, drop_frac=0.02, ordered=True):
    """A Top-k-shaped payload of n elements in chunks: per chunk, k distinct chunk-local
    indices (ascending unless `ordered` is False); slots past a short last chunk's
    length and a few dropped slots hold 0xFFFF.  Code bytes are uniformly random; the
    per-chunk absmax is log-uniform in [1e-5, 1e-2], a fraction of them exactly zero.
    The indices are an int16 tensor holding the u16 patterns."""
    nch = -(-n // chunk)
    g = _gen(device, "sparse-payload", key, n, chunk, k, bits)
    r = torch.rand(nch, chunk, generator=g, device=device)
    last = n - (nch - 1) * chunk
    r[-1, last:] = -1.0  # positions past the end are picked only when k exceeds the length
    idx = r.topk(k, dim=1).indices
    if ordered:
        idx = idx.sort(dim=1).values
    unused = torch.rand(nch, k, generator=g, device=device) < drop_frac
    unused[-1] |= idx[-1] >= last
    idx = torch.where(unused, torch.full_like(idx, -1), idx).to(torch.int16)  # -1 is 0xFFFF
    codes = torch.randint(0, 256, (nch * ((k * bits + 7) // 8),), generator=g, device=device,
                          dtype=torch.int32).to(torch.uint8)
    u = torch.rand(nch, generator=g, device=device, dtype=torch.float32)
    absmax = torch.exp(math.log(1e-5) + u * (math.log(1e-2) - math.log(1e-5)))
    absmax[torch.rand(nch, generator=g, device=device) < zero_frac] = 0.0
    return idx.reshape(-1).contiguous(), codes, absmax


# -- SparseLoCo pseudo-gradient -------------------------------------------------

def sparseloco_grad(step, n=SPARSE_N, device="cpu", p_out=1e-3, sigma=1e-3):
    def draw(m, g):
        v = _normal(m, g, device) * sigma
        u = torch.rand(m, generator=g, device=device)
        sgn = torch.rand(m, generator=g, device=device) < 0.5
        out = torch.full((m,), 100.0 * sigma, dtype=torch.float32, device=device)
        out[sgn] = -100.0 * sigma
        return torch.where(u < p_out, out, v)
    return _fill(n, device, ("sparseloco", step, n), draw)
