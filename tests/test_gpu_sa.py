"""GPU parity of loco_sparse_aggregate (SparseLoCo's sparse aggregation) against the CPU
oracle.

Payloads come from the seeded generator (distinct chunk-local indices, unused 0xFFFF
slots, random code bytes, positive scales with some zero chunks), never from the GPU
path.  The output must be within 1e-6 relative (fp32) or 1 bf16 ulp of the oracle;
bitwise equality is expected, since both sides add the same fp32 values in peer order.
The output buffer has canaries on both sides.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import Guarded, assert_bf16_close, assert_f32_close, bf16_bits, host, say

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def host_payload(p):
    ix, c, a = p
    return host(ix).view(np.uint16), host(c), host(a)


def check(loco, peers, n, chunk, k, bits, od, scale, tag):
    out = Guarded(n, TD[od])
    loco.loco_sparse_aggregate([(ix.cuda(), c.cuda(), a.cuda()) for ix, c, a in peers], n, chunk=chunk, k=k,
                               bits=bits, out=out.t, out_scale=scale)
    torch.cuda.synchronize()
    want = oracle.sparse_aggregate([host_payload(p) for p in peers], n, chunk=chunk, k=k, bits=bits,
                                   out_scale=scale, out_dtype=od)
    if od == "f32":
        bw = assert_f32_close(host(out.t), want, np.zeros(n), tag)
    else:
        bw = assert_bf16_close(bf16_bits(out.t), want, tag)
    out.check(f"{tag} out")
    assert bw, f"{tag}: not bitwise equal"


@pytest.mark.parametrize("chunk", [256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("od", ["f32", "bf16"])
def test_sa_matrix(gpu_lib, chunk, bits, od):
    """Every chunk size, code width and output type; k from 1 to the whole chunk, with a
    short last chunk; 3 peers."""
    n = 3 * chunk + chunk // 3 + 5
    for k in sorted({1, 82 if chunk >= 82 else chunk // 2, chunk // 2 + 1, chunk}):
        say(f"sa matrix chunk={chunk} bits={bits} out={od} k={k} n={n}")
        peers = [W.random_sparse_payload(n, chunk, k, bits, key=("m", p)) for p in range(3)]
        check(gpu_lib, peers, n, chunk, k, bits, od, 1.0 / 3.0, f"chunk {chunk} bits {bits} {od} k {k}")


@pytest.mark.parametrize("npeers", [1, 2, 8, 9, 17, 128])
def test_sa_peer_counts(gpu_lib, npeers):
    """Peer batches of 8: one, a full batch, one past it, and the maximum."""
    n, chunk, k = 4096 * 5 + 1000, 4096, 82
    say(f"sa peers={npeers}")
    peers = [W.random_sparse_payload(n, chunk, k, 2, key=("p", npeers, p)) for p in range(npeers)]
    check(gpu_lib, peers, n, chunk, k, 2, "f32", 1.0 / npeers, f"{npeers} peers")


def test_sa_unordered_and_out_of_chunk_slots(gpu_lib):
    """Slots in any order, and indices that fall outside their chunk (past a short last
    chunk, or past the chunk size) are skipped, never written."""
    n, chunk, k, bits = 2048 * 3 + 77, 2048, 300, 4
    peers = []
    for p in range(4):
        ix, c, a = W.random_sparse_payload(n, chunk, k, bits, key=("u", p), ordered=False)
        u = ix.numpy().view(np.uint16).copy().reshape(-1, k)
        u[0, :3] = [2048, 4095, 60000]      # past a full chunk
        u[-1, :3] = [77, 100, 2047]          # past the short last chunk (77 elements)
        peers.append((torch.from_numpy(u.reshape(-1).view(np.int16).copy()), c, a))
    say("sa unordered + out-of-chunk slots")
    check(gpu_lib, peers, n, chunk, k, bits, "bf16", 0.25, "unordered")


def test_sa_edge_sizes(gpu_lib):
    """n smaller than one chunk, exactly one chunk, one element, and all-unused payloads."""
    for n in (1, 255, 256, 257, 4096):
        peers = [W.random_sparse_payload(n, 256, 16, 2, key=("e", n, p)) for p in range(3)]
        say(f"sa n={n}")
        check(gpu_lib, peers, n, 256, 16, 2, "f32", 0.5, f"n {n}")
    n, k = 1000, 8
    empty = (torch.full((4 * k,), -1, dtype=torch.int16), torch.zeros(4 * 2, dtype=torch.uint8),
             torch.ones(4, dtype=torch.float32))
    say("sa all-unused payload")
    check(gpu_lib, [empty, empty], n, 256, k, 2, "f32", 1.0, "all unused")


def test_sa_deterministic(gpu_lib):
    """Two calls give identical bytes (the sum order is fixed)."""
    n, chunk, k = 4096 * 16, 4096, 82
    peers = [tuple(x.cuda() for x in W.random_sparse_payload(n, chunk, k, 2, key=("d", p))) for p in range(8)]
    outs = []
    for _ in range(2):
        o = torch.empty(n, device="cuda")
        gpu_lib.loco_sparse_aggregate(peers, n, chunk=chunk, k=k, bits=2, out=o, out_scale=0.125)
        torch.cuda.synchronize()
        outs.append(host(o))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("od", ["f32", "bf16"])
def test_sa_many_chunks_per_workgroup(gpu_lib, od):
    """6,000 chunks and a short last one.  bf16 output: more chunks than the persistent
    grid has workgroups, so each walks several (its next payload loaded while the current
    chunk is applied).  fp32 output: the general kernel, one workgroup per chunk, after the
    pre-read of all the payloads."""
    chunk, k = 256, 82
    n = chunk * 6000 + 37
    say(f"sa many chunks per workgroup, n={n}, {od}")
    peers = [W.random_sparse_payload(n, chunk, k, 4, key=("w", p)) for p in range(8)]
    check(gpu_lib, peers, n, chunk, k, 4, od, 0.125, f"many chunks {od}")
