"""Refused calls with real device buffers: every entry point validates on the host before
any launch, so a refused call raises (LocoError with the C status) and leaves every
output buffer as it was.  The host-only ABI tests check the same statuses with fake
pointers on machines without a GPU; these run the binding end to end on the GPU."""
import pytest
import torch

import workloads as W
from bit_gradient_compression_amd import loco

pytestmark = pytest.mark.gpu

INV, ALIGN, UNSUP = loco.LOCO_ERR_INVALID, loco.LOCO_ERR_ALIGN, loco.LOCO_ERR_UNSUPPORTED


def refused(status, fn, *a, **kw):
    with pytest.raises(loco.LocoError) as ei:
        fn(*a, **kw)
    assert ei.value.status == status, str(ei.value)


def snapshot(*ts):
    torch.cuda.synchronize()
    return [t.clone() for t in ts]


def unchanged(before, *ts):
    torch.cuda.synchronize()
    for b, t in zip(before, ts):
        assert torch.equal(b.view(torch.uint8), t.view(torch.uint8))


def cq_buffers(n, bits=4, block=256, edt=torch.float32):
    e = torch.full((n,), 7, dtype=edt, device="cuda")
    c = torch.full((loco.code_bytes(n, bits),), 0xA5, dtype=torch.uint8, device="cuda")
    a = torch.full((loco.num_blocks(n, block),), -1.0, device="cuda")
    return e, c, a


def test_cq_refusals_leave_outputs_untouched(gpu_lib):
    n = 10_000
    g = W.shard7b_grad(0, n=n + 8, device="cuda", chain="errors")
    e, c, a = cq_buffers(n)
    before = snapshot(e, c, a)
    # a gradient view 2 bytes into its buffer is not 16-byte aligned
    refused(ALIGN, gpu_lib.loco_compensate_quantize, [(g[1:n + 1], e, c, a)], bits=4, block=256, beta=0.9)
    # codes inside the error buffer
    eb = e.view(torch.uint8)
    refused(INV, gpu_lib.loco_compensate_quantize, [(g[:n], e, eb[4096:4096 + c.numel()], a)], bits=4, block=256,
            beta=0.9)
    # two segments writing the same error buffer
    e2, c2, a2 = cq_buffers(n)
    refused(INV, gpu_lib.loco_compensate_quantize, [(g[:n], e, c, a), (g[:n], e, c2, a2)], bits=4, block=256,
            beta=0.9)
    # parameters
    refused(UNSUP, gpu_lib.loco_compensate_quantize, [(g[:n], e, c, a)], bits=3, block=256, beta=0.9)
    refused(UNSUP, gpu_lib.loco_compensate_quantize, [(g[:n], e, c, a)], bits=4, block=100, beta=0.9)
    refused(INV, gpu_lib.loco_compensate_quantize, [(g[:n], e, c, a)], bits=4, block=256, beta=1.5)
    # an 8-bit error needs a finite positive scale
    e8 = torch.zeros(n, dtype=torch.int8, device="cuda")
    refused(INV, gpu_lib.loco_compensate_quantize_ex, [(g[:n], e8, c, a)], bits=4, block=256, beta=0.9,
            err_scale=0.0)
    unchanged(before, e, c, a)


def test_dr_and_dra_refusals(gpu_lib):
    n, bits, block = 20_000, 4, 256
    pays = [tuple(x.cuda() for x in W.random_payload(n, bits, block, key=("errors", p))) for p in range(3)]
    out = torch.full((n,), 3.0, device="cuda")
    before = snapshot(out, *[x for p in pays for x in p])
    # the output overlapping a peer's codes
    big = torch.zeros(n * 4 + 64, dtype=torch.uint8, device="cuda")
    alias = [(big[:loco.code_bytes(n, bits)], pays[0][1]), pays[1]]
    refused(INV, gpu_lib.loco_dequant_reduce, alias, n, bits=bits, block=block, out=big[:n * 4].view(torch.float32),
            out_scale=1.0)
    # too many peers, and unsupported widths
    refused(UNSUP, gpu_lib.loco_dequant_reduce, [pays[0]] * 129, n, bits=bits, block=block, out=out, out_scale=1.0)
    refused(UNSUP, gpu_lib.loco_dequant_reduce, pays, n, bits=5, block=block, out=out, out_scale=1.0)
    # the fused Adam step: moments sharing storage, and an invalid delta
    th = torch.zeros(n, device="cuda")
    mv = torch.zeros(2 * n, device="cuda")
    refused(INV, gpu_lib.loco_dequant_reduce_adam, pays, n, bits=bits, block=block, out_scale=1.0, param=th,
            m=mv[:n], v=mv[n // 2:n // 2 + n], lr=1e-3, beta1=0.1, beta2=0.01, delta=1e-8)
    refused(INV, gpu_lib.loco_dequant_reduce_adam, pays, n, bits=bits, block=block, out_scale=1.0, param=th,
            m=mv[:n], v=mv[n:], lr=1e-3, beta1=0.1, beta2=0.01, delta=0.0)
    unchanged(before, out, *[x for p in pays for x in p])
    assert torch.count_nonzero(th) == 0 and torch.count_nonzero(mv) == 0


def test_topk_and_sparse_aggregate_refusals(gpu_lib):
    n, chunk, k = 3 * 4096, 4096, 82
    g = W.sparseloco_grad(0, n=n, device="cuda")
    e = torch.full((n,), 0.5, device="cuda")
    idx = torch.full((3 * k,), 7, dtype=torch.int16, device="cuda")
    codes = torch.full((3 * loco.code_bytes(k, 2),), 9, dtype=torch.uint8, device="cuda")
    am = torch.full((3,), -2.0, device="cuda")
    before = snapshot(e, idx, codes, am)
    refused(INV, gpu_lib.loco_topk_quantize, g, e, chunk=chunk, k=chunk + 1, idx=idx, codes=codes, absmax=am)
    refused(UNSUP, gpu_lib.loco_topk_quantize, g, e, chunk=3000, k=k, idx=idx, codes=codes, absmax=am)
    refused(INV, gpu_lib.loco_topk_quantize, g, e, chunk=chunk, k=k, idx=idx, codes=codes, absmax=am, ef_decay=2.0)
    # the error buffer aliasing the gradient
    refused(INV, gpu_lib.loco_topk_quantize, g, g, chunk=chunk, k=k, idx=idx, codes=codes, absmax=am)
    unchanged(before, e, idx, codes, am)
    pays = [tuple(x.cuda() for x in W.random_sparse_payload(n, chunk, k, 2, key=("errors", p))) for p in range(2)]
    out = torch.full((n,), 1.0, device="cuda")
    before = snapshot(out)
    refused(UNSUP, gpu_lib.loco_sparse_aggregate, [pays[0]] * 129, n, chunk=chunk, k=k, out=out, out_scale=1.0)
    refused(INV, gpu_lib.loco_sparse_aggregate, pays, n, chunk=chunk, k=0, out=out, out_scale=1.0)
    refused(INV, gpu_lib.loco_sparse_aggregate, pays, n, chunk=chunk, k=k, out=out, out_scale=float("inf"))
    unchanged(before, out)


def test_binding_refuses_host_tensors(gpu_lib):
    n = 1000
    g = torch.zeros(n)  # host memory
    e, c, a = cq_buffers(n)
    with pytest.raises(ValueError, match="device memory"):
        gpu_lib.loco_compensate_quantize([(g, e, c, a)], bits=4, block=256, beta=0.9)


def test_binding_refuses_short_tensors(gpu_lib):
    """The C ABI sees only pointers and n; the binding checks that every tensor holds the
    bytes the call would touch, and refuses (ValueError) before any call."""
    n = 10_000
    g = W.shard7b_grad(0, n=n, device="cuda", chain="short")
    e, c, a = cq_buffers(n)
    before = snapshot(e, c, a)
    with pytest.raises(ValueError, match="codes"):
        gpu_lib.loco_compensate_quantize([(g, e, c[:-1], a)], bits=4, block=256, beta=0.9)
    with pytest.raises(ValueError, match="absmax"):
        gpu_lib.loco_compensate_quantize([(g, e, c, a[:-1])], bits=4, block=256, beta=0.9)
    with pytest.raises(ValueError, match="elements"):
        gpu_lib.loco_compensate_quantize([(g, e[:-1], c, a)], bits=4, block=256, beta=0.9)
    unchanged(before, e, c, a)
    pays = [tuple(x.cuda() for x in W.random_payload(n, 4, 256, key=("short", p))) for p in range(2)]
    out = torch.zeros(n - 1, device="cuda")
    with pytest.raises(ValueError, match="out"):
        gpu_lib.loco_dequant_reduce(pays, n, bits=4, block=256, out=out, out_scale=0.5)
    with pytest.raises(ValueError, match="peer 1: codes"):
        gpu_lib.loco_dequant_reduce([pays[0], (pays[1][0][:-1], pays[1][1])], n, bits=4, block=256,
                                    out=torch.zeros(n, device="cuda"), out_scale=0.5)
    with pytest.raises(ValueError, match="v holds"):
        gpu_lib.loco_dequant_reduce_adam(pays, n, bits=4, block=256, out_scale=0.5, param=torch.zeros(n, device="cuda"),
                                         m=torch.zeros(n, device="cuda"), v=torch.zeros(n - 4, device="cuda"),
                                         lr=1e-3, beta1=0.1, beta2=0.01, delta=1e-8)
    nt, chunk, k = 2 * 4096 + 5, 4096, 82
    gt = torch.zeros(nt, device="cuda")
    with pytest.raises(ValueError, match="idx"):
        gpu_lib.loco_topk_quantize(gt, torch.zeros(nt, device="cuda"), chunk=chunk, k=k,
                                   idx=torch.zeros(3 * k - 1, dtype=torch.int16, device="cuda"),
                                   codes=torch.zeros(3 * 21, dtype=torch.uint8, device="cuda"),
                                   absmax=torch.zeros(3, device="cuda"))
    sp = [tuple(x.cuda() for x in W.random_sparse_payload(nt, chunk, k, 2, key=("short", 0)))]
    with pytest.raises(ValueError, match="out"):
        gpu_lib.loco_sparse_aggregate(sp, nt, chunk=chunk, k=k, out=torch.zeros(nt - 1, device="cuda"), out_scale=1.0)


def test_binding_missing_buffers(gpu_lib):
    """A missing output or payload buffer (None) reaches the C call as a null pointer, which
    refuses it (LOCO_ERR_INVALID) before any launch."""
    n = 4096
    pays = [tuple(x.cuda() for x in W.random_payload(n, 4, 256, key=("none", p))) for p in range(2)]
    refused(INV, gpu_lib.loco_dequant_reduce, pays, n, bits=4, block=256, out=None, out_scale=0.5)
    refused(INV, gpu_lib.loco_dequant_reduce, [pays[0], (pays[1][0], None)], n, bits=4, block=256,
            out=torch.zeros(n, device="cuda"), out_scale=0.5)
    sp = [tuple(x.cuda() for x in W.random_sparse_payload(n, 4096, 82, 2, key=("none", 0)))]
    refused(INV, gpu_lib.loco_sparse_aggregate, sp, n, chunk=4096, k=82, out=None, out_scale=1.0)
