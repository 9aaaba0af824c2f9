"""Seeded generators: determinism and the shape of each workload's values (CPU)."""
import numpy as np
import torch

import workloads as W


def test_deterministic_and_distinct():
    a = W.tiny_grad(3, n=100_000)
    b = W.tiny_grad(3, n=100_000)
    c = W.tiny_grad(4, n=100_000)
    assert torch.equal(a, b)
    assert not torch.equal(a, c)
    assert abs(a.std().item() - 1e-3) < 2e-5
    p = W.tiny_peer_grads(4, n=1000)
    assert len({x.sum().item() for x in p}) == 4


def test_llama_layer_shapes_and_scales():
    gs = W.llama_layer_grads(0, div=256)
    shapes = W.llama_layer_shapes(256)
    assert [x.numel() for x in gs] == [r * c for _, r, c in shapes]
    assert all(x.dtype == torch.bfloat16 for x in gs)
    for x in gs:
        med = x.float().abs().median().item()  # median |t3| ~ 0.77 times the scale
        assert 1e-5 * 0.5 < med < 1e-2 * 1.0
    full = W.llama_layer_shapes()
    assert sum(r * c for _, r, c in full) == 202_375_168


def test_moe_zero_rows_fixed():
    a = W.moe_grads(0, div=512, experts=2)
    b = W.moe_grads(1, div=512, experts=2)
    for (name, x, r, c), ga, gb in zip(W.moe_shapes(512, 2), a, b):
        za = (ga.view(r, c) == 0).all(dim=1)
        zb = (gb.view(r, c) == 0).all(dim=1)
        assert int(za.sum()) == int(round(0.3 * r))
        assert torch.equal(za, zb)
    assert sum(r * c for _, _, r, c in W.moe_shapes()) == 1_409_286_144


def test_sparseloco_outliers():
    g = W.sparseloco_grad(0, n=1 << 21)
    big = g.abs() > 0.05
    frac = big.float().mean().item()
    assert 0.0007 < frac < 0.0013
    assert torch.all(g[big].abs() == torch.tensor(0.1, dtype=torch.float32))
    assert abs(g[~big].std().item() - 1e-3) < 2e-5


def test_shard7b_small():
    g = W.shard7b_grad(0, n=10_000)
    assert g.dtype == torch.bfloat16 and g.numel() == 10_000
    assert W.SHARD7B_PEERS * W.SHARD7B_PART == W.SHARD7B_N
