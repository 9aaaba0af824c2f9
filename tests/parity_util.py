"""Helpers of the GPU parity tests: guarded device buffers and comparisons."""
import numpy as np
import torch

GUARD = 4096  # bytes of canary on each side of every output buffer
CANARY = 0xA5


class Guarded:
    """A device buffer with canary bytes before and after the part the library sees."""

    def __init__(self, n, dtype, device="cuda", init=None):
        es = torch.empty(0, dtype=dtype).element_size()
        pad = GUARD // es
        self.n, self.pad = n, pad
        self.full = torch.empty(n + 2 * pad, dtype=dtype, device=device)
        raw = self.full.view(torch.uint8)
        raw[:GUARD].fill_(CANARY)
        raw[GUARD + n * es:].fill_(CANARY)
        self.t = self.full[pad:pad + n]
        if init is not None:
            self.t.copy_(init)

    def check(self, what="buffer"):
        raw = self.full.view(torch.uint8).cpu().numpy()
        es = self.full.element_size()
        lo, hi = raw[:GUARD], raw[GUARD + self.n * es:]
        assert np.all(lo == CANARY) and np.all(hi == CANARY), f"{what}: write outside its bounds"


def host(t):
    return t.detach().cpu().numpy()


def bf16_bits(t):
    return host(t.view(torch.int16)).view(np.uint16)


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {got.size} differ; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")


def assert_f32_close(got, want, floor, what):
    """fp32 bar: |got - want| <= 1e-6 |want| + 1e-6 * floor (floor = the block's step).
    Returns True when the two are also bitwise equal."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    tol = 1e-6 * np.abs(want.astype(np.float64)) + 1e-6 * np.asarray(floor, np.float64)
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    if not np.all(err <= tol):
        i = int(np.argmax(err - tol))
        raise AssertionError(f"{what}: {int(np.sum(err > tol))} out of tolerance; worst at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")
    return bool(np.array_equal(got.view(np.uint32), want.view(np.uint32)))


def _ordered(u16):
    s = np.asarray(u16, np.uint16).view(np.int16).astype(np.int32)
    return np.where(s >= 0, s, -32768 - s)


def assert_bf16_close(got, want, what):
    """bf16 bar: at most 1 ulp apart.  Returns True when bitwise equal."""
    d = np.abs(_ordered(got) - _ordered(want))
    if not np.all(d <= 1):
        i = int(np.argmax(d))
        raise AssertionError(f"{what}: {int(np.sum(d > 1))} more than 1 ulp apart; worst at {i}")
    return bool(np.array_equal(np.asarray(got, np.uint16), np.asarray(want, np.uint16)))


def step_per_elem(absmax, bits, block, n):
    qmax = (1 << (bits - 1)) - 1
    return np.repeat(np.asarray(absmax, np.float64) / qmax, block)[:n]


def say(*a):
    print(*a, flush=True)
