"""Whole-array parity at the workloads' full sizes.

The unchanged oracle runs over slabs (whole scale blocks or chunks) in spawned worker
processes; blocks and chunks are independent, so the slabs together are the oracle's
result for the whole array.  Arrays are shared through files under /dev/shm (or the
temporary directory) that every process maps: the test copies the GPU's inputs and
outputs into them, each worker maps only its slab, runs the oracle, compares element by
element and reports what differs.  Free-running chains keep the oracle's own state
(error buffer, optimizer state) in such files too.

This module imports NumPy and the oracle only (no torch, no GPU runtime), so the workers
start quickly and never touch the device.
"""
from __future__ import annotations

import os
import shutil
import tempfile
import uuid

import numpy as np

import oracle

# storage dtype in the files: bf16 is kept as its 16-bit patterns
FILE_DTYPE = {"f32": np.float32, "bf16": np.int16, "i8": np.int8, "u8": np.uint8, "u16": np.int16}


class SharedArrays:
    """Flat arrays in files of one private directory, removed by close()."""

    def __init__(self):
        base = "/dev/shm" if os.path.isdir("/dev/shm") else tempfile.gettempdir()
        self.dir = os.path.join(base, f"loco-parity-{os.getpid()}-{uuid.uuid4().hex[:8]}")
        os.makedirs(self.dir)
        self.specs = {}

    def new(self, name, n, kind):
        """A zero-filled array of n elements of `kind` ('f32', 'bf16', 'i8', 'u8', 'u16')."""
        path = os.path.join(self.dir, name)
        dt = FILE_DTYPE[kind]
        with open(path, "wb") as f:
            f.truncate(max(1, n) * np.dtype(dt).itemsize)
        self.specs[name] = (path, kind, n)
        return np.memmap(path, dtype=dt, mode="r+", shape=(n,)) if n else np.zeros(0, dt)

    def spec(self, name):
        return self.specs[name]

    def close(self):
        shutil.rmtree(self.dir, ignore_errors=True)


def _slab(spec, lo, hi, write=False):
    """Elements [lo, hi) of a shared array, in the oracle's storage form (bf16 and u16 as
    uint16 patterns)."""
    path, kind, n = spec
    assert 0 <= lo <= hi <= n, (spec, lo, hi)
    dt = np.dtype(FILE_DTYPE[kind])
    if hi == lo:
        a = np.zeros(0, dt)
    else:
        a = np.memmap(path, dtype=dt, mode="r+" if write else "r", offset=lo * dt.itemsize, shape=(hi - lo,))
    if kind in ("bf16", "u16"):
        a = a.view(np.uint16)
    return a


def _f32_report(got, want, floor, what):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    tol = 1e-6 * np.abs(want.astype(np.float64)) + 1e-6 * np.asarray(floor, np.float64)
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bad = ~(err <= tol)
    if np.any(bad):
        i = int(np.flatnonzero(bad)[0])
        return f"{what}: {int(bad.sum())} out of tolerance; first at {i}: got {got[i]!r} want {want[i]!r}", False
    return None, bool(np.array_equal(got.view(np.uint32), want.view(np.uint32)))


def _bf16_report(got, want, what):
    def ordered(u):
        s = np.asarray(u, np.uint16).view(np.int16).astype(np.int32)
        return np.where(s >= 0, s, -32768 - s)
    d = np.abs(ordered(got) - ordered(want))
    if np.any(d > 1):
        i = int(np.flatnonzero(d > 1)[0])
        return f"{what}: {int((d > 1).sum())} more than 1 ulp apart; first at {i}", False
    return None, bool(np.array_equal(np.asarray(got, np.uint16), np.asarray(want, np.uint16)))


def _bytes_report(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    if got.shape != want.shape:
        return f"{what}: shape {got.shape} vs {want.shape}"
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        return f"{what}: {bad.size} of {got.size} differ; first at {bad[0]}: got {got[bad[0]]!r} want {want[bad[0]]!r}"
    return None


def cq_task(t):
    """One slab [lo, hi) of one segment of a compensate-quantize step: the oracle from its own
    error state, compared with the GPU's codes, absmax and error; the oracle's new error is
    written back to its state.  Element offsets `off` (g, e), byte offset `coff` (codes) and
    block offset `boff` (absmax) place the segment in the shared arrays."""
    lo, hi, bits, block = t["lo"], t["hi"], t["bits"], t["block"]
    off, coff, boff = t["off"], t["coff"], t["boff"]
    g = _slab(t["g"], off + lo, off + hi)
    e_state = _slab(t["e_ora"], off + lo, off + hi, write=True)
    ref = oracle.compensate_quantize(np.array(g), np.array(e_state), bits=bits, block=block, beta=t["beta"],
                                     grad_dtype=t["gd"], err_dtype=t["ed"], err_scale=t["err_scale"],
                                     reset=t["reset"])
    what = f"{t['tag']} segment {t['seg']} elements {lo}:{hi}"
    msgs = []
    c0, c1 = lo * bits // 8, (hi * bits + 7) // 8
    m = _bytes_report(_slab(t["codes"], coff + c0, coff + c1), ref["codes"], f"{what} codes")
    if m:
        msgs.append(m)
    b0, b1 = lo // block, -(-hi // block)
    am = _slab(t["absmax"], boff + b0, boff + b1)
    m = _bytes_report(np.asarray(am).view(np.uint32), ref["absmax"].view(np.uint32), f"{what} absmax")
    if m:
        msgs.append(m)
    got_e = _slab(t["e_gpu"], off + lo, off + hi)
    bitwise = True
    if t["ed"] == "i8":
        m = _bytes_report(got_e, ref["e_new"], f"{what} 8-bit error")
    elif t["ed"] == "f32":
        qmax = (1 << (bits - 1)) - 1
        floor = np.repeat(ref["absmax"].astype(np.float64) / qmax, block)[: hi - lo]
        m, bitwise = _f32_report(got_e, ref["e_new"], floor, f"{what} error")
    else:
        m, bitwise = _bf16_report(got_e, ref["e_new"], f"{what} error")
    if m:
        msgs.append(m)
    e_state[:] = ref["e_new"]
    e_state.flush()
    return {"n": hi - lo, "bad": msgs, "bitwise": bitwise}


def dr_task(t):
    """Slab [lo, hi) of a dequant-reduce: every peer's codes and absmax of the slab, the
    oracle's average, compared with the GPU's output."""
    lo, hi, bits, block = t["lo"], t["hi"], t["bits"], t["block"]
    c0, c1 = lo * bits // 8, (hi * bits + 7) // 8
    b0, b1 = lo // block, -(-hi // block)
    pays = [(np.array(_slab(t["codes"], co + c0, co + c1)), np.array(_slab(t["absmax"], bo + b0, bo + b1)))
            for co, bo in zip(t["coffs"], t["boffs"])]
    what = f"{t['tag']} elements {lo}:{hi}"
    if t.get("adam"):
        th = _slab(t["theta_ora"], lo, hi, write=True)
        mo = _slab(t["m_ora"], lo, hi, write=True)
        ve = _slab(t["v_ora"], lo, hi, write=True)
        ref = oracle.dequant_reduce_adam(pays, hi - lo, bits=bits, block=block, out_scale=t["out_scale"],
                                         theta=np.array(th), m=np.array(mo), v=np.array(ve), **t["adam"])
        msgs, bitwise = [], True
        z = np.zeros(hi - lo)
        for key in ("theta", "m", "v"):
            m, bw = _f32_report(_slab(t[f"{key}_gpu"], lo, hi), ref[key], z, f"{what} {key}")
            bitwise &= bw
            if m:
                msgs.append(m)
        m, bw = _bf16_report(_slab(t["tb_gpu"], lo, hi), ref["theta_bf16"], f"{what} theta bf16")
        bitwise &= bw
        if m:
            msgs.append(m)
        th[:], mo[:], ve[:] = ref["theta"], ref["m"], ref["v"]
        for a in (th, mo, ve):
            a.flush()
        return {"n": hi - lo, "bad": msgs, "bitwise": bitwise}
    want = oracle.dequant_reduce(pays, hi - lo, bits=bits, block=block, out_scale=t["out_scale"],
                                 out_dtype=t["out_dtype"])
    got = _slab(t["out"], lo, hi)
    if t["out_dtype"] == "bf16":
        m, bw = _bf16_report(got, want, what)
    else:
        m, bw = _f32_report(got, want, np.zeros(hi - lo), what)
    return {"n": hi - lo, "bad": [m] if m else [], "bitwise": bw}


def tk_task(t):
    """Chunks [c0, c1) of a Top-k step from the oracle's own error state: indices, codes,
    absmax bit-exact, error within the fp32 bar; the oracle's new error is written back."""
    c0, c1, C, k, bits = t["c0"], t["c1"], t["chunk"], t["k"], t["bits"]
    lo, hi = c0 * C, min(c1 * C, t["n"])
    nb = -(-k * bits // 8)
    e_state = _slab(t["e_ora"], lo, hi, write=True)
    ref = oracle.topk_quantize(np.array(_slab(t["g"], lo, hi)), np.array(e_state), chunk=C, k=k, bits=bits,
                               decay=t["decay"])
    what = f"{t['tag']} chunks {c0}:{c1}"
    msgs = []
    for m in (_bytes_report(_slab(t["idx"], c0 * k, c1 * k), ref["idx"], f"{what} idx"),
              _bytes_report(_slab(t["codes"], c0 * nb, c1 * nb), ref["codes"], f"{what} codes"),
              _bytes_report(np.asarray(_slab(t["absmax"], c0, c1)).view(np.uint32), ref["absmax"].view(np.uint32),
                            f"{what} absmax")):
        if m:
            msgs.append(m)
    floor = np.repeat(ref["absmax"].astype(np.float64), C)[: hi - lo]
    m, bitwise = _f32_report(_slab(t["e_gpu"], lo, hi), ref["e_new"], floor, f"{what} error")
    if m:
        msgs.append(m)
    e_state[:] = ref["e_new"]
    e_state.flush()
    return {"n": hi - lo, "bad": msgs, "bitwise": bitwise}


def sa_task(t):
    """Chunks [c0, c1) of a sparse aggregation: every peer's slots of those chunks, the
    oracle's result, compared with the GPU's output."""
    c0, c1, C, k, bits = t["c0"], t["c1"], t["chunk"], t["k"], t["bits"]
    lo, hi = c0 * C, min(c1 * C, t["n"])
    nb = -(-k * bits // 8)
    pays = [(np.array(_slab(t["idx"], io + c0 * k, io + c1 * k)), np.array(_slab(t["codes"], co + c0 * nb,
                                                                                 co + c1 * nb)),
             np.array(_slab(t["absmax"], ao + c0, ao + c1)))
            for io, co, ao in zip(t["ioffs"], t["coffs"], t["aoffs"])]
    want = oracle.sparse_aggregate(pays, hi - lo, chunk=C, k=k, bits=bits, out_scale=t["out_scale"])
    m, bw = _f32_report(_slab(t["out"], lo, hi), want, np.zeros(hi - lo), f"{t['tag']} chunks {c0}:{c1}")
    return {"n": hi - lo, "bad": [m] if m else [], "bitwise": bw}


def cq_layout(sizes, bits, block):
    """Offsets of each segment in the concatenated shared arrays: elements (g, e), code
    bytes, scale blocks; each list has one more entry than there are segments."""
    offs, coffs, boffs = [0], [0], [0]
    for n in sizes:
        offs.append(offs[-1] + n)
        coffs.append(coffs[-1] + (n * bits + 7) // 8)
        boffs.append(boffs[-1] + -(-n // block))
    return offs, coffs, boffs


def cq_tasks(S, sizes, slab, **kw):
    """One task per slab of `slab` elements (a multiple of the block) of every segment."""
    offs, coffs, boffs = cq_layout(sizes, kw["bits"], kw["block"])
    base = dict(g=S.spec("g"), e_ora=S.spec("e_ora"), e_gpu=S.spec("e_gpu"), codes=S.spec("codes"),
                absmax=S.spec("absmax"), **kw)
    return [dict(base, seg=s, off=offs[s], coff=coffs[s], boff=boffs[s], lo=lo, hi=min(lo + slab, n))
            for s, n in enumerate(sizes) for lo in range(0, n, slab)]


def run(pool, fn, tasks):
    """Run the tasks on the pool; returns (elements checked, first mismatches, all bitwise)."""
    n, bad, bitwise = 0, [], True
    for r in pool.map(fn, tasks, chunksize=1):
        n += r["n"]
        bad.extend(r["bad"])
        bitwise &= r["bitwise"]
    return n, bad[:8], bitwise
