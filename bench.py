"""Benchmark of LoCo's per-GPU gradient path on one MI355X.

A step is one pass of the rank's path on the 7B FSDP-shard workload:
  compensate-quantize of the rank's 842,000,000-element bf16 gradient (fp32 error,
  4-bit codes, block 256, beta 0.9), split into 8 partitions of 105,250,000 (one per
  destination, blocks restarting per partition), then
  dequant-reduce of the 8 peer payloads of the rank's own partition into bf16 (x 1/8).
Inputs are resident in HBM before the timed region; the error buffer carries over from
step to step.  Compensate-quantize on the LLaMA-7B layer and MoE-expert workloads, the
SparseLoCo-style Top-k mode (2^28 fp32, chunk 4096, k = 82, 2-bit),
its sparse aggregation of 8 peers' payloads, the 8-bit-code variant, the 8-bit-error
variant (LoCo Eqn. (7)) and dequant-reduce fused with the LoCo-Adam step (Eqn. (9)) are
timed in the same run and reported under "modes".  So is the tiny case (1,048,576 fp32,
compensate-quantize then dequant-reduce of 4 peers), which fits in the Infinity Cache and
is bound by launch latency: its time per step is reported eagerly and as replays of a HIP
graph, with no roofline claim.

Every kernel (the step's two and each mode) is timed back to back and again with a 1 GiB
read before each launch (which keeps its inputs out of the Infinity Cache and keeps other
launches' dirty lines out of its time), with median, p10 and p90; its GB/s use the slower
of the two averages.  Beside each kernel its traffic twin (libloco_twins.so: the same
loads and stores in the same launch shape, no compression arithmetic) is timed the same
way: frac_twin = twin time / kernel time is how close the kernel runs to the ceiling of
its own stream mix.

Prints one JSON line.  value = gradient GB/s = 842,000,000 x 2 bytes / step time.
roofline: the compensate-quantize kernel's algorithmic bytes / its launch time against
8 TB/s, the launch time being the slowest of its average inside the timed steps (HIP
events on its stream) and its back-to-back and cache-flushed averages.  copy_ceiling: a
hand-written streaming copy (one 16-byte vector per thread, 1 GiB in, 1 GiB out) for
context; every kernel also reports its GB/s over it (frac_copy).  cpu_baseline: the CPU
oracle on a bounded sample of the same workload on this host, in one process, and
(parallel) fanned out over the host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PARTS = 8
BITS, BLOCK, BETA = 4, 256, 0.9
TK_CHUNK, TK_K = 4096, 82
TINY_N, TINY_BLOCK, TINY_PEERS = 1 << 20, 128, 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_7b_shard.json")
CSRC = os.path.join(ROOT, "bit_gradient_compression_amd", "csrc")
KERNEL_FILES = {"compensate_quantize_4bit": ["cq.hip"], "dequant_reduce_8peers": ["dr.hip"],
                "compensate_quantize_8bit_7b_shard": ["cq.hip"], "compensate_quantize_4bit_i8err_7b_shard": ["cq.hip"],
                "compensate_quantize_4bit_llama_layer": ["cq.hip"], "compensate_quantize_4bit_moe": ["cq.hip"],
                "dequant_reduce_adam_8peers": ["dr.hip"],
                "sparseloco_topk_2bit": ["tk.hip"], "sparseloco_aggregate_8peers": ["sa.hip"],
                "sparseloco_aggregate_8peers_bf16": ["sa.hip"]}
COMMON_FILES = ["loco_device.hpp", "loco_internal.hpp"]


def kernel_source_hash(kernel: str) -> str:
    """Hash of the sources a kernel is built from; counter summaries carry it so that a
    summary taken before the kernel changed is not used."""
    h = hashlib.sha256()
    for f in KERNEL_FILES[kernel] + COMMON_FILES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cq_bytes(sizes, gs, es, bits, block):
    return sum(n * (gs + 2 * es) + (n * bits + 7) // 8 + 4 * (-(-n // block)) for n in sizes)


def dr_bytes(n, peers, bits, block, out_bytes):
    return peers * ((n * bits + 7) // 8 + 4 * (-(-n // block))) + n * out_bytes


def tk_bytes(n, chunk, k, bits):
    chunks = -(-n // chunk)
    return n * 12 + chunks * (2 * k + (k * bits + 7) // 8 + 4)


def sa_bytes(n, peers, chunk, k, bits, out_bytes):
    chunks = -(-n // chunk)
    return peers * chunks * (2 * k + (k * bits + 7) // 8 + 4) + n * out_bytes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def load_traffic():
    """Measured HBM bytes per launch, per kernel, from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain-copy calibration).  A kernel whose
    sources changed since the counters were taken gets no entry."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    return {k: v for k, v in t.get("kernels", {}).items()
            if k in KERNEL_FILES and v.get("source_hash") == kernel_source_hash(k)}


def cpu_baseline(g_dev, payloads_dev, slab, min_seconds=10.0):
    """The oracle, as it stands, on consecutive slabs of the rank's shard: per slab, two
    compensate-quantize steps (error carried) on `slab` elements as one segment, and the
    dequant-reduce of the matching slab/8 elements of every peer payload.  Slabs are
    added until at least `min_seconds` of oracle time (or the whole shard) is done."""
    import numpy as np
    import torch

    import oracle
    part = slab // PARTS
    n = g_dev.numel()
    done = 0
    spent = 0.0
    steps = 2
    while done + slab <= n and spent < min_seconds:
        g = g_dev[done:done + slab].cpu().view(torch.int16).numpy().view(np.uint16)
        off = done // PARTS
        pays = [(c[(off * BITS) // 8:((off + part) * BITS + 7) // 8].cpu().numpy(),
                 a[off // BLOCK:-(-(off + part) // BLOCK)].cpu().numpy()) for c, a in payloads_dev]
        e = np.zeros(slab, np.float32)
        t0 = time.perf_counter()
        for _ in range(steps):
            r = oracle.compensate_quantize(g, e, bits=BITS, block=BLOCK, beta=BETA, grad_dtype="bf16")
            e = r["e_new"]
            oracle.dequant_reduce(pays, part, bits=BITS, block=BLOCK, out_scale=1.0 / PARTS, out_dtype="bf16")
        spent += time.perf_counter() - t0
        done += slab
    per_step = spent / steps
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": round(done * 2 / per_step / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done:,} of the shard's {n:,} elements in slabs of {slab:,} (one segment each) + the "
                      f"matching 1/8 of each of the 8 peer payloads, 2 steps per slab, {spent:.1f} s of oracle "
                      f"time; NumPy element-wise, one thread ({avail} cores available to the process, {model})"}



def _oracle_worker(slabs, barrier):
    """One worker of the parallel oracle timing: the oracle, unchanged, over its slabs
    (the same two steps per slab as cpu_baseline), started when every worker is ready.
    Returns its wall-clock span and the gradient elements it covered."""
    import numpy as np

    import oracle
    part = slabs[0][0].size // PARTS
    # untimed warm-up on the first 2^16 elements (first calls into NumPy are slow)
    g0, pays0 = slabs[0]
    w = 1 << 16
    oracle.compensate_quantize(g0[:w], np.zeros(w, np.float32), bits=BITS, block=BLOCK, beta=BETA, grad_dtype="bf16")
    oracle.dequant_reduce([(c[:(w // PARTS * BITS) // 8], a[:w // PARTS // BLOCK]) for c, a in pays0], w // PARTS,
                          bits=BITS, block=BLOCK, out_scale=1.0 / PARTS, out_dtype="bf16")
    barrier.wait()
    t0 = time.time()
    for g, pays in slabs:
        e = np.zeros(g.size, np.float32)
        for _ in range(2):
            r = oracle.compensate_quantize(g, e, bits=BITS, block=BLOCK, beta=BETA, grad_dtype="bf16")
            e = r["e_new"]
            oracle.dequant_reduce(pays, part, bits=BITS, block=BLOCK, out_scale=1.0 / PARTS, out_dtype="bf16")
    return t0, time.time(), sum(g.size for g, _ in slabs)


def cpu_baseline_parallel(g_dev, payloads_dev, slab, per_worker=4):
    """The same oracle fanned out over slabs across the host's cores (blocks and slabs are
    independent, so the results are the ones the single process computes): one spawned
    process per core (at most 16), each taking `per_worker` consecutive slabs.  Throughput
    = gradient bytes of all slabs / (2 steps) / the span from the first worker's start
    to the last one's end."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np
    import torch
    workers = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count())
    n = g_dev.numel()
    part = slab // PARTS
    nslab = min(workers * per_worker, n // slab)
    slabs = []
    for s in range(nslab):
        lo = s * slab
        g = g_dev[lo:lo + slab].cpu().view(torch.int16).numpy().view(np.uint16)
        off = lo // PARTS
        pays = [(c[(off * BITS) // 8:((off + part) * BITS + 7) // 8].cpu().numpy(),
                 a[off // BLOCK:-(-(off + part) // BLOCK)].cpu().numpy()) for c, a in payloads_dev]
        slabs.append((g, pays))
    jobs = [slabs[w::workers] for w in range(workers) if slabs[w::workers]]
    # spawned (not forked) workers: none inherits this process's GPU runtime; a worker that
    # dies raises here instead of being replaced.  A barrier starts them together, so the
    # span is their common compute time, not their start-up skew.
    ctx = multiprocessing.get_context("spawn")
    with ctx.Manager() as mgr, ProcessPoolExecutor(len(jobs), mp_context=ctx) as pool:
        barrier = mgr.Barrier(len(jobs), timeout=600)
        res = list(pool.map(_oracle_worker, jobs, [barrier] * len(jobs)))
    span = max(r[1] for r in res) - min(r[0] for r in res)
    elems = sum(r[2] for r in res)
    return {"value": round(elems * 2 / (span / 2) / 1e9, 4), "unit": "GB/s", "cores": len(jobs),
            "sample": f"{elems:,} elements in {nslab} slabs of {slab:,}, {per_worker} per process, 2 steps each, "
                      f"{span:.1f} s from the processes' common start to the last one's end"}


def _host_bf16(t):
    """A bf16 device tensor as its uint16 bit patterns on the host."""
    import numpy as np
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)



def oracle_module():
    import oracle
    return oracle


def _cq_job(gh, err, bits, block):
    """One compensate-quantize step of the oracle on host gradient bits `gh` (bf16), from a
    zero error of kind `err`."""
    import numpy as np
    zero = {"f32": np.zeros(gh.size, np.float32), "bf16": np.zeros(gh.size, np.uint16),
            "i8": np.zeros(gh.size, np.int8)}[err]
    return lambda: oracle_module().compensate_quantize(gh, zero, bits=bits, block=block, beta=BETA, grad_dtype="bf16",
                                                       err_dtype=err, err_scale=2.0 ** 17 if err == "i8" else 0.0)

def run_oracle_jobs(jobs, modes):
    """Time each mode's oracle call (one call on a bounded sample of that mode's own
    inputs, taken while they were on the device) and attach the GB/s of the sample's
    algorithmic bytes to the mode: the oracle timed beside every kernel."""
    for name, call, alg, sample in jobs:
        t0 = time.perf_counter()
        call()
        dt = time.perf_counter() - t0
        modes[name]["cpu_oracle"] = {"GBps": round(alg / dt / 1e9, 4), "seconds": round(dt, 3), "cores": 1,
                                     "sample": sample}

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-sample", type=int, default=1 << 23,
                    help="slab size of the CPU-oracle baseline (0: skip it)")
    ap.add_argument("--no-modes", action="store_true", help="skip the 8-bit and Top-k modes")
    ap.add_argument("--copy-probe", action="store_true",
                    help="kept for the counter commands: the 1 GiB device copy that calibrates the HBM byte "
                         "counters now runs on every call")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (peers are simulated "
              "in memory); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from bit_gradient_compression_amd import build as B
    if not os.path.exists(B.LIB_PATH):
        B.build()
    from bit_gradient_compression_amd import loco
    from bit_gradient_compression_amd import twins
    loco.load()
    twins.load()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    n = W.SHARD7B_N
    part = W.SHARD7B_PART
    sizes = [part] * PARTS

    log(f"bench: generating the 7B-shard workload ({n:,} bf16) on {torch.cuda.get_device_name(dev)}")
    g = W.shard7b_grad(0, n=n, device=dev)
    e = torch.zeros(n, dtype=torch.float32, device=dev)
    codes = [torch.empty((part * BITS + 7) // 8 + 16, dtype=torch.uint8, device=dev) for _ in range(PARTS)]
    absmax = [torch.empty(-(-part // BLOCK), dtype=torch.float32, device=dev) for _ in range(PARTS)]
    segs = [(g[i * part:(i + 1) * part], e[i * part:(i + 1) * part], codes[i][:(part * BITS + 7) // 8], absmax[i])
            for i in range(PARTS)]

    # the 8 peer payloads of this rank's partition: each peer quantised its own gradient
    # (one launch of the same shape as the timed one: 8 segments of 105,250,000)
    peer_g = W.shard7b_peer_grads(PARTS, n=part, device=dev)
    peer_e = torch.zeros(n, dtype=torch.float32, device=dev)
    payloads = [(torch.empty((part * BITS + 7) // 8, dtype=torch.uint8, device=dev),
                 torch.empty(-(-part // BLOCK), dtype=torch.float32, device=dev)) for _ in range(PARTS)]
    loco.loco_compensate_quantize([(peer_g[i], peer_e[i * part:(i + 1) * part], *payloads[i]) for i in range(PARTS)],
                                  bits=BITS, block=BLOCK, beta=BETA)
    torch.cuda.synchronize()
    del peer_g, peer_e
    out = torch.empty(part, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    # the streaming ceiling for context: a hand-written copy of 1 GiB into 1 GiB (one 16-byte
    # vector per thread, non-temporal); its launches also calibrate the HBM byte counters
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        twins.copy(src, dst)
    torch.cuda.synchronize()
    cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in cevs:
        a.record(stream)
        twins.copy(src, dst)
        b.record(stream)
    torch.cuda.synchronize()
    copy_ms = sorted(a.elapsed_time(b) for a, b in cevs)[len(cevs) // 2]
    copy_gbps = 2 * src.numel() * 4 / copy_ms / 1e6
    del src, dst

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        loco.loco_compensate_quantize(segs, bits=BITS, block=BLOCK, beta=BETA, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        loco.loco_dequant_reduce(payloads, part, bits=BITS, block=BLOCK, out=out, out_scale=1.0 / PARTS,
                                 stream=stream)
        if evs is not None:
            evs[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cq_ms = sorted(ev[0].elapsed_time(ev[1]) for ev in evs)
    dr_ms = sorted(ev[1].elapsed_time(ev[2]) for ev in evs)
    avg = lambda xs: sum(xs) / len(xs)  # noqa: E731
    ms_per_step = wall * 1e3 / args.steps
    cq_alg = cq_bytes(sizes, 2, 4, BITS, BLOCK)
    dr_alg = dr_bytes(part, PARTS, BITS, BLOCK, 2)
    reps = max(10, args.steps // 2)
    # the same two kernels by the modes' protocol (back to back, and cache-flushed), then
    # their traffic twins on the same buffers (the twins overwrite the error buffer and
    # the shard, which nothing reads afterwards)
    cq_call = lambda: loco.loco_compensate_quantize(segs, bits=BITS, block=BLOCK, beta=BETA, stream=stream)  # noqa: E731
    dr_call = lambda: loco.loco_dequant_reduce(payloads, part, bits=BITS, block=BLOCK, out=out,  # noqa: E731
                                               out_scale=1.0 / PARTS, stream=stream)
    cq_prot = timed(cq_call, stream, reps)
    cq_timing = spread()
    dr_prot = timed(dr_call, stream, reps)
    dr_timing = spread()
    # the roofline takes the slowest of the in-step average and the two protocol averages
    cq_time_ms = max(avg(cq_ms), cq_prot)
    cq_source = "timed steps" if cq_time_ms == avg(cq_ms) else "protocol"
    achieved = cq_alg / (cq_time_ms / 1e3) / 1e9
    dr_time_ms = max(avg(dr_ms), dr_prot)
    codes_cat = torch.empty(n * BITS // 8, dtype=torch.uint8, device=dev)
    absmax_cat = torch.empty(-(-n // BLOCK), dtype=torch.float32, device=dev)
    cq_twin = twin_of(lambda: twins.cq(g, e, codes_cat, absmax_cat, bits=BITS, block=BLOCK), stream, reps, cq_alg,
                      cq_time_ms)
    del codes_cat, absmax_cat
    dr_twin = twin_of(lambda: twins.dr(payloads, part, bits=BITS, block=BLOCK, out=out), stream, reps, dr_alg,
                      dr_time_ms)

    kernels = {
        "compensate_quantize_4bit": {"avg_ms_timed_steps": round(avg(cq_ms), 4),
                                     "p10_ms_timed_steps": round(cq_ms[len(cq_ms) // 10], 4),
                                     "p90_ms_timed_steps": round(cq_ms[(len(cq_ms) * 9) // 10], 4),
                                     **cq_timing, "ms": round(cq_time_ms, 4), "alg_bytes": cq_alg,
                                     "GBps": round(achieved, 1), "frac_hbm": round(achieved / HBM_PEAK_GBPS, 4),
                                     **cq_twin},
        "dequant_reduce_8peers": {"avg_ms_timed_steps": round(avg(dr_ms), 4), **dr_timing, "ms": round(dr_time_ms, 4),
                                  "alg_bytes": dr_alg, "GBps": round(dr_alg / dr_time_ms / 1e6, 1),
                                  "frac_hbm": round(dr_alg / dr_time_ms / 1e6 / HBM_PEAK_GBPS, 4), **dr_twin},
    }
    measured = load_traffic()
    traffic = measured.get("compensate_quantize_4bit", {}).get("hbm_bytes")
    for k, v in measured.items():
        if k in kernels:
            kernels[k]["hbm_bytes_measured"] = v["hbm_bytes"]

    modes = {}
    jobs = []  # (mode, oracle call on host copies of a sample of its inputs, sample's algorithmic bytes, what)
    SAMPLE = 1 << 24
    if not args.no_modes:
        # 8-bit codes on the same shard and error-buffer layout
        codes8 = [torch.empty(part, dtype=torch.uint8, device=dev) for _ in range(PARTS)]
        e8 = torch.zeros(n, dtype=torch.float32, device=dev)
        segs8 = [(g[i * part:(i + 1) * part], e8[i * part:(i + 1) * part], codes8[i], absmax[i])
                 for i in range(PARTS)]
        ms = timed(lambda: loco.loco_compensate_quantize(segs8, bits=8, block=BLOCK, beta=BETA, stream=stream),
                   stream, reps)
        b8 = cq_bytes(sizes, 2, 4, 8, BLOCK)
        modes["compensate_quantize_8bit_7b_shard"] = {"avg_ms": round(ms, 4), **spread(), "alg_bytes": b8,
                                                      "GBps": round(b8 / ms / 1e6, 1),
                                                      "frac_hbm": round(b8 / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                                      "grad_GBps": round(n * 2 / ms / 1e6, 1)}
        c8 = torch.empty(n, dtype=torch.uint8, device=dev)
        a8 = torch.empty(-(-n // BLOCK), dtype=torch.float32, device=dev)
        modes["compensate_quantize_8bit_7b_shard"].update(
            twin_of(lambda: twins.cq(g, e8, c8, a8, bits=8, block=BLOCK), stream, reps, b8, ms))
        del c8, a8
        jobs.append(("compensate_quantize_8bit_7b_shard", _cq_job(_host_bf16(g[:SAMPLE]), "f32", 8, BLOCK),
                     cq_bytes([SAMPLE], 2, 4, 8, BLOCK), f"the shard's first {SAMPLE:,} elements, one step"))
        del codes8, e8, segs8
        # the LLaMA-7B layer (7 bf16 gradients as 7 segments, fp32 error) and the MoE experts
        # (24 bf16 matrices with 30% zero rows, bf16 error): 4-bit, block 128
        for name, grads_of, edt in (("llama_layer", lambda: W.llama_layer_grads(0, device=dev), torch.float32),
                                    ("moe", lambda: W.moe_grads(0, device=dev), torch.bfloat16)):
            xg = grads_of()
            xs = [t.numel() for t in xg]
            sample_host = _host_bf16(xg[0].reshape(-1)[:SAMPLE])
            xsegs = [(t, torch.zeros(m, dtype=edt, device=dev), torch.empty((m * 4 + 7) // 8, dtype=torch.uint8,
                      device=dev), torch.empty(-(-m // 128), device=dev)) for t, m in zip(xg, xs)]
            ms = timed(lambda: loco.loco_compensate_quantize(xsegs, bits=4, block=128, beta=BETA, stream=stream),
                       stream, reps)
            bx = cq_bytes(xs, 2, 2 if edt == torch.bfloat16 else 4, 4, 128)
            modes[f"compensate_quantize_4bit_{name}"] = {
                "workload": f"{sum(xs):,} bf16 in {len(xs)} segments, {'bf16' if edt == torch.bfloat16 else 'fp32'} "
                            "error, 4-bit, block 128",
                "avg_ms": round(ms, 4), **spread(), "alg_bytes": bx, "GBps": round(bx / ms / 1e6, 1),
                "frac_hbm": round(bx / ms / 1e6 / HBM_PEAK_GBPS, 4), "grad_GBps": round(sum(xs) * 2 / ms / 1e6, 1)}
            # the twin streams the same bytes as one segment (scratch buffers of the total size)
            del xsegs
            tg = torch.cat([t.reshape(-1) for t in xg])
            del xg
            te = torch.zeros(tg.numel(), dtype=edt, device=dev)
            tc = torch.empty(tg.numel() // 2, dtype=torch.uint8, device=dev)
            ta = torch.empty(-(-tg.numel() // 128), dtype=torch.float32, device=dev)
            modes[f"compensate_quantize_4bit_{name}"].update(
                twin_of(lambda: twins.cq(tg, te, tc, ta, bits=4, block=128), stream, reps, bx, ms))
            del tg, te, tc, ta
            xe = "bf16" if edt == torch.bfloat16 else "f32"
            jobs.append((f"compensate_quantize_4bit_{name}", _cq_job(sample_host, xe, 4, 128),
                         cq_bytes([SAMPLE], 2, 2 if xe == "bf16" else 4, 4, 128),
                         f"the first tensor's first {SAMPLE:,} elements, one step"))
        # the paper's 8-bit error (LoCo Eqn. (7), s_e = 2^17) with 4-bit codes, same shard
        ei8 = torch.zeros(n, dtype=torch.int8, device=dev)
        segs_i8 = [(g[i * part:(i + 1) * part], ei8[i * part:(i + 1) * part], *segs[i][2:]) for i in range(PARTS)]
        ms = timed(lambda: loco.loco_compensate_quantize_ex(segs_i8, bits=BITS, block=BLOCK, beta=BETA,
                                                            err_scale=2.0 ** 17, stream=stream),
                   stream, reps)
        bi8 = cq_bytes(sizes, 2, 1, BITS, BLOCK)
        modes["compensate_quantize_4bit_i8err_7b_shard"] = {"avg_ms": round(ms, 4), **spread(), "alg_bytes": bi8,
                                                            "GBps": round(bi8 / ms / 1e6, 1),
                                                            "frac_hbm": round(bi8 / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                                            "grad_GBps": round(n * 2 / ms / 1e6, 1),
                                                            "err_scale": 2.0 ** 17}
        ci = torch.empty(n * BITS // 8, dtype=torch.uint8, device=dev)
        ai = torch.empty(-(-n // BLOCK), dtype=torch.float32, device=dev)
        modes["compensate_quantize_4bit_i8err_7b_shard"].update(
            twin_of(lambda: twins.cq(g, ei8, ci, ai, bits=BITS, block=BLOCK), stream, reps, bi8, ms))
        del ci, ai
        jobs.append(("compensate_quantize_4bit_i8err_7b_shard", _cq_job(_host_bf16(g[:SAMPLE]), "i8", BITS, BLOCK),
                     cq_bytes([SAMPLE], 2, 1, BITS, BLOCK), f"the shard's first {SAMPLE:,} elements, one step"))
        del ei8, segs_i8
        # the partition's payloads averaged straight into one LoCo-Adam step (Eqns. (8)-(9)):
        # fp32 weights and moments updated in place, plus the bf16 weight copy
        th = torch.randn(part, device=dev) * 0.02
        m_ = torch.zeros(part, device=dev)
        v_ = torch.zeros(part, device=dev)
        tb = torch.empty(part, dtype=torch.bfloat16, device=dev)
        ms = timed(lambda: loco.loco_dequant_reduce_adam(payloads, part, bits=BITS, block=BLOCK, out_scale=1.0 / PARTS,
                                                         param=th, m=m_, v=v_, lr=1e-4, beta1=0.1, beta2=0.01,
                                                         delta=1e-8, param_bf16=tb, stream=stream),
                   stream, reps)
        bda = dr_bytes(part, PARTS, BITS, BLOCK, 0) + 26 * part
        modes["dequant_reduce_adam_8peers"] = {"workload": f"8 peer 4-bit payloads of {part:,} averaged into one "
                                                           "Adam step (fp32 weights, m, v; bf16 weight copy)",
                                               "avg_ms": round(ms, 4), **spread(), "alg_bytes": bda,
                                               "GBps": round(bda / ms / 1e6, 1),
                                               "frac_hbm": round(bda / ms / 1e6 / HBM_PEAK_GBPS, 4)}
        ns = SAMPLE // 4
        th_h = th[:ns].cpu().numpy()  # before the twin overwrites the weights
        modes["dequant_reduce_adam_8peers"].update(
            twin_of(lambda: twins.dr(payloads, part, bits=BITS, block=BLOCK, theta=th, m=m_, v=v_, theta_bf16=tb),
                    stream, reps, bda, ms))
        spl = [(c[:ns * BITS // 8].cpu().numpy(), a[:ns // BLOCK].cpu().numpy()) for c, a in payloads]
        jobs.append(("dequant_reduce_adam_8peers",
                     lambda spl=spl, th_h=th_h, ns=ns: oracle_module().dequant_reduce_adam(
                         spl, ns, bits=BITS, block=BLOCK, out_scale=1.0 / PARTS, theta=th_h,
                         m=np.zeros(ns, np.float32), v=np.zeros(ns, np.float32), lr=1e-4, beta1=0.1, beta2=0.01,
                         delta=1e-8),
                     dr_bytes(ns, PARTS, BITS, BLOCK, 0) + 26 * ns, f"the partition's first {ns:,} elements"))
        del th, m_, v_, tb
        # SparseLoCo-style mode on its own workload
        nt = W.SPARSE_N
        gt = W.sparseloco_grad(0, n=nt, device=dev)
        et = torch.zeros(nt, dtype=torch.float32, device=dev)
        chunks = nt // TK_CHUNK
        idx = torch.empty(chunks * TK_K, dtype=torch.int16, device=dev)
        tcodes = torch.empty(chunks * ((TK_K * 2 + 7) // 8), dtype=torch.uint8, device=dev)
        tabs = torch.empty(chunks, dtype=torch.float32, device=dev)
        ms = timed(lambda: loco.loco_topk_quantize(gt, et, chunk=TK_CHUNK, k=TK_K, idx=idx, codes=tcodes,
                                                   absmax=tabs, bits=2, ef_decay=1.0, stream=stream),
                   stream, reps)
        bt = tk_bytes(nt, TK_CHUNK, TK_K, 2)
        modes["sparseloco_topk_2bit"] = {"workload": f"{nt:,} fp32 N(0,1e-3) + 0.1% +-0.1 outliers, chunk 4096, "
                                                     f"k=82, 2-bit, fp32 error feedback",
                                         "avg_ms": round(ms, 4), **spread(), "alg_bytes": bt, "GBps": round(bt / ms / 1e6, 1),
                                         "frac_hbm": round(bt / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                         "grad_GBps": round(nt * 4 / ms / 1e6, 1)}
        nts = 1024 * TK_CHUNK
        gts = gt[:nts].cpu().numpy()
        modes["sparseloco_topk_2bit"].update(
            twin_of(lambda: twins.tk(gt, et, idx, tcodes, tabs, k=TK_K, bits=2), stream, reps, bt, ms))
        jobs.append(("sparseloco_topk_2bit",
                     lambda gts=gts: oracle_module().topk_quantize(gts, np.zeros(gts.size, np.float32), chunk=TK_CHUNK,
                                                                  k=TK_K, bits=2, decay=1.0),
                     tk_bytes(nts, TK_CHUNK, TK_K, 2), f"the first 1,024 chunks ({nts:,} elements)"))
        del gt, et, idx, tcodes, tabs
        # SparseLoCo's sparse aggregation: 8 peers' Top-k payloads of the same shape into fp32 x 1/8
        spays = [W.random_sparse_payload(nt, TK_CHUNK, TK_K, 2, key=("bench", p), device=dev) for p in range(PARTS)]
        sout = torch.empty(nt, dtype=torch.float32, device=dev)
        ms = timed(lambda: loco.loco_sparse_aggregate(spays, nt, chunk=TK_CHUNK, k=TK_K, bits=2, out=sout,
                                                      out_scale=1.0 / PARTS, stream=stream),
                   stream, reps)
        bs = sa_bytes(nt, PARTS, TK_CHUNK, TK_K, 2, 4)
        modes["sparseloco_aggregate_8peers"] = {"workload": f"8 peers' Top-k payloads of {nt:,} (chunk 4096, k=82, "
                                                            f"2-bit) into fp32 x 1/8",
                                                "avg_ms": round(ms, 4), **spread(), "alg_bytes": bs,
                                                "GBps": round(bs / ms / 1e6, 1),
                                                "frac_hbm": round(bs / ms / 1e6 / HBM_PEAK_GBPS, 4)}
        modes["sparseloco_aggregate_8peers"].update(
            twin_of(lambda: twins.sa(spays, nt, k=TK_K, bits=2, out=sout), stream, reps, bs, ms))
        cb2, sch = (TK_K * 2 + 7) // 8, 8192
        sps = [(ix[:sch * TK_K].cpu().numpy().view(np.uint16), c[:sch * cb2].cpu().numpy(), a[:sch].cpu().numpy())
               for ix, c, a in spays]
        jobs.append(("sparseloco_aggregate_8peers",
                     lambda sps=sps: oracle_module().sparse_aggregate(sps, sch * TK_CHUNK, chunk=TK_CHUNK, k=TK_K,
                                                                     bits=2, out_scale=1.0 / PARTS),
                     sa_bytes(sch * TK_CHUNK, PARTS, TK_CHUNK, TK_K, 2, 4), f"the first {sch:,} chunks of the 8 payloads"))
        del sout
        # the same aggregation into bf16, which takes the library's other kernel (the
        # persistent streaming one, with its read passes); no traffic twin has its shape
        sob = torch.empty(nt, dtype=torch.bfloat16, device=dev)
        ms = timed(lambda: loco.loco_sparse_aggregate(spays, nt, chunk=TK_CHUNK, k=TK_K, bits=2, out=sob,
                                                      out_scale=1.0 / PARTS, stream=stream),
                   stream, reps)
        bsb = sa_bytes(nt, PARTS, TK_CHUNK, TK_K, 2, 2)
        modes["sparseloco_aggregate_8peers_bf16"] = {
            "workload": f"8 peers' Top-k payloads of {nt:,} (chunk 4096, k=82, 2-bit) into bf16 x 1/8",
            "avg_ms": round(ms, 4), **spread(), "alg_bytes": bsb, "GBps": round(bsb / ms / 1e6, 1),
            "frac_hbm": round(bsb / ms / 1e6 / HBM_PEAK_GBPS, 4)}
        jobs.append(("sparseloco_aggregate_8peers_bf16",
                     lambda sps=sps: oracle_module().sparse_aggregate(sps, sch * TK_CHUNK, chunk=TK_CHUNK, k=TK_K,
                                                                     bits=2, out_scale=1.0 / PARTS, out_dtype="bf16"),
                     sa_bytes(sch * TK_CHUNK, PARTS, TK_CHUNK, TK_K, 2, 2), f"the first {sch:,} chunks of the 8 payloads"))
        del spays, sob

        # the tiny case: 1,048,576 fp32 elements, one compensate-quantize (4-bit, block 128)
        # and the dequant-reduce of 4 peers into fp32 x 1/4 per step.  Its 19.6 MB sit in the
        # Infinity Cache and launch latency bounds it, so it gets no roofline claim: the time
        # per step over 200 back-to-back steps, launched eagerly and as replays of a HIP
        # graph that holds 20 steps.
        tn = TINY_N
        tg = W.tiny_grad(0, n=tn).to(dev)
        te = torch.zeros(tn, device=dev)
        tcd = torch.empty(loco.code_bytes(tn, BITS), dtype=torch.uint8, device=dev)
        tam = torch.empty(loco.num_blocks(tn, TINY_BLOCK), device=dev)
        tpays = []
        for pgr in W.tiny_peer_grads(TINY_PEERS, n=tn):
            tp = (torch.empty_like(tcd), torch.empty_like(tam))
            loco.loco_compensate_quantize([(pgr.to(dev), torch.zeros(tn, device=dev), *tp)], bits=BITS,
                                          block=TINY_BLOCK, beta=BETA)
            tpays.append(tp)
        tout = torch.empty(tn, device=dev)

        def tiny_step():  # on the current stream
            loco.loco_compensate_quantize([(tg, te, tcd, tam)], bits=BITS, block=TINY_BLOCK, beta=BETA)
            loco.loco_dequant_reduce(tpays, tn, bits=BITS, block=TINY_BLOCK, out=tout, out_scale=1.0 / TINY_PEERS)

        def per_step_us(launch, steps_per_launch, launches):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                for _ in range(3):
                    launch()
                a.record(stream)
                for _ in range(launches):
                    launch()
                b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / (steps_per_launch * launches)

        torch.cuda.synchronize()
        eager_us = per_step_us(tiny_step, 1, 200)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(20):
                tiny_step()
        torch.cuda.synchronize()
        graph_us = per_step_us(graph.replay, 20, 10)
        bt = cq_bytes([tn], 4, 4, BITS, TINY_BLOCK) + dr_bytes(tn, TINY_PEERS, BITS, TINY_BLOCK, 4)
        modes["tiny_1m_cq_dr_4peers"] = {
            "workload": f"{tn:,} fp32 N(0,1e-3), fp32 error, 4-bit block {TINY_BLOCK}; then dequant-reduce of "
                        f"{TINY_PEERS} peer payloads into fp32 x 1/{TINY_PEERS}",
            "cache_resident": True, "us_per_step_eager": round(eager_us, 2), "us_per_step_graph": round(graph_us, 2),
            "alg_bytes": bt, "GBps": round(bt / graph_us / 1e3, 1),
            "note": "launch-latency bound, inside the Infinity Cache: no roofline claim; GBps from the graph replays"}
        tgh, tph = tg.cpu().numpy(), [(c.cpu().numpy(), a.cpu().numpy()) for c, a in tpays]
        jobs.append(("tiny_1m_cq_dr_4peers",
                     lambda: (oracle_module().compensate_quantize(tgh, np.zeros(tn, np.float32), bits=BITS,
                                                                  block=TINY_BLOCK, beta=BETA),
                              oracle_module().dequant_reduce(tph, tn, bits=BITS, block=TINY_BLOCK,
                                                             out_scale=1.0 / TINY_PEERS)),
                     bt, f"the whole step ({tn:,} elements)"))
        del graph, tg, te, tcd, tam, tpays, tout

    for k, v in measured.items():
        if k in modes:
            modes[k]["hbm_bytes_measured"] = v["hbm_bytes"]
            modes[k]["hbm_over_alg"] = round(v["hbm_bytes"] / modes[k]["alg_bytes"], 4)

    for table in (kernels, modes):
        for v in table.values():
            if not v.get("cache_resident"):
                v["frac_copy"] = round(v["GBps"] / copy_gbps, 4)

    cpu = None
    if args.cpu_sample > 0:
        log(f"bench: CPU oracle on slabs of {args.cpu_sample:,} elements (>= 10 s)")
        cpu = cpu_baseline(g, payloads, args.cpu_sample)
        log("bench: the same oracle fanned out over the host's cores")
        cpu["parallel"] = cpu_baseline_parallel(g, payloads, args.cpu_sample)
        log("bench: the oracle on a sample of every mode's inputs")
        run_oracle_jobs(jobs, modes)

    value = n * 2 / (ms_per_step / 1e3) / 1e9
    line = {
        "metric": "gradient GB/s through compensate+quantize (and dequant-reduce), % of HBM peak",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "7B FSDP shard: 842,000,000 bf16 grad (1e-3 * Student-t(3)), fp32 error, "
                               "4-bit block-256 codes in 8 partitions of 105,250,000, beta 0.9; then "
                               "dequant-reduce of 8 peer 4-bit payloads of 105,250,000 into bf16 x 1/8",
                   "grad_elems": n, "partitions": PARTS, "bits": BITS, "block": BLOCK, "peers": PARTS,
                   "peer_elems": part},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "compensate_quantize_4bit", "alg_bytes_per_launch": cq_alg,
                     "launch_ms": round(cq_time_ms, 4), "launch_ms_from": cq_source,
                     "frac_twin": kernels["compensate_quantize_4bit"]["frac_twin"]},
        "cpu_baseline": cpu,
        "copy_ceiling": {"GBps": round(copy_gbps, 1), "frac_hbm": round(copy_gbps / HBM_PEAK_GBPS, 4),
                         "what": "1 GiB read + 1 GiB write by a hand-written streaming copy (libloco_twins.so, one "
                                 "16-byte vector per thread), bytes / median time of 10; each kernel's frac_copy is "
                                 "its GB/s over this"},
        "kernels": kernels,
        "modes": modes,
        "pct_hbm_peak_step": round(100 * (cq_alg + dr_alg) / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBPS, 2),
    }
    print(json.dumps(line), flush=True)


_FLUSH = None


def timed(fn, stream, reps):
    """Launch time in ms (HIP events on `stream`) of a mode, measured two ways after 2
    warm-ups, `reps` launches each:
      steady  - launches back to back: a launch may find the previous one's inputs in the
                256 MB Infinity Cache, and pays for writing back the previous one's dirty
                lines;
      flushed - a 1 GiB read before each launch (outside the timed pair): no launch finds
                its inputs cached, and none writes back another's dirty lines.
    Returns the slower of the two averages (the conservative one); the sorted per-launch
    times of both are kept in timed.last."""
    import torch
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    res = {}
    for mode in ("steady", "flushed"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        with torch.cuda.stream(stream):
            for a, b in evs:
                if mode == "flushed":
                    _FLUSH.sum()
                a.record(stream)
                fn()
                b.record(stream)
        torch.cuda.synchronize()
        res[mode] = sorted(a.elapsed_time(b) for a, b in evs)
    timed.last = res
    return max(sum(v) / reps for v in res.values())


def twin_of(fn, stream, reps, alg, kernel_ms):
    """Time a traffic twin by the same protocol as its kernel (the slower of back-to-back and
    cache-flushed averages) and relate the kernel to it: frac_twin = twin time / kernel time."""
    ms = timed(fn, stream, reps)
    return {"twin": {"ms": round(ms, 4), "GBps": round(alg / ms / 1e6, 1), **spread()},
            "frac_twin": round(ms / kernel_ms, 4)}


def spread():
    """Median, p10 and p90 (ms) of both ways of the last timed() call, and their averages."""
    out = {}
    for mode, ms in timed.last.items():
        out[mode] = {"avg_ms": round(sum(ms) / len(ms), 4), "median_ms": round(ms[len(ms) // 2], 4),
                     "p10_ms": round(ms[len(ms) // 10], 4), "p90_ms": round(ms[(len(ms) * 9) // 10], 4)}
    return {"timing": out}


if __name__ == "__main__":
    main()
