"""The algorithmic bytes bench.py divides by kernel time (the roofline numerators), against
the oracle's own byte counts and against totals worked out by hand per workload.

Per element: a bf16 gradient is 2 bytes read, an fp32 error 4 read + 4 written (bf16:
2 + 2, int8: 1 + 1), 4-bit codes half a byte written; plus 4 bytes of absmax per block.
"""
import bench
import oracle
import workloads as W


def test_compensate_quantize_bytes():
    part = W.SHARD7B_PART                      # 105,250,000 per partition, 8 partitions
    blocks = -(-part // 256)                   # 411,133 blocks of 256 (the last one 208 elements)
    assert blocks == 411_133
    # 7B shard, 4-bit: 10.5 bytes per element + 4 per block, per partition
    want = 8 * (part * 21 // 2 + 4 * blocks)
    assert want == 8_854_156_256
    assert bench.cq_bytes([part] * 8, 2, 4, 4, 256) == want
    assert 8 * oracle.cq_algorithmic_bytes(part, 2, 4, 4, 256) == want
    # 8-bit codes: one more half byte per element
    assert bench.cq_bytes([part] * 8, 2, 4, 8, 256) == want + 8 * part // 2 == 9_275_156_256
    # 8-bit error: 2 + 1 + 1 + 0.5 bytes per element
    assert bench.cq_bytes([part] * 8, 2, 1, 4, 256) == 8 * (part * 9 // 2 + 4 * blocks) == 3_802_156_256
    # LLaMA-7B layer: 7 tensors, block 128
    sizes = [r * c for _, r, c in W.llama_layer_shapes()]
    assert sum(sizes) == 202_375_168
    assert bench.cq_bytes(sizes, 2, 4, 4, 128) == sum(n * 21 // 2 + 4 * (n // 128) for n in sizes) == 2_131_263_488
    # MoE experts: bf16 error, 2 + 2 + 2 + 0.5 bytes per element, block 128
    sizes = [r * c for _, _, r, c in W.moe_shapes()]
    assert sum(sizes) == 1_409_286_144
    assert bench.cq_bytes(sizes, 2, 2, 4, 128) == sum(n * 13 // 2 + 4 * (n // 128) for n in sizes) == 9_204_400_128
    assert sum(oracle.cq_algorithmic_bytes(n, 2, 2, 4, 128) for n in sizes) == 9_204_400_128


def test_dequant_reduce_bytes():
    part = W.SHARD7B_PART
    # 8 peers' 4-bit codes and absmax read, bf16 out written
    want = 8 * (part // 2 + 4 * 411_133) + 2 * part
    assert want == 644_656_256
    assert bench.dr_bytes(part, 8, 4, 256, 2) == want == oracle.dr_algorithmic_bytes(part, 8, 4, 256, 2)
    # fused with the Adam step: theta, m, v read and written (24 bytes), the bf16 copy written
    dra = bench.dr_bytes(part, 8, 4, 256, 0) + 26 * part
    assert dra == 8 * (part // 2 + 4 * 411_133) + 26 * part == 3_170_656_256
    assert oracle.dra_algorithmic_bytes(part, 8, 4, 256, param_bf16=True) == dra


def test_tiny_bytes():
    # 1,048,576 fp32 gradient and error, 4-bit codes, block 128: 12.5 bytes per element + 4
    # per block; dequant-reduce of 4 peers into fp32
    n = bench.TINY_N
    assert n == W.TINY_N == 1 << 20
    assert bench.cq_bytes([n], 4, 4, 4, 128) == n * 25 // 2 + 4 * (n // 128) == 13_139_968
    assert bench.dr_bytes(n, 4, 4, 128, 4) == 4 * (n // 2 + 4 * (n // 128)) + 4 * n == 6_422_528
    assert oracle.cq_algorithmic_bytes(n, 4, 4, 4, 128) == 13_139_968
    assert oracle.dr_algorithmic_bytes(n, 4, 4, 128, 4) == 6_422_528


def test_sparseloco_bytes():
    n, C, k = 1 << 28, 4096, 82
    chunks = n // C
    # Top-k: g and e read, e written (12 bytes per element); per chunk 82 u16 indices, 21 bytes
    # of 2-bit codes and a 4-byte scale
    assert bench.tk_bytes(n, C, k, 2) == 12 * n + chunks * (164 + 21 + 4) == 3_233_611_776
    assert oracle.tk_algorithmic_bytes(n, C, k, 2) == 3_233_611_776
    # sparse aggregation: 8 peers' payloads read, fp32 out written
    assert bench.sa_bytes(n, 8, C, k, 2, 4) == 8 * chunks * (164 + 21 + 4) + 4 * n == 1_172_832_256
    assert bench.sa_bytes(n, 8, C, k, 2, 2) == 8 * chunks * (164 + 21 + 4) + 2 * n == 635_961_344
    assert oracle.sa_algorithmic_bytes(n, 8, C, k, 2, 4) == 1_172_832_256


def test_traffic_summary_dropped_when_kernel_changes(tmp_path, monkeypatch):
    """bench.py reports a kernel's measured HBM bytes only while the kernel's sources hash
    to what the counter summary recorded; a summary taken before a change gives null."""
    import json
    kernels = {k: {"hbm_bytes": 1000 + i, "source_hash": bench.kernel_source_hash(k)}
               for i, k in enumerate(sorted(bench.KERNEL_FILES))}
    stale = "compensate_quantize_4bit"
    kernels[stale]["source_hash"] = "0" * 16
    kernels["not_a_kernel"] = {"hbm_bytes": 1, "source_hash": "x"}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernels": kernels}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    got = bench.load_traffic()
    assert set(got) == set(bench.KERNEL_FILES) - {stale}
    # every kernel's hash covers source files that exist, plus the shared headers
    import os
    for k, files in bench.KERNEL_FILES.items():
        assert files and all(os.path.isfile(os.path.join(bench.CSRC, x)) for x in files + bench.COMMON_FILES)
        assert len(bench.kernel_source_hash(k)) == 16
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic() == {}
