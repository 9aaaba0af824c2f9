"""Every kernel of the built libraries keeps its values in registers: no scratch memory
(spills cost HBM writes on every wave that stores them) and no VGPR spills.  Read from
the compiler's per-kernel resource remarks that the build records; skipped when no build
has run here."""
import json
import os

import pytest

from bit_gradient_compression_amd import build as B

RES = os.path.join(B.BUILD_DIR, "resources.json")


@pytest.fixture(scope="module")
def resources():
    if not os.path.exists(RES):
        pytest.skip("no build has run in this tree")
    with open(RES) as f:
        return json.load(f)


def test_every_source_reported(resources):
    srcs = {v["source"] for v in resources.values()}
    assert set(B.SOURCES) - {"abi.hip"} <= srcs


def test_no_scratch_and_no_spills(resources):
    bad = {k: v for k, v in resources.items()
           if v.get("scratch_bytes_per_lane", 0) or v.get("vgpr_spill", 0)}
    assert not bad, f"kernels using scratch: {sorted(bad)[:5]}"


def test_hot_kernels_occupancy(resources):
    """The timed kernels keep the occupancy their launch shapes were tuned for."""
    want = {"cq_kernelILi1ELi0ELi4ELi256ELb0E": 8, "dr_kernelILi4ELi256ELb0ELi1E": 8,
            "dr_kernelILi4ELi256ELb0ELi2E": 5, "tk_kernelILi16ELi2ELb1E": 6}
    for frag, waves in want.items():
        got = [v["waves_per_simd"] for k, v in resources.items() if frag in k]
        assert got and min(got) >= waves, (frag, got)
