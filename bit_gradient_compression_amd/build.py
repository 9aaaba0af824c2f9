"""Build libloco.so (gfx950) in-tree with hipcc.

Every translation unit is compiled in parallel, then linked.  Flags that fix the
arithmetic: no fused multiply-add contraction, no fast math, IEEE division and denormals
kept, and no packed-fp32 instructions.
"""

from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libloco.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["abi.hip", "cq.hip", "dr.hip", "tk.hip", "sa.hip"]
# Traffic twins of the kernels, for the benchmark only: a library of their own, outside
# the API that include/loco.h declares.
TWINS_SOURCES = ["twins.hip"]
TWINS_PATH = os.path.join(PKG, "libloco_twins.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def compile_flags(extra=()):
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-fno-gpu-flush-denormals-to-zero",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}", *extra]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


# The compiler's per-kernel resource remarks (-Rpass-analysis=kernel-resource-usage), kept
# as one JSON file per build: VGPRs, scratch bytes per lane, occupancy and LDS per kernel.
RESOURCE_FLAG = "-Rpass-analysis=kernel-resource-usage"
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"LDS Size \[bytes/block\]|VGPRs Spill):\s+(\S+)")
_KEYS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
         "Occupancy [waves/SIMD]": "waves_per_simd", "LDS Size [bytes/block]": "lds_bytes", "VGPRs Spill": "vgpr_spill"}


def parse_resources(text: str) -> dict:
    """Kernel name -> its resource figures, from the compiler's remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(text):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[_KEYS[key]] = int(val)
    return out


def build(out_path: str = LIB_PATH, extra_flags=(), jobs: int | None = None, verbose=False,
          build_dir: str = BUILD_DIR, twins_path: str | None = TWINS_PATH) -> str:
    """Compile and link the library (and, unless twins_path is None, the benchmark's
    traffic twins); returns the path of the library's .so."""
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    flags = compile_flags(extra_flags)
    objs = []
    cmds = []
    for src in SOURCES + (TWINS_SOURCES if twins_path else []):
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *flags, RESOURCE_FLAG, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
    resources = {}
    with ThreadPoolExecutor(jobs) as ex:
        for src, r in zip(SOURCES + (TWINS_SOURCES if twins_path else []), ex.map(_run, cmds)):
            resources.update({k: {**v, "source": src} for k, v in parse_resources(r.stderr).items()})
            if verbose and r.stderr:
                print(r.stderr, file=sys.stderr)
    with open(os.path.join(build_dir, "resources.json"), "w") as f:
        json.dump(resources, f, indent=0, sort_keys=True)
    links = [(out_path, objs[:len(SOURCES)])]
    if twins_path:
        links.append((twins_path, objs[len(SOURCES):]))
    for path, os_ in links:
        tmp = path + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *os_, "-o", tmp])
        os.replace(tmp, path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
