"""The C ABI without a GPU: the library loads, exports every function include/loco.h
declares, and refuses bad arguments on the host before any HIP call.

Every call here either fails validation or has nothing to do (n == 0), so nothing is
launched; the fake pointers are never dereferenced.  The exception: calls with the most
peers a call accepts pass validation and build their kernel arguments on the host, then
fail to launch (no GPU here, LOCO_ERR_HIP); they check that building the peer tables
stays inside them.
"""
import ctypes
import glob
import math
import os
import re
import subprocess

import pytest
import torch

if torch.cuda.is_available():
    # Fake pointers must never reach a real device: these checks run only where no GPU is.
    pytest.skip("host-only validation tests (fake device pointers)", allow_module_level=True)

from bit_gradient_compression_amd import build as B  # noqa: E402
from bit_gradient_compression_amd import loco  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INV, ALIGN, UNSUP = loco.LOCO_OK, loco.LOCO_ERR_INVALID, loco.LOCO_ERR_ALIGN, loco.LOCO_ERR_UNSUPPORTED
F32, BF16 = loco.LOCO_F32, loco.LOCO_BF16
NAN = float("nan")


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(loco_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libloco.so is not built (run __graft_entry__.build())")
    return loco.load()


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for fn in ("loco_compensate_quantize", "loco_dequant_reduce", "loco_topk_quantize", "loco_status_string"):
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(loco_\w+)$", out, flags=re.M))
    for fn in declared_functions():
        assert fn in exported, fn
        assert getattr(lib, fn) is not None
    assert set(loco.SYMBOLS) == set(declared_functions())
    # nothing else leaks out of the library with a loco_ prefix
    assert exported == set(declared_functions())


def test_status_strings(lib):
    for s in (OK, INV, ALIGN, UNSUP, loco.LOCO_ERR_HIP):
        assert loco.status_string(s).startswith("LOCO_")
    assert loco.status_string(-99) == "unknown status"
    assert lib.loco_version() >= 10000


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(loco, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        loco.load("/nonexistent/libloco.so")


A = 0x10000  # fake, 16-byte aligned, far-apart device addresses
Bp, Cp, Dp = 0x20000000, 0x40000000, 0x60000000


def seg(g=A, e=Bp, c=Cp, a=Dp, n=1000):
    return loco.CqSegment(g, e, c, a, n)


def cq(lib, segs, gd=F32, ed=F32, bits=4, block=128, beta=0.9, fixed=0.0, nseg=None):
    arr = (loco.CqSegment * max(1, len(segs)))(*segs) if segs else None
    return lib.loco_compensate_quantize(arr, len(segs) if nseg is None else nseg, gd, ed, bits, block,
                                        beta, fixed, None)


@pytest.mark.parametrize("kwargs,want", [
    (dict(nseg=-1), INV),
    (dict(gd=2), INV), (dict(ed=-1), INV),
    (dict(bits=0), INV), (dict(bits=9), INV), (dict(bits=3), UNSUP), (dict(bits=1), UNSUP),
    (dict(beta=-0.1), INV), (dict(beta=1.1), INV), (dict(beta=NAN), INV),
    (dict(fixed=-1.0), INV), (dict(fixed=math.inf), INV),
    (dict(block=0), INV), (dict(block=-128), INV), (dict(block=100), UNSUP), (dict(block=1024), UNSUP),
])
def test_cq_parameter_checks(lib, kwargs, want):
    assert cq(lib, [seg()], **kwargs) == want


@pytest.mark.parametrize("s,want", [
    (seg(n=-1), INV),
    (seg(g=0), INV), (seg(e=0), INV), (seg(c=0), INV), (seg(a=0), INV),
    (seg(g=A + 2), ALIGN), (seg(e=Bp + 8), ALIGN), (seg(c=Cp + 4), ALIGN), (seg(a=Dp + 4), ALIGN),
    (seg(e=A + 16), INV),                 # err overlaps grad
    (seg(c=A + 1000 * 4 - 16), INV),      # codes overlap the last 16 bytes of grad (f32)
    (seg(a=Cp + 256), INV),               # absmax overlaps codes (500 bytes at 4 bits)
])
def test_cq_segment_checks(lib, s, want):
    assert cq(lib, [s]) == want


def test_cq_noop_and_mixed(lib):
    assert cq(lib, []) == OK
    assert cq(lib, [seg(n=0), seg(g=0, n=0)]) == OK     # empty segments are never touched
    # one bad segment refuses the whole call, wherever it is
    assert cq(lib, [seg(), seg(g=A + 4 * 4096, e=Bp + 4 * 4096, c=Cp + 4096, a=Dp + 4096, n=-5)]) == INV
    # fixed-scale mode: absmax may be NULL and block is ignored, but everything else is checked
    assert cq(lib, [seg(a=0, g=A + 2)], fixed=2.0 ** 19, block=7) == ALIGN


def test_cq_buffers_of_different_segments(lib):
    """A buffer one segment writes must not overlap any buffer of another segment."""
    s0 = seg()
    off = 1 << 20
    # the second segment's error overlaps the first one's codes (500 bytes at 4 bits)
    assert cq(lib, [s0, seg(g=A + off, e=Cp + 256, c=Cp + off, a=Dp + off)]) == INV
    # the second segment's codes overlap the first one's gradient
    assert cq(lib, [s0, seg(g=A + off, e=Bp + off, c=A + 64, a=Dp + off)]) == INV
    # the second segment's absmax overlaps the first one's error, and the order does not matter
    bad = seg(g=A + off, e=Bp + off, c=Cp + off, a=Bp + 128)
    assert cq(lib, [s0, bad]) == INV
    assert cq(lib, [bad, s0]) == INV
    # two segments writing the same error buffer
    assert cq(lib, [s0, seg(g=A + off, c=Cp + off, a=Dp + off)]) == INV


def pl(c=Cp, a=Dp):
    return loco.Payload(c, a)


def dr(lib, peers, n=1000, bits=4, block=128, fixed=0.0, scale=0.25, out=A, od=F32, npeers=None):
    arr = (loco.Payload * max(1, len(peers)))(*peers) if peers else None
    return lib.loco_dequant_reduce(arr, len(peers) if npeers is None else npeers, n, bits, block, fixed,
                                   scale, out, od, None)


@pytest.mark.parametrize("kwargs,want", [
    (dict(npeers=0), INV), (dict(n=-1), INV), (dict(bits=3), UNSUP), (dict(bits=0), INV),
    (dict(block=100), UNSUP), (dict(block=0), INV), (dict(fixed=-2.0), INV),
    (dict(scale=NAN), INV), (dict(scale=math.inf), INV), (dict(od=7), INV),
    (dict(out=0), INV), (dict(out=A + 4), ALIGN),
    (dict(out=Cp + 16), INV),             # output overlaps a payload
])
def test_dr_checks(lib, kwargs, want):
    assert dr(lib, [pl(), pl(Cp + 4096, Dp + 4096)], **kwargs) == want


def test_dr_peer_checks(lib):
    assert dr(lib, [pl(c=0)]) == INV
    assert dr(lib, [pl(a=0)]) == INV
    assert dr(lib, [pl(c=Cp + 1)]) == ALIGN
    assert dr(lib, [pl()] * 129) == UNSUP
    assert dr(lib, [], npeers=1) == INV
    assert dr(lib, [pl()], n=0) == OK


def tk(lib, g=A, e=Bp, n=10000, chunk=4096, k=82, bits=2, decay=1.0, idx=Cp, codes=Dp, absmax=0x70000000):
    return lib.loco_topk_quantize(g, e, n, chunk, k, bits, decay, idx, codes, absmax, None)


@pytest.mark.parametrize("kwargs,want", [
    (dict(n=-1), INV), (dict(chunk=0), INV), (dict(chunk=70000), INV), (dict(chunk=1000), UNSUP),
    (dict(chunk=8192), UNSUP), (dict(k=0), INV), (dict(k=4097), INV), (dict(bits=3), UNSUP),
    (dict(bits=10), INV), (dict(decay=1.5), INV), (dict(decay=NAN), INV),
    (dict(g=0), INV), (dict(idx=0), INV), (dict(absmax=0), INV),
    (dict(e=Bp + 4), ALIGN), (dict(codes=Dp + 1), ALIGN),
    (dict(e=A + 64), INV),                # err overlaps grad
    (dict(codes=Cp + 16), INV),           # codes overlap the index array
])
def test_tk_checks(lib, kwargs, want):
    assert tk(lib, **kwargs) == want


def test_tk_noop(lib):
    assert tk(lib, n=0) == OK
    assert tk(lib, n=0, g=0) == OK


I8 = loco.LOCO_I8


def cqx(lib, segs, gd=F32, ed=I8, bits=4, block=128, beta=0.9, fixed=0.0, err_scale=256.0, reset=0,
        opt=True):
    arr = (loco.CqSegment * max(1, len(segs)))(*segs) if segs else None
    o = loco.CqOptions(bits, block, beta, fixed, err_scale, reset)
    return lib.loco_compensate_quantize_ex(arr, len(segs), gd, ed, ctypes.byref(o) if opt else None, None)


@pytest.mark.parametrize("kwargs,want", [
    (dict(opt=False), INV),
    (dict(gd=I8), INV), (dict(ed=3), INV),
    (dict(err_scale=0.0), INV), (dict(err_scale=-4.0), INV), (dict(err_scale=NAN), INV),
    (dict(err_scale=math.inf), INV),
    (dict(err_scale=1e-37), INV),          # 256 / s_e overflows binary32
    (dict(bits=3), UNSUP), (dict(block=100), UNSUP), (dict(beta=2.0), INV), (dict(fixed=-1.0), INV),
    (dict(reset=1, bits=5), UNSUP),
])
def test_cq_ex_parameter_checks(lib, kwargs, want):
    assert cqx(lib, [seg()], **kwargs) == want


def test_cq_ex_err_scale_ignored_for_float_errors(lib):
    # a float error never reads s_e: only the segment's misalignment is reported
    assert cqx(lib, [seg(g=A + 2)], ed=F32, err_scale=0.0) == ALIGN
    assert cqx(lib, [seg(g=A + 2)], ed=BF16, err_scale=NAN) == ALIGN


def test_cq_old_entry_refuses_int8_error(lib):
    assert cq(lib, [seg()], ed=I8) == INV


def test_cq_ex_int8_error_is_one_byte_per_element(lib):
    # codes start 1008 bytes after an int8 error of 1000 elements: no overlap at one byte
    # per element (an f32 error would cover 4000 bytes and overlap them).  The second
    # segment is misaligned, so the call stops at ALIGN and launches nothing.
    first = seg(e=Bp, c=Bp + 1008, a=Dp)
    bad = seg(g=A + 8192 + 2, e=Bp + 65536, c=Cp, a=Dp + 65536)
    assert cqx(lib, [first, bad]) == ALIGN
    assert cqx(lib, [first, bad], ed=F32) == INV
    # and an overlap inside the int8 error's 1000 bytes is still refused
    assert cqx(lib, [seg(e=Bp, c=Bp + 992)]) == INV


def spl(ix=Cp, c=Dp, a=0x70000000):
    return loco.SparsePayload(ix, c, a)


def sa(lib, peers, n=10000, chunk=4096, k=82, bits=2, scale=0.125, out=A, od=F32, npeers=None):
    arr = (loco.SparsePayload * max(1, len(peers)))(*peers) if peers else None
    return lib.loco_sparse_aggregate(arr, len(peers) if npeers is None else npeers, n, chunk, k, bits, scale,
                                     out, od, None)


@pytest.mark.parametrize("kwargs,want", [
    (dict(npeers=0), INV), (dict(n=-1), INV), (dict(chunk=0), INV), (dict(chunk=70000), INV),
    (dict(chunk=1000), UNSUP), (dict(chunk=8192), UNSUP), (dict(k=0), INV), (dict(k=4097), INV),
    (dict(bits=3), UNSUP), (dict(bits=0), INV), (dict(scale=NAN), INV), (dict(scale=-math.inf), INV),
    (dict(od=I8), INV), (dict(out=0), INV), (dict(out=A + 8), ALIGN),
    (dict(out=Cp + 64), INV),             # output overlaps a peer's index array
])
def test_sa_checks(lib, kwargs, want):
    assert sa(lib, [spl(), spl(Cp + 0x100000, Dp + 0x100000, 0x70100000)], **kwargs) == want


def test_sa_peer_checks(lib):
    assert sa(lib, [spl(ix=0)]) == INV
    assert sa(lib, [spl(c=0)]) == INV
    assert sa(lib, [spl(a=0)]) == INV
    assert sa(lib, [spl(ix=Cp + 2)]) == ALIGN
    assert sa(lib, [spl(a=0x70000000 + 4)]) == ALIGN
    assert sa(lib, [spl()] * 129) == UNSUP
    assert sa(lib, [], npeers=1) == INV
    assert sa(lib, [spl()], n=0) == OK
    # a peer's scales inside the last 16 bytes of the output
    assert sa(lib, [spl(a=A + 10000 * 4 - 16)]) == INV


HIP = loco.LOCO_ERR_HIP


def test_max_peers_build_their_arguments(lib):
    """128 peers (the maximum) pass validation and fill the kernel arguments' peer tables
    on the host; with no GPU the launch then fails.  (A table written past its end on the
    host stack crashed the process here.)"""
    pls = [pl(Cp + i * 0x100000, Dp + i * 0x100000) for i in range(128)]
    assert dr(lib, pls, n=1000) == HIP
    assert dra(lib, pls, n=1000) == HIP
    spls = [spl(Cp + i * 0x100000, Dp + i * 0x100000, 0x70000000 + i * 0x100000) for i in range(128)]
    assert sa(lib, spls, n=10000) == HIP


def dra(lib, peers, n=1000, bits=4, block=128, fixed=0.0, scale=0.25, hp=(1e-4, 0.1, 0.01, 1e-8), param=A,
        m=0x7000000, v=0x7100000, pb=0, npeers=None, null_hp=False):
    arr = (loco.Payload * max(1, len(peers)))(*peers) if peers else None
    h = loco.AdamParams(*hp)
    return lib.loco_dequant_reduce_adam(arr, len(peers) if npeers is None else npeers, n, bits, block, fixed, scale,
                                        None if null_hp else ctypes.byref(h), param, m, v, pb or None, None)


@pytest.mark.parametrize("kwargs,want", [
    (dict(npeers=0), INV), (dict(n=-1), INV), (dict(bits=3), UNSUP), (dict(block=100), UNSUP),
    (dict(scale=NAN), INV), (dict(null_hp=True), INV),
    (dict(hp=(NAN, 0.1, 0.01, 1e-8)), INV), (dict(hp=(1e-4, 1.5, 0.01, 1e-8)), INV),
    (dict(hp=(1e-4, 0.1, -0.1, 1e-8)), INV), (dict(hp=(1e-4, 0.1, 0.01, 0.0)), INV),
    (dict(hp=(1e-4, 0.1, 0.01, math.inf)), INV),
    (dict(param=0), INV), (dict(m=0), INV), (dict(v=0), INV),
    (dict(param=A + 4), ALIGN), (dict(pb=0x7200000 + 2), ALIGN),
    (dict(m=A + 16), INV),                 # m overlaps param
    (dict(pb=0x7100000 + 64), INV),        # the bf16 copy overlaps v
    (dict(v=Cp + 32), INV),                # v overlaps a payload's codes
])
def test_dra_checks(lib, kwargs, want):
    assert dra(lib, [pl(), pl(Cp + 4096, Dp + 4096)], **kwargs) == want


def test_dra_noop(lib):
    assert dra(lib, [pl()], n=0) == OK
    assert dra(lib, [pl()], n=0, param=0) == OK


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "loco.h"

/* Only calls that fail validation or have nothing to do: nothing is launched. */
int main(void) {
    int bad = 0;
    loco_cq_segment_t seg;
    loco_payload_t pay;
    loco_sparse_payload_t sp;
    loco_cq_options_t opt;
    loco_adam_t adam = {1e-3f, 0.1f, 0.01f, 1e-8f};
    memset(&seg, 0, sizeof seg);
    memset(&pay, 0, sizeof pay);
    memset(&sp, 0, sizeof sp);
    memset(&opt, 0, sizeof opt);
    opt.bits = 4; opt.block = 256; opt.beta = 0.9f;
    if (loco_version() <= 0) bad |= 1;
    if (strlen(loco_status_string(LOCO_ERR_ALIGN)) == 0) bad |= 2;
    /* a null segment array with one segment, and a zero-length segment */
    if (loco_compensate_quantize(NULL, 1, LOCO_BF16, LOCO_F32, 4, 256, 0.9f, 0.0f, NULL) != LOCO_ERR_INVALID) bad |= 4;
    if (loco_compensate_quantize(&seg, 1, LOCO_BF16, LOCO_F32, 4, 256, 0.9f, 0.0f, NULL) != LOCO_OK) bad |= 8;
    if (loco_compensate_quantize_ex(&seg, 1, LOCO_BF16, LOCO_F32, NULL, NULL) != LOCO_ERR_INVALID) bad |= 16;
    if (loco_compensate_quantize_ex(&seg, 1, LOCO_BF16, LOCO_F32, &opt, NULL) != LOCO_OK) bad |= 32;
    if (loco_dequant_reduce(&pay, 0, 16, 4, 256, 0.0f, 1.0f, NULL, LOCO_F32, NULL) != LOCO_ERR_INVALID) bad |= 64;
    if (loco_dequant_reduce_adam(&pay, 1, 16, 4, 256, 0.0f, 1.0f, &adam, NULL, NULL, NULL, NULL, NULL)
        != LOCO_ERR_INVALID) bad |= 128;
    if (loco_topk_quantize(NULL, NULL, 0, 4096, 82, 2, 1.0f, NULL, NULL, NULL, NULL) != LOCO_OK) bad |= 256;
    if (loco_sparse_aggregate(&sp, 1, 16, 4096, 82, 3, 1.0f, NULL, LOCO_F32, NULL) != LOCO_ERR_UNSUPPORTED)
        bad |= 512;
    printf("bad=%d\n", bad);
    return bad != 0;
}
"""


@pytest.mark.parametrize("lang", ["c99", "c++17"])
def test_header_compiles_and_links_from_c(lib, tmp_path, lang):
    """include/loco.h is plain C (and C++ through its extern "C" block): a program built
    with warnings as errors links against the library and gets the documented statuses
    from calls that only validate."""
    cxx = lang.startswith("c++")
    src = tmp_path / ("prog.cpp" if cxx else "prog.c")
    src.write_text(C_PROGRAM)
    exe = tmp_path / "prog"
    libdir = os.path.dirname(B.LIB_PATH)
    cmd = ["g++" if cxx else "gcc", f"-std={lang}", "-Wall", "-Wextra", "-Werror", "-pedantic",
           f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe), f"-L{libdir}", "-lloco",
           f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "bad=0" in r.stdout, r.stdout + r.stderr


def test_twins_library_is_separate_and_loads():
    """The benchmark's traffic twins live in their own library: it loads, exports its five
    entry points, and refuses a shape it has no twin for before any launch."""
    from bit_gradient_compression_amd import twins
    if not os.path.exists(B.TWINS_PATH):
        pytest.fail("libloco_twins.so is not built (run __graft_entry__.build())")
    tl = twins.load()
    out = subprocess.run(["nm", "-D", "--defined-only", B.TWINS_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(loco_\w+)$", out, flags=re.M))
    assert exported == {"loco_twin_copy", "loco_twin_cq", "loco_twin_dr", "loco_twin_tk", "loco_twin_sa"}
    assert tl.loco_twin_copy(None, None, 0, None) == -1
    assert tl.loco_twin_cq(None, None, None, None, 0, 2, 0, 4, 256, None) == -1
