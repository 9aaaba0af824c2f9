"""ctypes binding of the benchmark's traffic twins (libloco_twins.so).

Each twin issues the loads and stores of one of the library's kernels, in its launch
shape, with no compression arithmetic; bench.py times them beside the kernels to report
each kernel's fraction of its own stream mix's ceiling, and the streaming copy as the
plain ceiling.  Not part of the library's API; nothing here is used by the data path.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

_lib = None
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def load(path: str | None = None):
    global _lib
    if _lib is None:
        path = path or _build.TWINS_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run bit_gradient_compression_amd.build.build()")
        lib = ctypes.CDLL(path)
        lib.loco_twin_copy.argtypes = [_p, _p, _i64, _p]
        lib.loco_twin_cq.argtypes = [_p, _p, _p, _p, _i64, _int, _int, _int, _int, _p]
        lib.loco_twin_dr.argtypes = [ctypes.POINTER(_p), ctypes.POINTER(_p), _int, _i64, _int, _int, _int,
                                     _p, _p, _p, _p, _p, _p]
        lib.loco_twin_tk.argtypes = [_p, _p, _p, _p, _p, _i64, _int, _int, _p]
        lib.loco_twin_sa.argtypes = [ctypes.POINTER(_p), ctypes.POINTER(_p), ctypes.POINTER(_p), _int, _i64, _int,
                                     _int, _p, _p]
        for f in (lib.loco_twin_copy, lib.loco_twin_cq, lib.loco_twin_dr, lib.loco_twin_tk, lib.loco_twin_sa):
            f.restype = _int
        _lib = lib
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(name, st):
    if st != 0:
        raise RuntimeError(f"{name}: status {st}")


def copy(src, dst):
    _check("copy", load().loco_twin_copy(_ptr(src), _ptr(dst), min(src.numel() * src.element_size(),
                                                                   dst.numel() * dst.element_size()), _stream()))


def cq(g, e, codes, absmax, *, bits, block):
    ekind = {torch.float32: 0, torch.bfloat16: 1, torch.int8: 2}[e.dtype]
    _check("cq", load().loco_twin_cq(_ptr(g), _ptr(e), _ptr(codes), _ptr(absmax), g.numel(), g.element_size(),
                                     ekind, bits, block, _stream()))


def _arr(ts):
    return (_p * len(ts))(*[t.data_ptr() for t in ts])


def dr(payloads, n, *, bits, block, out=None, theta=None, m=None, v=None, theta_bf16=None):
    codes = _arr([c for c, _ in payloads])
    absmax = _arr([a for _, a in payloads])
    mode = 2 if theta is not None else (1 if out.dtype == torch.bfloat16 else 0)
    _check("dr", load().loco_twin_dr(codes, absmax, len(payloads), n, bits, block, mode, _ptr(out), _ptr(theta),
                                     _ptr(m), _ptr(v), _ptr(theta_bf16), _stream()))


def tk(g, e, idx, codes, absmax, *, k, bits):
    _check("tk", load().loco_twin_tk(_ptr(g), _ptr(e), _ptr(idx), _ptr(codes), _ptr(absmax), g.numel(), k, bits,
                                     _stream()))


def sa(payloads, n, *, k, bits, out):
    _check("sa", load().loco_twin_sa(_arr([i for i, _, _ in payloads]), _arr([c for _, c, _ in payloads]),
                                     _arr([a for _, _, a in payloads]), len(payloads), n, k, bits, _ptr(out),
                                     _stream()))
