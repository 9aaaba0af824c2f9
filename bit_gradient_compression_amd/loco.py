"""Python binding of libloco.so (ctypes): argument marshalling only.

Every function takes torch tensors (device memory) and passes their pointers, sizes and
the current HIP stream to the C ABI of the same name; every step of the computation
runs in the library's HIP kernels.  There is no fallback: if the library is missing or
a call returns an error status, the call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

LOCO_F32 = 0
LOCO_BF16 = 1
LOCO_I8 = 2
LOCO_OK = 0
LOCO_ERR_INVALID = -1
LOCO_ERR_ALIGN = -2
LOCO_ERR_UNSUPPORTED = -3
LOCO_ERR_HIP = -4
LOCO_MAX_PEERS = 128

SYMBOLS = ["loco_compensate_quantize", "loco_compensate_quantize_ex", "loco_dequant_reduce",
           "loco_dequant_reduce_adam", "loco_topk_quantize", "loco_sparse_aggregate", "loco_status_string",
           "loco_version"]


class LocoError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} ({status})")


class CqSegment(ctypes.Structure):
    _fields_ = [("grad", ctypes.c_void_p), ("err", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("absmax", ctypes.c_void_p), ("n", ctypes.c_int64)]


class CqOptions(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int), ("block", ctypes.c_int), ("beta", ctypes.c_float),
                ("fixed_scale", ctypes.c_float), ("err_scale", ctypes.c_float),
                ("reset_error", ctypes.c_int)]


class Payload(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p)]


class AdamParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("delta", ctypes.c_float)]


class SparsePayload(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return _build.LIB_PATH


def load(path: str | None = None):
    """Load libloco.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.loco_compensate_quantize.argtypes = [ctypes.POINTER(CqSegment), ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                             ctypes.c_float, ctypes.c_void_p]
    lib.loco_compensate_quantize.restype = ctypes.c_int
    lib.loco_compensate_quantize_ex.argtypes = [ctypes.POINTER(CqSegment), ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.POINTER(CqOptions), ctypes.c_void_p]
    lib.loco_compensate_quantize_ex.restype = ctypes.c_int
    lib.loco_dequant_reduce.argtypes = [ctypes.POINTER(Payload), ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p]
    lib.loco_dequant_reduce.restype = ctypes.c_int
    lib.loco_dequant_reduce_adam.argtypes = [ctypes.POINTER(Payload), ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.POINTER(AdamParams),
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p]
    lib.loco_dequant_reduce_adam.restype = ctypes.c_int
    lib.loco_topk_quantize.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.loco_topk_quantize.restype = ctypes.c_int
    lib.loco_sparse_aggregate.argtypes = [ctypes.POINTER(SparsePayload), ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.loco_sparse_aggregate.restype = ctypes.c_int
    lib.loco_status_string.argtypes = [ctypes.c_int]
    lib.loco_status_string.restype = ctypes.c_char_p
    lib.loco_version.argtypes = []
    lib.loco_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().loco_status_string(int(status)).decode()


loco_status_string = status_string


def _check(fn, status):
    if status != LOCO_OK:
        raise LocoError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t is None:  # a missing buffer: the C call refuses its null pointer
        return LOCO_F32
    if t.dtype == torch.float32:
        return LOCO_F32
    if t.dtype == torch.bfloat16:
        return LOCO_BF16
    if t.dtype == torch.int8:
        return LOCO_I8
    raise TypeError(f"unsupported dtype {t.dtype}")


try:  # the current stream's handle without building a Stream object (~2.5 us less per call)
    _current_raw_stream = torch._C._cuda_getCurrentRawStream
except AttributeError:  # pragma: no cover - a torch without it
    _current_raw_stream = None


def _device() -> int:
    """The current device: every call launches there, so its tensors must live there."""
    return torch.cuda.current_device()


def _ptr(t, dev):
    if t is None:
        return None
    d = t.get_device()
    if d != dev:
        if d < 0:
            raise ValueError("tensor must be in device memory")
        raise ValueError(f"tensor is on cuda:{d}; the call runs on the current device, cuda:{dev}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream, dev):
    if stream is None:
        if _current_raw_stream is not None:
            return _current_raw_stream(dev)
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def code_bytes(n: int, bits: int) -> int:
    return (n * bits + 7) // 8


def num_blocks(n: int, block: int) -> int:
    return -(-n // block)


# Sizes the C calls accept; for these, the binding checks that every tensor holds the bytes
# the call will read or write (the C ABI sees only pointers and n).  Other values go to
# the C call unchecked, which refuses them with its own status.
_BITS = (2, 4, 8)
_BLOCKS = (64, 128, 256, 512)
_CHUNKS = (256, 512, 1024, 2048, 4096)


def _need(t, nbytes: int, what: str) -> None:
    if t is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what} holds {t.numel() * t.element_size()} bytes; the call needs {nbytes}")


def _segments(segments, dev, bits=None, block=None, fixed=False):
    segs = list(segments)
    arr = (CqSegment * max(1, len(segs)))()
    gd = ed = None
    for i, (g, e, c, a) in enumerate(segs):
        gi, ei = _dtype_code(g), _dtype_code(e)
        gd = gi if gd is None else gd
        ed = ei if ed is None else ed
        if gi != gd or ei != ed:
            raise TypeError("all segments must share grad and err dtypes")
        n = g.numel()
        if e.numel() != n:
            raise ValueError(f"segment {i}: err has {e.numel()} elements, grad {n}")
        if n > 0 and bits in _BITS:
            _need(c, code_bytes(n, bits), f"segment {i}: codes")
            if not fixed and block in _BLOCKS:
                _need(a, 4 * num_blocks(n, block), f"segment {i}: absmax")
        arr[i] = CqSegment(_ptr(g, dev), _ptr(e, dev), _ptr(c, dev), _ptr(a, dev), n)
    return arr, len(segs), gd, ed


def _payloads(peers, dev, n, bits, block, fixed):
    ps = list(peers)
    arr = (Payload * max(1, len(ps)))()
    for i, (c, a) in enumerate(ps):
        if n > 0 and bits in _BITS:
            _need(c, code_bytes(n, bits), f"peer {i}: codes")
            if not fixed and block in _BLOCKS:
                _need(a, 4 * num_blocks(n, block), f"peer {i}: absmax")
        arr[i] = Payload(_ptr(c, dev), _ptr(a, dev))
    return arr, ps


def loco_compensate_quantize(segments, *, bits: int, block: int, beta: float, fixed_scale: float = 0.0,
                             stream=None, grad_dtype=None, err_dtype=None) -> None:
    """segments: iterable of (grad, err, codes, absmax) tensors; absmax may be None in
    fixed-scale mode.  n of a segment is grad.numel()."""
    dev = _device()
    arr, nseg, gd, ed = _segments(segments, dev, bits, block, fixed_scale > 0)
    gd = gd if grad_dtype is None else grad_dtype
    ed = ed if err_dtype is None else err_dtype
    st = load().loco_compensate_quantize(arr, nseg, LOCO_F32 if gd is None else gd,
                                         LOCO_F32 if ed is None else ed, bits, block, beta,
                                         fixed_scale, _stream(stream, dev))
    _check("loco_compensate_quantize", st)


def loco_compensate_quantize_ex(segments, *, bits: int, block: int, beta: float, fixed_scale: float = 0.0,
                                err_scale: float = 0.0, reset_error: bool = False, stream=None,
                                grad_dtype=None, err_dtype=None) -> None:
    """As loco_compensate_quantize; an int8 err tensor holds the 8-bit error of scale
    err_scale, and reset_error stores a zero error this step."""
    dev = _device()
    arr, nseg, gd, ed = _segments(segments, dev, bits, block, fixed_scale > 0)
    gd = gd if grad_dtype is None else grad_dtype
    ed = ed if err_dtype is None else err_dtype
    opt = CqOptions(bits, block, beta, fixed_scale, err_scale, 1 if reset_error else 0)
    st = load().loco_compensate_quantize_ex(arr, nseg, LOCO_F32 if gd is None else gd,
                                            LOCO_F32 if ed is None else ed, ctypes.byref(opt),
                                            _stream(stream, dev))
    _check("loco_compensate_quantize_ex", st)


def loco_dequant_reduce(peers, n: int, *, bits: int, block: int, out, out_scale: float,
                        fixed_scale: float = 0.0, stream=None) -> None:
    """peers: iterable of (codes, absmax) tensors (absmax None in fixed-scale mode)."""
    dev = _device()
    arr, ps = _payloads(peers, dev, n, bits, block, fixed_scale > 0)
    if out is not None:
        _need(out, n * out.element_size(), "out")
    st = load().loco_dequant_reduce(arr if ps else None, len(ps), n, bits, block, fixed_scale, out_scale,
                                    _ptr(out, dev), _dtype_code(out), _stream(stream, dev))
    _check("loco_dequant_reduce", st)


def loco_dequant_reduce_adam(peers, n: int, *, bits: int, block: int, out_scale: float, param, m, v,
                             lr: float, beta1: float, beta2: float, delta: float, param_bf16=None,
                             fixed_scale: float = 0.0, stream=None) -> None:
    """peers as loco_dequant_reduce; param, m, v float32 tensors of n elements, updated in
    place; param_bf16 an optional bfloat16 tensor that receives the new param."""
    for t in (param, m, v):
        if t.dtype != torch.float32:
            raise TypeError("param, m and v must be float32")
    if param_bf16 is not None and param_bf16.dtype != torch.bfloat16:
        raise TypeError("param_bf16 must be bfloat16")
    dev = _device()
    arr, ps = _payloads(peers, dev, n, bits, block, fixed_scale > 0)
    for t, what in ((param, "param"), (m, "m"), (v, "v")):
        _need(t, 4 * n, what)
    _need(param_bf16, 2 * n, "param_bf16")
    hp = AdamParams(lr, beta1, beta2, delta)
    st = load().loco_dequant_reduce_adam(arr if ps else None, len(ps), n, bits, block, fixed_scale, out_scale,
                                         ctypes.byref(hp), _ptr(param, dev), _ptr(m, dev), _ptr(v, dev),
                                         _ptr(param_bf16, dev), _stream(stream, dev))
    _check("loco_dequant_reduce_adam", st)


def loco_topk_quantize(grad, err, *, chunk: int, k: int, idx, codes, absmax, bits: int = 2,
                       ef_decay: float = 1.0, stream=None) -> None:
    if grad.dtype != torch.float32 or err.dtype != torch.float32:
        raise TypeError("grad and err must be float32")
    dev = _device()
    n = grad.numel()
    if err.numel() != n:
        raise ValueError(f"err has {err.numel()} elements, grad {n}")
    if n > 0 and chunk in _CHUNKS and 1 <= k <= chunk and bits in _BITS:
        chunks = num_blocks(n, chunk)
        _need(idx, 2 * chunks * k, "idx")
        _need(codes, chunks * code_bytes(k, bits), "codes")
        _need(absmax, 4 * chunks, "absmax")
    st = load().loco_topk_quantize(_ptr(grad, dev), _ptr(err, dev), grad.numel(), chunk, k, bits, ef_decay,
                                   _ptr(idx, dev), _ptr(codes, dev), _ptr(absmax, dev), _stream(stream, dev))
    _check("loco_topk_quantize", st)


def loco_sparse_aggregate(peers, n: int, *, chunk: int, k: int, out, out_scale: float, bits: int = 2,
                          stream=None) -> None:
    """peers: iterable of (idx int16/uint16, codes uint8, absmax float32) tensors, as
    loco_topk_quantize writes them."""
    dev = _device()
    ps = list(peers)
    arr = (SparsePayload * max(1, len(ps)))()
    check = n > 0 and chunk in _CHUNKS and 1 <= k <= chunk and bits in _BITS
    chunks = num_blocks(n, chunk) if check else 0
    for i, (ix, c, a) in enumerate(ps):
        if check:
            _need(ix, 2 * chunks * k, f"peer {i}: idx")
            _need(c, chunks * code_bytes(k, bits), f"peer {i}: codes")
            _need(a, 4 * chunks, f"peer {i}: absmax")
        arr[i] = SparsePayload(_ptr(ix, dev), _ptr(c, dev), _ptr(a, dev))
    if check and out is not None:
        _need(out, n * out.element_size(), "out")
    st = load().loco_sparse_aggregate(arr if ps else None, len(ps), n, chunk, k, bits, out_scale, _ptr(out, dev),
                                      _dtype_code(out), _stream(stream, dev))
    _check("loco_sparse_aggregate", st)


# short names
compensate_quantize = loco_compensate_quantize
compensate_quantize_ex = loco_compensate_quantize_ex
dequant_reduce = loco_dequant_reduce
dequant_reduce_adam = loco_dequant_reduce_adam
topk_quantize = loco_topk_quantize
sparse_aggregate = loco_sparse_aggregate
