"""MI355X (gfx950) implementation of LoCo's per-GPU gradient path.

The work happens in hand-written HIP kernels behind the C ABI declared in
include/loco.h (libloco.so); `loco` is its thin Python binding.
"""
from . import loco  # noqa: F401
from .loco import (loco_compensate_quantize, loco_dequant_reduce, loco_topk_quantize,  # noqa: F401
                   loco_status_string, LocoError)

__all__ = ["loco", "loco_compensate_quantize", "loco_dequant_reduce", "loco_topk_quantize",
           "loco_status_string", "LocoError"]
