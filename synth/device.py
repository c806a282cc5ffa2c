"""Device side of the synthetic-input generator: fills torch GPU tensors with
the same streams as the host functions in ``synth`` (bit for bit)."""
from __future__ import annotations

import ctypes
import os

import torch

from . import (KIND_BYTES, KIND_FP8_CODES, KIND_INT_BF16, KIND_NORMAL_BF16, KIND_NORMAL_F32,
               KIND_POS_SCALE, KIND_POW2_E4M3)

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcskv_synth.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: run `python synth/build.py`")
_lib = ctypes.CDLL(_LIB_PATH)
_lib.synth_fill.restype = ctypes.c_int
_lib.synth_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int,
                            ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]

_ELEM = {KIND_NORMAL_F32: torch.float32, KIND_POS_SCALE: torch.float32, KIND_NORMAL_BF16: torch.bfloat16,
         KIND_INT_BF16: torch.bfloat16, KIND_BYTES: torch.uint8, KIND_POW2_E4M3: torch.uint8,
         KIND_FP8_CODES: torch.uint8}


def fill(t: torch.Tensor, kind: int, key: int, offset: int = 0, a: int = 0, emin: int = 0, emax: int = 0) -> torch.Tensor:
    """Overwrites the contiguous GPU tensor t with elements offset.. of a stream."""
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("fill needs a contiguous GPU tensor")
    if t.element_size() != torch.tensor([], dtype=_ELEM[kind]).element_size():
        raise TypeError(f"kind {kind} writes {_ELEM[kind]} elements, tensor is {t.dtype}")
    rc = _lib.synth_fill(kind, key, offset, t.numel(), a, emin, emax, ctypes.c_void_p(t.data_ptr()),
                         ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill failed ({rc})")
    return t


def new(shape, kind: int, key: int, device="cuda", offset: int = 0, a: int = 0, emin: int = 0, emax: int = 0) -> torch.Tensor:
    t = torch.empty(shape, dtype=_ELEM[kind], device=device)
    return fill(t, kind, key, offset, a, emin, emax)
