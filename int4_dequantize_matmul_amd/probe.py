"""Python binding of libq4_probe (``include/q4_probe.h``): the ceilings the
benchmark measures libq4's kernels against.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

from . import OK, Q4Error, _ptr, _stream

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libq4_probe.so")
_P, _I = ctypes.c_void_p, ctypes.c_int64
_SIG = {
    "q4_probe_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _I, _I, _P]),
    "q4_probe_mfma_i8": (ctypes.c_int, [_P, _I, _I, _P]),
}
EXPORTS = tuple(_SIG)
_LIB = None


def raw():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m int4_dequantize_matmul_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _LIB = lib
    return _LIB


def q4_probe_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int, threads: int, nbytes: int | None = None):
    """Stream nbytes (default: all) of buf once; sink is a uint32 tensor of >= blocks."""
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    st = raw().q4_probe_read(_ptr(buf), n, _ptr(sink), blocks, threads, _stream(buf))
    if st != OK:
        raise Q4Error("q4_probe_read", st)


def q4_probe_mfma_i8(out: torch.Tensor, blocks: int, iters: int):
    """out: uint64-sized tensor of >= 8 * blocks elements (per wave: cycles, 100 MHz ticks)."""
    st = raw().q4_probe_mfma_i8(_ptr(out), blocks, iters, _stream(out))
    if st != OK:
        raise Q4Error("q4_probe_mfma_i8", st)
