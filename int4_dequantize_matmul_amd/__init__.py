"""Python binding of libq4, the fused packed-int4 linear for MI355X (gfx950).

Argument marshalling only: every function calls the C entry point of the same
name in ``lib/libq4.so`` (declared in ``include/q4.h``); all arithmetic runs
in that library's host code or HIP kernels.  torch provides device memory and
the current stream; outputs are allocated here with torch.

The library must be built first (``python -m int4_dequantize_matmul_amd.build``);
importing the compute functions without it raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # loaded before libq4 so both share torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
# Q4_LIB names another build of the same library (the mutation check of the
# test suite loads libraries with a planted mistake this way).
LIB_PATH = os.environ.get("Q4_LIB") or os.path.join(_PKG, "lib", "libq4.so")

OK, EINVAL, ESHAPE, EDEVICE, EMISMATCH = 0, 1, 2, 3, 4
ENC = {"twos": 0, "excess8": 1}
DT = {"f32": 0, "bf16": 1}
PATHS = {"auto": 0, "generic": 1, "gemv": 2, "tiled": 3, "gemv_mc": 4}
PATH_NAMES = {v: k for k, v in PATHS.items()}
OPS = {"w4a32": 0, "w4a16": 1, "w4a16_zp": 2, "w4a8": 3, "w4a8_zp": 4, "w8a8": 5}
W4A8_MAX_K = 1048576
W8A8_MAX_K = 131071
MULTI_MAX = 64
NOALLOC_SCRATCH_BYTES = 8388608


class Q4Error(RuntimeError):
    """A libq4 call returned a status other than Q4_OK."""

    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib().q4_status_string(status).decode()
        super().__init__(f"{fn}: status {status} ({msg})")


_LIB = None

_P = ctypes.c_void_p
_I = ctypes.c_int64
_SIG = {
    "q4_quantize_row": (ctypes.c_int, [_P, _I, _P, _P]),
    "q8_quantize_row": (ctypes.c_int, [_P, _I, _P, _P]),
    "q4_pack": (ctypes.c_int, [_P, _I, _I, ctypes.c_int, _P]),
    "q8_quantize_rows": (ctypes.c_int, [_P, ctypes.c_int, _I, _I, _P, _P, _P]),
    "q4_linear_w4a32": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _P]),
    "q4_linear_w4a16": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _P]),
    "q4_linear_w4a8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _P]),
    "q4_linear_w4a16_zp": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "q4_linear_w4a8_zp": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "q4_w4a8_dynamic_workspace": (ctypes.c_size_t, [_I, _I]),
    "q4_linear_w4a8_dynamic": (ctypes.c_int, [_P, ctypes.c_int, _P, _P, _P, _I, _I, _I, _I,
                                              ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "q4_linear_w4a8_dynamic_noalloc": (ctypes.c_int, [_P, ctypes.c_int, _P, _P, _P, _I, _I, _I, _I,
                                                      ctypes.c_int, _P]),
    "q4_linear_w4a8_dynamic_multi": (ctypes.c_int, [_P, _I, ctypes.c_int, _I, _P]),
    "q8_linear_w8a8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "q8_linear_w8a32": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _P]),
    "q8_linear_w8a16": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "q4_selftest_workspace": (ctypes.c_size_t, []),
    "q4_selftest": (ctypes.c_int, [_P, ctypes.c_size_t, _P]),
    "q4_selftest_report": (ctypes.c_char_p, []),
    "q4_set_path": (ctypes.c_int, [ctypes.c_int]),
    "q4_get_path": (ctypes.c_int, []),
    "q4_last_path": (ctypes.c_int, []),
    "q4_route_plan": (ctypes.c_int, [ctypes.c_int, _I, _I, _I, _I, ctypes.c_int32, _P]),
    "q4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}
EXPORTS = tuple(_SIG)


def _lib():
    """Load lib/libq4.so once and declare the signatures; raise if missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m int4_dequantize_matmul_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _LIB = lib
    return _LIB


def raw():
    """The ctypes handle itself, for tests that pass raw pointers."""
    return _lib()


def _check(fn: str, st: int):
    if st != OK:
        raise Q4Error(fn, st)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


_DUMMY = {}


def _ptr(t):
    """Address of a numpy array or tensor.  A zero-size tensor may have no
    storage; it is given the address of a small placeholder allocation on
    its device (a zero-byte range overlaps nothing and is never read)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return ctypes.c_void_p(t.ctypes.data)
    if t.numel() == 0:
        d = _DUMMY.get(t.device)
        if d is None:
            d = _DUMMY[t.device] = torch.empty(64, dtype=torch.uint8, device=t.device)
        return ctypes.c_void_p(d.data_ptr())
    return ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtypes, ndim: int):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")
    return t


_U16 = (torch.uint16, torch.int16, torch.float16, torch.bfloat16)


# ---------------------------------------------------------------------------
# host calls
# ---------------------------------------------------------------------------

def q4_quantize_row(w: np.ndarray):
    """One weight row (f32 [K]) -> (packed uint8 [ceil(K/2)], f32 scale)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K = w.shape[0]
    packed = np.empty((K + 1) // 2, np.uint8)
    s = np.zeros(1, np.float32)
    _check("q4_quantize_row", _lib().q4_quantize_row(_ptr(w), K, _ptr(packed), _ptr(s)))
    return packed, s[0]


def q4_quantize_matrix(W: np.ndarray):
    """Rows of W [N, K] through q4_quantize_row -> (packed [N, ceil(K/2)], scales [N])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    packed = np.empty((N, (K + 1) // 2), np.uint8)
    scales = np.empty(N, np.float32)
    f = _lib().q4_quantize_row
    base_w, base_p, base_s = W.ctypes.data, packed.ctypes.data, scales.ctypes.data
    kb = (K + 1) // 2
    for n in range(N):
        st = f(ctypes.c_void_p(base_w + 4 * n * K), K, ctypes.c_void_p(base_p + n * kb),
               ctypes.c_void_p(base_s + 4 * n))
        _check("q4_quantize_row", st)
    return packed, scales


def q8_quantize_row(x: np.ndarray):
    """One row (f32 [K]) -> (int8 [K], f32 scale)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.empty(x.shape[0], np.int8)
    s = np.zeros(1, np.float32)
    _check("q8_quantize_row", _lib().q8_quantize_row(_ptr(x), x.shape[0], _ptr(q), _ptr(s)))
    return q, s[0]


def q4_pack(codes: np.ndarray, enc: str = "excess8"):
    """int codes [N, K] in [-8, 7] -> packed uint8 [N, ceil(K/2)]."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    N, K = codes.shape
    out = np.empty((N, (K + 1) // 2), np.uint8)
    _check("q4_pack", _lib().q4_pack(_ptr(codes), N, K, ENC[enc], _ptr(out)))
    return out


# ---------------------------------------------------------------------------
# device calls (torch tensors on the GPU; results ready after a stream sync)
# ---------------------------------------------------------------------------

def q8_quantize_rows(x: torch.Tensor):
    """Activation rows (f32 or bf16 [M, K]) -> (int8 [M, K], f32 scales [M])."""
    _dev(x, "x", (torch.float32, torch.bfloat16), 2)
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    sx = torch.empty(M, dtype=torch.float32, device=x.device)
    if M == 0:
        return xq, sx
    dt = DT["bf16"] if x.dtype == torch.bfloat16 else DT["f32"]
    _check("q8_quantize_rows", _lib().q8_quantize_rows(_ptr(x), dt, M, K, _ptr(xq), _ptr(sx), _stream(x)))
    return xq, sx


def q4_linear_w4a32(x, wq, scales_f16, G: int, enc: str = "twos"):
    """f32 x [M, K], packed int4 wq [N, K/2], f16 scales [N, K/G] -> f32 y [M, N]."""
    _dev(x, "x", (torch.float32,), 2)
    _dev(wq, "wq", (torch.uint8,), 2)
    _dev(scales_f16, "scales_f16", _U16, 2)
    M, K = x.shape
    N = wq.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if M == 0 or N == 0:
        return y
    _check("q4_linear_w4a32", _lib().q4_linear_w4a32(_ptr(x), _ptr(wq), _ptr(scales_f16), _ptr(y),
                                                      M, N, K, G, ENC[enc], _stream(x)))
    return y


def q4_linear_w4a16(x, wq, scales_bf16, G: int, enc: str = "excess8", want_f32: bool = False):
    """bf16 x [M, K], packed int4 [N, K/2], bf16 scales [N, K/G] -> (bf16 y, f32 y or None)."""
    _dev(x, "x", _U16, 2)
    _dev(wq, "wq", (torch.uint8,), 2)
    _dev(scales_bf16, "scales_bf16", _U16, 2)
    M, K = x.shape
    N = wq.shape[0]
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    yf = torch.empty((M, N), dtype=torch.float32, device=x.device) if want_f32 else None
    if M == 0 or N == 0:
        return yb, yf
    _check("q4_linear_w4a16", _lib().q4_linear_w4a16(_ptr(x), _ptr(wq), _ptr(scales_bf16), _ptr(yb),
                                                      _ptr(yf), M, N, K, G, ENC[enc], _stream(x)))
    return yb, yf


def q4_linear_w4a8(xq, sx, wq, sw, G: int = 0, enc: str = "excess8", y=None):
    """int8 xq [M, K] + sx [M], packed int4 [N, ceil(K/2)], sw [N] or [N, K/G] -> f32 y [M, N]."""
    _dev(xq, "xq", (torch.int8,), 2)
    _dev(sx, "sx", (torch.float32,), 1)
    _dev(wq, "wq", (torch.uint8,), 2)
    _dev(sw, "sw", (torch.float32,), sw.dim())
    M, K = xq.shape
    N = wq.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    if M == 0 or N == 0:
        return y
    _check("q4_linear_w4a8", _lib().q4_linear_w4a8(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(y),
                                                    M, N, K, G, ENC[enc], _stream(xq)))
    return y


def q4_linear_w4a16_zp(x, wq, scales_bf16, zeros, G: int, want_f32: bool = False):
    """bf16 x [M, K], packed nibbles [N, K/2], bf16 scales and uint8 zero points
    [N, K/G] -> (bf16 y, f32 y or None); weight = s * (u - z)."""
    _dev(x, "x", _U16, 2)
    _dev(wq, "wq", (torch.uint8,), 2)
    _dev(scales_bf16, "scales_bf16", _U16, 2)
    _dev(zeros, "zeros", (torch.uint8,), 2)
    M, K = x.shape
    N = wq.shape[0]
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    yf = torch.empty((M, N), dtype=torch.float32, device=x.device) if want_f32 else None
    if M == 0 or N == 0:
        return yb, yf
    _check("q4_linear_w4a16_zp", _lib().q4_linear_w4a16_zp(_ptr(x), _ptr(wq), _ptr(scales_bf16), _ptr(zeros),
                                                            _ptr(yb), _ptr(yf), M, N, K, G, _stream(x)))
    return yb, yf


def q4_linear_w4a8_zp(xq, sx, wq, sw, zeros, G: int, y=None):
    """Grouped W4A8 with uint8 zero points [N, K/G] -> f32 y [M, N]."""
    _dev(xq, "xq", (torch.int8,), 2)
    _dev(sx, "sx", (torch.float32,), 1)
    _dev(wq, "wq", (torch.uint8,), 2)
    _dev(sw, "sw", (torch.float32,), sw.dim())
    _dev(zeros, "zeros", (torch.uint8,), 2)
    M, K = xq.shape
    N = wq.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    if M == 0 or N == 0:
        return y
    _check("q4_linear_w4a8_zp", _lib().q4_linear_w4a8_zp(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(zeros),
                                                          _ptr(y), M, N, K, G, _stream(xq)))
    return y


def q8_linear_w8a32(x, wq, sw):
    """f32 x [M, K], int8 weights [N, K], f32 row scales [N] -> f32 y [M, N]."""
    _dev(x, "x", (torch.float32,), 2)
    _dev(wq, "wq", (torch.int8,), 2)
    _dev(sw, "sw", (torch.float32,), 1)
    M, K = x.shape
    N = wq.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if M == 0 or N == 0:
        return y
    _check("q8_linear_w8a32", _lib().q8_linear_w8a32(_ptr(x), _ptr(wq), _ptr(sw), _ptr(y), M, N, K, _stream(x)))
    return y


def q8_linear_w8a16(x, wq, sw, want_f32: bool = False):
    """bf16 x [M, K], int8 weights [N, K], f32 row scales [N] -> (bf16 y, f32 y or None)."""
    _dev(x, "x", _U16, 2)
    _dev(wq, "wq", (torch.int8,), 2)
    _dev(sw, "sw", (torch.float32,), 1)
    M, K = x.shape
    N = wq.shape[0]
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    yf = torch.empty((M, N), dtype=torch.float32, device=x.device) if want_f32 else None
    if M == 0 or N == 0:
        return yb, yf
    _check("q8_linear_w8a16", _lib().q8_linear_w8a16(_ptr(x), _ptr(wq), _ptr(sw), _ptr(yb), _ptr(yf),
                                                      M, N, K, _stream(x)))
    return yb, yf


def q4_w4a8_dynamic_workspace(M: int, K: int) -> int:
    return int(_lib().q4_w4a8_dynamic_workspace(M, K))


def q4_linear_w4a8_dynamic(x, wq, sw, G: int = 0, enc: str = "excess8", ws=None, y=None):
    """f32/bf16 x [M, K] -> quantize rows into ws, then W4A8 -> f32 y [M, N]."""
    _dev(x, "x", (torch.float32, torch.bfloat16), 2)
    _dev(wq, "wq", (torch.uint8,), 2)
    M, K = x.shape
    N = wq.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if M == 0 or N == 0:
        return y
    need = q4_w4a8_dynamic_workspace(M, K)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    dt = DT["bf16"] if x.dtype == torch.bfloat16 else DT["f32"]
    _check("q4_linear_w4a8_dynamic",
           _lib().q4_linear_w4a8_dynamic(_ptr(x), dt, _ptr(wq), _ptr(sw), _ptr(y), M, N, K, G,
                                         ENC[enc], _ptr(ws), ws.numel() * ws.element_size(), _stream(x)))
    return y


def q4_linear_w4a8_dynamic_noalloc(x, wq, sw, G: int = 0, enc: str = "excess8", y=None):
    """As q4_linear_w4a8_dynamic, with the activation codes in the library's
    own per-device scratch array (no workspace; the C call allocates
    nothing).  Pass y to keep this wrapper from allocating the output."""
    _dev(x, "x", (torch.float32, torch.bfloat16), 2)
    _dev(wq, "wq", (torch.uint8,), 2)
    M, K = x.shape
    N = wq.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if M == 0 or N == 0:
        return y
    dt = DT["bf16"] if x.dtype == torch.bfloat16 else DT["f32"]
    _check("q4_linear_w4a8_dynamic_noalloc",
           _lib().q4_linear_w4a8_dynamic_noalloc(_ptr(x), dt, _ptr(wq), _ptr(sw), _ptr(y), M, N, K, G,
                                                 ENC[enc], _stream(x)))
    return y


class W4A8Problem(ctypes.Structure):
    """q4_w4a8_problem: one linear of q4_linear_w4a8_dynamic_multi."""
    _fields_ = [("x", _P), ("wq", _P), ("sw", _P), ("y", _P), ("N", _I), ("K", _I)]


def w4a8_problems(items):
    """(x, wq, sw, y) tensor tuples -> a ctypes array of q4_w4a8_problem
    (the tensors must outlive every call that uses the array)."""
    arr = (W4A8Problem * max(len(items), 1))()
    for i, (x, wq, sw, y) in enumerate(items):
        arr[i] = W4A8Problem(_ptr(x).value, _ptr(wq).value, _ptr(sw).value, _ptr(y).value,
                             wq.shape[0], x.shape[1])
    return arr


def q4_linear_w4a8_dynamic_multi(problems, ys=None):
    """Independent per-channel W4A8 linears in one launch.  problems: a
    sequence of (x [M, K_i] f32/bf16, wq [N_i, ceil(K_i/2)] uint8 excess-8,
    sw [N_i] f32), all with the same M and x dtype.  Returns the f32 outputs
    [M, N_i] (or fills ys)."""
    if not problems:
        return []
    x0 = problems[0][0]
    _dev(x0, "x", (torch.float32, torch.bfloat16), 2)
    M = x0.shape[0]
    items = []
    for i, (x, wq, sw) in enumerate(problems):
        _dev(x, f"x[{i}]", (x0.dtype,), 2)
        _dev(wq, f"wq[{i}]", (torch.uint8,), 2)
        _dev(sw, f"sw[{i}]", (torch.float32,), 1)
        if x.shape[0] != M:
            raise ValueError("every problem must have the same number of rows M")
        y = ys[i] if ys is not None else torch.empty((M, wq.shape[0]), dtype=torch.float32, device=x.device)
        items.append((x, wq, sw, y))
    out = [it[3] for it in items]
    if M == 0:
        return out
    dt = DT["bf16"] if x0.dtype == torch.bfloat16 else DT["f32"]
    arr = w4a8_problems(items)
    _check("q4_linear_w4a8_dynamic_multi",
           _lib().q4_linear_w4a8_dynamic_multi(arr, len(items), dt, M, _stream(x0)))
    return out


def q8_linear_w8a8(xq, sx, wq, sw, y=None):
    """int8 xq [M, K] + sx [M], int8 wq [N, K] + sw [N] -> f32 y [M, N]."""
    _dev(xq, "xq", (torch.int8,), 2)
    _dev(wq, "wq", (torch.int8,), 2)
    M, K = xq.shape
    N = wq.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    if M == 0 or N == 0:
        return y
    _check("q8_linear_w8a8", _lib().q8_linear_w8a8(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(y),
                                                    M, N, K, _stream(xq)))
    return y


def q4_selftest(device="cuda:0") -> str:
    """Run the all-extreme route checks on `device`; returns the report,
    raises Q4Error (with the report) if a check fails."""
    lib = _lib()
    ws = torch.empty(int(lib.q4_selftest_workspace()), dtype=torch.uint8, device=device)
    st = lib.q4_selftest(_ptr(ws), ws.numel(), _stream(ws))
    report = lib.q4_selftest_report().decode()
    if st != OK:
        raise Q4Error(f"q4_selftest ({report})", st)
    return report


def q4_set_path(path: str):
    _check("q4_set_path", _lib().q4_set_path(PATHS[path]))


def q4_get_path() -> str:
    return PATH_NAMES[_lib().q4_get_path()]


def q4_last_path() -> str:
    return PATH_NAMES[_lib().q4_last_path()]


class RoutePlan(ctypes.Structure):
    """q4_plan: the route of one call shape, and the tiled work split."""
    _fields_ = [("path", ctypes.c_int), ("decode_max", ctypes.c_int32), ("whole_tiles", ctypes.c_int32),
                ("piece_rows", ctypes.c_int32), ("pieces", ctypes.c_int32)]


def q4_route_plan(op: str, M: int, N: int, K: int, G: int = 0, cus: int = 0) -> dict:
    """The route a call of this shape takes under the current route setting
    (host only; cus = 0 asks the current device for its compute units)."""
    plan = RoutePlan()
    _check("q4_route_plan", _lib().q4_route_plan(OPS[op], M, N, K, G, cus, ctypes.byref(plan)))
    return {"path": PATH_NAMES[plan.path], "decode_max": plan.decode_max, "whole_tiles": plan.whole_tiles,
            "piece_rows": plan.piece_rows, "pieces": plan.pieces}


def q4_status_string(st: int) -> str:
    return _lib().q4_status_string(st).decode()
