"""Helpers for the GPU parity tests: moving arrays, comparing results."""
from __future__ import annotations

import numpy as np
import torch

import oracle.errors as E

DEV = "cuda:0"


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    """numpy array -> contiguous tensor on the GPU (uint16 bits stay 16-bit)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
        t = t.view(torch.bfloat16) if dtype is None else t.view(dtype)
    else:
        t = torch.from_numpy(a)
    return t.to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def assert_bitwise(got: np.ndarray, want: np.ndarray, what: str = ""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype.kind == "f":
        g, w = got.view(np.uint32 if got.itemsize == 4 else np.uint16), want.astype(got.dtype).view(
            np.uint32 if got.itemsize == 4 else np.uint16)
    else:
        g, w = got, want
    bad = np.argwhere(g != w)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: " \
                          f"got {got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}"


def assert_close(got, y_ref, abs_terms, tol: float, what: str = ""):
    e = E.normwise(got, y_ref)
    c = E.conditioned(got, y_ref, abs_terms)
    assert e <= tol and c <= tol, f"{what}: normwise {e:.3g}, conditioned {c:.3g}, tol {tol}"
    return e, c
