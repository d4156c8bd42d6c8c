"""Seeded synthetic inputs shared by the HIP library's tests/bench and the oracle.

This package holds no attention arithmetic.  It draws counter-based random
numbers (SplitMix64 + Box-Muller, defined in ``synth.c``), shapes them into the
tensors the HiLS-Attention forward pass takes, and plants "needle" keys.  Both
the GPU path and the float64 oracle receive exactly these host buffers.

bf16 tensors are returned as ``numpy.uint16`` arrays holding the raw bf16 bit
patterns; f32 tensors as ``numpy.float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

OUT_BF16, OUT_F32, OUT_F64 = 0, 1, 2

# Stream ids: one independent random stream per tensor role.
STREAM_Q, STREAM_K, STREAM_V, STREAM_QLM = 1, 2, 3, 4
STREAM_H, STREAM_WDOWN, STREAM_WUP = 5, 6, 7
STREAM_NEEDLE, STREAM_NEEDLE_DIR = 8, 9
STREAM_KSUM, STREAM_BSUM = 10, 11


def build(force: bool = False) -> str:
    """Compile libsynth.so with the host C compiler (no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, _SRC,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_int]
        lib.synth_normal.restype = None
        lib.synth_uniform.argtypes = lib.synth_normal.argtypes
        lib.synth_uniform.restype = None
        lib.synth_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_u64.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _alloc(shape, dtype: str):
    if dtype == "bf16":
        return np.empty(shape, dtype=np.uint16), OUT_BF16
    if dtype == "f32":
        return np.empty(shape, dtype=np.float32), OUT_F32
    if dtype == "f64":
        return np.empty(shape, dtype=np.float64), OUT_F64
    raise ValueError(dtype)


def normal(shape, seed: int, stream: int, std: float = 1.0, mean: float = 0.0,
           dtype: str = "bf16", nthreads: int | None = None) -> np.ndarray:
    out, t = _alloc(shape, dtype)
    _load().synth_normal(seed, stream, out.size, mean, std, t,
                         out.ctypes.data, nthreads or default_threads())
    return out


def uniform(shape, seed: int, stream: int, lo: float, hi: float, dtype: str = "f32",
            nthreads: int | None = None) -> np.ndarray:
    out, t = _alloc(shape, dtype)
    _load().synth_uniform(seed, stream, out.size, lo, hi, t,
                          out.ctypes.data, nthreads or default_threads())
    return out


def u64(seed: int, stream: int, index: int) -> int:
    return int(_load().synth_u64(seed, stream, index & 0xFFFFFFFFFFFFFFFF))


# ---------------------------------------------------------------------------
# bf16 <-> float conversions (storage plumbing, exact in the widening direction)
# ---------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = (u & 0x7F800000) == 0x7F800000
    if np.any(nan):
        r = np.where(nan, ((u >> 16) | np.where(u & 0xFFFF, 0x40, 0)).astype(np.uint16), r)
    return r


def as_f64(arr: np.ndarray) -> np.ndarray:
    """Exact float64 view of a bf16-bits / f32 / f64 array."""
    if arr.dtype == np.uint16:
        return bf16_to_f64(arr)
    return arr.astype(np.float64)


def store_like(ref: np.ndarray, x64: np.ndarray) -> np.ndarray:
    """Store float64 values in the storage type of ``ref`` (bf16 bits or f32)."""
    if ref.dtype == np.uint16:
        return f32_to_bf16(x64.astype(np.float32))
    return x64.astype(ref.dtype)


from .workloads import (Workload, WORKLOADS, prefill_inputs, decode_inputs,  # noqa: E402
                        synthetic_summaries)

__all__ = ["build", "normal", "uniform", "u64", "bf16_to_f32", "bf16_to_f64",
           "f32_to_bf16", "as_f64", "store_like", "Workload", "WORKLOADS",
           "prefill_inputs", "decode_inputs", "synthetic_summaries"]
