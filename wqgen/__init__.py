"""Seeded synthetic inputs shared by the oracle side and the GPU side.

Counter-based SplitMix64 + Box–Muller (see ``wqgen.c``).  This module draws
f32 values and raw random bytes only: it never rounds to f16, never quantises
and never multiplies, so it holds none of the matmul's arithmetic.

Stream convention: activations A come from stream 0 and weights B from
stream 1 of the same seed, so a workload is fixed by (seed, shapes).  Q4_0
weight bytes (no Q4_0 encoder is on the pages) come straight from stream 2 as
random codes and scale bit patterns.  Residual-stream values (the C that a
residual epilogue adds into) come from stream 3.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wqgen.c")
_LIB = os.path.join(_HERE, "libwqgen.so")

STREAM_A = 0
STREAM_B = 1
STREAM_Q4 = 2
STREAM_R = 3
WEIGHT_STD = 0.02  # B ~ N(0, 0.02): 0.02 is the standard deviation


def build() -> str:
    """Compile ``libwqgen.so`` with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-std=c11", "-Wall",
         "-Wextra", "-o", tmp, _SRC, "-lm"],
        check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.wqgen_normal_f32.restype = ctypes.c_int
        lib.wqgen_normal_f32.argtypes = [
            ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
            ctypes.c_uint64, ctypes.c_double, ctypes.c_double, ctypes.c_int]
        lib.wqgen_u64.restype = ctypes.c_uint64
        lib.wqgen_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.wqgen_stream_key.restype = ctypes.c_uint64
        lib.wqgen_stream_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.wqgen_u64_fill.restype = ctypes.c_int
        lib.wqgen_u64_fill.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.c_uint64]
        lib.wqgen_normal_at.restype = ctypes.c_double
        lib.wqgen_normal_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(shape, seed: int = 0, stream: int = 0, mean: float = 0.0,
           std: float = 1.0, offset: int = 0) -> np.ndarray:
    """float32 array of the given shape: elements offset.. of stream (seed, stream)."""
    shape = tuple(int(s) for s in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    count = int(np.prod(shape, dtype=np.int64)) if shape else 1
    out = np.empty(shape, dtype=np.float32)
    if count:
        rc = _load().wqgen_normal_f32(out.ctypes.data, count, seed, stream, offset,
                                      float(mean), float(std), _threads())
        if rc != 0:
            raise RuntimeError("wqgen_normal_f32 failed")
    return out


def activations(m: int, k: int, seed: int = 0) -> np.ndarray:
    """A ~ N(0, 1), float32 [m, k], row-major; row i is the same for every m > i."""
    return normal((m, k), seed=seed, stream=STREAM_A)


def residual(m: int, n: int, seed: int = 0) -> np.ndarray:
    """Residual stream R ~ N(0, 1), float32 [m, n]."""
    return normal((m, n), seed=seed, stream=STREAM_R)


def weights(n: int, k: int, seed: int = 0, std: float = WEIGHT_STD) -> np.ndarray:
    """B ~ N(0, std^2) as float32 [n, k] (before any f16 cast or Q8_0 quantisation)."""
    return normal((n, k), seed=seed, stream=STREAM_B, std=std)


def weight_rows(rows, k: int, seed: int = 0, std: float = WEIGHT_STD) -> np.ndarray:
    """Selected rows of ``weights(n, k)`` without drawing the others."""
    rows = [int(r) for r in rows]
    out = np.empty((len(rows), k), dtype=np.float32)
    for i, r in enumerate(rows):
        out[i] = normal((k,), seed=seed, stream=STREAM_B, std=std, offset=r * k)
    return out


def u64_array(count: int, seed: int = 0, stream: int = 0, offset: int = 0) -> np.ndarray:
    """uint64 [count]: raw outputs offset .. offset+count-1 of stream (seed, stream)."""
    out = np.empty(int(count), dtype=np.uint64)
    if count and _load().wqgen_u64_fill(out.ctypes.data, int(count), seed, stream, offset) != 0:
        raise RuntimeError("wqgen_u64_fill failed")
    return out


Q4_BLOCK_BYTES = 18


def q4_0_bytes(n: int, k: int, seed: int = 0, row0: int = 0) -> np.ndarray:
    """Synthetic Q4_0 weight bytes, uint8 [n, k/32*18] (k % 32 == 0), for rows
    row0 .. row0+n-1 of the matrix drawn with this seed.

    Block b (row-major over rows and blocks) uses outputs 3b, 3b+1, 3b+2 of
    stream 2: the first two give the 16 code bytes (two uniform 4-bit codes per
    byte, in little-endian byte order), the third the scale's bit pattern:
    0x1C00 | (u & 0x3FF) with the sign bit set from bit 10 of u, i.e. scales of
    either sign with magnitude in [2^-8, 2^-7) -- the size a Q4_0 scale of
    N(0, 0.02) weights has (largest |w| about 0.06 over 8 steps)."""
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    nb = k // 32
    u = u64_array(3 * n * nb, seed, STREAM_Q4, 3 * row0 * nb).reshape(n * nb, 3)
    out = np.empty((n * nb, Q4_BLOCK_BYTES), dtype=np.uint8)
    scale = (np.uint64(0x1C00) | (u[:, 2] & np.uint64(0x3FF)) |
             (((u[:, 2] >> np.uint64(10)) & np.uint64(1)) << np.uint64(15))).astype("<u2")
    out[:, 0:2] = scale.view(np.uint8).reshape(-1, 2)
    out[:, 2:18] = np.ascontiguousarray(u[:, 0:2]).astype("<u8").view(np.uint8).reshape(-1, 16)
    return out.reshape(n, nb * Q4_BLOCK_BYTES)


def raw_u64(seed: int, stream: int, i: int) -> int:
    """The i-th raw SplitMix64 output of stream (seed, stream)."""
    lib = _load()
    return int(lib.wqgen_u64(lib.wqgen_stream_key(seed, stream), i))
