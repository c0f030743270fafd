"""CPU oracle for C[M,N] = A[M,K] · B[N,K]^T with f16, Q8_0 or Q4_0 weights,
and for the residual and SwiGLU epilogues on that product.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library (``gemm_wq_gemv_amd``) never imports it and shares no code with it.

The arithmetic lives in ``wqref.c`` (plain C, f64 accumulation, built with
``-O2 -fno-fast-math -ffp-contract=off``); this module only marshals numpy
arrays.  Every function cites the passage it follows in ``wqref.c``.

Parity status of each function (what pins it, see ``tests/test_oracle.py``):
  f16_value      exhaustive over all 65536 patterns against ``struct '<e'``
  f16_bits       against numpy's float16 cast on every exponent/rounding case
  q8_0_quantize  hand-derived golden blocks, round-trip bounds, tie rounding
  decode         hand-built blocks, one-hot / identity products
  matmul         exact rational brute force, identity, one-hot, linearity,
                 permutation, numpy float64 matmul on the decoded weights
  silu           closed forms: silu(0) = 0, silu(ln 3) = (3/4) ln 3,
                 silu(x) - silu(-x) = x, limits at +-inf, sign
  decode_attention  L = 1 gives v of the mapped KV head exactly; equal keys or
                 scale 0 give the mean of v; a dominant key gives its v (also
                 at scores of 1e4, which overflow without the max shift); numpy
                 float64 softmax attention; joint token permutation; L = 0
  topk           numpy lexsort on random and tie-heavy logits, hand cases with
                 ties, NaN, +-inf, k > n (sentinel padding)
  matmul_epilogue  residual: exact hand sums on the worked example, linearity;
                 SwiGLU: hand-derived values (gate ln 3 / 0 / +-40), which half
                 is gate, the identity out(g) - out(-g) = g * u
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wqref.c")
_LIB = os.path.join(_HERE, "libwqref.so")

FMT_F16 = 0
FMT_Q8_0 = 1
FMT_Q4_0 = 2
EPI_NONE = 0
EPI_RESIDUAL = 1
EPI_SWIGLU = 2
KV_F32 = 0
KV_F16 = 1
QK = 32
BLOCK_BYTES = 34

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
          "-pthread", "-std=c11", "-Wall", "-Wextra"]


def build(out: str | None = None, defines: tuple = ()) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    out = out or _LIB
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, *[f"-D{d}" for d in defines], "-o", tmp, _SRC, "-lm"],
                   check=True)
    os.replace(tmp, out)
    return out


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class Oracle:
    """ctypes view of one build of ``wqref.c``."""

    def __init__(self, path: str = _LIB):
        if not os.path.exists(path):
            if path != _LIB:
                raise FileNotFoundError(path)
            build()
        lib = ctypes.CDLL(path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.wqref_f16_value.restype = ctypes.c_double
        lib.wqref_f16_value.argtypes = [ctypes.c_uint16]
        lib.wqref_f16_bits.restype = ctypes.c_uint16
        lib.wqref_f16_bits.argtypes = [ctypes.c_float]
        lib.wqref_f16_bits_array.restype = None
        lib.wqref_f16_bits_array.argtypes = [P, P, I64]
        lib.wqref_f16_value_array.restype = None
        lib.wqref_f16_value_array.argtypes = [P, P, I64]
        lib.wqref_q8_0_quantize.restype = I
        lib.wqref_q8_0_quantize.argtypes = [P, P, I64]
        lib.wqref_decode.restype = I
        lib.wqref_decode.argtypes = [P, I, I64, I64, P]
        lib.wqref_matmul.restype = I
        lib.wqref_matmul.argtypes = [P, P, I, I64, I64, I64, P, P, I]
        lib.wqref_matmul_entries.restype = I
        lib.wqref_matmul_entries.argtypes = [P, P, I, I64, I64, I64, P, P, I64, P, P, I]
        lib.wqref_silu.restype = ctypes.c_double
        lib.wqref_silu.argtypes = [ctypes.c_double]
        lib.wqref_silu_array.restype = None
        lib.wqref_silu_array.argtypes = [P, P, I64]
        lib.wqref_epilogue.restype = I
        lib.wqref_epilogue.argtypes = [I, P, P, I64, I64, P, P, P]
        lib.wqref_topk.restype = I
        lib.wqref_topk.argtypes = [P, I64, I64, P, P]
        lib.wqref_decode_attention.restype = I
        lib.wqref_decode_attention.argtypes = [P, P, P, I, I64, I64, I64, I64, ctypes.c_float, P, P]
        self.lib = lib
        self.path = path

    # -- f16 (f32_to_f16 / f16_to_f32, lattice-inference 0.1.2 page) --------
    def f16_bits(self, x) -> np.ndarray:
        """float32 -> binary16 bit patterns, round to nearest even."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.wqref_f16_bits_array(x.ctypes.data, out.ctypes.data, x.size)
        return out

    def f16_value(self, bits) -> np.ndarray:
        """binary16 bit patterns -> exact float64 values."""
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self.lib.wqref_f16_value_array(bits.ctypes.data, out.ctypes.data, bits.size)
        return out

    # -- Q8_0 (quantize_row_q8_0, lattice-inference 0.1.2 page) --------------
    def q8_0_quantize(self, w) -> np.ndarray:
        """float32 [..., K] (K % 32 == 0) -> uint8 [..., K/32*34] Q8_0 bytes."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        k = w.shape[-1]
        if k % QK:
            raise ValueError("last dimension must be a multiple of 32")
        out = np.empty(w.shape[:-1] + (k // QK * BLOCK_BYTES,), dtype=np.uint8)
        if self.lib.wqref_q8_0_quantize(w.ctypes.data, out.ctypes.data, w.size) != 0:
            raise ValueError("quantize failed")
        return out

    # -- decode and product (dispatch_matmul_half / gemm_q8 statements) -----
    def decode(self, b, fmt: int, n: int, k: int) -> np.ndarray:
        """Exact weights [n, k] (float64) of an f16, Q8_0 or Q4_0 matrix."""
        b = np.ascontiguousarray(b)
        out = np.empty((n, k), dtype=np.float64)
        if self.lib.wqref_decode(b.ctypes.data, fmt, n, k, out.ctypes.data) != 0:
            raise ValueError("decode: bad arguments")
        return out

    def encode(self, w, fmt: int) -> np.ndarray:
        """Weight bytes of float32 w [n, k] in the given format, by the oracle's own encoders."""
        if fmt == FMT_F16:
            return self.f16_bits(w)
        if fmt == FMT_Q8_0:
            return self.q8_0_quantize(w)
        raise ValueError(f"unknown format {fmt}")

    def matmul(self, a, b, fmt: int, m: int, n: int, k: int, threads: int | None = None):
        """(C, bound): C[m,n] = sum_k a[m,k] w[n,k] in float64 and the per-element
        tolerance 1e-5 * sum_k |a[m,k] w[n,k]| + 1e-6."""
        a = np.ascontiguousarray(a, dtype=np.float32)
        b = np.ascontiguousarray(b)
        if a.size < m * k:
            raise ValueError("a too small")
        c = np.empty((m, n), dtype=np.float64)
        bound = np.empty((m, n), dtype=np.float64)
        rc = self.lib.wqref_matmul(a.ctypes.data, b.ctypes.data, fmt, m, n, k, c.ctypes.data,
                                   bound.ctypes.data, threads or _threads())
        if rc != 0:
            raise ValueError("matmul: bad arguments")
        return c, bound

    def matmul_entries(self, a, b, fmt: int, m: int, n: int, k: int, rows, cols,
                       threads: int | None = None):
        """(c, bound) for the selected outputs (rows[i], cols[i]) only."""
        a = np.ascontiguousarray(a, dtype=np.float32)
        b = np.ascontiguousarray(b)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape:
            raise ValueError("rows/cols shape mismatch")
        c = np.empty(rows.shape, dtype=np.float64)
        bound = np.empty(rows.shape, dtype=np.float64)
        rc = self.lib.wqref_matmul_entries(a.ctypes.data, b.ctypes.data, fmt, m, n, k,
                                           rows.ctypes.data, cols.ctypes.data, rows.size,
                                           c.ctypes.data, bound.ctypes.data,
                                           threads or _threads())
        if rc != 0:
            raise ValueError("matmul_entries: bad arguments")
        return c, bound

    # -- epilogues (silu_mul / residual GEMM statements, see wqref.c) ---------
    def silu(self, x) -> np.ndarray:
        """silu(x) = x / (1 + exp(-x)) in float64."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.float64)
        self.lib.wqref_silu_array(x.ctypes.data, out.ctypes.data, x.size)
        return out

    def epilogue(self, epi: int, acc, acc_bound, m: int, n: int, resid=None):
        """(out, bound) of epilogue epi (1 residual, 2 SwiGLU) on product sums
        acc [m, n] (residual) or [m, 2n] (SwiGLU: gate sums, then up sums)."""
        acc = np.ascontiguousarray(acc, dtype=np.float64)
        acc_bound = np.ascontiguousarray(acc_bound, dtype=np.float64)
        if acc.size != (2 if epi == EPI_SWIGLU else 1) * m * n or acc_bound.size != acc.size:
            raise ValueError("epilogue: acc has the wrong size")
        r = None
        if epi == EPI_RESIDUAL:
            r = np.ascontiguousarray(resid, dtype=np.float32)
            if r.size != m * n:
                raise ValueError("epilogue: residual has the wrong size")
        out = np.empty((m, n), dtype=np.float64)
        bound = np.empty((m, n), dtype=np.float64)
        rc = self.lib.wqref_epilogue(epi, acc.ctypes.data, acc_bound.ctypes.data, m, n,
                                     None if r is None else r.ctypes.data,
                                     out.ctypes.data, bound.ctypes.data)
        if rc != 0:
            raise ValueError("epilogue: bad arguments")
        return out, bound

    def matmul_epilogue(self, a, b, fmt: int, m: int, n: int, k: int, epi: int, resid=None,
                        threads: int | None = None):
        """(out, bound) of the product with an epilogue: EPI_NONE as matmul;
        EPI_RESIDUAL resid + A.B^T (resid f32 [m, n]); EPI_SWIGLU with b holding
        2n rows (gate rows, then up rows) and out = silu(A.gate^T) * (A.up^T)."""
        if epi == EPI_NONE:
            return self.matmul(a, b, fmt, m, n, k, threads)
        rows = 2 * n if epi == EPI_SWIGLU else n
        acc, bnd = self.matmul(a, b, fmt, m, rows, k, threads)
        return self.epilogue(epi, acc, bnd, m, n, resid)

    def epilogue_entries(self, a, b, fmt: int, m: int, n: int, k: int, epi: int, rows, cols,
                         resid=None, threads: int | None = None):
        """(out, bound) of the epilogue product at the entries (rows[i], cols[i]);
        resid, when given, is the full f32 [m, n] residual."""
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if epi == EPI_NONE:
            return self.matmul_entries(a, b, fmt, m, n, k, rows, cols, threads)
        if epi == EPI_RESIDUAL:
            s, bs = self.matmul_entries(a, b, fmt, m, n, k, rows, cols, threads)
            r = np.asarray(resid, dtype=np.float32).reshape(m, n)[rows, cols]
            out, bound = self.epilogue(EPI_RESIDUAL, s, bs, rows.size, 1, r)
            return out.reshape(-1), bound.reshape(-1)
        both_rows = np.stack([rows, rows], axis=1).reshape(-1)
        both_cols = np.stack([cols, cols + n], axis=1).reshape(-1)  # (gate, up) per entry
        s, bs = self.matmul_entries(a, b, fmt, m, 2 * n, k, both_rows, both_cols, threads)
        out, bound = self.epilogue(EPI_SWIGLU, s, bs, rows.size, 1)
        return out.reshape(-1), bound.reshape(-1)

    # -- top-k (TopKCandidate / topk_better, lattice-inference 0.1.2 page) ----
    def topk(self, logits, topk: int):
        """(vals float64 [topk], ids int64 [topk]): the topk best logits, higher first,
        equal logits by lower id, NaN left out, padded with (-inf, 4294967295)."""
        x = np.ascontiguousarray(logits, dtype=np.float64).reshape(-1)
        vals = np.empty(topk, dtype=np.float64)
        ids = np.empty(topk, dtype=np.int64)
        if self.lib.wqref_topk(x.ctypes.data, x.size, topk, vals.ctypes.data, ids.ctypes.data) != 0:
            raise ValueError("topk: bad arguments")
        return vals, ids

    def lm_head_topk(self, a, b, fmt: int, n: int, k: int, topk: int, threads: int | None = None):
        """The LM-head product for one token, logits[j] = sum_k a[k] w[j, k], then
        its top-k: (vals, ids, logits, bound) with the full float64 logits and their
        per-row tolerance 1e-5 * sum_k |a_k w_jk| + 1e-6."""
        logits, bound = self.matmul(np.asarray(a, np.float32).reshape(1, -1), b, fmt, 1, n, k, threads)
        vals, ids = self.topk(logits[0], topk)
        return vals, ids, logits[0], bound[0]

    # -- decode attention (decode_attention / flash partial + reduce, engine page)
    def decode_attention(self, q, k, v, kvfmt: int, L: int, D: int, Hq: int, Hkv: int, scale: float):
        """(out, bound), float64 [Hq, D]: one query token's grouped-query attention over
        an L-token K/V cache [L, Hkv*D] (kvfmt 0 f32, 1 f16 bits); head h reads KV head
        h // (Hq // Hkv)."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        dt = np.float32 if kvfmt == KV_F32 else np.uint16
        k = np.ascontiguousarray(k, dtype=dt)
        v = np.ascontiguousarray(v, dtype=dt)
        if q.size < Hq * D or k.size < L * Hkv * D or v.size < L * Hkv * D:
            raise ValueError("decode_attention: input too small")
        out = np.empty((Hq, D), dtype=np.float64)
        bound = np.empty((Hq, D), dtype=np.float64)
        rc = self.lib.wqref_decode_attention(q.ctypes.data, k.ctypes.data, v.ctypes.data, kvfmt, L, D, Hq, Hkv,
                                             scale, out.ctypes.data, bound.ctypes.data)
        if rc != 0:
            raise ValueError("decode_attention: bad arguments")
        return out, bound


_default: Oracle | None = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def f16_bits(x):
    return get().f16_bits(x)


def f16_value(bits):
    return get().f16_value(bits)


def q8_0_quantize(w):
    return get().q8_0_quantize(w)


def decode(b, fmt, n, k):
    return get().decode(b, fmt, n, k)


def matmul(a, b, fmt, m, n, k, threads=None):
    return get().matmul(a, b, fmt, m, n, k, threads)


def matmul_entries(a, b, fmt, m, n, k, rows, cols, threads=None):
    return get().matmul_entries(a, b, fmt, m, n, k, rows, cols, threads)


def encode(w, fmt: int) -> np.ndarray:
    """Weight bytes of float32 w [n, k] in the given format, by the oracle's own encoders."""
    return get().encode(w, fmt)


def silu(x):
    return get().silu(x)


def matmul_epilogue(a, b, fmt, m, n, k, epi, resid=None, threads=None):
    return get().matmul_epilogue(a, b, fmt, m, n, k, epi, resid, threads)


def epilogue_entries(a, b, fmt, m, n, k, epi, rows, cols, resid=None, threads=None):
    return get().epilogue_entries(a, b, fmt, m, n, k, epi, rows, cols, resid, threads)


def topk(logits, k):
    return get().topk(logits, k)


def lm_head_topk(a, b, fmt, n, k, topk_, threads=None):
    return get().lm_head_topk(a, b, fmt, n, k, topk_, threads)


def decode_attention(q, k, v, kvfmt, L, D, Hq, Hkv, scale):
    return get().decode_attention(q, k, v, kvfmt, L, D, Hq, Hkv, scale)
