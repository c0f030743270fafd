"""Python binding of libwqmm (argument marshalling only).

Each function has the name and argument order of the C entry point declared in
``include/wqmm.h`` and forwards to it through ctypes: tensors become device
pointers, the stream becomes a ``hipStream_t``.  All computation happens in
the library's HIP kernels; there is no fallback of any kind, and importing
this module fails loudly if ``libwqmm.so`` is missing and cannot be built.

PyTorch supplies device memory and streams.  ``torch`` is imported before the
library is loaded so that libwqmm binds to the HIP runtime torch already
loaded (both carry the soname ``libamdhip64.so.7``): one runtime per process,
so torch's stream handles and device pointers are valid in the library.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading libwqmm, see above)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwqmm.so")

WQ_FMT_F16 = 0
WQ_FMT_Q8_0 = 1
WQ_FMT_Q4_0 = 2

WQ_OK = 0
WQ_ERR_NULL = 1
WQ_ERR_SHAPE = 2
WQ_ERR_K = 3
WQ_ERR_FORMAT = 4
WQ_ERR_ALIGN = 5
WQ_ERR_LAUNCH = 6
WQ_ERR_ALIAS = 7
WQ_ERR_ROUTE = 8
WQ_ERR_EPILOGUE = 9
WQ_ERR_TOPK = 10
WQ_ERR_WORKSPACE = 11
WQ_TOPK_MAX = 64
WQ_ATTN_MAX_GROUP = 8
WQ_KV_F32 = 0
WQ_KV_F16 = 1
WQ_TOPK_NO_ID = 0xFFFFFFFF

WQ_ROUTE_AUTO = 0
WQ_ROUTE_GEMV = 1
WQ_ROUTE_GEMM = 2
WQ_ROUTE_SKINNY = 3
WQ_ROUTE_STREAM = 4
WQ_ROUTE_GEMM_HL = 5

WQ_EPI_NONE = 0
WQ_EPI_RESIDUAL = 1
WQ_EPI_SWIGLU = 2

Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_WEIGHTS = 32
Q4_0_BLOCK_BYTES = 18


class WQError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sigs = {
        "wq_gemv_f16": (I, [P, P, P, I64, I64, P]),
        "wq_gemv_q8_0": (I, [P, P, P, I64, I64, P]),
        "wq_gemv_q4_0": (I, [P, P, P, I64, I64, P]),
        "wq_gemm_f16": (I, [P, P, P, I64, I64, I64, P]),
        "wq_gemm_q8_0": (I, [P, P, P, I64, I64, I64, P]),
        "wq_gemm_q4_0": (I, [P, P, P, I64, I64, I64, P]),
        "wq_matmul": (I, [P, P, P, I64, I64, I64, I, P]),
        "wq_matmul_ex": (I, [P, P, P, I64, I64, I64, I, I, P]),
        "wq_lm_head_topk": (I, [P, P, I64, I64, I, I, P, P, P]),
        "wq_lm_head_topk_noalloc": (I, [P, P, I64, I64, I, I, P, P, P]),
        "wq_noalloc_workspace_bytes": (ctypes.c_size_t, []),
        "wq_topk": (I, [P, I64, I, P, P, P]),
        "wq_decode_attention": (I, [P, P, P, P, I64, I, I, I, I, ctypes.c_float, P]),
        "wq_set_attn_partition": (I, [I64]),
        "wq_pack_f16": (I, [P, P, I64, P]),
        "wq_quantize_q8_0": (I, [P, P, I64, P]),
        "wq_read_probe": (I, [P, I64, P, I, P]),
        "wq_route_for": (I, [I64, I64, I64, I]),
        "wq_gemm_plan": (I, [I64, I64, I64, I, I, P, P, P]),
        "wq_set_gemm_plan": (I, [I, I, I]),
        "wq_hgemm_plan": (I, [I64, I64, I64, I, I, P, P, P]),
        "wq_set_hgemm_plan": (I, [I, I, I]),
        "wq_set_gemv_plan": (I, [I, I, I]),
        "wq_set_stream_plan": (I, [I, I]),
        "wq_set_forced_route": (I, [I]),
        "wq_route_count": (ctypes.c_uint64, [I]),
        "wq_reset_route_counts": (None, []),
        "wq_status_str": (ctypes.c_char_p, [I]),
        "wq_abi_version": (I, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


# ----------------------------------------------------------------- helpers --
def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() or None


_raw_stream = torch._C._cuda_getCurrentRawStream


def _stream(stream, like=None):
    """hipStream_t for `stream` (a torch.cuda.Stream or a raw handle); None is
    torch's current stream on the device of tensor `like` (else the current
    device)."""
    if stream is None:
        dev = like.get_device() if like is not None and like.is_cuda else torch.cuda.current_device()
        return _raw_stream(dev)
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def _need(t, nbytes: int, what: str):
    if t is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")


def _dtype(t, dtypes, what):
    if t is not None and t.dtype not in dtypes:
        raise TypeError(f"{what} must be one of {dtypes}, got {t.dtype}")


_F32 = (torch.float32,)
_H = (torch.uint16, torch.int16, torch.float16)
_U8 = (torch.uint8, torch.int8)


def weight_bytes(n: int, k: int, fmt: int) -> int:
    """Bytes of an [n, k] weight matrix in the given format."""
    if fmt == WQ_FMT_F16:
        return 2 * n * k
    if fmt == WQ_FMT_Q4_0:
        return n * (k // Q8_0_BLOCK_WEIGHTS) * Q4_0_BLOCK_BYTES
    return n * (k // Q8_0_BLOCK_WEIGHTS) * Q8_0_BLOCK_BYTES


def _check(status: int, what: str):
    if status != WQ_OK:
        raise WQError(status, what)


def _sizes(a, b, c, m, n, k, fmt, weight_rows=None):
    if m > 0 and n > 0:
        _dtype(a, _F32, "a")
        _dtype(c, _F32, "c")
        _dtype(b, _H if fmt == WQ_FMT_F16 else _U8, "b")
        _need(a, 4 * m * k, "a")
        _need(c, 4 * m * n, "c")
        if k >= 0 and (fmt == WQ_FMT_F16 or k % 32 == 0):
            _need(b, weight_bytes(n if weight_rows is None else weight_rows, k, fmt), "b")


# ------------------------------------------------------------ entry points --
def wq_gemv_f16(a, b, c, n: int, k: int, stream=None) -> None:
    _sizes(a, b, c, 1, n, k, WQ_FMT_F16)
    _check(_lib.wq_gemv_f16(_ptr(a), _ptr(b), _ptr(c), n, k, _stream(stream, c)), "wq_gemv_f16")


def wq_gemv_q8_0(a, b, c, n: int, k: int, stream=None) -> None:
    _sizes(a, b, c, 1, n, k, WQ_FMT_Q8_0)
    _check(_lib.wq_gemv_q8_0(_ptr(a), _ptr(b), _ptr(c), n, k, _stream(stream, c)), "wq_gemv_q8_0")


def wq_gemv_q4_0(a, b, c, n: int, k: int, stream=None) -> None:
    _sizes(a, b, c, 1, n, k, WQ_FMT_Q4_0)
    _check(_lib.wq_gemv_q4_0(_ptr(a), _ptr(b), _ptr(c), n, k, _stream(stream, c)), "wq_gemv_q4_0")


def wq_gemm_f16(a, b, c, m: int, n: int, k: int, stream=None) -> None:
    _sizes(a, b, c, m, n, k, WQ_FMT_F16)
    _check(_lib.wq_gemm_f16(_ptr(a), _ptr(b), _ptr(c), m, n, k, _stream(stream, c)), "wq_gemm_f16")


def wq_gemm_q8_0(a, b, c, m: int, n: int, k: int, stream=None) -> None:
    _sizes(a, b, c, m, n, k, WQ_FMT_Q8_0)
    _check(_lib.wq_gemm_q8_0(_ptr(a), _ptr(b), _ptr(c), m, n, k, _stream(stream, c)), "wq_gemm_q8_0")


def wq_gemm_q4_0(a, b, c, m: int, n: int, k: int, stream=None) -> None:
    _sizes(a, b, c, m, n, k, WQ_FMT_Q4_0)
    _check(_lib.wq_gemm_q4_0(_ptr(a), _ptr(b), _ptr(c), m, n, k, _stream(stream, c)), "wq_gemm_q4_0")


def wq_matmul(a, b, c, m: int, n: int, k: int, fmt: int, stream=None) -> None:
    if fmt in (WQ_FMT_F16, WQ_FMT_Q8_0, WQ_FMT_Q4_0):
        _sizes(a, b, c, m, n, k, fmt)
    _check(_lib.wq_matmul(_ptr(a), _ptr(b), _ptr(c), m, n, k, fmt, _stream(stream, c)), "wq_matmul")


def wq_matmul_ex(a, b, c, m: int, n: int, k: int, fmt: int, epi: int, stream=None) -> None:
    """wq_matmul with a fused epilogue: WQ_EPI_RESIDUAL (c += a.b^T) or
    WQ_EPI_SWIGLU (b holds 2n rows, gate then up; c = silu(gate) * up)."""
    if fmt in (WQ_FMT_F16, WQ_FMT_Q8_0, WQ_FMT_Q4_0) and epi in (WQ_EPI_NONE, WQ_EPI_RESIDUAL, WQ_EPI_SWIGLU):
        _sizes(a, b, c, m, n, k, fmt, 2 * n if epi == WQ_EPI_SWIGLU else n)
    _check(_lib.wq_matmul_ex(_ptr(a), _ptr(b), _ptr(c), m, n, k, fmt, epi, _stream(stream, c)), "wq_matmul_ex")


def _topk_out(vals, ids, topk):
    if 1 <= topk <= WQ_TOPK_MAX:
        _dtype(vals, _F32, "vals")
        _dtype(ids, (torch.uint32, torch.int32), "ids")
        _need(vals, 4 * topk, "vals")
        _need(ids, 4 * topk, "ids")


def wq_lm_head_topk(a, b, n: int, k: int, fmt: int, topk: int, vals, ids, stream=None) -> None:
    """Fused LM-head GEMV + top-k for one token: vals / ids (topk entries, rank
    order) of logits[j] = sum_k a[k] w[j, k]."""
    if fmt in (WQ_FMT_F16, WQ_FMT_Q8_0, WQ_FMT_Q4_0) and n > 0:
        _dtype(a, _F32, "a")
        _dtype(b, _H if fmt == WQ_FMT_F16 else _U8, "b")
        _need(a, 4 * k, "a")
        if k >= 0 and (fmt == WQ_FMT_F16 or k % 32 == 0):
            _need(b, weight_bytes(n, k, fmt), "b")
    _topk_out(vals, ids, topk)
    _check(_lib.wq_lm_head_topk(_ptr(a), _ptr(b), n, k, fmt, topk, _ptr(vals), _ptr(ids), _stream(stream, vals)),
           "wq_lm_head_topk")


def wq_lm_head_topk_noalloc(a, b, n: int, k: int, fmt: int, topk: int, vals, ids, stream=None) -> None:
    """wq_lm_head_topk without any allocation (fixed per-GPU workspace)."""
    if fmt in (WQ_FMT_F16, WQ_FMT_Q8_0, WQ_FMT_Q4_0) and n > 0:
        _dtype(a, _F32, "a")
        _dtype(b, _H if fmt == WQ_FMT_F16 else _U8, "b")
        _need(a, 4 * k, "a")
        if k >= 0 and (fmt == WQ_FMT_F16 or k % 32 == 0):
            _need(b, weight_bytes(n, k, fmt), "b")
    _topk_out(vals, ids, topk)
    _check(_lib.wq_lm_head_topk_noalloc(_ptr(a), _ptr(b), n, k, fmt, topk, _ptr(vals), _ptr(ids),
                                        _stream(stream, vals)), "wq_lm_head_topk_noalloc")


def wq_noalloc_workspace_bytes() -> int:
    return int(_lib.wq_noalloc_workspace_bytes())


def wq_topk(logits, n: int, topk: int, vals, ids, stream=None) -> None:
    """Top-k of an f32 logits vector [n] (device)."""
    if n > 0:
        _dtype(logits, _F32, "logits")
        _need(logits, 4 * n, "logits")
    _topk_out(vals, ids, topk)
    _check(_lib.wq_topk(_ptr(logits), n, topk, _ptr(vals), _ptr(ids), _stream(stream, vals)), "wq_topk")


def wq_decode_attention(q, k_cache, v_cache, out, cache_len: int, head_dim: int, num_q_heads: int,
                        num_kv_heads: int, kv_fmt: int, scale: float, stream=None) -> None:
    """One query token's grouped-query attention over a [cache_len, num_kv_heads*head_dim]
    K/V cache (f32 or f16 bits): out [num_q_heads, head_dim]."""
    if num_q_heads > 0 and head_dim > 0:
        _dtype(q, _F32, "q")
        _dtype(out, _F32, "out")
        _need(q, 4 * num_q_heads * head_dim, "q")
        _need(out, 4 * num_q_heads * head_dim, "out")
        if cache_len > 0 and num_kv_heads > 0 and kv_fmt in (WQ_KV_F32, WQ_KV_F16):
            kv = (_F32 if kv_fmt == WQ_KV_F32 else _H)
            nbytes = cache_len * num_kv_heads * head_dim * (4 if kv_fmt == WQ_KV_F32 else 2)
            _dtype(k_cache, kv, "k_cache")
            _dtype(v_cache, kv, "v_cache")
            _need(k_cache, nbytes, "k_cache")
            _need(v_cache, nbytes, "v_cache")
    _check(_lib.wq_decode_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), cache_len, head_dim,
                                    num_q_heads, num_kv_heads, kv_fmt, scale, _stream(stream, out)),
           "wq_decode_attention")


def wq_set_attn_partition(tokens: int) -> None:
    """Force the attention partition size (tokens); 0 = automatic."""
    _check(_lib.wq_set_attn_partition(tokens), "wq_set_attn_partition")


def wq_pack_f16(w, out, count: int, stream=None) -> None:
    if count > 0:
        _dtype(w, _F32, "w")
        _dtype(out, _H, "out")
        _need(w, 4 * count, "w")
        _need(out, 2 * count, "out")
    _check(_lib.wq_pack_f16(_ptr(w), _ptr(out), count, _stream(stream, out)), "wq_pack_f16")


def wq_quantize_q8_0(w, out, count: int, stream=None) -> None:
    if count > 0 and count % 32 == 0:
        _dtype(w, _F32, "w")
        _dtype(out, _U8, "out")
        _need(w, 4 * count, "w")
        _need(out, count // 32 * Q8_0_BLOCK_BYTES, "out")
    _check(_lib.wq_quantize_q8_0(_ptr(w), _ptr(out), count, _stream(stream, out)), "wq_quantize_q8_0")


def wq_read_probe(p, nbytes: int, out, variant: int = 2, stream=None) -> None:
    """Measurement hook: stream `nbytes` bytes of tensor p once (plain read);
    out (uint32/int32, ceil(nbytes / 1024) elements) receives per-wave checksums."""
    if nbytes > 0:
        _need(p, nbytes, "p")
        _dtype(out, (torch.uint32, torch.int32), "out")
        _need(out, 4 * ((nbytes + 1023) // 1024), "out")
    _check(_lib.wq_read_probe(_ptr(p), nbytes, _ptr(out), variant, _stream(stream, out)), "wq_read_probe")


def wq_route_for(m: int, n: int, k: int, fmt: int) -> int:
    return int(_lib.wq_route_for(m, n, k, fmt))


def wq_gemm_plan(m: int, n: int, k: int, fmt: int, cus: int = 256):
    """(bm, bn, splits) the GEMM uses for this problem on `cus` compute units."""
    bm, bn, sp = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(_lib.wq_gemm_plan(m, n, k, fmt, cus, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(sp)),
           "wq_gemm_plan")
    return bm.value, bn.value, sp.value


def wq_set_gemm_plan(bm: int, bn: int, splits: int) -> None:
    _check(_lib.wq_set_gemm_plan(bm, bn, splits), "wq_set_gemm_plan")


def wq_hgemm_plan(m: int, n: int, k: int, fmt: int, cus: int = 256):
    """(bm, bn, splits) the f16 matrix-core GEMM uses for this problem."""
    bm, bn, sp = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(_lib.wq_hgemm_plan(m, n, k, fmt, cus, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(sp)),
           "wq_hgemm_plan")
    return bm.value, bn.value, sp.value


def wq_set_hgemm_plan(bm: int, bn: int, splits: int) -> None:
    _check(_lib.wq_set_hgemm_plan(bm, bn, splits), "wq_set_hgemm_plan")


HGEMM_TILES = [(128, 128), (128, 64), (64, 128), (64, 64)]


def wq_set_gemv_plan(rb: int, nf: int, nr: int) -> None:
    _check(_lib.wq_set_gemv_plan(rb, nf, nr), "wq_set_gemv_plan")


def wq_set_stream_plan(shape: int, splits: int) -> None:
    _check(_lib.wq_set_stream_plan(shape, splits), "wq_set_stream_plan")


# (tiles per wave, K sub-ranges per workgroup, tile groups, weights staged in LDS)
STREAM_SHAPES = [(1, 4, 1, 0), (1, 8, 1, 0), (2, 4, 1, 0), (1, 2, 2, 0), (2, 1, 4, 0), (1, 1, 4, 0), (2, 8, 1, 0),
                 (1, 4, 1, 1), (1, 1, 4, 1), (2, 1, 4, 1), (1, 8, 1, 1), (1, 2, 2, 1), (1, 1, 8, 1), (2, 1, 8, 1)]


GEMM_TILES = [(128, 128), (128, 96), (128, 64), (64, 128), (64, 64), (32, 128), (16, 128), (16, 64)]
GEMV_PLANS = [(8, 2, 1), (4, 2, 1), (4, 3, 1), (4, 1, 1), (8, 1, 1), (16, 1, 1), (2, 2, 1)]


def wq_set_forced_route(route: int) -> int:
    return int(_lib.wq_set_forced_route(route))


def wq_route_count(route: int) -> int:
    return int(_lib.wq_route_count(route))


def wq_reset_route_counts() -> None:
    _lib.wq_reset_route_counts()


def status_str(status: int) -> str:
    return _lib.wq_status_str(status).decode()


wq_status_str = status_str


def wq_abi_version() -> int:
    return int(_lib.wq_abi_version())


# ------------------------------------------------------- tensor conveniences --
def pack_f16(w: torch.Tensor, stream=None) -> torch.Tensor:
    """f32 [n, k] device tensor -> binary16 bits (uint16 [n, k]) via wq_pack_f16."""
    out = torch.empty(w.shape, dtype=torch.uint16, device=w.device)
    wq_pack_f16(w, out, w.numel(), stream)
    return out


def quantize_q8_0(w: torch.Tensor, stream=None) -> torch.Tensor:
    """f32 [n, k] device tensor (k % 32 == 0) -> Q8_0 bytes (uint8 [n, k/32*34])."""
    n, k = w.shape
    out = torch.empty((n, k // 32 * Q8_0_BLOCK_BYTES), dtype=torch.uint8, device=w.device)
    wq_quantize_q8_0(w, out, w.numel(), stream)
    return out


def matmul(a: torch.Tensor, b: torch.Tensor, n: int, k: int, fmt: int, out=None, stream=None) -> torch.Tensor:
    """C = A . B^T for f32 a [m, k] and encoded weights b (via wq_matmul)."""
    m = a.numel() // k if k else a.shape[0]
    c = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=a.device)
    wq_matmul(a, b, c, m, n, k, fmt, stream)
    return c


def lm_head_topk(a: torch.Tensor, b: torch.Tensor, n: int, k: int, fmt: int, topk: int, stream=None):
    """(vals f32 [topk], ids int32 [topk]) via wq_lm_head_topk; ids hold the uint32
    token ids as int32 bit patterns (the sentinel WQ_TOPK_NO_ID reads as -1)."""
    vals = torch.empty(topk, dtype=torch.float32, device=a.device)
    ids = torch.empty(topk, dtype=torch.int32, device=a.device)
    wq_lm_head_topk(a, b, n, k, fmt, topk, vals, ids, stream)
    return vals, ids
