"""The C-ABI boundary on the CPU: symbols, validation, routing (no kernel runs).

Every call here returns from libwqmm's argument checks before any HIP call,
so it runs in a container without a GPU.  Pointers are plain integers: the
library never dereferences them on these paths.
"""
import os
import re

import pytest

import gemm_wq_gemv_amd as wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wqmm.h")
L = wq._lib

# Fake, suitably aligned device addresses far apart from each other.
A, B, C = 0x100000, 0x900000, 0x1100000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for want in ("wq_gemv_f16", "wq_gemv_q8_0", "wq_gemv_q4_0", "wq_gemm_f16", "wq_gemm_q8_0",
                 "wq_gemm_q4_0", "wq_matmul", "wq_matmul_ex", "wq_lm_head_topk", "wq_topk",
                 "wq_decode_attention", "wq_pack_f16", "wq_quantize_q8_0"):
        assert want in names


def test_library_exports_every_declared_symbol():
    for name in _declared():
        assert hasattr(L, name), name


def test_binding_has_every_entry_point_by_the_same_name():
    for name in _declared():
        assert callable(getattr(wq, name, None)), name


def test_single_hip_runtime_in_process():
    # torch is imported first, so libwqmm reuses torch's libamdhip64.so.7.
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs


def test_abi_and_status_strings():
    assert wq.wq_abi_version() == 108
    for st in range(0, 11):
        assert wq.status_str(st)
    assert wq.status_str(99) == "unknown status"


@pytest.mark.parametrize("fmt", [wq.WQ_FMT_F16, wq.WQ_FMT_Q8_0, wq.WQ_FMT_Q4_0])
def test_empty_outputs_are_noops(fmt):
    # m == 0 or n == 0: nothing to do, pointers are not even looked at.
    assert L.wq_matmul(None, None, None, 0, 16, 64, fmt, None) == wq.WQ_OK
    assert L.wq_matmul(None, None, None, 4, 0, 64, fmt, None) == wq.WQ_OK
    assert L.wq_gemm_f16(None, None, None, 0, 0, 0, None) == wq.WQ_OK
    assert L.wq_gemv_q8_0(None, None, None, 0, 33, None) == wq.WQ_OK  # n == 0 first, as on the page


def test_q8_and_q4_k_rules():
    for k in (0, 16, 33, 48, 1000):
        assert L.wq_gemv_q8_0(A, B, C, 8, k, None) == wq.WQ_ERR_K
        assert L.wq_gemm_q8_0(A, B, C, 2, 8, k, None) == wq.WQ_ERR_K
        assert L.wq_matmul(A, B, C, 2, 8, k, wq.WQ_FMT_Q8_0, None) == wq.WQ_ERR_K
        assert L.wq_gemv_q4_0(A, B, C, 8, k, None) == wq.WQ_ERR_K
        assert L.wq_gemm_q4_0(A, B, C, 2, 8, k, None) == wq.WQ_ERR_K
        assert L.wq_matmul(A, B, C, 2, 8, k, wq.WQ_FMT_Q4_0, None) == wq.WQ_ERR_K
    assert L.wq_quantize_q8_0(A, B, 33, None) == wq.WQ_ERR_K


def test_shape_format_null_align_alias():
    assert L.wq_matmul(A, B, C, -1, 8, 64, 0, None) == wq.WQ_ERR_SHAPE
    assert L.wq_matmul(A, B, C, 1, -8, 64, 0, None) == wq.WQ_ERR_SHAPE
    assert L.wq_matmul(A, B, C, 1, 8, -64, 0, None) == wq.WQ_ERR_SHAPE
    assert L.wq_matmul(A, B, C, 1 << 40, 1 << 40, 64, 0, None) == wq.WQ_ERR_SHAPE  # overflow
    assert L.wq_matmul(A, B, C, 1, 8, 64, 3, None) == wq.WQ_ERR_FORMAT
    assert L.wq_matmul(A, B, C, 1, 8, 64, -1, None) == wq.WQ_ERR_FORMAT
    assert L.wq_gemv_f16(None, B, C, 8, 64, None) == wq.WQ_ERR_NULL
    assert L.wq_gemv_f16(A, None, C, 8, 64, None) == wq.WQ_ERR_NULL
    assert L.wq_gemv_f16(A, B, None, 8, 64, None) == wq.WQ_ERR_NULL
    assert L.wq_gemm_f16(None, None, None, 2, 8, 0, None) == wq.WQ_ERR_NULL  # K == 0 still writes c
    assert L.wq_gemv_f16(A + 2, B, C, 8, 64, None) == wq.WQ_ERR_ALIGN
    assert L.wq_gemv_f16(A, B + 1, C, 8, 64, None) == wq.WQ_ERR_ALIGN
    assert L.wq_gemv_f16(A, B, C + 2, 8, 64, None) == wq.WQ_ERR_ALIGN
    # c overlapping a or b
    assert L.wq_gemv_f16(A, B, A + 64, 8, 64, None) == wq.WQ_ERR_ALIAS
    assert L.wq_gemm_q8_0(A, B, B + 4, 2, 8, 64, None) == wq.WQ_ERR_ALIAS
    assert L.wq_gemv_q4_0(A, B + 1, C, 8, 64, None) == wq.WQ_ERR_ALIGN
    # Q4_0 b spans n*(k/32)*18 = 288 bytes here: c starting inside it overlaps
    assert L.wq_gemv_q4_0(A, B, B + 8 * 2 * 18 - 4, 8, 64, None) == wq.WQ_ERR_ALIAS
    assert L.wq_pack_f16(A, A + 8, 64, None) == wq.WQ_ERR_ALIAS
    assert L.wq_pack_f16(A, B, -1, None) == wq.WQ_ERR_SHAPE
    assert L.wq_pack_f16(A, B, 0, None) == wq.WQ_OK
    assert L.wq_pack_f16(None, B, 5, None) == wq.WQ_ERR_NULL
    assert L.wq_quantize_q8_0(A, B + 1, 64, None) == wq.WQ_ERR_ALIGN


def test_epilogue_validation():
    EX = L.wq_matmul_ex
    # An unknown epilogue is reported before anything else is looked at.
    for epi in (-1, 3, 99):
        assert EX(A, B, C, 2, 8, 64, wq.WQ_FMT_F16, epi, None) == wq.WQ_ERR_EPILOGUE
        assert EX(None, None, None, -1, 8, 64, 7, epi, None) == wq.WQ_ERR_EPILOGUE
    for epi in (wq.WQ_EPI_NONE, wq.WQ_EPI_RESIDUAL, wq.WQ_EPI_SWIGLU):
        assert EX(None, None, None, 0, 8, 64, wq.WQ_FMT_Q8_0, epi, None) == wq.WQ_OK  # m == 0
        assert EX(None, None, None, 4, 0, 64, wq.WQ_FMT_Q4_0, epi, None) == wq.WQ_OK  # n == 0
        assert EX(A, B, C, 2, 8, 48, wq.WQ_FMT_Q8_0, epi, None) == wq.WQ_ERR_K
        assert EX(A, B, C, 2, 8, 64, 5, epi, None) == wq.WQ_ERR_FORMAT
        assert EX(A, B, None, 2, 8, 64, wq.WQ_FMT_F16, epi, None) == wq.WQ_ERR_NULL
        assert EX(A, B, C + 2, 2, 8, 64, wq.WQ_FMT_F16, epi, None) == wq.WQ_ERR_ALIGN
        assert EX(A, B, A + 8, 2, 8, 64, wq.WQ_FMT_F16, epi, None) == wq.WQ_ERR_ALIAS
    # SwiGLU weights span 2n rows: for f16 n = 8, K = 64 that is 2048 bytes, so a
    # c starting 1536 bytes into b overlaps the up half.
    assert EX(A, B, B + 1536, 1, 8, 64, wq.WQ_FMT_F16, wq.WQ_EPI_SWIGLU, None) == wq.WQ_ERR_ALIAS
    assert EX(A, B, B + 1020, 1, 8, 64, wq.WQ_FMT_F16, wq.WQ_EPI_NONE, None) == wq.WQ_ERR_ALIAS
    # Q4_0 up half: b spans 2 * 8 * 2 * 18 = 576 bytes.
    assert EX(A, B, B + 500, 1, 8, 64, wq.WQ_FMT_Q4_0, wq.WQ_EPI_SWIGLU, None) == wq.WQ_ERR_ALIAS
    # 2n rows overflow int64.
    assert EX(A, B, C, 1, 1 << 62, 64, wq.WQ_FMT_F16, wq.WQ_EPI_SWIGLU, None) == wq.WQ_ERR_SHAPE
    import torch
    with pytest.raises(ValueError):  # the binding checks b against 2n rows for SwiGLU
        wq.wq_matmul_ex(torch.zeros(64), torch.zeros(8 * 64, dtype=torch.uint16), torch.zeros(8), 1, 8, 64,
                        wq.WQ_FMT_F16, wq.WQ_EPI_SWIGLU)


def test_topk_validation():
    LM, TK = L.wq_lm_head_topk, L.wq_topk
    V, I = 0x1900000, 0x1A00000  # output pointers
    for topk in (0, -1, 65, 1000):
        assert LM(A, B, 100, 64, wq.WQ_FMT_F16, topk, V, I, None) == wq.WQ_ERR_TOPK
        assert TK(A, 100, topk, V, I, None) == wq.WQ_ERR_TOPK
    assert LM(A, B, 100, 64, 3, 1, V, I, None) == wq.WQ_ERR_FORMAT
    assert LM(A, B, -1, 64, wq.WQ_FMT_F16, 1, V, I, None) == wq.WQ_ERR_SHAPE
    assert LM(A, B, 100, -64, wq.WQ_FMT_F16, 1, V, I, None) == wq.WQ_ERR_SHAPE
    assert LM(A, B, 1 << 32, 64, wq.WQ_FMT_F16, 1, V, I, None) == wq.WQ_ERR_SHAPE  # ids would reach the sentinel
    assert TK(A, (1 << 32) - 1, 1, V, I, None) == wq.WQ_ERR_SHAPE
    assert TK(A, -5, 1, V, I, None) == wq.WQ_ERR_SHAPE
    for k in (0, 48):
        assert LM(A, B, 100, k, wq.WQ_FMT_Q8_0, 1, V, I, None) == wq.WQ_ERR_K
        assert LM(A, B, 100, k, wq.WQ_FMT_Q4_0, 1, V, I, None) == wq.WQ_ERR_K
    assert LM(A, B, 100, 64, wq.WQ_FMT_F16, 1, None, I, None) == wq.WQ_ERR_NULL
    assert LM(A, B, 100, 64, wq.WQ_FMT_F16, 1, V, None, None) == wq.WQ_ERR_NULL
    assert LM(None, B, 100, 64, wq.WQ_FMT_F16, 1, V, I, None) == wq.WQ_ERR_NULL
    assert LM(A, None, 100, 64, wq.WQ_FMT_F16, 1, V, I, None) == wq.WQ_ERR_NULL
    assert TK(None, 100, 1, V, I, None) == wq.WQ_ERR_NULL
    assert LM(A, B, 100, 64, wq.WQ_FMT_F16, 1, V + 2, I, None) == wq.WQ_ERR_ALIGN
    assert LM(A, B, 100, 64, wq.WQ_FMT_F16, 1, V, I + 1, None) == wq.WQ_ERR_ALIGN
    assert LM(A + 2, B, 100, 64, wq.WQ_FMT_F16, 1, V, I, None) == wq.WQ_ERR_ALIGN
    assert TK(A + 1, 100, 1, V, I, None) == wq.WQ_ERR_ALIGN
    assert LM(A, B, 100, 64, wq.WQ_FMT_F16, 8, V, V + 16, None) == wq.WQ_ERR_ALIAS   # vals / ids overlap
    assert LM(A, B, 100, 64, wq.WQ_FMT_F16, 8, A + 64, I, None) == wq.WQ_ERR_ALIAS   # vals inside a
    assert LM(A, B, 100, 64, wq.WQ_FMT_F16, 8, V, B + 1000, None) == wq.WQ_ERR_ALIAS  # ids inside b
    assert TK(A, 100, 8, A + 396, I, None) == wq.WQ_ERR_ALIAS                       # vals inside logits


def test_decode_attention_validation():
    AT = L.wq_decode_attention
    Q, K, V, O = 0x100000, 0x2000000, 0x4000000, 0x6000000

    def call(q=Q, k=K, v=V, o=O, L_=4096, D=256, hq=8, hkv=2, fmt=wq.WQ_KV_F32):
        return AT(q, k, v, o, L_, D, hq, hkv, fmt, 0.0625, None)
    assert call(fmt=2) == wq.WQ_ERR_FORMAT
    assert call(fmt=-1) == wq.WQ_ERR_FORMAT
    for bad in (dict(L_=-1), dict(D=96), dict(D=512), dict(D=0), dict(hq=0), dict(hkv=0), dict(hq=6, hkv=4),
                dict(hq=18, hkv=2), dict(hq=2, hkv=4), dict(L_=1 << 60)):
        assert call(**bad) == wq.WQ_ERR_SHAPE, bad
    assert call(q=None) == wq.WQ_ERR_NULL
    assert call(o=None) == wq.WQ_ERR_NULL
    assert call(k=None) == wq.WQ_ERR_NULL
    assert call(v=None) == wq.WQ_ERR_NULL
    assert call(q=Q + 2) == wq.WQ_ERR_ALIGN
    assert call(o=O + 1) == wq.WQ_ERR_ALIGN
    assert call(k=K + 8) == wq.WQ_ERR_ALIGN      # caches need 16 bytes
    assert call(v=V + 4, fmt=wq.WQ_KV_F16) == wq.WQ_ERR_ALIGN
    assert call(o=Q + 64) == wq.WQ_ERR_ALIAS
    assert call(o=K + 4096 * 512 * 4 - 16) == wq.WQ_ERR_ALIAS   # inside the f32 K cache
    assert call(o=V + 100 * 16) == wq.WQ_ERR_ALIAS
    assert L.wq_set_attn_partition(-1) == wq.WQ_ERR_SHAPE
    assert L.wq_set_attn_partition(0) == wq.WQ_OK


def test_routing_rule():
    """M = 1: GEMV; quantized with K % 256 == 0: 2..16 the f16 matrix-core
    stream (two Q8_0 rows the register-chunk GEMV takes with few units: GEMV); other quantized K: 2..4 small-M; f16: 2..8 small-M; more: the
    tiled f16 matrix-core GEMM (which hands calls it cannot take to the fp32
    GEMM at launch)."""
    for fmt in (wq.WQ_FMT_F16, wq.WQ_FMT_Q8_0, wq.WQ_FMT_Q4_0):
        for k in (4096, 4128):
            assert wq.wq_route_for(1, 4096, k, fmt) == wq.WQ_ROUTE_GEMV
            if fmt != wq.WQ_FMT_F16 and k % 256 == 0:
                small, top = wq.WQ_ROUTE_STREAM, 16
            else:
                small, top = wq.WQ_ROUTE_SKINNY, 8 if fmt == wq.WQ_FMT_F16 else 4
            for m in range(2, top + 1):
                # Two Q8_0 rows at N = K = 4096: the register-chunk plan (8, 1, 1)
                # keeps two units per wave, so the GEMV route takes them.
                two_rows = fmt == wq.WQ_FMT_Q8_0 and m == 2 and k % 256 == 0
                assert wq.wq_route_for(m, 4096, k, fmt) == (wq.WQ_ROUTE_GEMV if two_rows else small)
            for m in (top + 1, 17, 64, 512):
                assert wq.wq_route_for(m, 4096, k, fmt) == wq.WQ_ROUTE_GEMM_HL
    # Two Q8_0 rows: GEMV where the register-chunk plan has at most three
    # units per wave (K <= 8448 at Q8_0's 34 bytes per 32 columns), the stream
    # otherwise (K = 11008: four units).
    for (n, k), route in (((11008, 4096), wq.WQ_ROUTE_GEMV), ((151936, 2048), wq.WQ_ROUTE_GEMV),
                          ((6144, 2048), wq.WQ_ROUTE_GEMV), ((2048, 6144), wq.WQ_ROUTE_GEMV),
                          ((2048, 2048), wq.WQ_ROUTE_GEMV), ((1000, 8448), wq.WQ_ROUTE_GEMV),
                          ((4096, 11008), wq.WQ_ROUTE_STREAM), ((11008, 8704), wq.WQ_ROUTE_STREAM)):
        assert wq.wq_route_for(2, n, k, wq.WQ_FMT_Q8_0) == route, (n, k)
        assert wq.wq_route_for(2, n, k, wq.WQ_FMT_Q4_0) == wq.WQ_ROUTE_STREAM, (n, k)
        assert wq.wq_route_for(3, n, k, wq.WQ_FMT_Q8_0) == wq.WQ_ROUTE_STREAM, (n, k)
    assert wq.wq_route_for(2, 8, 33, wq.WQ_FMT_Q8_0) == -wq.WQ_ERR_K
    assert wq.wq_route_for(2, 8, 48, wq.WQ_FMT_Q4_0) == -wq.WQ_ERR_K
    assert wq.wq_route_for(2, 8, 32, 5) == -wq.WQ_ERR_FORMAT
    assert wq.wq_route_for(-2, 8, 32, 0) == -wq.WQ_ERR_SHAPE


def test_forced_route_setting():
    prev = wq.wq_set_forced_route(wq.WQ_ROUTE_GEMM)
    try:
        assert prev == wq.WQ_ROUTE_AUTO
        assert wq.wq_set_forced_route(wq.WQ_ROUTE_GEMV) == wq.WQ_ROUTE_GEMM
        assert wq.wq_set_forced_route(wq.WQ_ROUTE_SKINNY) == wq.WQ_ROUTE_GEMV
        assert wq.wq_set_forced_route(wq.WQ_ROUTE_STREAM) == wq.WQ_ROUTE_SKINNY
        assert wq.wq_set_forced_route(wq.WQ_ROUTE_GEMM_HL) == wq.WQ_ROUTE_STREAM
        assert wq.wq_set_forced_route(7) == -wq.WQ_ERR_ROUTE
        assert wq.wq_set_forced_route(-1) == -wq.WQ_ERR_ROUTE
    finally:
        wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)
    wq.wq_reset_route_counts()
    for r in (wq.WQ_ROUTE_GEMV, wq.WQ_ROUTE_GEMM, wq.WQ_ROUTE_SKINNY, wq.WQ_ROUTE_STREAM, wq.WQ_ROUTE_GEMM_HL):
        assert wq.wq_route_count(r) == 0
    assert wq.wq_route_count(99) == 0


def test_python_binding_rejects_host_and_short_tensors():
    import torch
    a = torch.zeros(64)
    with pytest.raises(ValueError):
        wq.wq_gemv_f16(a, torch.zeros(64, dtype=torch.uint16), torch.zeros(1), 1, 64)  # host tensors
    with pytest.raises(ValueError):
        wq.wq_gemv_f16(a, torch.zeros(10, dtype=torch.uint16), torch.zeros(1), 1, 64)  # b too short
    with pytest.raises(TypeError):
        wq.wq_gemv_f16(a.double(), torch.zeros(64, dtype=torch.uint16), torch.zeros(1), 1, 64)


def test_product_path_does_not_touch_the_oracle():
    """The library and its binding never import, include or load the oracle or
    the input generator; the oracle never includes library code."""
    pkg = os.path.join(ROOT, "gemm_wq_gemv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b|wqref|wqgen", text), f
    src = open(os.path.join(ROOT, "oracle", "wqref.c")).read()
    assert "#include \"" not in src and "wqmm" not in src and "hip" not in src.lower().replace("ship", "")


def test_gemm_planner_invariants():
    """Every plan uses a compiled tile, no split is empty, tiny M uses 16-row
    tiles, and the M = 512 prefill shapes get the tilings measured fastest."""
    for m in (1, 2, 7, 16, 33, 64, 130, 512, 4096):
        for n in (1, 97, 2048, 11008):
            for k in (32, 1000, 2048, 11008):
                for fmt in (wq.WQ_FMT_F16, wq.WQ_FMT_Q8_0):
                    if fmt == wq.WQ_FMT_Q8_0 and k % 32:
                        continue
                    bm, bn, sp = wq.wq_gemm_plan(m, n, k, fmt)
                    assert (bm, bn) in wq.GEMM_TILES
                    kt = -(-k // 32)
                    assert 1 <= sp <= kt
                    kts = -(-kt // sp)
                    assert (sp - 1) * kts < kt          # the last split is not empty
                    if m <= 16:
                        assert bm == 16
    assert wq.wq_gemm_plan(512, 6144, 2048, wq.WQ_FMT_F16) == (64, 64, 1)
    assert wq.wq_gemm_plan(512, 4096, 11008, wq.WQ_FMT_Q8_0) == (128, 128, 4)
    assert wq.wq_gemm_plan(16, 11008, 4096, wq.WQ_FMT_Q8_0) == (16, 128, 8)


def test_gemv_plan_override_hook():
    try:
        for pl in wq.GEMV_PLANS:
            wq.wq_set_gemv_plan(*pl)
        wq.wq_set_gemv_plan(-1, 0, 0)
        for bad in ((3, 2, 1), (8, 2, 2), (16, 2, 1), (-1, 1, 0)):
            with pytest.raises(wq.WQError):
                wq.wq_set_gemv_plan(*bad)
    finally:
        wq.wq_set_gemv_plan(0, 0, 0)


def test_stream_plan_override_hook():
    try:
        for p, sp in ((1, 0), (14, 0), (0, 3), (2, 43)):
            wq.wq_set_stream_plan(p, sp)
        for bad in ((15, 0), (-1, 0), (1, -2)):
            with pytest.raises(wq.WQError):
                wq.wq_set_stream_plan(*bad)
    finally:
        wq.wq_set_stream_plan(0, 0)


def test_gemm_plan_override_hook():
    try:
        wq.wq_set_gemm_plan(32, 128, 3)
        assert wq.wq_gemm_plan(512, 6144, 2048, wq.WQ_FMT_F16) == (32, 128, 3)
        assert wq.wq_gemm_plan(5, 10, 64, wq.WQ_FMT_F16) == (32, 128, 2)   # capped at 2 k-steps
        with pytest.raises(wq.WQError):
            wq.wq_set_gemm_plan(48, 64, 1)
        with pytest.raises(wq.WQError):
            wq.wq_set_gemm_plan(64, 64, 0)
    finally:
        wq.wq_set_gemm_plan(0, 0, 0)
    assert wq.wq_gemm_plan(512, 6144, 2048, wq.WQ_FMT_F16) == (64, 64, 1)
    assert L.wq_gemm_plan(0, 1, 1, 0, 256, None, None, None) == wq.WQ_ERR_SHAPE


def test_hgemm_planner_invariants():
    """The f16 matrix-core GEMM's plans: a compiled tile, no empty split, no
    128-row tile for M <= 64, and the measured-fastest tilings of the M = 512
    prefill shapes."""
    for m in (2, 17, 33, 64, 130, 512, 4096):
        for n in (1, 97, 2048, 11008):
            for k in (32, 1024, 2048, 11008):
                for fmt in (wq.WQ_FMT_F16, wq.WQ_FMT_Q8_0, wq.WQ_FMT_Q4_0):
                    bm, bn, sp = wq.wq_hgemm_plan(m, n, k, fmt)
                    assert (bm, bn) in wq.HGEMM_TILES
                    kt = k // 32
                    assert 1 <= sp <= kt
                    assert (sp - 1) * (-(-kt // sp)) < kt
                    if m <= 64:
                        assert bm == 64
    assert wq.wq_hgemm_plan(512, 6144, 2048, wq.WQ_FMT_F16) == (64, 128, 2)
    assert wq.wq_hgemm_plan(512, 2048, 6144, wq.WQ_FMT_F16) == (64, 128, 4)
    assert wq.wq_hgemm_plan(512, 4096, 11008, wq.WQ_FMT_Q8_0) == (64, 128, 2)


def test_hgemm_plan_override_hook():
    try:
        wq.wq_set_hgemm_plan(128, 64, 3)
        assert wq.wq_hgemm_plan(512, 6144, 2048, wq.WQ_FMT_F16) == (128, 64, 3)
        assert wq.wq_hgemm_plan(5, 10, 64, wq.WQ_FMT_F16) == (128, 64, 2)   # capped at 2 k-steps
        for bad in ((32, 128, 1), (96, 64, 1), (64, 64, 0), (64, 64, 65)):
            with pytest.raises(wq.WQError):
                wq.wq_set_hgemm_plan(*bad)
    finally:
        wq.wq_set_hgemm_plan(0, 0, 0)
    assert wq.wq_hgemm_plan(512, 6144, 2048, wq.WQ_FMT_F16) == (64, 128, 2)
    assert L.wq_hgemm_plan(0, 1, 1, 0, 256, None, None, None) == wq.WQ_ERR_SHAPE
    assert L.wq_hgemm_plan(4, 1, 48, 0, 256, None, None, None) == wq.WQ_ERR_K
