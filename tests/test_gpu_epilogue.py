"""GPU parity of the fused epilogues (wq_matmul_ex) against the CPU oracle.

WQ_EPI_RESIDUAL adds the product into C (C holds a seeded residual on entry);
WQ_EPI_SWIGLU reads a fused gate||up weight of 2n rows and writes
silu(gate) * up into C [m, n].  Each case runs on every route (decode GEMV,
small-M kernel, tiled GEMM) and every weight format, with ragged N, a K tail
and split K, and is compared element by element with the oracle's float64
epilogue within the oracle's bound (the product's 1e-5 * sum|a w| + 1e-6,
propagated through the epilogue).  Outputs that the epilogue overwrites are
poisoned with NaN first.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import gemm_wq_gemv_amd as wq
import oracle
import wqgen

pytestmark = pytest.mark.gpu

F16, Q8, Q4 = wq.WQ_FMT_F16, wq.WQ_FMT_Q8_0, wq.WQ_FMT_Q4_0
ALL = [F16, Q8, Q4]
RES, GLU = wq.WQ_EPI_RESIDUAL, wq.WQ_EPI_SWIGLU
ROUTES = {"gemv": wq.WQ_ROUTE_GEMV, "skinny": wq.WQ_ROUTE_SKINNY, "gemm": wq.WQ_ROUTE_GEMM,
          "stream": wq.WQ_ROUTE_STREAM, "gemm_hl": wq.WQ_ROUTE_GEMM_HL, "auto": wq.WQ_ROUTE_AUTO}


def say(msg: str):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)
    wq.wq_set_gemm_plan(0, 0, 0)
    yield
    wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)
    wq.wq_set_gemm_plan(0, 0, 0)


@functools.lru_cache(maxsize=4)
def encoded(rows, k, fmt, seed):
    """(oracle bytes, library bytes on the GPU) of the same [rows, k] weights."""
    if fmt == Q4:
        raw = wqgen.q4_0_bytes(rows, k, seed)
        return raw, torch.from_numpy(raw).cuda()
    w = wqgen.weights(rows, k, seed)
    ref = oracle.encode(w, fmt)
    wd = torch.from_numpy(w).cuda()
    dev = wq.pack_f16(wd) if fmt == F16 else wq.quantize_q8_0(wd)
    torch.cuda.synchronize()
    return ref, dev


def assert_close(c, c_ref, bound, what):
    err = np.abs(c.astype(np.float64) - c_ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        det = [(tuple(i), float(c[tuple(i)]), float(c_ref[tuple(i)]), float(bound[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, e.g. {det}")


def run_ex(a_np, b_dev, m, n, k, fmt, epi, resid=None, stream=None):
    a = torch.from_numpy(np.ascontiguousarray(a_np)).cuda()
    if epi == RES:
        c = torch.from_numpy(np.ascontiguousarray(resid)).cuda()
    else:
        c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    wq.wq_matmul_ex(a, b_dev, c, m, n, k, fmt, epi, stream)
    torch.cuda.synchronize()
    return c.cpu().numpy()


def case(fmt, epi, m, n, k, seed=0, route="auto"):
    say(f"epi={epi} route={route} fmt={fmt} m={m} n={n} k={k} seed={seed}")
    rows = 2 * n if epi == GLU else n
    ref_b, dev_b = encoded(rows, k, fmt, seed)
    a = wqgen.activations(m, k, seed)
    r = wqgen.residual(m, n, seed) if epi == RES else None
    prev = wq.wq_set_forced_route(ROUTES[route])
    try:
        c = run_ex(a, dev_b, m, n, k, fmt, epi, r)
    finally:
        wq.wq_set_forced_route(prev)
    c_ref, bound = oracle.matmul_epilogue(a, ref_b, fmt, m, n, k, epi, r)
    assert_close(c, c_ref, bound, f"epi={epi} route={route} fmt={fmt} {m}x{n}x{k}")


SHAPES = {F16: [(1, 37, 1000), (3, 300, 2048), (13, 129, 96), (37, 97, 1003), (5, 1000, 8192)],
          Q8: [(1, 37, 992), (3, 300, 2048), (13, 129, 96), (37, 97, 1024), (5, 1000, 8192)],
          Q4: [(1, 37, 992), (3, 300, 2048), (13, 129, 96), (37, 97, 1024), (5, 1000, 8192)]}


@pytest.mark.parametrize("route", ["gemv", "skinny", "gemm", "stream", "gemm_hl", "auto"])
@pytest.mark.parametrize("epi", [RES, GLU], ids=["residual", "swiglu"])
@pytest.mark.parametrize("fmt", ALL)
def test_epilogue_every_route(fmt, epi, route):
    """Ragged N (not a multiple of any tile), K tails (f16 K % 32 != 0), K split
    across workgroups (small N, large K), and every small-M row-group count."""
    for m, n, k in SHAPES[fmt]:
        if route in ("skinny", "stream") and m > 16:
            continue
        case(fmt, epi, m, n, k, seed=m + n, route=route)


@pytest.mark.parametrize("epi", [RES, GLU], ids=["residual", "swiglu"])
@pytest.mark.parametrize("fmt", ALL)
def test_epilogue_small_m_every_row_group(fmt, epi):
    for m in (2, 4, 5, 8, 9, 12, 16):
        case(fmt, epi, m, 200, 1024, seed=20 + m, route="skinny")
        case(fmt, epi, m, 200, 1024, seed=20 + m, route="stream")


@pytest.mark.parametrize("fmt", [Q8, Q4])
def test_residual_stream_split_k(fmt):
    """The f16 matrix-core stream adds the residual in the last arrival of a
    split-K row group (forced splits) as well as in a single split."""
    try:
        for p, sp in ((1, 1), (5, 3), (2, 8)):
            wq.wq_set_stream_plan(p, sp)
            for m in (1, 5, 16):
                case(fmt, RES, m, 333, 2048, seed=40 + m, route="stream")
    finally:
        wq.wq_set_stream_plan(0, 0)


PLAN = [(F16, 37, 300, 640), (Q8, 130, 97, 1024), (Q4, 37, 300, 640), (F16, 5, 77, 1003)]


@pytest.mark.parametrize("epi", [RES, GLU], ids=["residual", "swiglu"])
@pytest.mark.parametrize("p", PLAN, ids=[f"fmt{f}-{m}x{n}x{k}" for f, m, n, k in PLAN])
def test_epilogue_every_gemm_tiling_and_split(p, epi):
    """Every compiled tile with 1, 2 and 5 K splits: the epilogue in the GEMM's
    store (one split) and in the split reduction.  SwiGLU pairs gate and up
    fragments inside a tile, so tiles with an odd fragment count per wave fall
    back to the planner's choice; the result must match either way."""
    fmt, m, n, k = p
    rows = 2 * n if epi == GLU else n
    ref_b, dev_b = encoded(rows, k, fmt, 31)
    a = wqgen.activations(m, k, 31)
    r = wqgen.residual(m, n, 31) if epi == RES else None
    c_ref, bound = oracle.matmul_epilogue(a, ref_b, fmt, m, n, k, epi, r)
    prev = wq.wq_set_forced_route(wq.WQ_ROUTE_GEMM)
    try:
        for bm, bn in wq.GEMM_TILES:
            for sp in (1, 2, 5):
                say(f"plan {bm}x{bn}/{sp} epi={epi} fmt={fmt} {m}x{n}x{k}")
                wq.wq_set_gemm_plan(bm, bn, sp)
                c = run_ex(a, dev_b, m, n, k, fmt, epi, r)
                assert_close(c, c_ref, bound, f"plan {bm}x{bn}/{sp} epi={epi}")
    finally:
        wq.wq_set_gemm_plan(0, 0, 0)
        wq.wq_set_forced_route(prev)


@pytest.mark.parametrize("fmt", ALL)
def test_decode_ffn_shapes(fmt):
    """Decode (M = 1) at the FFN shapes: gate||up [2 x 11008, 4096] with SwiGLU and
    the down projection [4096, 11008] added into the residual stream."""
    case(fmt, GLU, 1, 11008, 4096, seed=41)
    case(fmt, RES, 1, 4096, 11008, seed=42)
    case(fmt, RES, 1, 2048, 6144, seed=43)


GEMV_K = {F16: [64, 1000, 2048, 4096, 8192, 10000, 16384, 24584, 32768, 32776, 1001, 12],
          Q8: [256, 768, 1024, 1536, 2048, 4096, 6144, 8192, 10240, 992],
          Q4: [256, 768, 1024, 1536, 2048, 4096, 6144, 8192, 10240, 992]}


@pytest.mark.parametrize("epi", [RES, GLU], ids=["residual", "swiglu"])
@pytest.mark.parametrize("fmt", ALL)
def test_decode_every_gemv_variant(fmt, epi):
    """M = 1 over every GEMV kernel family: f16 K-split blocks of 1..16 waves
    with 1, 2 or 4 chunk slots per lane (K a multiple of the split or not, up
    to K = 32768; 32776 takes the plain kernel), 16/32/64 lanes per quantized
    row with 1..4 blocks per lane (SwiGLU fused in the GEMV), and the shapes
    that take one GEMV over all 2n rows plus an element-wise pass (quantized
    K > 8192 or K % 256 != 0, f16 K % 8 != 0 or K > 32768)."""
    for k in GEMV_K[fmt]:
        for n in (37, 1000):
            case(fmt, epi, 1, n, k, seed=k + n, route="gemv")


@pytest.mark.parametrize("epi", [RES, GLU], ids=["residual", "swiglu"])
@pytest.mark.parametrize("fmt", ALL)
def test_prefill_full(fmt, epi):
    """M = 512 prefill at the FFN shapes (gate||up 2 x 11008 rows with SwiGLU, down
    11008 -> 4096 into the residual): every output against the oracle."""
    m, k = 512, 4096
    n = 11008 if epi == GLU else 4096
    kk = k if epi == GLU else 11008
    say(f"prefill epi={epi} fmt={fmt} {m}x{n}x{kk}")
    rows = 2 * n if epi == GLU else n
    ref_b, dev_b = encoded(rows, kk, fmt, 51)
    a = wqgen.activations(m, kk, 51)
    r = wqgen.residual(m, n, 51) if epi == RES else None
    c = run_ex(a, dev_b, m, n, kk, fmt, epi, r)
    c_ref, bound = oracle.matmul_epilogue(a, ref_b, fmt, m, n, kk, epi, r)
    assert_close(c, c_ref, bound, f"prefill epi={epi} fmt={fmt}")


@pytest.mark.parametrize("fmt", ALL)
def test_swiglu_split_k_is_deterministic(fmt):
    """Split partial sums are reduced in split order: two runs agree bit for bit."""
    m, n, k = 3, 64, 8192
    ref_b, dev_b = encoded(2 * n, k, fmt, 61)
    a = wqgen.activations(m, k, 61)
    prev = wq.wq_set_forced_route(wq.WQ_ROUTE_GEMM)
    try:
        say(f"determinism fmt={fmt}")
        c1 = run_ex(a, dev_b, m, n, k, fmt, GLU)
        c2 = run_ex(a, dev_b, m, n, k, fmt, GLU)
    finally:
        wq.wq_set_forced_route(prev)
    assert np.array_equal(c1, c2)


def test_residual_accumulates_in_place():
    """Two residual calls add the product twice: C = R + 2 A.B^T."""
    m, n, k = 4, 300, 2048
    ref_b, dev_b = encoded(n, k, F16, 71)
    a = wqgen.activations(m, k, 71)
    r = wqgen.residual(m, n, 71)
    at = torch.from_numpy(a).cuda()
    c = torch.from_numpy(r.copy()).cuda()
    say("residual twice")
    for _ in range(2):
        wq.wq_matmul_ex(at, dev_b, c, m, n, k, F16, RES)
    torch.cuda.synchronize()
    s, sb = oracle.matmul(a, ref_b, F16, m, n, k)
    want = r.astype(np.float64) + 2 * s
    assert_close(c.cpu().numpy(), want, 2 * sb + 2.0 ** -22 * (np.abs(r) + 2 * np.abs(s)), "residual twice")


@pytest.mark.parametrize("fmt", ALL)
def test_sub_matrix_of_fused_buffer(fmt):
    """Offsets into a fused weight buffer need no extra argument: b advanced by
    whole rows (the up half of gate||up, as dispatch_gemm_at binds it) gives the
    product with those rows alone, on every route."""
    n, k = 300, 1024
    ref_b, dev_b = encoded(2 * n, k, fmt, 81)
    up_ref, up_dev = ref_b[n:], dev_b[n:]
    assert up_dev.is_contiguous()
    for m in (1, 3, 40):
        a = wqgen.activations(m, k, 81)
        say(f"sub-matrix fmt={fmt} m={m}")
        c = torch.full((m, n), float("nan"), device="cuda")
        wq.wq_matmul(torch.from_numpy(a).cuda(), up_dev, c, m, n, k, fmt)
        torch.cuda.synchronize()
        c_ref, bound = oracle.matmul(a, np.ascontiguousarray(up_ref), fmt, m, n, k)
        assert_close(c.cpu().numpy(), c_ref, bound, f"up half m={m}")


def test_k0_epilogues():
    """K == 0 (f16): the empty sum is 0, so NONE and SWIGLU write zeros and
    RESIDUAL leaves C unchanged."""
    m, n = 3, 17
    a = torch.empty(0, device="cuda")
    b = torch.empty(0, dtype=torch.uint16, device="cuda")
    r = wqgen.residual(m, n, 91)
    say("k=0 epilogues")
    for epi in (wq.WQ_EPI_NONE, RES, GLU):
        c = torch.from_numpy(r.copy()).cuda()
        wq.wq_matmul_ex(a, b, c, m, n, 0, F16, epi)
        torch.cuda.synchronize()
        want = r if epi == RES else np.zeros_like(r)
        assert np.array_equal(c.cpu().numpy(), want), epi
