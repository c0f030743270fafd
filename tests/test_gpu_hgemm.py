"""GPU parity of the tiled product on the f16 matrix cores (WQ_ROUTE_GEMM_HL):
each row of A is scaled by a power of two and carried as two f16 halves, the
weights as exact f16 numbers (f16 weights, or Q8_0 / Q4_0 codes with the block
scale applied in f32).

Every case compares against the CPU oracle's float64 product element by
element, |c - c_ref| <= 1e-5 * sum_k |a_k w_k| + 1e-6, with outputs poisoned
with NaN before the launch.  Cases: shapes spanning several tiles with ragged
M and N tails, every compiled tile with 1..5 K splits, rows of A with extreme
and mixed magnitudes (the per-row scale), zero rows, infinite entries, the
residual and SwiGLU epilogues, hand-built blocks through A = I (bit-exact),
and the M = 512 prefill shapes at full size.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gemm_wq_gemv_amd as wq
import oracle
import wqgen
from test_gpu_parity import assert_close, encoded, say, weights_f32

pytestmark = pytest.mark.gpu

F16, Q8, Q4 = wq.WQ_FMT_F16, wq.WQ_FMT_Q8_0, wq.WQ_FMT_Q4_0
ALL = [F16, Q8, Q4]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    prev = wq.wq_set_forced_route(wq.WQ_ROUTE_GEMM_HL)
    wq.wq_set_hgemm_plan(0, 0, 0)
    yield
    wq.wq_set_hgemm_plan(0, 0, 0)
    wq.wq_set_forced_route(prev)


def run(a_np, b_dev, m, n, k, fmt, epi=wq.WQ_EPI_NONE, c_init=None):
    a = torch.from_numpy(np.ascontiguousarray(a_np, dtype=np.float32)).cuda()
    if c_init is None:
        c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    else:
        c = torch.from_numpy(np.ascontiguousarray(c_init, dtype=np.float32)).cuda()
    wq.wq_reset_route_counts()
    wq.wq_matmul_ex(a, b_dev, c, m, n, k, fmt, epi)
    torch.cuda.synchronize()
    assert wq.wq_route_count(wq.WQ_ROUTE_GEMM_HL) == 1, "the call did not take the f16 matrix-core GEMM"
    return c.cpu().numpy()


# The last K is past the split pass's one-read limit (16384 columns): that row
# is read twice.
SHAPES = [(17, 100, 96), (64, 128, 256), (65, 300, 1056), (130, 257, 2080), (200, 520, 512), (512, 640, 384),
          (33, 90, 4128), (20, 70, 16448)]


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_matches_oracle(fmt, m, n, k):
    say(f"hgemm fmt={fmt} {m}x{n}x{k}")
    ref_b, dev_b = encoded(n, k, fmt, 3)
    a = wqgen.activations(m, k, 3)
    c = run(a, dev_b, m, n, k, fmt)
    c_ref, bound = oracle.matmul(a, ref_b, fmt, m, n, k)
    assert_close(c, c_ref, bound, f"hgemm fmt={fmt} {m}x{n}x{k}")


@pytest.mark.parametrize("fmt", ALL)
def test_every_tile_and_split(fmt):
    m, n, k = 150, 270, 800
    ref_b, dev_b = encoded(n, k, fmt, 4)
    a = wqgen.activations(m, k, 4)
    c_ref, bound = oracle.matmul(a, ref_b, fmt, m, n, k)
    try:
        for bm, bn in wq.HGEMM_TILES:
            for sp in (1, 2, 3, 5):
                say(f"hgemm tile {bm}x{bn} splits={sp} fmt={fmt}")
                wq.wq_set_hgemm_plan(bm, bn, sp)
                c = run(a, dev_b, m, n, k, fmt)
                assert_close(c, c_ref, bound, f"tile {bm}x{bn}/{sp} fmt={fmt}")
    finally:
        wq.wq_set_hgemm_plan(0, 0, 0)


def wide_range_rows(m, k, seed):
    """Rows whose magnitudes differ by many decades, within a row and across
    rows: the per-row power-of-two scale and both halves must hold them."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((m, k)).astype(np.float32)
    expo = rng.integers(-30, 30, size=(m, 1))
    a *= np.float32(10.0) ** expo.astype(np.float32)
    a[1] *= np.where(np.arange(k) % 7 == 0, 1e6, 1e-6).astype(np.float32)  # mixed within a row
    a[2] = 0.0                                                              # all-zero row
    a[3] = np.float32(1.0e36) * np.sign(a[3])                              # near the top of f32
    a[4] = np.float32(1e-40) * np.sign(a[4])                               # subnormal f32
    a[5, 0] = np.float32(2.0 ** 20)                                         # one dominant entry
    return a


@pytest.mark.parametrize("fmt", ALL)
def test_rows_of_extreme_magnitude(fmt):
    m, n, k = 40, 96, 512
    ref_b, dev_b = encoded(n, k, fmt, 5)
    a = wide_range_rows(m, k, 5)
    c = run(a, dev_b, m, n, k, fmt)
    c_ref, bound = oracle.matmul(a, ref_b, fmt, m, n, k)
    fin = np.isfinite(c_ref)
    assert_close(c[fin], c_ref[fin], bound[fin], f"extreme rows fmt={fmt}")
    assert np.array_equal(np.isinf(c), np.isinf(c_ref)) and np.array_equal(np.isnan(c), np.isnan(c_ref))


def test_infinite_entries_propagate():
    """An infinite entry of A gives +-inf (or NaN against a zero weight) in its
    row, as an f32 product would; other rows are untouched."""
    m, n, k = 20, 64, 256
    ref_b, dev_b = encoded(n, k, F16, 6)
    a = wqgen.activations(m, k, 6).copy()
    a[7, 10] = np.inf
    c = run(a, dev_b, m, n, k, F16)
    c_ref, bound = oracle.matmul(a, ref_b, F16, m, n, k)
    ok = np.arange(m) != 7
    assert_close(c[ok], c_ref[ok], bound[ok], "rows without inf")
    assert np.array_equal(np.isinf(c[7]), np.isinf(c_ref[7]))
    assert np.array_equal(np.sign(c[7][np.isinf(c[7])]), np.sign(c_ref[7][np.isinf(c_ref[7])]))


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("plan", [(0, 0, 0), (128, 128, 1), (64, 64, 3), (128, 64, 2)])
def test_epilogues(fmt, plan):
    """Residual (c += a . b^T) and SwiGLU (2n weight rows, gate then up) on the
    tile's own store (one split) and on the split-sum pass."""
    m, n, k = 70, 160, 640
    a = wqgen.activations(m, k, 7)
    try:
        wq.wq_set_hgemm_plan(*plan)
        for epi, rows in ((wq.WQ_EPI_RESIDUAL, n), (wq.WQ_EPI_SWIGLU, 2 * n)):
            say(f"hgemm epilogue {epi} fmt={fmt} plan={plan}")
            ref_b, dev_b = encoded(rows, k, fmt, 7)
            r = wqgen.residual(m, n, 7) if epi == wq.WQ_EPI_RESIDUAL else None
            c = run(a, dev_b, m, n, k, fmt, epi, c_init=r)
            c_ref, bound = oracle.matmul_epilogue(a, ref_b, fmt, m, n, k, epi, r)
            assert_close(c, c_ref, bound, f"epilogue {epi} fmt={fmt} plan={plan}")
    finally:
        wq.wq_set_hgemm_plan(0, 0, 0)


def test_identity_a_returns_the_decoded_weights_bit_for_bit():
    """A = I (and a scaled identity) through every tile: the f32 result is
    exactly the oracle's decode of each weight (hand-built Q8_0 / Q4_0 blocks
    with zero, subnormal, negative and largest scales included)."""
    n, k = 96, 96
    raw8 = oracle.encode(weights_f32(n, k, 11), Q8).copy()
    raw8[0, 0:2] = (0x00, 0x00)      # zero scale
    raw8[1, 0:2] = (0x01, 0x00)      # smallest subnormal
    raw8[2, 0:2] = (0xFF, 0x03)      # largest subnormal
    raw8[3, 0:2] = (0x00, 0xC0)      # -2
    raw8[4, 0:2] = (0xFF, 0x7B)      # 65504
    raw8[5, 2:34] = np.arange(-128, -96, dtype=np.int8).view(np.uint8)
    raw4 = wqgen.q4_0_bytes(n, k, 11).copy()
    raw4[0, 0:2] = (0x01, 0x00)
    raw4[1, 0:2] = (0x00, 0x80)      # -0
    raw4[2, 0:2] = (0x00, 0xBC)      # -1
    raw4[3, 2:18] = np.arange(16, dtype=np.uint8) * 17
    f16w = oracle.encode(weights_f32(n, k, 11), F16).copy()
    cases = [(F16, f16w), (Q8, raw8), (Q4, raw4)]
    for fmt, raw in cases:
        w = oracle.decode(raw, fmt, n, k)
        dev = torch.from_numpy(np.ascontiguousarray(raw)).cuda()
        for scale in (1.0, 2.0 ** -20):
            a = np.eye(k, dtype=np.float32) * np.float32(scale)
            for bm, bn in wq.HGEMM_TILES:
                say(f"identity fmt={fmt} scale={scale} tile {bm}x{bn}")
                wq.wq_set_hgemm_plan(bm, bn, 1)
                try:
                    c = run(a, dev, k, n, k, fmt)
                finally:
                    wq.wq_set_hgemm_plan(0, 0, 0)
                assert np.array_equal(c.astype(np.float64), (w.T * scale)), f"fmt={fmt} scale={scale} {bm}x{bn}"


@pytest.mark.parametrize("fmt,m,n,k", [(F16, 512, 6144, 2048), (F16, 512, 2048, 6144), (Q8, 512, 4096, 11008),
                                       (Q4, 512, 11008, 4096), (Q8, 64, 11008, 4096)])
def test_full_size_automatic_plan(fmt, m, n, k):
    """The benchmark's shapes with the planner's own tiling, every output
    against the oracle."""
    say(f"hgemm full size fmt={fmt} {m}x{n}x{k} plan={wq.wq_hgemm_plan(m, n, k, fmt)}")
    ref_b, dev_b = encoded(n, k, fmt, 0)
    a = wqgen.activations(m, k, 0)
    c = run(a, dev_b, m, n, k, fmt)
    c_ref, bound = oracle.matmul(a, ref_b, fmt, m, n, k)
    assert_close(c, c_ref, bound, f"full size fmt={fmt} {m}x{n}x{k}")
