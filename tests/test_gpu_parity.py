"""GPU parity: libwqmm (through its C ABI) against the CPU oracle.

Both sides draw the same seeded f32 inputs from ``wqgen``; each side encodes
the weights with its own code (the library's wq_pack_f16 / wq_quantize_q8_0 on
the GPU, the oracle's encoders on the CPU) and the encoded bytes must agree
bit for bit.  Products must satisfy, per element,
    |c - c_ref| <= 1e-5 * sum_k |a_k w_k| + 1e-6,
with c_ref the oracle's float64 result.  Outputs are poisoned with NaN before
every launch, so an element that is never written fails.

Sizes: the oracle computes every output of every case, the M = 512 prefill and
the M = 512 sweep (5.6 M outputs) included.  Hand-built Q8_0 / Q4_0 blocks the
quantiser never writes (zero, subnormal, negative and largest scales, code
-128) go through every route with one-hot rows of A and must come back bit for
bit.
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
DECODE_SHAPES = [(6144, 2048), (2048, 6144), (2048, 2048), (151936, 2048)]
SWEEP_SHAPES = [(11008, 4096), (4096, 11008)]
SWEEP_M = [1, 2, 4, 8, 16, 64, 512]


def say(msg: str):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)
    yield
    wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)


# ------------------------------------------------------------------ inputs --
@functools.lru_cache(maxsize=6)
def weights_f32(n, k, seed=0):
    return wqgen.weights(n, k, seed)


@functools.lru_cache(maxsize=6)
def acts(m, k, seed=0):
    return wqgen.activations(m, k, seed)


@functools.lru_cache(maxsize=6)
def encoded(n, k, fmt, seed=0):
    """(oracle bytes, library bytes on the GPU) for the same f32 weights; for
    Q4_0 (no encoder on the pages) the same synthetic bytes on both sides."""
    if fmt == Q4:
        raw = wqgen.q4_0_bytes(n, k, seed)
        dev = torch.from_numpy(raw).cuda()
        torch.cuda.synchronize()
        return raw, dev
    w = weights_f32(n, k, seed)
    ref = oracle.encode(w, fmt)
    wd = torch.from_numpy(w).cuda()
    dev = wq.pack_f16(wd) if fmt == F16 else wq.quantize_q8_0(wd)
    torch.cuda.synchronize()
    del wd
    return ref, dev


def _entry(name, fmt):
    if name == "gemv":
        f = {F16: wq.wq_gemv_f16, Q8: wq.wq_gemv_q8_0, Q4: wq.wq_gemv_q4_0}[fmt]
        return lambda a, b, c, m, n, k: f(a, b, c, n, k)
    if name == "gemm":
        f = {F16: wq.wq_gemm_f16, Q8: wq.wq_gemm_q8_0, Q4: wq.wq_gemm_q4_0}[fmt]
        return lambda a, b, c, m, n, k: f(a, b, c, m, n, k)
    return lambda a, b, c, m, n, k: wq.wq_matmul(a, b, c, m, n, k, fmt)


def run_gpu(entry, fmt, a_np, b_dev, m, n, k, stream=None):
    a = torch.from_numpy(np.ascontiguousarray(a_np)).cuda()
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    fn = _entry(entry, fmt)
    if stream is None:
        fn(a, b_dev, c, m, n, k)
    else:
        with torch.cuda.stream(stream):
            fn(a, b_dev, c, m, n, k)
    torch.cuda.synchronize()
    return c.cpu().numpy()


def assert_close(c, c_ref, bound, what):
    err = np.abs(c.astype(np.float64) - c_ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        det = [(tuple(i), float(c[tuple(i)]), float(c_ref[tuple(i)]), float(bound[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, e.g. {det}")
    return float(np.max(err / bound)) if err.size else 0.0


def full_case(entry, fmt, m, n, k, seed=0):
    say(f"{entry} fmt={fmt} m={m} n={n} k={k} seed={seed}")
    ref_b, dev_b = encoded(n, k, fmt, seed)
    a = acts(m, k, seed)
    c = run_gpu(entry, fmt, a, dev_b, m, n, k)
    c_ref, bound = oracle.matmul(a, ref_b, fmt, m, n, k)
    return assert_close(c, c_ref, bound, f"{entry} fmt={fmt} {m}x{n}x{k}")


# ------------------------------------------------------- weight encoding --
@pytest.mark.parametrize("fmt", [F16, Q8])
@pytest.mark.parametrize("nk", [(1024, 1024), (6144, 2048), (2048, 6144), (151936, 2048), (4096, 11008), (3, 96)])
def test_weight_encoding_bit_exact(fmt, nk):
    n, k = nk
    say(f"encode fmt={fmt} n={n} k={k}")
    ref, dev = encoded(n, k, fmt)
    got = dev.cpu().numpy()
    assert got.shape == ref.shape
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))


def test_pack_f16_special_values():
    say("pack_f16 special values")
    x = np.array([1.0, -2.0, 65504.0, 65519.875, 65520.0, 1e6, -1e6, 2.0 ** -14, 2.0 ** -24, 2.0 ** -25,
                  1.5 * 2.0 ** -24, 1023.5 * 2.0 ** -24, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -149,
                  -2.0 ** -149, -0.0, 0.0, np.inf, -np.inf, 0.1, 0.02], dtype=np.float32)
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 32, size=1 << 18, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([x, bits.view(np.float32)])
    finite_or_inf = ~np.isnan(x)
    got = wq.pack_f16(torch.from_numpy(x).cuda()).cpu().numpy()
    ref = oracle.f16_bits(x)
    assert np.array_equal(got[finite_or_inf], ref[finite_or_inf])
    g = got[~finite_or_inf]
    assert np.all((g & 0x7c00) == 0x7c00) and np.all((g & 0x3ff) != 0)  # NaN stays NaN


def test_quantize_q8_0_golden_and_edges():
    say("quantize_q8_0 ties, zero blocks, tiny and huge scales")
    rng = np.random.default_rng(11)
    blocks = [
        np.array([127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 0.49] + [0] * 24, np.float32),
        np.zeros(32, np.float32),
        (rng.standard_normal(32) * 1e-30).astype(np.float32),
        (rng.standard_normal(32) * 1e4).astype(np.float32),
        (rng.standard_normal(32) * 2e7).astype(np.float32),    # d beyond the f16 range: scale inf
        np.full(32, -3.0, np.float32),
    ]
    x = np.concatenate(blocks + [rng.standard_normal(32 * 4096).astype(np.float32)])
    got = wq.quantize_q8_0(torch.from_numpy(x.reshape(1, -1)).cuda()).cpu().numpy()
    ref = oracle.q8_0_quantize(x.reshape(1, -1))
    assert np.array_equal(got, ref)


# ---------------------------------------------------------- configurations --
def test_gemv_f16_1024():
    """GEMV M=1, K=1024, N=1024, f16 weights, seed 0."""
    full_case("matmul", F16, 1, 1024, 1024)
    full_case("gemv", F16, 1, 1024, 1024)


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("nk", DECODE_SHAPES)
def test_decode_suite(fmt, nk):
    """Decode GEMV at hidden 2048: gate/up, down, o_proj, LM head."""
    n, k = nk
    full_case("matmul", fmt, 1, n, k)


@pytest.mark.parametrize("nk", [(6144, 2048), (2048, 6144)])
def test_prefill_f16_m512(nk):
    """The f16 prefill at M = 512: every one of the 3.1 M outputs against the oracle."""
    n, k = nk
    full_case("matmul", F16, 512, n, k)


@pytest.mark.parametrize("fmt", [Q8, Q4])
@pytest.mark.parametrize("nk", SWEEP_SHAPES)
@pytest.mark.parametrize("m", SWEEP_M)
def test_quant_sweep(fmt, nk, m):
    """The M sweep, every output against the oracle (up to 5.6 M at M = 512)."""
    n, k = nk
    full_case("matmul", fmt, m, n, k)


# ---------------------------------------------------------- ragged / edges --
RAGGED = [(1, 1, 32), (1, 7, 96), (1, 129, 1056), (1, 1000, 4128), (1, 33, 256), (1, 65, 8192),
          (2, 5, 64), (3, 77, 160), (17, 130, 288), (130, 97, 320), (257, 300, 512), (33, 1, 2048),
          (1, 300, 20480), (5, 4099, 256)]


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("mnk", RAGGED, ids=[f"{m}x{n}x{k}" for m, n, k in RAGGED])
def test_ragged(fmt, mnk):
    m, n, k = mnk
    full_case("matmul", fmt, m, n, k, seed=1)
    if m == 1:
        full_case("gemm", fmt, m, n, k, seed=1)


# Quantized GEMV rows of more than 128 blocks split K over the waves of a
# workgroup (one 64-block slice per wave): slices of 8 blocks at the end
# (K = 4352), 16 waves with one row per workgroup (K = 32768), row counts
# that leave the last workgroup partial, and the down / sweep shapes.
LONG_K = [(1, 4352), (3, 4352), (5, 6144), (513, 6144), (2048, 6144), (77, 11008), (4096, 11008), (9, 32768),
          (130, 16640)]


@pytest.mark.parametrize("fmt", [Q8, Q4])
@pytest.mark.parametrize("nk", LONG_K, ids=[f"{n}x{k}" for n, k in LONG_K])
def test_gemv_long_k_split(fmt, nk):
    n, k = nk
    full_case("gemv", fmt, 1, n, k, seed=11)


@pytest.mark.parametrize("fmt", [Q8, Q4])
def test_gemv_long_k_onehot_bit_exact(fmt):
    """a = e_j through the K-split GEMV returns column j of the decoded weights
    exactly, for a block in every wave's slice and at slice edges."""
    n, k = 515, 6144
    ref_b, dev_b = encoded(n, k, fmt, 12)
    w = oracle.decode(ref_b, fmt, n, k)
    for j in (0, 31, 32, 2047, 2048, 2080, 4095, 4096, 6143):
        say(f"long-K one-hot fmt={fmt} j={j}")
        a = np.zeros((1, k), np.float32)
        a[0, j] = 1.0
        c = run_gpu("gemv", fmt, a, dev_b, 1, n, k)
        assert np.array_equal(c[0].astype(np.float64), w[:, j]), f"gemv column {j}"


@pytest.mark.parametrize("fmt", [Q8, Q4])
def test_gemv_long_k_deterministic_and_linear(fmt):
    """The K-split GEMV sums its wave partials in a fixed order: repeated calls
    are bitwise identical, C(2a) = 2 C(a) and C(-a) = -C(a)."""
    n, k = 515, 11008
    say(f"long-K determinism fmt={fmt}")
    _, dev_b = encoded(n, k, fmt, 13)
    a = acts(1, k, 13)
    c1 = run_gpu("gemv", fmt, a, dev_b, 1, n, k)
    assert np.array_equal(c1, run_gpu("gemv", fmt, a, dev_b, 1, n, k))
    assert np.array_equal(run_gpu("gemv", fmt, 2 * a, dev_b, 1, n, k), 2 * c1)
    assert np.array_equal(run_gpu("gemv", fmt, -a, dev_b, 1, n, k), -c1)


@pytest.mark.parametrize("mnk", [(1, 37, 1), (1, 50, 7), (2, 19, 33), (1, 64, 1001), (9, 40, 999), (1, 8, 4100)])
def test_f16_any_k(mnk):
    """K not a multiple of 8 (or of 32): the general code paths."""
    m, n, k = mnk
    full_case("matmul", F16, m, n, k, seed=2)
    full_case("gemm", F16, m, n, k, seed=2)


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("entry", ["gemv", "gemm", "matmul"])
def test_misaligned_pointers(fmt, entry):
    """a offset by 4 bytes and b by 2 bytes from 16-byte alignment (wq_matmul
    at M = 3 takes the small-M kernel's scalar-load variant)."""
    m, n, k = (3 if entry == "matmul" else 1, 300, 2048)
    say(f"misaligned {entry} fmt={fmt}")
    ref_b, dev_b = encoded(n, k, fmt, 3)
    a = acts(m, k, 3)
    raw = dev_b.view(-1).view(torch.uint8)
    b_buf = torch.empty(raw.numel() + 2, dtype=torch.uint8, device="cuda")
    b_buf[2:].copy_(raw)
    a_buf = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
    a_buf[1:].copy_(torch.from_numpy(a.ravel()))
    c = torch.full((m, n), float("nan"), device="cuda")
    # Shifted pointers go through the C ABI directly (the binding takes whole tensors).
    L = wq._lib
    s = torch.cuda.current_stream().cuda_stream
    bp = b_buf.data_ptr() + 2
    if entry == "gemv":
        fn = {F16: L.wq_gemv_f16, Q8: L.wq_gemv_q8_0, Q4: L.wq_gemv_q4_0}[fmt]
        st = fn(a_buf.data_ptr() + 4, bp, c.data_ptr(), n, k, s)
    elif entry == "matmul":
        st = L.wq_matmul(a_buf.data_ptr() + 4, bp, c.data_ptr(), m, n, k, fmt, s)
    else:
        fn = {F16: L.wq_gemm_f16, Q8: L.wq_gemm_q8_0, Q4: L.wq_gemm_q4_0}[fmt]
        st = fn(a_buf.data_ptr() + 4, bp, c.data_ptr(), m, n, k, s)
    assert st == wq.WQ_OK
    torch.cuda.synchronize()
    c_ref, bound = oracle.matmul(a, ref_b, fmt, m, n, k)
    assert_close(c.cpu().numpy(), c_ref, bound, "misaligned")


@pytest.mark.parametrize("fmt", ALL)
def test_onehot_a_dequant_bit_exact(fmt):
    """a = e_j gives c[n] = w[n, j] exactly: the decode is bit-exact, through the
    GEMV and through the GEMM."""
    n, k = 4099, 2048
    say(f"one-hot a fmt={fmt}")
    ref_b, dev_b = encoded(n, k, fmt, 4)
    w = oracle.decode(ref_b, fmt, n, k)
    js = [0, 1, 31, 32, 33, 1000, 2047]
    a = np.zeros((len(js), k), np.float32)
    for i, j in enumerate(js):
        a[i, j] = 1.0
    for i, j in enumerate(js):
        c = run_gpu("gemv", fmt, a[i:i + 1], dev_b, 1, n, k)
        assert np.array_equal(c[0].astype(np.float64), w[:, j]), f"gemv column {j}"
    c = run_gpu("gemm", fmt, a, dev_b, len(js), n, k)
    for i, j in enumerate(js):
        assert np.array_equal(c[i].astype(np.float64), w[:, j]), f"gemm column {j}"


@pytest.mark.parametrize("fmt", ALL)
def test_identity_a_gives_transposed_weights(fmt):
    """A = I (M = K) gives C = W^T exactly: checks the matrix-core lane layout
    and every tile edge of the GEMM."""
    for (n, k) in [(96, 256), (300, 160)]:
        say(f"identity a fmt={fmt} n={n} k={k}")
        ref_b, dev_b = encoded(n, k, fmt, 5)
        w = oracle.decode(ref_b, fmt, n, k)
        c = run_gpu("gemm", fmt, np.eye(k, dtype=np.float32), dev_b, k, n, k)
        assert np.array_equal(c.astype(np.float64), w.T)


@pytest.mark.parametrize("fmt", ALL)
def test_empty_and_k0(fmt):
    say(f"empty outputs fmt={fmt}")
    c = torch.full((4, 8), float("nan"), device="cuda")
    a = torch.zeros(4 * 64, device="cuda")
    b = torch.zeros(8 * 64 * 2, dtype=torch.uint8, device="cuda")
    wq.wq_matmul(a, b, c, 0, 8, 64, fmt)
    wq.wq_matmul(a, b, c, 4, 0, 64, fmt)
    torch.cuda.synchronize()
    assert torch.isnan(c).all()
    if fmt == F16:
        wq.wq_matmul(None, None, c, 4, 8, 0, F16)
        wq.wq_gemv_f16(None, None, c, 8, 0)
        torch.cuda.synchronize()
        assert (c == 0).all()
    else:
        with pytest.raises(wq.WQError):
            wq.wq_matmul(a, b, c, 4, 8, 0, fmt)


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("m", [1, 7, 512])
def test_deterministic_and_linear(fmt, m):
    """Repeated calls are bitwise identical; C(2A) = 2 C(A) and C(-A) = -C(A)
    (on the f16 matrix-core route up to the rounding of the matrix core)."""
    n, k = 2048, 2048
    say(f"determinism fmt={fmt} m={m}")
    _, dev_b = encoded(n, k, fmt, 6)
    a = acts(m, k, 6)
    c1 = run_gpu("matmul", fmt, a, dev_b, m, n, k)
    c2 = run_gpu("matmul", fmt, a, dev_b, m, n, k)
    assert np.array_equal(c1, c2)
    assert np.array_equal(run_gpu("matmul", fmt, 2 * a, dev_b, m, n, k), 2 * c1)
    cneg = run_gpu("matmul", fmt, -a, dev_b, m, n, k)
    if wq.wq_route_for(m, n, k, fmt) in (wq.WQ_ROUTE_STREAM, wq.WQ_ROUTE_GEMM_HL):
        # The f16 matrix core's internal sums do not round symmetrically
        # (negating the operands can move a result by an ulp); the result is
        # still within the oracle's bound of the negated product.
        c_ref, bound = oracle.matmul(-a, encoded(n, k, fmt, 6)[0], fmt, m, n, k)
        assert_close(cneg, c_ref, bound, "C(-A)")
        assert_close(-cneg, -c_ref, bound, "-C(-A) against C(A)'s reference")
        assert np.all(np.abs(cneg + c1) <= bound), "C(-A) + C(A) beyond the tolerance"
    else:
        assert np.array_equal(cneg, -c1)


@pytest.mark.parametrize("fmt", ALL)
def test_routes_agree_and_are_counted(fmt):
    """Every route gives the oracle's product for any M, and the path-proof
    counters show which kernels ran: the GEMV once per row of A (once for 2
    to 4 Q8_0 rows, which the register-chunk kernel takes together), either
    GEMM once, the small-M kernels once per 16 rows of A."""
    n, k = 1000, 1024
    ref_b, dev_b = encoded(n, k, fmt, 7)
    ms = (1, 2, 3, 20)
    c_ref = {m: oracle.matmul(acts(m, k, 7), ref_b, fmt, m, n, k) for m in ms}
    routes = (wq.WQ_ROUTE_GEMV, wq.WQ_ROUTE_GEMM, wq.WQ_ROUTE_SKINNY, wq.WQ_ROUTE_STREAM, wq.WQ_ROUTE_GEMM_HL)
    skinny = {1: (0, 0, 1, 0, 0), 2: (0, 0, 1, 0, 0), 3: (0, 0, 1, 0, 0), 20: (0, 0, 2, 0, 0)}
    stream = skinny if fmt == F16 else {m: (0, 0, 0, 1 if m <= 16 else 2, 0) for m in ms}
    gemm, hl = {m: (0, 1, 0, 0, 0) for m in ms}, {m: (0, 0, 0, 0, 1) for m in ms}
    expect = {
        wq.WQ_ROUTE_GEMV: {1: (1, 0, 0, 0, 0), 2: (2 if fmt == F16 else 1, 0, 0, 0, 0),
                           3: (1 if fmt == Q8 else 3, 0, 0, 0, 0), 20: (20, 0, 0, 0, 0)},
        wq.WQ_ROUTE_GEMM: gemm,
        wq.WQ_ROUTE_SKINNY: skinny,
        wq.WQ_ROUTE_STREAM: stream,
        wq.WQ_ROUTE_GEMM_HL: hl,
        # Two Q8_0 rows at K = 1024: the register-chunk GEMV (plan 4 x 2 x 1).
        wq.WQ_ROUTE_AUTO: {1: (1, 0, 0, 0, 0), 2: (1, 0, 0, 0, 0) if fmt == Q8 else stream[2],
                           3: stream[3], 20: hl[20]},
    }
    try:
        for route, per_call in expect.items():
            wq.wq_set_forced_route(route)
            for m in ms:
                say(f"route={route} fmt={fmt} m={m}")
                wq.wq_reset_route_counts()
                c = run_gpu("matmul", fmt, acts(m, k, 7), dev_b, m, n, k)
                assert_close(c, *c_ref[m], f"route {route} m={m}")
                assert tuple(wq.wq_route_count(r) for r in routes) == per_call[m]
    finally:
        wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)


def test_nondefault_stream():
    n, k = 2048, 2048
    say("non-default stream")
    ref_b, dev_b = encoded(n, k, F16, 8)
    s = torch.cuda.Stream()
    for m in (1, 64):
        a = acts(m, k, 8)
        c = run_gpu("matmul", F16, a, dev_b, m, n, k, stream=s)
        c_ref, bound = oracle.matmul(a, ref_b, F16, m, n, k)
        assert_close(c, c_ref, bound, f"stream m={m}")


# Quantized shapes with K % 256 == 0 take the staged small-M kernel: one step
# (K = 256, 512), a partial last step (K = 768: 16 + 8 blocks, K = 8448), ragged
# row tiles (N = 37, 300, 4099) and K split across workgroups (small N).
SKINNY_SHAPES = {F16: [(1, 8), (37, 1000), (300, 2048), (4099, 136), (19, 33), (64, 1001)],
                 Q8: [(1, 32), (37, 992), (300, 2080), (4099, 160), (64, 4096), (37, 512), (300, 768),
                      (4099, 256), (70, 8448), (1000, 2048)],
                 Q4: [(1, 32), (37, 992), (300, 2080), (4099, 160), (64, 4096), (37, 512), (300, 768),
                      (4099, 256), (70, 8448), (1000, 2048)]}


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("m", [1, 2, 4, 5, 8, 9, 12, 13, 16])
def test_small_m_kernel_every_row_group(fmt, m):
    """The small-M kernel (forced route) for every group count of A rows
    (MB = 1..4), ragged N, K with and without a partial step, K split across
    workgroups (small N), and K % 8 != 0 (f16 scalar-load variant)."""
    try:
        wq.wq_set_forced_route(wq.WQ_ROUTE_SKINNY)
        for n, k in SKINNY_SHAPES[fmt]:
            full_case("matmul", fmt, m, n, k, seed=10)
    finally:
        wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)


# The f16 matrix-core weight stream (quantized, K % 256 == 0): every row count
# of A up to 16, ragged N (row groups of 64 and 128 rows, tiles of 16), one
# superblock, odd superblock counts, K split across workgroups with the
# arrival ticket (including one superblock per split and more splits than row
# groups), and the automatic plan; K = 16384 at M > 12 is beyond the kernel's
# staging and falls back to the small-M kernel.
STREAM_SHAPES = [(1, 256), (37, 512), (300, 2048), (4099, 256), (64, 4096), (70, 8448), (1000, 2048),
                 (129, 11008), (16, 1792), (37, 16384)]
STREAM_PLANS = [(0, 0)] + [(i + 1, sp) for i in range(len(wq.STREAM_SHAPES)) for sp in (1, 3)] + [(1, 43), (5, 5)]


@pytest.mark.parametrize("fmt", [Q8, Q4])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 11, 16])
def test_stream_kernel_every_row_count(fmt, m):
    try:
        wq.wq_set_forced_route(wq.WQ_ROUTE_STREAM)
        for n, k in STREAM_SHAPES:
            full_case("matmul", fmt, m, n, k, seed=12)
    finally:
        wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)


@pytest.mark.parametrize("fmt", [Q8, Q4])
@pytest.mark.parametrize("plan", STREAM_PLANS, ids=[f"p{p}-s{s}" for p, s in STREAM_PLANS])
def test_stream_kernel_every_plan(fmt, plan):
    """Forced plans (every workgroup shape, K splits) agree with the oracle and
    are bitwise repeatable (wave partials and split partials are summed in a
    fixed order)."""
    try:
        wq.wq_set_forced_route(wq.WQ_ROUTE_STREAM)
        wq.wq_set_stream_plan(*plan)
        for m, n, k in ((1, 300, 2048), (7, 1000, 11008), (16, 4099, 4096), (3, 64, 256)):
            ref_b, dev_b = encoded(n, k, fmt, 13)
            a = acts(m, k, 13)
            say(f"stream plan {plan} fmt={fmt} {m}x{n}x{k}")
            c1 = run_gpu("matmul", fmt, a, dev_b, m, n, k)
            c2 = run_gpu("matmul", fmt, a, dev_b, m, n, k)
            assert np.array_equal(c1, c2), "not repeatable"
            c_ref, bound = oracle.matmul(a, ref_b, fmt, m, n, k)
            assert_close(c1, c_ref, bound, f"stream plan {plan}")
    finally:
        wq.wq_set_stream_plan(0, 0)
        wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)


def test_stream_kernel_on_many_streams():
    """Streams past the eighth get a private scratch allocation for the split
    partials; every stream must give the oracle's product."""
    m, n, k = 4, 1000, 4096
    ref_b, dev_b = encoded(n, k, Q8, 14)
    a = acts(m, k, 14)
    c_ref, bound = oracle.matmul(a, ref_b, Q8, m, n, k)
    streams = [torch.cuda.Stream() for _ in range(10)]
    try:
        wq.wq_set_forced_route(wq.WQ_ROUTE_STREAM)
        wq.wq_set_stream_plan(1, 4)
        for i, st in enumerate(streams):
            say(f"stream route on stream {i}")
            c = run_gpu("matmul", Q8, a, dev_b, m, n, k, stream=st)
            assert_close(c, c_ref, bound, f"stream {i}")
    finally:
        wq.wq_set_stream_plan(0, 0)
        wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)


PLAN_CASES = [(F16, 37, 300, 640), (Q8, 37, 300, 640), (F16, 130, 97, 1000), (F16, 5, 77, 1003),
              (Q8, 300, 129, 2080), (Q4, 37, 300, 640), (Q4, 300, 129, 2080)]


@pytest.mark.parametrize("case", PLAN_CASES, ids=[f"fmt{f}-{m}x{n}x{k}" for f, m, n, k in PLAN_CASES])
def test_every_gemm_tiling_and_split(case):
    """Every compiled tile shape with 1, 2, 3 and 5 K splits (forced through the
    plan hook) matches the oracle, including the K tail (K % 32 != 0) and the
    unaligned-K general path."""
    fmt, m, n, k = case
    ref_b, dev_b = encoded(n, k, fmt, 9)
    a = acts(m, k, 9)
    c_ref, bound = oracle.matmul(a, ref_b, fmt, m, n, k)
    try:
        for bm, bn in wq.GEMM_TILES:
            for sp in (1, 2, 3, 5):
                say(f"plan {bm}x{bn}/{sp} fmt={fmt} {m}x{n}x{k}")
                wq.wq_set_gemm_plan(bm, bn, sp)
                assert wq.wq_gemm_plan(m, n, k, fmt)[:2] == (bm, bn)
                c = run_gpu("gemm", fmt, a, dev_b, m, n, k)
                assert_close(c, c_ref, bound, f"plan {bm}x{bn}/{sp}")
    finally:
        wq.wq_set_gemm_plan(0, 0, 0)


# ------------------------------------------------------------ edge blocks --
# Hand-built blocks the quantiser never writes: zero, subnormal, negative,
# largest-magnitude and negative-zero scales, and every int8 code -128 .. 127
# (Q4_0: every nibble 0 .. 15).  The pages' kernels read the scale as a raw
# half, so any finite f16 is a valid scale.  One-hot rows of A make each output
# a single decoded weight, which every route must return bit for bit.
Q8_EDGE_SCALES = [0x0000, 0x0001, 0x03FF, 0xC000, 0x8000, 0x3C00, 0x7BFF, 0x0400, 0x8001, 0x2E66, 0xFBFF, 0x0200]
Q4_EDGE_SCALES = [0x0000, 0x0001, 0x03FF, 0x8400, 0xBC00, 0x3C00, 0x7BFF, 0x8001, 0xFBFF, 0x8000]


def edge_weights(fmt, n, k, seed=0):
    """Weight bytes [n, k/32 * bytes] of hand-built blocks: block j of row r takes
    scale list[(r + 3j) % len] and codes that run through every value."""
    nb = k // 32
    r = np.arange(n)[:, None, None]
    j = np.arange(nb)[None, :, None]
    scales = np.array(Q8_EDGE_SCALES if fmt == Q8 else Q4_EDGE_SCALES, np.uint16)
    sc = scales[(r[:, :, 0] + 3 * j[:, :, 0]) % len(scales)]                    # [n, nb]
    if fmt == Q8:
        raw = np.empty((n, nb, 34), np.uint8)
        i = np.arange(32)[None, None, :]
        raw[:, :, 2:] = ((7 * r + 13 * j + i + seed) % 256).astype(np.uint8)     # every code value
    else:
        raw = np.empty((n, nb, 18), np.uint8)
        i = np.arange(16)[None, None, :]
        lo, hi = (3 * r + 5 * j + i + seed) % 16, (11 * r + 7 * j + 2 * i + seed + 1) % 16
        raw[:, :, 2:] = (lo | (hi << 4)).astype(np.uint8)
    raw[:, :, 0] = (sc & 0xFF).astype(np.uint8)
    raw[:, :, 1] = (sc >> 8).astype(np.uint8)
    return raw.reshape(n, -1)


def onehot_positions(k, rng):
    """Columns hitting the first, second, a middle and the last block at code
    positions 0, 1, 15, 16 and 31, and a few random columns."""
    nb = k // 32
    blocks = sorted({0, min(1, nb - 1), nb // 2, nb - 1})
    pos = sorted({32 * b + i for b in blocks for i in (0, 1, 15, 16, 31)} | set(rng.integers(0, k, 6).tolist()))
    return pos


@pytest.mark.parametrize("fmt", [Q8, Q4])
@pytest.mark.parametrize("k", [96, 256, 1024, 2048, 2080, 8448])
def test_edge_blocks_every_route_bit_exact(fmt, k):
    """Hand-built edge blocks through the GEMV (staged: K = 256, 1024, 2048; K split
    over waves: K = 8448; plain: K = 96, 2080), the small-M kernel and the GEMM, with
    one-hot rows of A: each output equals the oracle's decoded weight exactly."""
    n = 37
    raw = edge_weights(fmt, n, k)
    w = oracle.decode(raw, fmt, n, k)
    pos = onehot_positions(k, np.random.default_rng(k))
    a = np.zeros((len(pos), k), np.float32)
    a[np.arange(len(pos)), pos] = 1.0
    want = w[:, pos].T                                        # [rows of A, n]
    dev_b = torch.from_numpy(raw).cuda()
    routes = ((wq.WQ_ROUTE_GEMV, "gemv"), (wq.WQ_ROUTE_SKINNY, "small-M"), (wq.WQ_ROUTE_STREAM, "stream"),
              (wq.WQ_ROUTE_GEMM, "gemm"), (wq.WQ_ROUTE_GEMM_HL, "f16 matrix-core gemm"))
    try:
        for route, name in routes:
            wq.wq_set_forced_route(route)
            for m0 in range(0, len(pos), 16):                 # the small-M kernel takes up to 16 rows
                rows = slice(m0, min(len(pos), m0 + 16))
                say(f"edge blocks fmt={fmt} k={k} route={name} rows {rows.start}..{rows.stop - 1}")
                c = run_gpu("matmul", fmt, a[rows], dev_b, rows.stop - rows.start, n, k)
                assert np.array_equal(c.astype(np.float64), want[rows]), f"{name} rows {rows}"
    finally:
        wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)
    if k in (256, 2080):
        try:
            for bm, bn in wq.GEMM_TILES:
                for sp in (1, 3):
                    say(f"edge blocks fmt={fmt} k={k} plan {bm}x{bn}/{sp}")
                    wq.wq_set_gemm_plan(bm, bn, sp)
                    c = run_gpu("gemm", fmt, a, dev_b, len(pos), n, k)
                    assert np.array_equal(c.astype(np.float64), want), f"plan {bm}x{bn}/{sp}"
        finally:
            wq.wq_set_gemm_plan(0, 0, 0)
        try:
            wq.wq_set_forced_route(wq.WQ_ROUTE_GEMM_HL)
            for bm, bn in wq.HGEMM_TILES:
                for sp in (1, 3):
                    say(f"edge blocks fmt={fmt} k={k} f16 matrix-core plan {bm}x{bn}/{sp}")
                    wq.wq_set_hgemm_plan(bm, bn, sp)
                    c = run_gpu("matmul", fmt, a, dev_b, len(pos), n, k)
                    assert np.array_equal(c.astype(np.float64), want), f"hl plan {bm}x{bn}/{sp}"
        finally:
            wq.wq_set_hgemm_plan(0, 0, 0)
            wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)


def chunk_plan_fits(fmt, k, rb, nf, nr):
    """Whether the register-chunk GEMV takes K with plan (rb, nf, nr): rows of
    C = B K / 512 16-byte chunks (B = 34 bytes per Q8_0 block, 18 per Q4_0
    block), C // 64 full units and rb groups of remainder lanes (C % 64
    rounded up to a power of two each) over at most four waves."""
    if k % 256:
        return False
    c = (34 if fmt == Q8 else 18) * (k // 32) // 16
    q, rem = c // 64, c % 64
    r2 = 1 << (rem - 1).bit_length() if rem else 0
    return max(-(-q // nf), -(-(r2 * rb) // (64 * nr)), 1) <= 4


CHUNK_K = [256, 1024, 2048, 2304, 3328, 4096, 6144, 11008]


@pytest.mark.parametrize("fmt", [Q8, Q4])
@pytest.mark.parametrize("plan", wq.GEMV_PLANS, ids=[f"{r}x{f}x{g}" for r, f, g in wq.GEMV_PLANS])
def test_chunk_gemv_every_plan(plan, fmt):
    """The register-chunk Q8_0 / Q4_0 GEMV under every plan it instantiates, at
    every K of CHUNK_K the plan takes (rows whose last chunks fill a whole unit
    or part of one, one to three remainder units, invalid full units in the
    last wave) and row counts that leave the last workgroup partial: full
    compares against the oracle, then one-hot rows of A over hand-built edge
    blocks, bit for bit."""
    ks = [k for k in CHUNK_K if chunk_plan_fits(fmt, k, *plan)]
    assert len(ks) >= 3, ks
    try:
        wq.wq_set_gemv_plan(*plan)
        for k in ks:
            for n in (1, 5, 37, 133):
                full_case("gemv", fmt, 1, n, k, seed=n + k)
            # Equal rows give equal f32 sums wherever they sit in a workgroup.
            raw1 = encoded(1, k, fmt, k)[0]
            same = np.ascontiguousarray(np.repeat(raw1, 37, axis=0))
            a1 = acts(1, k, k + 1)
            c = run_gpu("gemv", fmt, a1, torch.from_numpy(same).cuda(), 1, 37, k)
            assert np.all(c[0] == c[0, 0]), f"plan {plan} k={k}: equal rows differ {np.unique(c[0])}"
            n = 21
            raw = edge_weights(fmt, n, k, seed=2)
            w = oracle.decode(raw, fmt, n, k)
            dev_b = torch.from_numpy(raw).cuda()
            for col in onehot_positions(k, np.random.default_rng(k)):
                a = np.zeros((1, k), np.float32)
                a[0, col] = 1.0
                c = run_gpu("gemv", fmt, a, dev_b, 1, n, k)
                assert np.array_equal(c[0].astype(np.float64), w[:, col]), f"plan {plan} k={k} column {col}"
            say(f"chunk plan {plan} fmt={fmt} k={k} edge blocks")
    finally:
        wq.wq_set_gemv_plan(0, 0, 0)


# Plans the register-chunk GEMV compiles for 2 and 4 rows of A (its activation
# windows take NU * rows * 16 or 32 registers): (format, rows of A, plan).
ROW_PLANS = ([(Q8, 2, p) for p in ((16, 1, 1), (8, 1, 1), (4, 2, 1), (4, 3, 1))]
             + [(Q4, 2, p) for p in ((8, 1, 1), (4, 1, 1), (4, 2, 1))]
             + [(Q8, 4, p) for p in ((8, 1, 1), (4, 1, 1))])


@pytest.mark.parametrize("case", ROW_PLANS, ids=[f"fmt{f}-mr{r}-{p[0]}x{p[1]}x{p[2]}" for f, r, p in ROW_PLANS])
def test_chunk_gemv_several_rows_every_plan(case):
    """2 <= M <= 4 rows of A through one register-chunk launch (the GEMV route),
    under every plan compiled for that many rows, at every K of CHUNK_K the
    plan takes and row counts that leave the last workgroup partial: full
    compares against the oracle at every row count the kernel serves (3 rows
    on the 4-row kernel leave one padding row), equal weight rows giving equal sums,
    the residual epilogue, and hand-built edge blocks bit for bit through one
    one-hot row of A per row."""
    fmt, mr, plan = case
    ks = [k for k in CHUNK_K if chunk_plan_fits(fmt, k, *plan)]
    assert len(ks) >= 2, ks
    try:
        wq.wq_set_forced_route(wq.WQ_ROUTE_GEMV)
        wq.wq_set_gemv_plan(*plan)
        for k in ks:
            for m in range(mr // 2 + 1, mr + 1):
                for n in (5, 37, 133):
                    full_case("matmul", fmt, m, n, k, seed=n + k + m)
            say(f"rows fmt={fmt} mr={mr} plan {plan} k={k}")
            raw1 = encoded(1, k, fmt, k)[0]
            same = np.ascontiguousarray(np.repeat(raw1, 37, axis=0))
            a2 = acts(mr, k, k + 1)
            c = run_gpu("matmul", fmt, a2, torch.from_numpy(same).cuda(), mr, 37, k)
            for i in range(mr):
                assert np.all(c[i] == c[i, 0]), f"plan {plan} k={k} row {i}: equal rows differ"
            n = 21
            raw = edge_weights(fmt, n, k, seed=2)
            w = oracle.decode(raw, fmt, n, k)
            dev_b = torch.from_numpy(raw).cuda()
            cols = onehot_positions(k, np.random.default_rng(k))
            for j in range(0, len(cols) - mr + 1, mr):
                a = np.zeros((mr, k), np.float32)
                for i in range(mr):
                    a[i, cols[j + i]] = 1.0
                c = run_gpu("matmul", fmt, a, dev_b, mr, n, k)
                for i in range(mr):
                    assert np.array_equal(c[i].astype(np.float64), w[:, cols[j + i]]), (plan, k, cols[j + i])
        m, n, k = mr, 133, ks[-1]
        ref_b, dev_b = encoded(n, k, fmt, 4)
        a = acts(m, k, 4)
        c0 = np.random.default_rng(4).standard_normal((m, n)).astype(np.float32)
        c = torch.from_numpy(c0).cuda()
        wq.wq_matmul_ex(torch.from_numpy(a).cuda(), dev_b, c, m, n, k, fmt, wq.WQ_EPI_RESIDUAL)
        torch.cuda.synchronize()
        c_ref, bound = oracle.matmul(a, ref_b, fmt, m, n, k)
        assert_close(c.cpu().numpy() - c0, c_ref, bound + 1e-6 * np.abs(c0), "residual, several rows")
    finally:
        wq.wq_set_gemv_plan(0, 0, 0)
        wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)


@pytest.mark.parametrize("fmt", [Q8, Q4])
def test_chunk_gemv_residual_and_large_n(fmt):
    """Residual epilogue through the chunk kernel, and the automatic plans at the
    shapes they are chosen for (the LM head's plan on a 70000-row matrix)."""
    for n, k in ((70000, 2048), (9000, 4096), (300, 6144), (4096, 11008)):
        say(f"chunk auto plan fmt={fmt} n={n} k={k}")
        full_case("gemv", fmt, 1, n, k, seed=3)
    n, k = 133, 4096
    ref_b, dev_b = encoded(n, k, fmt, 4)
    a = acts(1, k, 4)
    c0 = np.random.default_rng(4).standard_normal((1, n)).astype(np.float32)
    c = torch.from_numpy(c0).cuda()
    wq.wq_matmul_ex(torch.from_numpy(a).cuda(), dev_b, c, 1, n, k, fmt, wq.WQ_EPI_RESIDUAL)
    torch.cuda.synchronize()
    c_ref, bound = oracle.matmul(a, ref_b, fmt, 1, n, k)
    assert_close(c.cpu().numpy() - c0, c_ref, bound + 1e-6 * np.abs(c0), "residual")


@pytest.mark.parametrize("fmt", [Q8, Q4])
def test_identity_a_edge_blocks(fmt):
    """A = I (M = K = 256) on the edge blocks: C = W^T exactly through the GEMM and the
    small-M kernel (16 launches of 16 rows)."""
    n, k = 45, 256
    raw = edge_weights(fmt, n, k, seed=5)
    w = oracle.decode(raw, fmt, n, k)
    dev_b = torch.from_numpy(raw).cuda()
    try:
        for route in (wq.WQ_ROUTE_GEMM, wq.WQ_ROUTE_SKINNY, wq.WQ_ROUTE_STREAM, wq.WQ_ROUTE_GEMM_HL):
            wq.wq_set_forced_route(route)
            say(f"identity a, edge blocks fmt={fmt} route={route}")
            c = run_gpu("matmul", fmt, np.eye(k, dtype=np.float32), dev_b, k, n, k)
            assert np.array_equal(c.astype(np.float64), w.T)
    finally:
        wq.wq_set_forced_route(wq.WQ_ROUTE_AUTO)


@pytest.mark.parametrize("fmt", [Q8, Q4])
@pytest.mark.parametrize("m", [1, 3, 16])
def test_partial_step_does_not_read_the_next_row(fmt, m):
    """K = 2080 (one 32-column block past the last full 256-column step) with a
    misaligned a (the small-M kernel's scalar-load variant) and b: the first eight
    blocks of every odd row have an infinite scale, so a kernel whose partial step
    let the next row's blocks into a row's sum would turn the even rows' outputs
    into inf or NaN.  Even rows must match the oracle."""
    n, k = 300, 2080
    raw = (wqgen.q4_0_bytes(n, k, 14) if fmt == Q4 else oracle.encode(weights_f32(n, k, 14), Q8)).copy()
    blk = 18 if fmt == Q4 else 34
    for j in range(8):
        raw[1::2, j * blk] = 0x00
        raw[1::2, j * blk + 1] = 0x7C                                  # +inf scale
    a = acts(m, k, 14)
    c_ref, bound = oracle.matmul(a, raw, fmt, m, n, k)
    dev = torch.from_numpy(raw.ravel()).cuda()
    b_buf = torch.empty(dev.numel() + 2, dtype=torch.uint8, device="cuda")
    b_buf[2:].copy_(dev)
    a_buf = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
    a_buf[1:].copy_(torch.from_numpy(a.ravel()))
    L = wq._lib
    s = torch.cuda.current_stream().cuda_stream
    for route in (wq.WQ_ROUTE_AUTO, wq.WQ_ROUTE_SKINNY, wq.WQ_ROUTE_GEMM, wq.WQ_ROUTE_GEMM_HL):
        say(f"partial step, next row inf, fmt={fmt} m={m} route={route}")
        c = torch.full((m, n), float("nan"), device="cuda")
        prev = wq.wq_set_forced_route(route)
        try:
            assert L.wq_matmul(a_buf.data_ptr() + 4, b_buf.data_ptr() + 2, c.data_ptr(), m, n, k, fmt, s) == wq.WQ_OK
            torch.cuda.synchronize()
        finally:
            wq.wq_set_forced_route(prev)
        got = c.cpu().numpy()
        assert_close(got[:, 0::2], c_ref[:, 0::2], bound[:, 0::2], f"route {route} even rows")
