"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself or with the GPU library.  Each
pin checks the oracle against one of:
  * values derived by hand from the pages (tests/golden/*.txt, cited there),
  * a library routine (struct's and numpy's binary16 codecs, numpy float64
    matmul on weights decoded by numpy),
  * exact rational arithmetic (fractions.Fraction) on small inputs,
  * invariants of the product (identity, one-hot, linearity, permutation).

``PINS`` is also run against deliberately broken copies of the oracle
(test_mutants_are_caught) to show that a plausible mistake anywhere in it --
a dropped term, a wrong sign, index or byte order, a wrong rounding rule --
fails at least one pin.
"""
from __future__ import annotations

import os
import shutil
import struct
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
import wqgen
from oracle import FMT_F16, FMT_Q4_0, FMT_Q8_0

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------- helpers --
def _parse_float(tok: str) -> float:
    if tok in ("inf", "-inf", "nan"):
        return float(tok)
    if "0x" in tok:
        return float.fromhex(tok)
    return float(tok)


def _golden_f16():
    rows = []
    with open(os.path.join(GOLDEN, "f16_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            rows.append((_parse_float(tok[0]), int(tok[1], 16)))
    return rows


def _golden_q8():
    blocks = []
    with open(os.path.join(GOLDEN, "q8_0_blocks.txt")) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    i = 0
    while i < len(lines):
        assert lines[i].startswith("block ")
        vals = [_parse_float(t) for t in lines[i + 1].split()]
        byts = bytes(int(t, 16) for t in lines[i + 2].split())
        blocks.append((lines[i][6:], np.array(vals, dtype=np.float32), byts))
        i += 3
    return blocks


def _golden_q4():
    blocks = []
    with open(os.path.join(GOLDEN, "q4_0_blocks.txt")) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    for i in range(0, len(lines), 3):
        assert lines[i].startswith("block ")
        byts = bytes(int(t, 16) for t in lines[i + 1].split())
        vals = [_parse_float(t) for t in lines[i + 2].split()]
        assert len(byts) == 18 and len(vals) == 32, lines[i]
        blocks.append((lines[i][6:], byts, np.array(vals, dtype=np.float64)))
    return blocks


def _golden_matmul():
    a, f16, q8, q4, c = {}, {}, {}, {}, {}
    dims = None
    with open(os.path.join(GOLDEN, "matmul_tiny.txt")) as f:
        for line in f:
            tok = line.split()
            if not tok or tok[0].startswith("#"):
                continue
            if tok[0] == "dims":
                dims = tuple(int(t) for t in tok[1:4])
            elif tok[0] == "a":
                a[(int(tok[1]), int(tok[2]))] = float(tok[3])
            elif tok[0] == "f16":
                f16[(int(tok[1]), int(tok[2]))] = int(tok[3], 16)
            elif tok[0] == "q8":
                q8[int(tok[1])] = bytes(int(t, 16) for t in tok[2:])
            elif tok[0] == "q4":
                q4[int(tok[1])] = bytes(int(t, 16) for t in tok[2:])
            elif tok[0] == "c":
                c[(int(tok[1]), int(tok[2]))] = float(tok[3])
    M, N, K = dims
    A = np.zeros((M, K), np.float32)
    for (m, k), v in a.items():
        A[m, k] = v
    B16 = np.zeros((N, K), np.uint16)
    for (n, k), v in f16.items():
        B16[n, k] = v
    B8 = np.frombuffer(b"".join(q8[n] for n in range(N)), dtype=np.uint8).reshape(N, -1)
    B4 = np.frombuffer(b"".join(q4[n] for n in range(N)), dtype=np.uint8).reshape(N, -1)
    C = np.zeros((M, N))
    for (m, n), v in c.items():
        C[m, n] = v
    return M, N, K, A, B16, B8, B4, C


def _numpy_decode(b, fmt, n, k):
    """Weights decoded with numpy's own binary16 codec (independent of the oracle)."""
    if fmt == FMT_F16:
        return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float64).reshape(n, k)
    if fmt == FMT_Q4_0:
        raw = np.ascontiguousarray(b, dtype=np.uint8).reshape(n, k // 32, 18)
        d = raw[:, :, 0:2].copy().view("<f2").astype(np.float64)          # [n, nb, 1]
        codes = np.empty((n, k // 32, 32), np.int64)
        codes[:, :, 0::2] = raw[:, :, 2:18] & 0x0F
        codes[:, :, 1::2] = raw[:, :, 2:18] >> 4
        return (d * (codes - 8)).reshape(n, k)
    raw = np.ascontiguousarray(b, dtype=np.uint8).reshape(n, k // 32, 34)
    d = raw[:, :, 0:2].copy().view("<f2").astype(np.float64)          # [n, nb, 1]
    q = raw[:, :, 2:34].copy().view(np.int8).astype(np.float64)       # [n, nb, 32]
    return (d * q).reshape(n, k)


def _dyadic_inputs(rng, m, n, k, fmt):
    a = (rng.integers(-4, 5, size=(m, k)) * 0.5).astype(np.float32)
    if fmt == FMT_F16:
        vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0, 0.25, -0.25], np.float16)
        b = vals[rng.integers(0, len(vals), size=(n, k))].view(np.uint16)
    elif fmt == FMT_Q4_0:
        blocks = []
        for _ in range(n * k // 32):
            d = [0x3800, 0x3c00, 0x3400, 0xb800][rng.integers(0, 4)]
            blocks.append(struct.pack("<H", d) + rng.integers(0, 256, size=16).astype(np.uint8).tobytes())
        b = np.frombuffer(b"".join(blocks), np.uint8).reshape(n, -1)
    else:
        blocks = []
        for _ in range(n * k // 32):
            d = [0x3800, 0x3c00, 0x3400][rng.integers(0, 3)]
            q = rng.integers(-4, 5, size=32).astype(np.int8)
            blocks.append(struct.pack("<H", d) + q.tobytes())
        b = np.frombuffer(b"".join(blocks), np.uint8).reshape(n, -1)
    return a, b


def _weights(orc, fmt, n, k, seed):
    """Encoded weights for the random-input pins: the oracle's f16 / Q8_0
    encoders on N(0, 0.02) draws, and wqgen's synthetic bytes for Q4_0 (the
    pages give no Q4_0 encoder)."""
    if fmt == FMT_Q4_0:
        return wqgen.q4_0_bytes(n, k, seed)
    return orc.encode(wqgen.normal((n, k), seed=seed, stream=1, std=0.02), fmt)


# ------------------------------------------------------------------- pins --
def pin_f16_decode_exhaustive(orc):
    """All 65536 binary16 patterns against struct's '<e' decoder."""
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.f16_value(bits)
    want = np.array([struct.unpack("<e", int(b).to_bytes(2, "little"))[0] for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_f16_encode_golden(orc):
    """Hand-derived patterns of tests/golden/f16_values.txt."""
    rows = _golden_f16()
    x = np.array([r[0] for r in rows], dtype=np.float32)
    want = np.array([r[1] for r in rows], dtype=np.uint16)
    got = orc.f16_bits(x)
    bad = [(float(x[i]).hex(), hex(got[i]), hex(want[i])) for i in range(len(x)) if got[i] != want[i]]
    assert not bad, bad


def pin_f16_encode_vs_numpy(orc):
    """Every exponent, with the fraction bits at and around each rounding point,
    against numpy's float32 -> float16 cast (round to nearest even)."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001,
                     0x3000, 0x4000, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(1234)
    u = np.concatenate([u, rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)])
    x = u.view(np.float32)
    finite = ~np.isnan(x)
    got = orc.f16_bits(x)
    with np.errstate(over="ignore", invalid="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got[finite], want[finite])
    # NaN keeps its sign, sets the quiet bit and stays NaN.
    g = got[~finite]
    assert np.all((g & 0x7c00) == 0x7c00) and np.all((g & 0x0200) == 0x0200)
    assert np.array_equal(g >> 15, (u[~finite] >> 31).astype(np.uint16))


def pin_q8_golden(orc):
    """Hand-derived blocks of tests/golden/q8_0_blocks.txt (ties round away from zero,
    little-endian scale, zero block, subnormal scale, clamp at +-127)."""
    for name, vals, byts in _golden_q8():
        assert vals.size == 32 and len(byts) == 34, name
        got = orc.q8_0_quantize(vals.reshape(1, 32)).tobytes()
        assert got == byts, (name, got.hex(" "), byts.hex(" "))


def pin_q8_roundtrip(orc):
    """Round trip of the quantiser on N(0, 0.02) and N(0, 1) weights.  With d the
    f32 scale the quantiser divides by (amax/127) and h = f16(d) the stored one:
      |x - d*q| <= d/2 + d*2^-16 (the slack covers the f32 product x * (1/d));
      the decoded weight is exactly h*q;
      |x - h*q| <= d/2 + 127*|d - h| + tiny."""
    for std in (0.02, 1.0):
        w = wqgen.normal((64, 256), seed=7, stream=9, std=std)
        b = orc.q8_0_quantize(w)
        raw = b.reshape(64, 8, 34)
        q = raw[:, :, 2:].copy().view(np.int8).astype(np.float64).reshape(64, 256)
        h = orc.f16_value(raw[:, :, 0].astype(np.uint16) | (raw[:, :, 1].astype(np.uint16) << 8))
        amax = np.abs(w.reshape(64, 8, 32)).max(axis=2)
        d = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float64)
        dd = np.repeat(d, 32, axis=1)
        hh = np.repeat(h, 32, axis=1)
        x = w.astype(np.float64)
        assert np.all(np.abs(x - dd * q) <= dd / 2 + dd * 2.0 ** -16)
        assert np.array_equal(orc.decode(b, FMT_Q8_0, 64, 256), hh * q)
        assert np.all(np.abs(x - hh * q) <= dd / 2 + 127 * np.abs(dd - hh) + 1e-12)
        assert np.all(np.abs(q) <= 127)
        # the largest |x| of every block maps to +-127
        idx = np.abs(w.reshape(64, 8, 32)).argmax(axis=2)
        qmax = np.take_along_axis(q.reshape(64, 8, 32), idx[:, :, None], axis=2)[:, :, 0]
        assert np.all(np.abs(qmax) == 127)


def pin_q8_decode_handbuilt(orc):
    """Blocks built byte by byte: scale 1.0, 0.5 and -2.0, every int8 code -128..127
    (the decoder accepts -128 though the quantiser never writes it)."""
    codes = np.arange(-128, 128, dtype=np.int8)
    for hbits, dval in ((0x3c00, 1.0), (0x3800, 0.5), (0xc000, -2.0)):
        blocks = b"".join(struct.pack("<H", hbits) + codes[i:i + 32].tobytes()
                          for i in range(0, 256, 32))
        b = np.frombuffer(blocks, np.uint8).reshape(1, -1)
        got = orc.decode(b, FMT_Q8_0, 1, 256)[0]
        assert np.array_equal(got, dval * codes.astype(np.float64))


def pin_q4_golden(orc):
    """Q4_0 blocks decoded by hand from the pages' Q4_0 kernels (tests/golden/q4_0_blocks.txt):
    little-endian scale, low nibble = even weight, code offset 8, negative and
    subnormal scales; a row of all the blocks and each block alone."""
    blocks = _golden_q4()
    row = np.frombuffer(b"".join(byts for _, byts, _ in blocks), np.uint8).reshape(1, -1)
    got = orc.decode(row, FMT_Q4_0, 1, 32 * len(blocks))[0]
    assert np.array_equal(got, np.concatenate([vals for _, _, vals in blocks]))
    for name, byts, vals in blocks:
        got = orc.decode(np.frombuffer(byts, np.uint8).reshape(1, 18), FMT_Q4_0, 1, 32)[0]
        assert np.array_equal(got, vals), name


def pin_matmul_golden(orc):
    """The hand-worked 2x3x32 example of tests/golden/matmul_tiny.txt, all three formats."""
    M, N, K, A, B16, B8, B4, C = _golden_matmul()
    for fmt, b in ((FMT_F16, B16), (FMT_Q8_0, B8), (FMT_Q4_0, B4)):
        c, _ = orc.matmul(A, b, fmt, M, N, K)
        assert np.array_equal(c, C), (fmt, c)


def pin_bruteforce_fraction(orc):
    """Tiny dyadic inputs: every product and sum is exact, so the oracle must equal
    exact rational arithmetic bit for bit; and on N(0,1) activations it must be
    within K * 2^-52 * sum|p| of the exact sum."""
    rng = np.random.default_rng(5)
    for fmt in (FMT_F16, FMT_Q8_0, FMT_Q4_0):
        for m in (1, 2, 3):
            for n in (1, 2, 3):
                for k in (32, 64):
                    a, b = _dyadic_inputs(rng, m, n, k, fmt)
                    w = _numpy_decode(b, fmt, n, k)
                    c, _ = orc.matmul(a, b, fmt, m, n, k)
                    for i in range(m):
                        for j in range(n):
                            exact = sum(Fraction(float(a[i, t])) * Fraction(float(w[j, t]))
                                        for t in range(k))
                            assert c[i, j] == float(exact)
        a = wqgen.normal((2, 96), seed=1, stream=0)
        b = _weights(orc, fmt, 3, 96, seed=1)
        w = _numpy_decode(b, fmt, 3, 96)
        c, _ = orc.matmul(a, b, fmt, 2, 3, 96)
        for i in range(2):
            for j in range(3):
                terms = [Fraction(float(a[i, t])) * Fraction(float(w[j, t])) for t in range(96)]
                exact = sum(terms)
                scale = float(sum(abs(t) for t in terms))
                assert abs(Fraction(c[i, j]) - exact) <= Fraction(96 * scale) * Fraction(1, 2 ** 52)


def pin_identity_and_onehot(orc):
    """B = I gives C = A exactly; a one-hot B row n (weight v at column j(n)) gives
    c[m,n] = a[m,j(n)] * v exactly, for f16 (incl. subnormal v) and Q8_0."""
    K = 64
    a = wqgen.normal((3, K), seed=2, stream=0)
    eye16 = np.where(np.eye(K, dtype=bool), 0x3c00, 0).astype(np.uint16)
    c, _ = orc.matmul(a, eye16, FMT_F16, 3, K, K)
    assert np.array_equal(c, a.astype(np.float64))
    blocks = []
    for n in range(K):
        for j in range(K // 32):
            q = np.zeros(32, np.int8)
            if n // 32 == j:
                q[n % 32] = 1
            blocks.append(struct.pack("<H", 0x3c00) + q.tobytes())
    eye8 = np.frombuffer(b"".join(blocks), np.uint8).reshape(K, -1)
    c, _ = orc.matmul(a, eye8, FMT_Q8_0, 3, K, K)
    assert np.array_equal(c, a.astype(np.float64))
    # one-hot rows
    N = 40
    cols = [(7 * n + 3) % K for n in range(N)]
    vals16 = [0x0001, 0x03ff, 0x0400, 0x3c00, 0xbc00, 0x7bff, 0x3555, 0xc001] * 5
    b16 = np.zeros((N, K), np.uint16)
    for n in range(N):
        b16[n, cols[n]] = vals16[n]
    c, _ = orc.matmul(a, b16, FMT_F16, 3, N, K)
    v = np.array([struct.unpack("<e", struct.pack("<H", h))[0] for h in vals16])
    assert np.array_equal(c, a[:, cols].astype(np.float64) * v[None, :])
    blocks = []
    qs = [1, -1, 127, -128, 5, -77, 64, 3] * 5
    ds = [0x3c00, 0x0001, 0x2e66, 0xc000, 0x7bff, 0x3800, 0x0400, 0x251f] * 5
    for n in range(N):
        for j in range(K // 32):
            q = np.zeros(32, np.int8)
            if cols[n] // 32 == j:
                q[cols[n] % 32] = qs[n]
            blocks.append(struct.pack("<H", ds[n]) + q.tobytes())
    b8 = np.frombuffer(b"".join(blocks), np.uint8).reshape(N, -1)
    c, _ = orc.matmul(a, b8, FMT_Q8_0, 3, N, K)
    dv = np.array([struct.unpack("<e", struct.pack("<H", h))[0] for h in ds])
    assert np.array_equal(c, a[:, cols].astype(np.float64) * (dv * np.array(qs))[None, :])
    # Q4_0: identity (code 9 = +1 on the diagonal, 8 = 0 elsewhere), then one-hot
    # rows with codes 0..15 (weights -8..7 times the scale)
    def q4_row(n_codes, d):
        nib = np.array(n_codes, np.uint8).reshape(-1, 32)
        packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        return b"".join(struct.pack("<H", d) + blk.tobytes() for blk in packed)
    eye4 = b"".join(q4_row([9 if t == n else 8 for t in range(K)], 0x3c00) for n in range(K))
    c, _ = orc.matmul(a, np.frombuffer(eye4, np.uint8).reshape(K, -1), FMT_Q4_0, 3, K, K)
    assert np.array_equal(c, a.astype(np.float64))
    us = [(3 * n) % 16 for n in range(N)]
    b4 = b"".join(q4_row([us[n] if t == cols[n] else 8 for t in range(K)], ds[n]) for n in range(N))
    c, _ = orc.matmul(a, np.frombuffer(b4, np.uint8).reshape(N, -1), FMT_Q4_0, 3, N, K)
    assert np.array_equal(c, a[:, cols].astype(np.float64) * (dv * (np.array(us) - 8))[None, :])


def pin_invariants(orc):
    """GEMV(a_m) equals GEMM row m; C(2A) = 2C(A) and C(-A) = -C(A) exactly;
    permuting the rows of B permutes the columns of C; entries match the full product."""
    M, N, K = 5, 37, 96
    a = wqgen.normal((M, K), seed=4, stream=0)
    for fmt in (FMT_F16, FMT_Q8_0, FMT_Q4_0):
        b = _weights(orc, fmt, N, K, seed=4)
        c, bound = orc.matmul(a, b, fmt, M, N, K)
        for m in range(M):
            cm, _ = orc.matmul(a[m:m + 1], b, fmt, 1, N, K)
            assert np.array_equal(cm[0], c[m])
        c2, _ = orc.matmul(2 * a, b, fmt, M, N, K)
        assert np.array_equal(c2, 2 * c)
        cn, _ = orc.matmul(-a, b, fmt, M, N, K)
        assert np.array_equal(cn, -c)
        perm = np.random.default_rng(0).permutation(N)
        cp, _ = orc.matmul(a, np.ascontiguousarray(b[perm]), fmt, M, N, K)
        assert np.array_equal(cp, c[:, perm])
        rows = np.array([0, 4, 2, 1, 3])
        cols = np.array([36, 0, 17, 5, 20])
        ce, be = orc.matmul_entries(a, b, fmt, M, N, K, rows, cols)
        assert np.array_equal(ce, c[rows, cols]) and np.array_equal(be, bound[rows, cols])


def pin_numpy_matmul(orc):
    """Against numpy float64 A @ W.T with W decoded by numpy (library routines only),
    including ragged shapes, K = 0 and the tolerance scale 1e-5*sum|a w| + 1e-6."""
    for (M, N, K) in ((1, 300, 256), (7, 129, 320), (33, 65, 1024)):
        a = wqgen.normal((M, K), seed=M, stream=0)
        for fmt in (FMT_F16, FMT_Q8_0, FMT_Q4_0):
            b = _weights(orc, fmt, N, K, seed=M)
            w = _numpy_decode(b, fmt, N, K)
            c, bound = orc.matmul(a, b, fmt, M, N, K)
            a64 = a.astype(np.float64)
            ref = a64 @ w.T
            sabs = np.abs(a64) @ np.abs(w).T
            assert np.all(np.abs(c - ref) <= 1e-12 * sabs + 1e-300)
            assert np.allclose(bound, 1e-5 * sabs + 1e-6, rtol=1e-12, atol=0)
    c, bound = orc.matmul(np.zeros((2, 0), np.float32), np.zeros((3, 0), np.uint16), FMT_F16, 2, 3, 0)
    assert np.array_equal(c, np.zeros((2, 3))) and np.allclose(bound, 1e-6)


# ------------------------------------------------------------- epilogues --
LN3 = float(np.log(3.0))


def pin_silu_closed_forms(orc):
    """silu(x) = x * sigma(x) with sigma(x) = 1 / (1 + e^-x) (silu_mul, lattice-inference
    0.1.2 page).  Closed forms: sigma(0) = 1/2 so silu(0) = 0; sigma(ln 3) = 1/(1 + 1/3) = 3/4;
    sigma(1) = e / (1 + e); sigma(x) + sigma(-x) = 1 gives silu(x) - silu(-x) = x; silu(x) / x
    tends to 1 at +inf and silu(x) to 0- at -inf; 0 < silu(x) < x and silu(x) > x / 2 for x > 0."""
    assert orc.silu([0.0])[0] == 0.0
    assert abs(orc.silu([LN3])[0] - 0.75 * LN3) <= 1e-15
    assert abs(orc.silu([1.0])[0] - np.e / (1.0 + np.e)) <= 1e-15
    x = np.concatenate([np.geomspace(1e-6, 30.0, 200), [0.5, 2.0, 7.25]])
    assert np.all(np.abs(orc.silu(x) - orc.silu(-x) - x) <= 4e-16 * x + 1e-300)
    pos = orc.silu(x)
    assert np.all((pos > x / 2) & (pos < x))
    assert orc.silu([40.0])[0] == 40.0                      # 40 / (1 + e^-40), e^-40 < 2^-53
    v = orc.silu([-40.0])[0]
    assert -40.0 * np.exp(-40.0) <= v < -0.99 * 40.0 * np.exp(-40.0)
    assert orc.silu([-1000.0])[0] == 0.0 and orc.silu([1000.0])[0] == 1000.0


def pin_residual_golden(orc):
    """The worked 2x3x32 example (tests/golden/matmul_tiny.txt) added into a residual
    (gemm_q1_v7_residual, oxibonsai-kernels 0.1.4 page): out = r + C, each sum below
    exact and done by hand (the tolerance is pinned by pin_residual_bound)."""
    M, N, K, A, B16, B8, B4, C = _golden_matmul()
    r = np.array([[0.25, -1.0, 1e6], [0.5, -4.5, 7.0]], np.float32)
    want = np.array([[3.25, -1.0, 1000002.0], [0.0, 0.0, 2.0]])
    for fmt, b in ((FMT_F16, B16), (FMT_Q8_0, B8), (FMT_Q4_0, B4)):
        out, bound = orc.matmul_epilogue(A, b, fmt, M, N, K, oracle.EPI_RESIDUAL, r)
        assert np.array_equal(out, want), (fmt, out)
        rows, cols = np.array([1, 0, 1]), np.array([2, 2, 0])
        oe, be = orc.epilogue_entries(A, b, fmt, M, N, K, oracle.EPI_RESIDUAL, rows, cols, r)
        assert np.array_equal(oe, want[rows, cols]) and np.array_equal(be, bound[rows, cols])


def _swiglu_tiny():
    """A hand-built SwiGLU case, K = 32, n = 2: gate rows 0, 1 then up rows 2, 3 (f16
    one-hots) of the fused gate||up weight (gate at offset 0, up after it:
    dispatch_gemm_at, lattice-inference 0.9.0 page)."""
    K, n = 32, 2
    w = np.zeros((2 * n, K), np.uint16)
    w[0, 0] = 0x3C00   # gate 0 = a[0]
    w[1, 1] = 0xBC00   # gate 1 = -a[1]
    w[2, 0] = 0x4000   # up 0 = 2 a[0]
    w[3, 2] = 0x3800   # up 1 = a[2] / 2
    g = np.float32(LN3)  # the f32 nearest ln 3, |g - ln 3| < 2^-23
    a = np.zeros((3, K), np.float32)
    a[0, 0], a[0, 2] = g, 4.0            # gate (g, 0), up (2g, 2)
    a[1, 1], a[1, 2] = -g, 8.0           # gate (0, g), up (0, 4)
    a[2, 0], a[2, 1], a[2, 2] = -40.0, 40.0, -6.0  # gate (-40, -40), up (-80, -3)
    # out = silu(gate) * up:  row 0: (3/4 g * 2g, 0) = (1.5 g^2, 0); row 1: (0, 3/4 g * 4) = (0, 3g);
    # row 2: silu(-40) * (-80) and silu(-40) * (-3), both within 100 e^-40 of 0.
    want = np.array([[1.5 * LN3 * LN3, 0.0], [0.0, 3.0 * LN3], [0.0, 0.0]])
    return a, w, K, n, want


def pin_swiglu_golden(orc):
    """Hand values of _swiglu_tiny (sigma(ln 3) = 3/4; silu(0) = 0; silu(-40) ~ 0): which
    half is the gate, its pairing with the up row of the same index, and the sign of the
    exponent; the relative 1e-7 covers g being the f32 nearest ln 3."""
    a, w, K, n, want = _swiglu_tiny()
    out, bound = orc.matmul_epilogue(a, w, FMT_F16, 3, n, K, oracle.EPI_SWIGLU)
    assert out.shape == (3, n)
    assert np.all(np.abs(out - want) <= 1e-7 * np.abs(want) + 1e-13), out
    oe, be = orc.epilogue_entries(a, w, FMT_F16, 3, n, K, oracle.EPI_SWIGLU, [1, 0, 2], [1, 0, 1])
    assert np.array_equal(oe, out[[1, 0, 2], [1, 0, 1]]) and np.array_equal(be, bound[[1, 0, 2], [1, 0, 1]])


def pin_swiglu_identity(orc):
    """silu(g) u - silu(-g) u = g u (sigma(x) + sigma(-x) = 1): negating the gate rows
    (flipping their f16 sign bits) and subtracting must give g * u, with g and u from
    numpy on numpy-decoded weights, for random activations and weights."""
    M, n, K = 5, 37, 96
    a = wqgen.normal((M, K), seed=3, stream=0)
    w = _weights(orc, FMT_F16, 2 * n, K, seed=11)
    wneg = w.copy()
    wneg[:n] ^= np.uint16(0x8000)
    out, _ = orc.matmul_epilogue(a, w, FMT_F16, M, n, K, oracle.EPI_SWIGLU)
    outn, _ = orc.matmul_epilogue(a, wneg, FMT_F16, M, n, K, oracle.EPI_SWIGLU)
    wd = _numpy_decode(w, FMT_F16, 2 * n, K)
    a64 = a.astype(np.float64)
    g, u = a64 @ wd[:n].T, a64 @ wd[n:].T
    assert np.all(np.abs((out - outn) - g * u) <= 1e-12 * (np.abs(g) + 1) * (np.abs(u) + 1))
    # silu(g) u itself lies between 0 and g u for g > 0 and between g u and 0 for g < 0.
    gu = g * u
    assert np.all(np.minimum(0, gu) - 1e-12 <= out) and np.all(out <= np.maximum(0, gu) + 1e-12)


# ----------------------------------------------------------------- top-k --
UMAX = 4294967295


def pin_topk_hand(orc):
    """The ranking of the pages' TopKCandidate / topk_better (lattice-inference 0.1.2):
    higher logit first, equal logits by lower id, NaN never selected, sentinel
    (-inf, UINT_MAX) padding; -inf logits rank above the sentinel by their id.
    Every expected list below is worked out by hand."""
    x = [1.0, 3.0, float("nan"), 3.0, float("-inf"), 2.0]
    v, i = orc.topk(x, 7)
    assert list(i) == [1, 3, 5, 0, 4, UMAX, UMAX]
    assert list(v[:4]) == [3.0, 3.0, 2.0, 1.0] and np.all(np.isneginf(v[4:]))
    v, i = orc.topk(x, 1)
    assert list(i) == [1] and v[0] == 3.0
    v, i = orc.topk([float("nan")] * 3, 2)
    assert list(i) == [UMAX, UMAX] and np.all(np.isneginf(v))
    v, i = orc.topk([-1.0, float("inf"), 5.0, float("inf")], 3)
    assert list(i) == [1, 3, 2] and v[2] == 5.0
    v, i = orc.topk([0.0, -0.0, 0.0], 3)  # -0.0 == 0.0: ties by id
    assert list(i) == [0, 1, 2]
    v, i = orc.topk([], 2)
    assert list(i) == [UMAX, UMAX]


def pin_topk_vs_lexsort(orc):
    """Against numpy's lexsort (descending logit, then ascending id) with NaNs
    dropped, on tie-heavy integer logits and on N(0,1) logits, for k below, at and
    above the number of candidates."""
    rng = np.random.default_rng(12)
    for n in (1, 7, 63, 64, 65, 1000, 5000):
        for kind in ("ties", "normal"):
            x = rng.integers(-3, 4, n).astype(np.float64) if kind == "ties" else rng.standard_normal(n)
            if n > 10:
                x[rng.integers(0, n, n // 10)] = np.nan
            keep = np.flatnonzero(~np.isnan(x))
            order = keep[np.lexsort((keep, -x[keep]))]
            for k in (1, 5, 50, 64, n + 3):
                v, i = orc.topk(x, k)
                m = min(k, order.size)
                assert np.array_equal(i[:m], order[:m]), (n, kind, k)
                assert np.array_equal(v[:m], x[order[:m]])
                assert np.all(i[m:] == UMAX) and np.all(np.isneginf(v[m:]))


def pin_lm_head_topk(orc):
    """One-hot LM head: row j of the f16 weights holds w_j at column 0 and a = e_0, so
    logit j = w_j exactly; the top-k of chosen w_j (with ties and a NaN row) is known by
    hand.  Also the logits and bounds it returns are those of the product."""
    K = 32
    w = np.array([0.5, -2.0, 3.0, 3.0, float("nan"), 1.0, 3.0, -0.25], np.float32)
    b = np.zeros((w.size, K), np.uint16)
    b[:, 0] = w.astype(np.float16).view(np.uint16)
    a = np.zeros(K, np.float32)
    a[0] = 1.0
    v, i, logits, bound = orc.lm_head_topk(a, b, FMT_F16, w.size, K, 5)
    assert list(i) == [2, 3, 6, 5, 0] and list(v) == [3.0, 3.0, 3.0, 1.0, 0.5]
    c, bd = orc.matmul(a.reshape(1, K), b, FMT_F16, 1, w.size, K)
    assert np.array_equal(logits, c[0], equal_nan=True) and np.array_equal(bound, bd[0], equal_nan=True)


# ------------------------------------------------------ decode attention --
def _attn_inputs(L, D, Hq, Hkv, seed, kvfmt=oracle.KV_F32):
    q = wqgen.normal((Hq, D), seed=seed, stream=11)
    k = wqgen.normal((L, Hkv * D), seed=seed, stream=12)
    v = wqgen.normal((L, Hkv * D), seed=seed, stream=13)
    if kvfmt == oracle.KV_F16:
        k, v = k.astype(np.float16).view(np.uint16), v.astype(np.float16).view(np.uint16)
    return q, k, v


def _kv_numpy(c, kvfmt):
    return (c.view(np.float16) if kvfmt == oracle.KV_F16 else c).astype(np.float64)


def pin_attention_single_token(orc):
    """L = 1: softmax of one score is 1, so out[h] is the V row of the KV head that
    query head h reads (h // G, the page's qh_base = kvh * group_size) exactly, for f32
    and f16 caches (f16 decoded by numpy)."""
    for kvfmt in (oracle.KV_F32, oracle.KV_F16):
        for (D, Hq, Hkv) in ((256, 8, 2), (64, 6, 3), (128, 4, 4)):
            q, k, v = _attn_inputs(1, D, Hq, Hkv, 5, kvfmt)
            out, _ = orc.decode_attention(q, k, v, kvfmt, 1, D, Hq, Hkv, 0.0625)
            vn = _kv_numpy(v, kvfmt).reshape(Hkv, D)
            G = Hq // Hkv
            for h in range(Hq):
                assert np.array_equal(out[h], vn[h // G]), (kvfmt, D, Hq, Hkv, h)


def pin_attention_uniform(orc):
    """Equal keys, or scale 0, make every score equal, so p is uniform and out is the
    mean of the V rows (numpy mean)."""
    L, D, Hq, Hkv = 37, 64, 4, 2
    q, k, v = _attn_inputs(L, D, Hq, Hkv, 6)
    kk = np.repeat(k[:1], L, axis=0)
    G = Hq // Hkv
    for kc, scale in ((kk, 0.7), (k, 0.0)):
        out, _ = orc.decode_attention(q, kc, v, oracle.KV_F32, L, D, Hq, Hkv, scale)
        mean = v.astype(np.float64).reshape(L, Hkv, D).mean(axis=0)
        for h in range(Hq):
            assert np.allclose(out[h], mean[h // G], rtol=0, atol=1e-12)


def pin_attention_dominant_key(orc):
    """One key aligned with q and 60 (then 1e4) score units above the rest: its weight
    is 1 within e^-60, so out is its V row; at 1e4 the scores overflow exp unless the
    maximum is taken out first."""
    L, D, Hq, Hkv = 50, 64, 2, 1
    q, k, v = _attn_inputs(L, D, Hq, Hkv, 7)
    q[1] = q[0]
    k = np.zeros_like(k)
    t0 = 17
    for big in (60.0, 1e4):
        kk = k.copy()
        kk[t0] = q[0] * np.float32(big / float(np.dot(q[0].astype(np.float64), q[0])))
        out, _ = orc.decode_attention(q, kk, v, oracle.KV_F32, L, D, Hq, Hkv, 1.0)
        assert np.all(np.isfinite(out))
        assert np.allclose(out[0], v[t0].astype(np.float64), rtol=0, atol=1e-20 + 10 * np.exp(-59.0) * 10)


def pin_attention_numpy(orc):
    """Against float64 numpy softmax attention (matmul, exp, sum) on random inputs,
    f32 and f16 caches, ragged L."""
    for kvfmt in (oracle.KV_F32, oracle.KV_F16):
        for (L, D, Hq, Hkv) in ((1, 256, 8, 2), (100, 256, 8, 2), (513, 128, 8, 1), (77, 64, 3, 3)):
            q, k, v = _attn_inputs(L, D, Hq, Hkv, L + D, kvfmt)
            scale = 1.0 / np.sqrt(D)
            out, bound = orc.decode_attention(q, k, v, kvfmt, L, D, Hq, Hkv, scale)
            kn = _kv_numpy(k, kvfmt).reshape(L, Hkv, D)
            vn = _kv_numpy(v, kvfmt).reshape(L, Hkv, D)
            G = Hq // Hkv
            for h in range(Hq):
                s_ = np.float64(np.float32(scale)) * (kn[:, h // G, :] @ q[h].astype(np.float64))
                w = np.exp(s_ - s_.max())
                ref = (w / w.sum()) @ vn[:, h // G, :]
                assert np.allclose(out[h], ref, rtol=1e-12, atol=1e-14), (kvfmt, L, D, h)


def pin_attention_permutation_and_empty(orc):
    """Permuting the cache tokens (K and V together) leaves out unchanged; L = 0 gives 0."""
    L, D, Hq, Hkv = 64, 128, 4, 2
    q, k, v = _attn_inputs(L, D, Hq, Hkv, 8)
    perm = np.random.default_rng(1).permutation(L)
    a, _ = orc.decode_attention(q, k, v, oracle.KV_F32, L, D, Hq, Hkv, 0.1)
    b, _ = orc.decode_attention(q, k[perm], v[perm], oracle.KV_F32, L, D, Hq, Hkv, 0.1)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    z, bz = orc.decode_attention(q, k[:0], v[:0], oracle.KV_F32, 0, D, Hq, Hkv, 0.1)
    assert np.array_equal(z, np.zeros((Hq, D)))


# ------------------------------------------------- tolerance propagation --
# The product tolerance B = 1e-5 * sum_k |a_k w_k| + 1e-6 of the task fixes how
# far a kernel's f32 sum may sit from the exact one.  The oracle propagates it
# through the epilogues and through softmax attention.  These pins check each
# propagated bound against the thing it claims to cover -- every input moved by
# up to its own tolerance, in the worst directions, and evaluated in float32 by
# numpy -- and that it is not much looser than that worst case (a bound ten
# times too loose, or one missing a term, fails here).

def _f32_within(x, r):
    """The float32 values nearest x - r and x + r that stay inside [x - r, x + r]
    (x and r float64 arrays): what a float32 sum within r of x can be."""
    lo = (x - r).astype(np.float32)
    hi = (x + r).astype(np.float32)
    lo = np.where(lo.astype(np.float64) < x - r, np.nextafter(lo, np.float32(np.inf)), lo)
    hi = np.where(hi.astype(np.float64) > x + r, np.nextafter(hi, np.float32(-np.inf)), hi)
    return lo, hi


def pin_residual_bound(orc):
    """Residual (out = r + s): a float32 sum s' within B_s of the exact s, added to the
    f32 residual r in float32, lands within the oracle's bound of r + s; and where B_s
    dominates the bound is within 1.5x of that worst case (the f32 addition then
    rounds by at most half an ulp of the result)."""
    rng = np.random.default_rng(21)
    n = 4000
    r = (rng.standard_normal(n) * 10.0 ** rng.integers(-3, 4, n)).astype(np.float32)
    s = rng.standard_normal(n) * 10.0 ** rng.integers(-3, 4, n)
    for rel in (0.0, 1e-7, 1e-4):
        if rel == 0.0:
            s_ = s.astype(np.float32).astype(np.float64)    # exact f32 sums: only the addition rounds
        else:
            s_ = s
        bs = rel * np.abs(s_)
        out, bound = orc.epilogue(oracle.EPI_RESIDUAL, s_, bs, 1, n, r)
        exact = r.astype(np.float64) + s_
        assert np.array_equal(out[0], exact)
        dev = np.zeros(n)
        for sp in _f32_within(s_, bs):
            got = (r + sp).astype(np.float64)               # the f32 addition
            dev = np.maximum(dev, np.abs(got - exact))
        assert np.all(dev <= bound[0]), (rel, float(np.max(dev / bound[0])))
        if rel == 1e-4:
            dom = bs > 100.0 * 2.0 ** -23 * (np.abs(r) + np.abs(s_))   # B_s dominates the rounding
            assert dom.sum() > n // 4
            assert np.all(bound[0][dom] <= 1.5 * dev[dom]), float(np.max(bound[0][dom] / dev[dom]))
    # Rounding-only case with same-sign operands: the bound is at most 4 half-ulps.
    rr = np.abs(r)
    ss = np.abs(s).astype(np.float32).astype(np.float64)
    _, bound = orc.epilogue(oracle.EPI_RESIDUAL, ss, np.zeros(n), 1, n, rr)
    ulp = np.spacing((rr.astype(np.float64) + ss).astype(np.float32)).astype(np.float64)
    assert np.all(bound[0] <= 2.0 * ulp + 1e-300)


def _silu32(x):
    x = np.asarray(x, np.float32)
    return x / (np.float32(1.0) + np.exp(-x))


def pin_swiglu_bound(orc):
    """SwiGLU (out = silu(g) u): float32 gate and up sums within B_g and B_u of the
    exact g and u, put through silu and the product in float32, land within the
    oracle's bound of silu(g) u; for gates where silu' is far from 0 the bound is
    within 2x of the worst corner."""
    rng = np.random.default_rng(22)
    n = 3000
    g = rng.uniform(-12.0, 12.0, n)
    u = rng.standard_normal(n) * 3.0
    for rel in (0.0, 1e-6, 1e-3):
        bg, bu = rel * np.abs(g) + 1e-6, rel * np.abs(u) + 1e-6
        acc = np.concatenate([g, u]).reshape(1, 2 * n)
        accb = np.concatenate([bg, bu]).reshape(1, 2 * n)
        out, bound = orc.epilogue(oracle.EPI_SWIGLU, acc, accb, 1, n)
        exact = g / (1.0 + np.exp(-g)) * u
        assert np.allclose(out[0], exact, rtol=1e-14, atol=1e-300)
        dev = np.zeros(n)
        gs = _f32_within(g, bg) + (g.astype(np.float32),)
        us = _f32_within(u, bu) + (u.astype(np.float32),)
        for gp in gs:
            for up in us:
                got = (_silu32(gp) * up).astype(np.float64)
                dev = np.maximum(dev, np.abs(got - exact))
        assert np.all(dev <= bound[0]), (rel, float(np.max(dev / bound[0])))
        if rel == 1e-3:
            steep = g > 0.5           # silu' in (0.74, 1.1)
            assert np.all(bound[0][steep] <= 2.0 * dev[steep]), float(np.max(bound[0][steep] / dev[steep]))


def pin_attention_bound(orc):
    """Attention: every score moved by its own product tolerance B_t = |scale|(1e-5
    sum_d |q_d k_td| + 1e-6), in the direction that pushes each output furthest (up
    where v_td is above the output, down elsewhere, and the reverse), through a numpy
    float64 softmax, stays within the oracle's bound; and the bound's median excess
    over that worst case is below 4x (scores of spread ~4, B_t ~ 2e-4, where the
    expm1(2 max B) term dominates)."""
    rng = np.random.default_rng(23)
    for L, D, Hq, Hkv, sig in ((64, 64, 2, 1, 2.0), (300, 128, 4, 2, 2.0), (40, 64, 2, 2, 3.0)):
        q = (rng.standard_normal((Hq, D)) * sig).astype(np.float32)
        k = (rng.standard_normal((L, Hkv * D)) * sig).astype(np.float32)
        v = rng.standard_normal((L, Hkv * D)).astype(np.float32)
        scale = 0.125
        out, bound = orc.decode_attention(q, k, v, oracle.KV_F32, L, D, Hq, Hkv, scale)
        kn = k.astype(np.float64).reshape(L, Hkv, D)
        vn = v.astype(np.float64).reshape(L, Hkv, D)
        G = Hq // Hkv
        ratios = []
        for h in range(Hq):
            qh = q[h].astype(np.float64)
            kk, vv = kn[:, h // G, :], vn[:, h // G, :]
            s = scale * (kk @ qh)
            B = scale * (1e-5 * np.abs(kk * qh).sum(axis=1) + 1e-6)
            w = np.exp(s - s.max())
            o = (w / w.sum()) @ vv
            assert np.allclose(out[h], o, rtol=1e-12, atol=1e-14)
            dev = np.zeros(D)
            signs = [np.sign(vv - o), -np.sign(vv - o)] + [rng.choice([-1.0, 1.0], size=(L, 1)) for _ in range(4)]
            for sg in signs:
                s2 = s[:, None] + B[:, None] * sg
                w2 = np.exp(s2 - s2.max(axis=0))
                o2 = (w2 * vv).sum(axis=0) / w2.sum(axis=0)
                dev = np.maximum(dev, np.abs(o2 - o))
            assert np.all(dev <= bound[h]), float(np.max(dev / bound[h]))
            ratios.extend((bound[h] / dev).tolist())
        if sig == 2.0:
            assert np.median(ratios) <= 4.0, float(np.median(ratios))
    # One token whose key is long (B_t about 40x the others') but whose score is only
    # slightly above the rest, so it carries a large weight: the bound must follow the
    # largest B_t, not a typical one.
    L, D = 50, 64
    q = (rng.standard_normal((1, D)) * 2.0).astype(np.float32)
    k = (rng.standard_normal((L, D)) * 2.0).astype(np.float64)
    qd = q[0].astype(np.float64)
    z = rng.standard_normal(D)
    z -= (z @ qd) / (qd @ qd) * qd
    s_other = 0.125 * (k @ qd)
    k[7] = qd * ((np.delete(s_other, 7).max() + 0.5) / (0.125 * (qd @ qd))) + 40.0 * z
    k = k.astype(np.float32)
    v = rng.standard_normal((L, D)).astype(np.float32)
    out, bound = orc.decode_attention(q, k, v, oracle.KV_F32, L, D, 1, 1, 0.125)
    kk, vv = k.astype(np.float64), v.astype(np.float64)
    s = 0.125 * (kk @ qd)
    B = 0.125 * (1e-5 * np.abs(kk * qd).sum(axis=1) + 1e-6)
    w = np.exp(s - s.max())
    o = (w / w.sum()) @ vv
    for sg in (np.sign(vv - o), -np.sign(vv - o)):
        s2 = s[:, None] + B[:, None] * sg
        w2 = np.exp(s2 - s2.max(axis=0))
        dev = np.abs((w2 * vv).sum(axis=0) / w2.sum(axis=0) - o)
        assert np.all(dev <= bound[0]), float(np.max(dev / bound[0]))


PINS = [
    pin_f16_decode_exhaustive,
    pin_f16_encode_golden,
    pin_f16_encode_vs_numpy,
    pin_q8_golden,
    pin_q8_roundtrip,
    pin_q8_decode_handbuilt,
    pin_q4_golden,
    pin_matmul_golden,
    pin_bruteforce_fraction,
    pin_identity_and_onehot,
    pin_invariants,
    pin_numpy_matmul,
    pin_silu_closed_forms,
    pin_residual_golden,
    pin_swiglu_golden,
    pin_swiglu_identity,
    pin_topk_hand,
    pin_topk_vs_lexsort,
    pin_lm_head_topk,
    pin_attention_single_token,
    pin_attention_uniform,
    pin_attention_dominant_key,
    pin_attention_numpy,
    pin_attention_permutation_and_empty,
    pin_residual_bound,
    pin_swiglu_bound,
    pin_attention_bound,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_argument_errors(orc):
    a = np.zeros((1, 48), np.float32)
    with pytest.raises(ValueError):
        orc.matmul(a, np.zeros((1, 51), np.uint8), FMT_Q8_0, 1, 1, 48)  # K % 32 != 0
    with pytest.raises(ValueError):
        orc.matmul(a, np.zeros((1, 0), np.uint8), FMT_Q8_0, 1, 1, 0)    # Q8_0 with K == 0
    with pytest.raises(ValueError):
        orc.matmul(a, np.zeros((1, 27), np.uint8), FMT_Q4_0, 1, 1, 48)  # Q4_0, K % 32 != 0
    with pytest.raises(ValueError):
        orc.matmul(a, np.zeros((1, 48), np.uint16), 7, 1, 1, 48)        # unknown format
    with pytest.raises(ValueError):
        orc.q8_0_quantize(np.zeros((1, 40), np.float32))
    c, _ = orc.matmul(a, np.zeros((1, 48), np.uint16), FMT_F16, 0, 1, 48)
    assert c.shape == (0, 1)


# --------------------------------------------------------------- mutants --
# Each entry plants one plausible mistake in a copy of wqref.c.
MUTANTS = {
    "drop_last_k_term": ("for (int64_t k = 0; k < K; ++k) {\n        const double p",
                         "for (int64_t k = 0; k + 1 < K; ++k) {\n        const double p"),
    "reversed_k_index": ("((const uint16_t *)b)[n * K + k]", "((const uint16_t *)b)[n * K + (K - 1 - k)]"),
    "q8_code_sign": ("return wqref_f16_value(h) * (double)q;", "return wqref_f16_value(h) * (double)(-q);"),
    "q8_scale_big_endian": ("(uint16_t)(blk[0] | (blk[1] << 8))", "(uint16_t)(blk[1] | (blk[0] << 8))"),
    "q8_block_stride_32": ("(n * nb + k / WQREF_QK) * WQREF_BLOCK_BYTES", "(n * nb + k / WQREF_QK) * 32"),
    "f16_truncate": ("nearbyint(ldexp(ax, -q))", "floor(ldexp(ax, -q))"),
    "f16_flush_subnormal": ("if (q < -24) q = -24;", "if (q < -24) q = -24; if (e2 - 1 < -14) return sign;"),
    "f16_exponent_bias": ("(uint16_t)((E + 15) << 10)", "(uint16_t)((E + 16) << 10)"),
    "q8_round_ties_even": ("roundf(v[i] * id)", "rintf(v[i] * id)"),
    "q8_scale_over_128": ("amax / 127.0f", "amax / 128.0f"),
    "q8_scale_byte_order_write": ("o[0] = (uint8_t)(h & 0xff);\n        o[1] = (uint8_t)(h >> 8);",
                                  "o[1] = (uint8_t)(h & 0xff);\n        o[0] = (uint8_t)(h >> 8);"),
    "f32_accumulate": ("s += p;", "s = (double)(float)(s + p);"),
    "row_zero_only": ("dot(j->a + m * j->K, w", "dot(j->a + 0 * j->K, w"),
    "abs_sum_dropped": ("sa += fabs(p);", "sa += p;"),
    "q4_nibble_order": ("(i % 2 == 0) ? (byte & 0x0F) : (byte >> 4)", "(i % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    "q4_no_offset": ("(double)(u - 8)", "(double)(u)"),
    "q4_offset_7": ("(double)(u - 8)", "(double)(u - 7)"),
    "q4_block_20_bytes": ("* WQREF_Q4_BLOCK_BYTES;", "* 20;"),
    "q4_split_halves_layout": ("blk[2 + i / 2];\n    const int u = (i % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
                               "blk[2 + i % 16];\n    const int u = (i < 16) ? (byte & 0x0F) : (byte >> 4);"),
    "q4_signed_nibble": ("(byte & 0x0F) : (byte >> 4);", "((byte & 0x0F) ^ 8) : ((byte >> 4) ^ 8);"),
    "silu_exp_sign": ("x / (1.0 + exp(-x))", "x / (1.0 + exp(x))"),
    "silu_is_sigmoid": ("x / (1.0 + exp(-x))", "1.0 / (1.0 + exp(-x))"),
    "silu_no_gate_product": ("out[i * N + j] = sg * u;", "out[i * N + j] = sg;"),
    "glu_halves_swapped": ("gi = i * 2 * N + j, ui = gi + N;", "ui = i * 2 * N + j, gi = ui + N;"),
    "glu_interleaved": ("gi = i * 2 * N + j, ui = gi + N;", "gi = i * 2 * N + 2 * j, ui = gi + 1;"),
    "residual_dropped": ("out[i] = r + s;", "out[i] = s;"),
    "residual_subtracted": ("out[i] = r + s;", "out[i] = s - r;"),
    "residual_bound_no_rounding": ("acc_bound[i] + ldexp(fabs(r) + fabs(s), -23)", "acc_bound[i]"),
    "topk_ties_higher_id": ("return (a->id < b->id) ? -1 : (a->id > b->id) ? 1 : 0;",
                            "return (a->id > b->id) ? -1 : (a->id < b->id) ? 1 : 0;"),
    "topk_ascending": ("if (a->v > b->v) return -1;\n    if (a->v < b->v) return 1;",
                       "if (a->v < b->v) return -1;\n    if (a->v > b->v) return 1;"),
    "topk_keeps_nan": ("if (!isnan(logits[i])) {", "if (1) {"),
    "topk_sentinel_zero": ("vals[r] = r < cnt ? c[r].v : -INFINITY;", "vals[r] = r < cnt ? c[r].v : 0.0;"),
    "topk_sentinel_id": ("(int64_t)4294967295LL", "(int64_t)-1"),
    "attn_head_mod": ("const int64_t kvh = h / G;", "const int64_t kvh = h % Hkv;"),
    "attn_no_scale": ("s[t] = (double)scale * dot;", "s[t] = dot;"),
    "attn_no_max_shift": ("s[t] = exp(s[t] - smax);", "s[t] = exp(s[t]);"),
    "attn_k_for_v": ("const double vv = kv_value(v, kvfmt,", "const double vv = kv_value(k, kvfmt,"),
    "attn_last_token_dropped": ("for (int64_t t = 0; t < L; ++t) {\n            double dot",
                                "for (int64_t t = 0; t + 1 < L; ++t) {\n            double dot"),
    "attn_unnormalised": ("out[h * D + d] = L > 0 ? acc / z : 0.0;", "out[h * D + d] = L > 0 ? acc : 0.0;"),
    "attn_head_stride_kvdim": ("kv_value(k, kvfmt, t * kv_dim + kvh * D + d)", "kv_value(k, kvfmt, t * D + kvh * D + d)"),
    "residual_bound_x10": ("acc_bound[i] + ldexp(fabs(r) + fabs(s), -23)",
                           "10.0 * (acc_bound[i] + ldexp(fabs(r) + fabs(s), -23))"),
    "glu_bound_x10": ("bound[i * N + j] = 1.1 * bg * (fabs(u) + bu) + fabs(sg) * bu + ldexp(fabs(sg * u), -20);",
                      "bound[i * N + j] = 10.0 * (1.1 * bg * (fabs(u) + bu) + fabs(sg) * bu + ldexp(fabs(sg * u), -20));"),
    "glu_bound_no_gate_term": ("= 1.1 * bg * (fabs(u) + bu) + fabs(sg) * bu", "= fabs(sg) * bu"),
    "glu_bound_slope_half": ("= 1.1 * bg * (fabs(u) + bu)", "= 0.5 * bg * (fabs(u) + bu)"),
    "glu_bound_no_rounding": ("+ fabs(sg) * bu + ldexp(fabs(sg * u), -20);", "+ fabs(sg) * bu;"),
    "attn_bound_x10": ("(expm1(2.0 * bmax) + 1e-5) * (mag / z)", "10.0 * (expm1(2.0 * bmax) + 1e-5) * (mag / z)"),
    "attn_bound_no_expm1": ("(expm1(2.0 * bmax) + 1e-5) * (mag / z)", "(1e-5) * (mag / z)"),
    "attn_bound_mean_b": ("if (b[t] > bmax) bmax = b[t];", "bmax += b[t] / (double)L;"),
    "topk_drops_last": ("for (int64_t r = 0; r < topk; ++r) {\n        vals[r]",
                        "for (int64_t r = 0; r < topk; ++r) {\n        if (r == topk - 1 && r > 0) { vals[r] = -INFINITY; ids[r] = 4294967295LL; continue; }\n        vals[r]"),
}


@pytest.mark.slow
def test_mutants_are_caught():
    src = os.path.join(os.path.dirname(oracle.__file__), "wqref.c")
    text = open(src).read()
    tmp = tempfile.mkdtemp(prefix="wqref_mut_")
    try:
        survivors = []
        for name, (old, new) in MUTANTS.items():
            assert text.count(old) >= 1, f"mutation site missing: {name}"
            msrc = os.path.join(tmp, f"{name}.c")
            with open(msrc, "w") as f:
                f.write(text.replace(old, new))
            so = os.path.join(tmp, f"{name}.so")
            subprocess.run(["gcc", *oracle.CFLAGS, "-o", so, msrc, "-lm"], check=True)
            mut = oracle.Oracle(so)
            caught = False
            for pin in PINS:
                try:
                    pin(mut)
                except AssertionError:
                    caught = True
                    break
            if not caught:
                survivors.append(name)
        assert not survivors, f"mutants not caught by any pin: {survivors}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
