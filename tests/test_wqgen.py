"""The shared input generator: determinism, slicing and distribution."""
import math

import numpy as np
import pytest

import wqgen

pytestmark = pytest.mark.filterwarnings("ignore")


def _splitmix64_reference(state: int, count: int):
    """Sequential SplitMix64 as published (Steele, Lea & Flood 2014)."""
    out = []
    mask = (1 << 64) - 1
    for _ in range(count):
        state = (state + 0x9E3779B97F4A7C15) & mask
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        out.append(z ^ (z >> 31))
    return out


def test_counter_outputs_equal_sequential_splitmix64():
    lib = wqgen._load()
    key = lib.wqgen_stream_key(0, 1)
    got = [wqgen.raw_u64(0, 1, i) for i in range(16)]
    assert got == _splitmix64_reference(key, 16)


def test_known_splitmix64_value():
    # SplitMix64 from state 0: first output 0xE220A8397B1DCDAF (a widely
    # published test value of the generator).
    assert _splitmix64_reference(0, 1)[0] == 0xE220A8397B1DCDAF


def test_deterministic_and_sliceable():
    a = wqgen.normal((1000,), seed=3, stream=0)
    b = wqgen.normal((1000,), seed=3, stream=0)
    assert np.array_equal(a, b)
    part = wqgen.normal((301,), seed=3, stream=0, offset=357)
    assert np.array_equal(part, a[357:658])
    rows = wqgen.weight_rows([0, 5, 9], 64, seed=2)
    full = wqgen.weights(10, 64, seed=2)
    assert np.array_equal(rows, full[[0, 5, 9]])


def test_streams_and_seeds_differ():
    a = wqgen.normal((256,), seed=0, stream=0)
    assert not np.array_equal(a, wqgen.normal((256,), seed=0, stream=1))
    assert not np.array_equal(a, wqgen.normal((256,), seed=1, stream=0))


def test_activation_prefix_rows():
    a512 = wqgen.activations(512, 64)
    a4 = wqgen.activations(4, 64)
    assert np.array_equal(a512[:4], a4)


def test_moments():
    x = wqgen.normal((1 << 20,), seed=0, stream=0).astype(np.float64)
    assert abs(x.mean()) < 5.0 / math.sqrt(x.size)
    assert abs(x.std() - 1.0) < 0.005
    w = wqgen.weights(256, 1024).astype(np.float64)
    assert abs(w.std() - 0.02) < 0.0002
    # tail mass beyond 3 sigma for a normal: 0.0027
    assert abs(np.mean(np.abs(x) > 3.0) - 0.0027) < 0.0004


def test_q4_0_bytes_layout_and_determinism():
    b = wqgen.q4_0_bytes(5, 96, seed=3)
    assert b.shape == (5, 3 * 18) and b.dtype == np.uint8
    assert np.array_equal(b, wqgen.q4_0_bytes(5, 96, seed=3))
    assert np.array_equal(b[2:4], wqgen.q4_0_bytes(2, 96, seed=3, row0=2))
    assert not np.array_equal(b, wqgen.q4_0_bytes(5, 96, seed=4))
    blocks = b.reshape(-1, 18)
    scale = blocks[:, 0:2].copy().view("<u2").ravel()
    assert np.all((scale & 0x7C00) == 0x1C00)            # |d| in [2^-8, 2^-7)
    # codes of a big draw: all 16 values, both scale signs
    big = wqgen.q4_0_bytes(64, 1024, seed=0).reshape(-1, 18)
    codes = np.concatenate([big[:, 2:] & 0x0F, big[:, 2:] >> 4]).ravel()
    assert set(np.unique(codes)) == set(range(16))
    signs = big[:, 1] >> 7
    assert 0.4 < signs.mean() < 0.6
    with pytest.raises(ValueError):
        wqgen.q4_0_bytes(1, 48)
