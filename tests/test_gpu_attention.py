"""GPU parity of the split-KV decode attention (wq_decode_attention) against the oracle.

Inputs: q ~ N(0,1) [Hq, D], K and V caches ~ N(0,1) [L, Hkv*D] (f32, or the
same values rounded to f16 for the f16 cache, the bytes shared by both sides).
Each output must lie within the oracle's propagated tolerance
(expm1(2 max_t B_t) + 1e-5) * sum_t p_t |v_td| + 1e-6, B_t the product
tolerance of score t.  Outputs are poisoned with NaN before each call.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attn_cases
import gemm_wq_gemv_amd as wq
import oracle
import wqgen

pytestmark = pytest.mark.gpu

F32, F16 = wq.WQ_KV_F32, wq.WQ_KV_F16


def say(msg: str):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def inputs(L, D, Hq, Hkv, kvfmt, seed, kscale=1.0):
    q = wqgen.normal((Hq, D), seed=seed, stream=11)
    k = wqgen.normal((L, Hkv * D), seed=seed, stream=12) * np.float32(kscale)
    v = wqgen.normal((L, Hkv * D), seed=seed, stream=13)
    if kvfmt == F16:
        k, v = k.astype(np.float16).view(np.uint16), v.astype(np.float16).view(np.uint16)
    return q, k, v


def run(q, k, v, L, D, Hq, Hkv, kvfmt, scale, stream=None):
    qd = torch.from_numpy(q).cuda()
    kd = torch.from_numpy(np.ascontiguousarray(k)).cuda()
    vd = torch.from_numpy(np.ascontiguousarray(v)).cuda()
    out = torch.full((Hq, D), float("nan"), device="cuda")
    wq.wq_decode_attention(qd, kd, vd, out, L, D, Hq, Hkv, kvfmt, scale, stream)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(L, D, Hq, Hkv, kvfmt, seed=0, scale=None, kscale=1.0):
    scale = float(np.float32(1.0 / np.sqrt(D))) if scale is None else scale
    say(f"attention L={L} D={D} Hq={Hq} Hkv={Hkv} kv={kvfmt} scale={scale} kscale={kscale}")
    q, k, v = inputs(L, D, Hq, Hkv, kvfmt, seed, kscale)
    return check_inputs(q, k, v, L, D, Hq, Hkv, kvfmt, scale)


def check_inputs(q, k, v, L, D, Hq, Hkv, kvfmt, scale):
    out = run(q, k, v, L, D, Hq, Hkv, kvfmt, scale)
    ref, bound = oracle.decode_attention(q, k, v, kvfmt, L, D, Hq, Hkv, scale)
    err = np.abs(out.astype(np.float64) - ref)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} outside tolerance; worst "
                           f"{float((err / bound).max()):.3g} x bound at {np.unravel_index(np.argmax(err / bound), err.shape)}")
    return float((err / bound).max())


@pytest.mark.parametrize("kvfmt", [F32, F16], ids=["f32", "f16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_every_head_dim_and_group(D, kvfmt):
    """Group sizes 1..8 (padded to 1, 2, 4, 8 inside), ragged cache lengths around the
    8/16-token tiles, the 64-token partition step and the one-partition case."""
    for Hq, Hkv in ((1, 1), (2, 1), (3, 1), (4, 2), (5, 5), (6, 2), (7, 1), (8, 1), (8, 2), (16, 2)):
        for L in (1, 7, 17, 64, 65, 300):
            check(L, D, Hq, Hkv, kvfmt, seed=L + Hq)


@pytest.mark.parametrize("kvfmt", [F32, F16], ids=["f32", "f16"])
@pytest.mark.parametrize("L", [512, 4096, 32768])
def test_model_shape_long_cache(L, kvfmt):
    """The pages' head layout (head_dim 256, GQA group 4: 8 query heads over 2 KV
    heads, q_dim 2048) at growing cache lengths: many partitions and the merge pass."""
    check(L, 256, 8, 2, kvfmt, seed=L)


def test_peaky_and_flat_softmax():
    """Large logits (a few tokens carry all the weight) and scale 0 (uniform weights)."""
    check(1000, 256, 8, 2, F32, seed=3, kscale=8.0)
    check(1000, 128, 4, 1, F16, seed=4, kscale=6.0)
    check(777, 64, 8, 8, F32, seed=5, scale=0.0)


def test_empty_cache_writes_zeros():
    q = torch.randn(8, 256, device="cuda")
    out = torch.full((8, 256), float("nan"), device="cuda")
    say("empty cache")
    wq.wq_decode_attention(q, None, None, out, 0, 256, 8, 2, F32, 0.0625)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))


def test_deterministic_and_stream():
    """Two runs agree bit for bit (partitions merge in a fixed order); a non-default
    stream gives the same result."""
    L, D, Hq, Hkv = 20000, 256, 8, 2
    q, k, v = inputs(L, D, Hq, Hkv, F16, 9)
    say("determinism")
    a = run(q, k, v, L, D, Hq, Hkv, F16, 0.0625)
    b = run(q, k, v, L, D, Hq, Hkv, F16, 0.0625)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = run(q, k, v, L, D, Hq, Hkv, F16, 0.0625, stream=s)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_forced_partition_sizes():
    """The merge pass over many partitions (ptok 64 at 20K tokens: 313 partitions,
    more than one load round per wave), partitions that end inside a tile
    (ptok 100, 8 and 1), and one partition for a long cache."""
    try:
        for ptok, L in ((64, 20000), (100, 3001), (8, 1000), (1, 300), (1 << 20, 50000)):
            wq.wq_set_attn_partition(ptok)
            say(f"forced partition {ptok} tokens, L={L}")
            check(L, 256, 8, 2, F32, seed=ptok)
            check(L, 128, 4, 4, F16, seed=ptok + 1)
    finally:
        wq.wq_set_attn_partition(0)


@pytest.mark.parametrize("kvfmt", [F32, F16], ids=["f32", "f16"])
@pytest.mark.parametrize("L", [32768, 131072])
def test_long_cache_every_token_counts(L, kvfmt):
    """Scale 0 and one-hot V rows (tests/attn_cases.py): every token weighs 1/L and
    feeds one output alone, so a skipped token -- the first, the last, one at a
    partition or tile edge -- puts that output 7x (L = 131072) to 29x (L = 32768)
    outside the tolerance (tests/test_case_design.py checks this on the CPU)."""
    say(f"one-hot V, scale 0, L={L} kv={kvfmt}")
    q, k, v, scale = attn_cases.onehot_v(L, 256, 8, 2, kvfmt)
    check_inputs(q, k, v, L, 256, 8, 2, kvfmt, scale)


def test_dominant_keys_at_partition_edges():
    """Keys that each carry ~1/9 of the weight placed at the first and last token and
    at the first and last token of the second and the last partition, for forced
    partition sizes (ragged last partitions, partitions ending inside a tile) and the
    automatic size; also the one-hot V case under a forced partition size."""
    try:
        for part, L in ((1000, 32768), (64, 4096), (37, 3001), (8, 1000)):
            wq.wq_set_attn_partition(part)
            for kvfmt in (F32, F16):
                pos = attn_cases.edge_positions(L, part)
                say(f"dominant keys at {pos}, partition {part}, L={L} kv={kvfmt}")
                q, k, v, scale = attn_cases.dominant(L, 256, 8, 2, kvfmt, pos, seed=part)
                check_inputs(q, k, v, L, 256, 8, 2, kvfmt, scale)
        wq.wq_set_attn_partition(1000)
        say("one-hot V, scale 0, partition 1000, L=32768")
        q, k, v, scale = attn_cases.onehot_v(32768, 256, 8, 2, F16, seed=1)
        check_inputs(q, k, v, 32768, 256, 8, 2, F16, scale)
    finally:
        wq.wq_set_attn_partition(0)
    for L in (777, 4096, 32768):
        pos = sorted({0, L // 4, L // 2, L - 2, L - 1})
        say(f"dominant keys at {pos}, automatic partitions, L={L}")
        q, k, v, scale = attn_cases.dominant(L, 256, 8, 2, F32, pos, seed=L)
        check_inputs(q, k, v, L, 256, 8, 2, F32, scale)
