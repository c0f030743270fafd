"""CPU checks that the GPU parity cases can see the mistakes they are meant to
catch: the oracle's tolerance around the correct result must exclude the result
of a kernel that skipped a cache token (attention) -- computed here by the
oracle itself on the cache with that token removed.  No GPU involved."""
from __future__ import annotations

import numpy as np

import attn_cases
import oracle


def _outside(ref, bound, other) -> float:
    return float(np.max(np.abs(other - ref) / bound))


def test_onehot_v_sees_a_dropped_token():
    """Scale 0, one-hot V: dropping the first, the last or a middle token puts an
    output outside the tolerance, at L = 32768 (f16 cache, the GPU case's heads) and at
    L = 131072 (one head: each head's outputs are built the same way)."""
    for (L, Hq, Hkv, kvfmt, need) in ((32768, 8, 2, attn_cases.F16, 20.0), (131072, 1, 1, attn_cases.F32, 5.0)):
        q, k, v, scale = attn_cases.onehot_v(L, 256, Hq, Hkv, kvfmt)
        ref, bound = oracle.decode_attention(q, k, v, kvfmt, L, 256, Hq, Hkv, scale)
        for t in (0, L // 2 + 3, L - 1):
            kd, vd = np.delete(k, t, axis=0), np.delete(v, t, axis=0)
            other, _ = oracle.decode_attention(q, kd, vd, kvfmt, L - 1, 256, Hq, Hkv, scale)
            assert _outside(ref, bound, other) > need, (L, t)


def test_dominant_keys_see_a_dropped_edge_token():
    """Keys dominating at partition edges: dropping any one of them moves an output
    far outside the tolerance (at least 100x)."""
    L, part = 4096, 64
    pos = attn_cases.edge_positions(L, part)
    assert pos == sorted({0, 63, 64, 127, 4032, 4031, 4095})
    q, k, v, scale = attn_cases.dominant(L, 256, 8, 2, attn_cases.F16, pos, seed=part)
    ref, bound = oracle.decode_attention(q, k, v, attn_cases.F16, L, 256, 8, 2, scale)
    for t in pos:
        other, _ = oracle.decode_attention(q, np.delete(k, t, 0), np.delete(v, t, 0), attn_cases.F16, L - 1,
                                           256, 8, 2, scale)
        assert _outside(ref, bound, other) > 100.0, t
