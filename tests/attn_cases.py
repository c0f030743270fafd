"""Attention inputs built so that a kernel that skips a cache token fails the
tolerance check (shared by the GPU parity tests and the CPU check that each
case really has that property; no arithmetic of the method lives here).

* ``onehot_v``: scale 0 makes every softmax weight 1/L, and V row t of KV head
  h is the unit vector e_((t + 7h) mod D).  Output d of a head is then the
  fraction of tokens t with (t + 7h) mod D == d, so dropping any one token moves
  one output by about 1/L, while the tolerance there is about
  1e-5 * (1/D) + 1e-6 (the score tolerance vanishes with the scale).
* ``dominant``: every query head shares a direction u (entries +-1) plus a small
  random part, background keys are small random vectors (near-uniform weights),
  and the keys at the chosen positions are alpha * u with alpha set so that each
  of them scores ln(L) above the background: each then carries a weight of about
  1 / (count + 1), and dropping one moves the outputs by a large fraction of a V
  value.
"""
from __future__ import annotations

import numpy as np

import wqgen

F32, F16 = 0, 1


def _encode(x: np.ndarray, kvfmt: int) -> np.ndarray:
    return x.astype(np.float16).view(np.uint16) if kvfmt == F16 else x.astype(np.float32)


def onehot_v(L: int, D: int, Hq: int, Hkv: int, kvfmt: int, seed: int = 0):
    """(q, k, v, scale) with scale 0 and one-hot V rows."""
    q = wqgen.normal((Hq, D), seed=seed, stream=21)
    k = wqgen.normal((L, Hkv * D), seed=seed, stream=22)
    v = np.zeros((L, Hkv, D), np.float32)
    t = np.arange(L)
    for h in range(Hkv):
        v[t, h, (t + 7 * h) % D] = 1.0
    return q, _encode(k, kvfmt), _encode(v.reshape(L, Hkv * D), kvfmt), 0.0


def dominant(L: int, D: int, Hq: int, Hkv: int, kvfmt: int, positions, seed: int = 0):
    """(q, k, v, scale): keys at `positions` dominate the softmax of every head."""
    scale = float(np.float32(1.0 / np.sqrt(D)))
    u = np.where(wqgen.normal((D,), seed=seed, stream=23) >= 0, 1.0, -1.0).astype(np.float32)
    q = (u[None, :] + 0.1 * wqgen.normal((Hq, D), seed=seed, stream=24)).astype(np.float32)
    k = (0.05 * wqgen.normal((L, Hkv * D), seed=seed, stream=25)).reshape(L, Hkv, D)
    alpha = np.float32(np.log(L) / (scale * D))       # score of alpha * u: about ln(L)
    for t in positions:
        k[t, :, :] = alpha * u
    v = wqgen.normal((L, Hkv * D), seed=seed, stream=26)
    return q, _encode(k.reshape(L, Hkv * D), kvfmt), _encode(v, kvfmt), scale


def edge_positions(L: int, part: int):
    """The first and last token, and the first and last token of the second and of
    the last partition of `part` tokens."""
    last = (L - 1) // part * part
    return sorted({0, L - 1, part - 1, min(part, L - 1), min(2 * part - 1, L - 1), last, max(last - 1, 0)})
