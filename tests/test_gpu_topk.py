"""GPU parity of the LM-head top-k (wq_lm_head_topk, wq_topk) against the CPU oracle.

The ranking is the pages' TopKCandidate rule: higher logit first, equal logits
by the lower id, NaN never selected, (-inf, 0xFFFFFFFF) padding.

wq_topk takes logits the test draws itself, so its result must equal the
oracle's top-k of the same values bit for bit.  wq_lm_head_topk selects on the
f32 logits its own GEMV computes, which differ from the oracle's float64
logits by rounding, so where two logits lie within their tolerances of each
other either order is correct.  The check is then what is unique plus
validity:
  * every returned value is the oracle logit of its id within the product
    tolerance (1e-5 * sum|a w| + 1e-6), ids are distinct, the list is in rank
    order by its own values, and it holds min(topk, non-NaN rows) entries;
  * no row left out beats the last returned one by more than the two
    tolerances, and no returned row trails the oracle's k-th by more;
  * where the oracle's top-(k+1) logits are separated by more than the
    tolerances, the ids equal the oracle's exactly.
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
NO_ID = wq.WQ_TOPK_NO_ID


def say(msg: str):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@functools.lru_cache(maxsize=3)
def encoded(n, k, fmt, seed):
    if fmt == Q4:
        raw = wqgen.q4_0_bytes(n, k, seed)
        return raw, torch.from_numpy(raw).cuda()
    w = wqgen.weights(n, k, seed)
    ref = oracle.encode(w, fmt)
    wd = torch.from_numpy(w).cuda()
    dev = wq.pack_f16(wd) if fmt == F16 else wq.quantize_q8_0(wd)
    torch.cuda.synchronize()
    return ref, dev


def gpu_lm_head_topk(a_np, b_dev, n, k, fmt, topk):
    a = torch.from_numpy(np.ascontiguousarray(a_np, dtype=np.float32).reshape(-1)).cuda()
    vals = torch.full((topk,), float("nan"), device="cuda")
    ids = torch.full((topk,), 12345, dtype=torch.int32, device="cuda")
    wq.wq_lm_head_topk(a, b_dev, n, k, fmt, topk, vals, ids)
    torch.cuda.synchronize()
    return vals.cpu().numpy(), u32(ids)


def u32(ids):
    """Device int32 ids (uint32 bit patterns) -> int64 numpy."""
    return ids.cpu().numpy().view(np.uint32).astype(np.int64)


def check_topk(vals, ids, logits, bound, topk, what):
    """Validity of a GPU top-k against the oracle's float64 logits and bounds."""
    ov, oi = oracle.topk(logits, topk)
    valid = int(min(topk, np.count_nonzero(~np.isnan(logits))))
    assert np.all(ids[valid:] == NO_ID) and np.all(np.isneginf(vals[valid:])), f"{what}: padding"
    g, gv = ids[:valid], vals[:valid].astype(np.float64)
    assert np.all((g >= 0) & (g < logits.size)), f"{what}: id out of range"
    assert np.unique(g).size == valid, f"{what}: repeated id"
    ref = logits[g]
    ok = (np.abs(gv - ref) <= bound[g]) | (gv == ref)
    assert np.all(ok), f"{what}: value off: {gv[~ok]} vs {ref[~ok]}"
    # Rank order by the returned values themselves (exact).
    for r in range(valid - 1):
        assert gv[r] > gv[r + 1] or (gv[r] == gv[r + 1] and g[r] < g[r + 1]), f"{what}: order at {r}"
    if valid == 0:
        return
    # Nothing left out is clearly better than the last returned row ...
    last = g[-1]
    out = np.ones(logits.size, bool)
    out[g] = False
    out &= ~np.isnan(logits)
    slack = bound[out] + bound[last]
    assert np.all(logits[out] <= logits[last] + slack), f"{what}: a row left out beats the last one"
    # ... and nothing returned is clearly worse than the oracle's k-th.
    okth = oi[valid - 1]
    assert np.all(logits[g] >= logits[okth] - bound[g] - bound[okth]), f"{what}: a returned row trails"
    # Unambiguous prefix: exact ids.
    order = np.argsort(-np.nan_to_num(logits, nan=-np.inf), kind="stable")[: valid + 1]
    lv, lb = logits[order], bound[order]
    with np.errstate(invalid="ignore"):  # inf - inf: not separated
        sep = (lv[:-1] - lv[1:]) > (lb[:-1] + lb[1:]) if order.size > 1 else np.ones(0, bool)
    if sep.size == valid and np.all(sep[: valid]):
        assert np.array_equal(g, oi[:valid]), f"{what}: ids {g} vs oracle {oi[:valid]}"


def lm_case(fmt, n, k, topk, seed=0, b_override=None):
    say(f"lm_head_topk fmt={fmt} n={n} k={k} topk={topk} seed={seed}")
    ref_b, dev_b = b_override if b_override is not None else encoded(n, k, fmt, seed)
    a = wqgen.activations(1, k, seed)[0]
    vals, ids = gpu_lm_head_topk(a, dev_b, n, k, fmt, topk)
    _, _, logits, bound = oracle.lm_head_topk(a, ref_b, fmt, n, k, topk)
    check_topk(vals, ids, logits, bound, topk, f"fmt={fmt} n={n} k={k} topk={topk}")
    return vals, ids


@pytest.mark.parametrize("topk", [1, 2, 8, 50, 64])
@pytest.mark.parametrize("fmt", ALL)
def test_lm_head_full_vocab(fmt, topk):
    """The LM head at vocab 151936, hidden 2048 (the decode suite's largest GEMV)."""
    lm_case(fmt, 151936, 2048, topk, seed=1)


GEMV_K = {F16: [64, 1000, 2048, 4096, 8192, 16384, 24584, 1001, 12],
          Q8: [256, 768, 1024, 1536, 2048, 4096, 8192, 10240, 992],
          Q4: [256, 768, 1024, 1536, 2048, 4096, 8192, 10240, 992]}


@pytest.mark.parametrize("fmt", ALL)
def test_every_gemv_family(fmt):
    """Every GEMV kernel family feeds the merge right: f16 K-split logits
    (1..16 waves, 1, 2 or 4 chunk slots per lane) read 64 at a time, the
    quantized kernels' per-wave lists (16/32/64 lanes per row), the plain
    kernels' lists (odd or short K); ragged vocab sizes, fewer rows than k,
    fewer rows than waves."""
    for k in GEMV_K[fmt]:
        for n, topk in ((1, 1), (37, 50), (1000, 1), (5000, 64), (4099, 7)):
            lm_case(fmt, n, k, topk, seed=k + n)


def test_ties_go_to_the_lower_id():
    """Copies of the best row at higher and lower ids: equal f32 logits (every row is
    computed the same way), so the copies must come out in ascending id order."""
    n, k = 20000, 2048
    for fmt in ALL:
        ref_b, _ = encoded(n, k, fmt, 3)
        a = wqgen.activations(1, k, 3)[0]
        _, _, logits, _ = oracle.lm_head_topk(a, ref_b, fmt, n, k, 1)
        best = int(np.nanargmax(logits))
        b = np.array(ref_b, copy=True)
        copies = sorted({3, best, 9000, 19999})
        for c in copies:
            b[c] = b[best]
        say(f"ties fmt={fmt} best={best}")
        vals, ids = gpu_lm_head_topk(a, torch.from_numpy(b).cuda(), n, k, fmt, 6)
        assert list(ids[:len(copies)]) == copies, (fmt, ids)
        assert np.all(vals[:len(copies)] == vals[0])
        _, _, logits2, bound2 = oracle.lm_head_topk(a, b, fmt, n, k, 6)
        check_topk(vals, ids, logits2, bound2, 6, f"ties fmt={fmt}")


def test_nan_and_inf_rows():
    """A NaN weight makes its logit NaN: never selected.  A +inf weight against a
    positive activation gives +inf: ranked first (by id among equals)."""
    n, k = 3000, 1024
    ref_b, _ = encoded(n, k, F16, 4)
    a = wqgen.activations(1, k, 4)[0]
    _, _, logits, _ = oracle.lm_head_topk(a, ref_b, F16, n, k, 1)
    best = int(np.nanargmax(logits))
    b = np.array(ref_b, copy=True)
    b[best, 5] = 0x7E00                      # NaN
    col = int(np.flatnonzero(a > 0)[0])
    r1, r2 = [r for r in (700, 2500, 1500, 2999) if r != best][:2]
    for r in (r1, r2):
        b[r, :] = 0
        b[r, col] = 0x7C00                   # +inf * a[col] > 0 -> +inf
    say("nan / inf rows")
    vals, ids = gpu_lm_head_topk(a, torch.from_numpy(b).cuda(), n, k, F16, 4)
    assert list(ids[:2]) == [r1, r2] and np.all(np.isposinf(vals[:2]))
    assert best not in ids
    _, _, logits2, bound2 = oracle.lm_head_topk(a, b, F16, n, k, 4)
    check_topk(vals, ids, logits2, bound2, 4, "nan/inf")


def test_top1_ties_nan_inf_and_back_to_back_calls():
    """Top-1 of f16 rows on the K-split route, where the argmax is fused into the
    GEMV: copies of the best row go to the lowest id; a NaN best row is skipped;
    +inf rows win by id; all rows NaN gives the sentinel; all logits negative
    still gives the best one; and a call after a call with a larger maximum
    returns its own (nothing is left over from the previous call)."""
    n, k = 20000, 2048
    ref_b, dev_b = encoded(n, k, F16, 3)
    a = wqgen.activations(1, k, 3)[0]
    _, _, logits, _ = oracle.lm_head_topk(a, ref_b, F16, n, k, 1)
    best = int(np.nanargmax(logits))

    say("top1 ties")
    b = np.array(ref_b, copy=True)
    for c in (9000, 19999, 3):
        b[c] = b[best]
    vals, ids = gpu_lm_head_topk(a, torch.from_numpy(b).cuda(), n, k, F16, 1)
    assert ids[0] == 3
    _, _, logits2, bound2 = oracle.lm_head_topk(a, b, F16, n, k, 1)
    check_topk(vals, ids, logits2, bound2, 1, "top1 ties")

    say("top1 nan best row, then +inf rows")
    b = np.array(ref_b, copy=True)
    b[best, 7] = 0x7E00
    vals, ids = gpu_lm_head_topk(a, torch.from_numpy(b).cuda(), n, k, F16, 1)
    assert ids[0] != best
    _, _, logits2, bound2 = oracle.lm_head_topk(a, b, F16, n, k, 1)
    check_topk(vals, ids, logits2, bound2, 1, "top1 nan")
    col = int(np.flatnonzero(a > 0)[0])
    for r in (15001, 4321):
        b[r, :] = 0
        b[r, col] = 0x7C00
    vals, ids = gpu_lm_head_topk(a, torch.from_numpy(b).cuda(), n, k, F16, 1)
    assert ids[0] == 4321 and np.isposinf(vals[0])

    say("top1 all nan")
    b = np.full((n, k), 0x7E00, dtype=np.uint16)
    vals, ids = gpu_lm_head_topk(a, torch.from_numpy(b).cuda(), n, k, F16, 1)
    assert ids[0] == NO_ID and np.isneginf(vals[0])

    say("top1 all negative, after a call with a larger maximum")
    big = gpu_lm_head_topk(a, dev_b, n, k, F16, 1)
    neg = np.array(ref_b, copy=True)
    neg[:, :] = 0
    neg[:, col] = np.float16(-1.0).view(np.uint16)   # every logit = -a[col] ...
    neg[777, col] = np.float16(-0.5).view(np.uint16)  # ... but row 777's is -a[col] / 2
    vals, ids = gpu_lm_head_topk(a, torch.from_numpy(neg).cuda(), n, k, F16, 1)
    assert big[0][0] > 0 and ids[0] == 777 and vals[0] == np.float32(-0.5 * np.float32(a[col]))
    say("top1 ragged row counts")
    for nn in (1, 2, 3, 5, 4097):
        lm_case(F16, nn, 4096, 1, seed=nn)


def test_more_k_than_rows_and_empty():
    for fmt in ALL:
        lm_case(fmt, 5, 256, 8, seed=5)      # 3 sentinels
        lm_case(fmt, 1, 256, 64, seed=6)
    say("n = 0")
    a = torch.zeros(64, device="cuda")
    b = torch.zeros(0, dtype=torch.uint16, device="cuda")
    vals = torch.zeros(4, device="cuda")
    ids = torch.zeros(4, dtype=torch.int32, device="cuda")
    wq.wq_lm_head_topk(a, b, 0, 64, F16, 4, vals, ids)
    torch.cuda.synchronize()
    assert np.all(np.isneginf(vals.cpu().numpy())) and np.all(u32(ids) == NO_ID)
    say("K = 0")
    wq.wq_lm_head_topk(torch.empty(0, device="cuda"), torch.empty(0, dtype=torch.uint16, device="cuda"), 10, 0,
                       F16, 4, vals, ids)
    torch.cuda.synchronize()
    assert list(u32(ids)) == [0, 1, 2, 3] and np.all(vals.cpu().numpy() == 0)


@pytest.mark.parametrize("n", [1, 63, 64, 65, 4097, 151936])
def test_topk_of_given_logits_is_exact(n):
    """wq_topk on seeded logits (with ties, NaN and infinities) equals the oracle's
    top-k of the same values, ids and values bit for bit."""
    rng = np.random.default_rng(n)
    for kind in ("normal", "ties"):
        x = wqgen.normal((n,), seed=n, stream=9)
        if kind == "ties":
            x = np.round(x * 2).astype(np.float32)
        if n > 10:
            x[rng.integers(0, n, n // 50 + 1)] = np.nan
            x[rng.integers(0, n, 2)] = np.inf
            x[rng.integers(0, n, 2)] = -np.inf
        xd = torch.from_numpy(x).cuda()
        for topk in (1, 7, 50, 64):
            say(f"wq_topk n={n} {kind} topk={topk}")
            vals = torch.zeros(topk, device="cuda")
            ids = torch.zeros(topk, dtype=torch.int32, device="cuda")
            wq.wq_topk(xd, n, topk, vals, ids)
            torch.cuda.synchronize()
            ov, oi = oracle.topk(x.astype(np.float64), topk)
            assert np.array_equal(u32(ids), oi), (kind, topk)
            assert np.array_equal(vals.cpu().numpy().astype(np.float64), ov), (kind, topk)


@pytest.mark.parametrize("fmt", ALL)
def test_fused_equals_logits_then_topk(fmt):
    """The fused call selects on the same f32 logits as wq_matmul computes (the
    same GEMV kernel: the argmax and logits routes run the store kernel's
    arithmetic, the list routes the same row sums), so it equals wq_matmul
    followed by wq_topk bit for bit."""
    n, k = 151936, 2048
    _, dev_b = encoded(n, k, fmt, 1)
    a = torch.from_numpy(wqgen.activations(1, k, 1)).cuda()
    logits = torch.empty((1, n), device="cuda")
    wq.wq_matmul(a, dev_b, logits, 1, n, k, fmt)
    torch.cuda.synchronize()
    for topk in (1, 50):
        say(f"fused vs unfused fmt={fmt} topk={topk}")
        v1, i1 = wq.lm_head_topk(a, dev_b, n, k, fmt, topk)
        v2 = torch.empty(topk, device="cuda")
        i2 = torch.empty(topk, dtype=torch.int32, device="cuda")
        wq.wq_topk(logits, n, topk, v2, i2)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2) and torch.equal(v1, v2)
