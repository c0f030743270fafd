"""The allocation-free LM-head top-k (wq_lm_head_topk_noalloc) through the C ABI,
against the allocating entry point it mirrors (wq_lm_head_topk): the same
kernels, so the same result bit for bit.  Two calls in a row per weight format,
the second with a smaller input (the fixed workspace keeps the first call's
bytes), plus the rejection of a request larger than the workspace."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gemm_wq_gemv_amd as wq
import oracle
import wqgen

pytestmark = pytest.mark.gpu

F16, Q8, Q4 = wq.WQ_FMT_F16, wq.WQ_FMT_Q8_0, wq.WQ_FMT_Q4_0


def say(msg: str):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def weights(n, k, fmt, seed):
    if fmt == Q4:
        return torch.from_numpy(wqgen.q4_0_bytes(n, k, seed)).cuda()
    w = torch.from_numpy(wqgen.weights(n, k, seed)).cuda()
    return wq.pack_f16(w) if fmt == F16 else wq.quantize_q8_0(w)


def call(name, a, b, n, k, fmt, topk, a_ptr=None, b_ptr=None):
    """One call of entry point `name` through ctypes; returns (status, vals, ids)."""
    vals = torch.full((topk,), float("nan"), device="cuda")
    ids = torch.full((topk,), -7, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    fn = getattr(wq._lib, name)
    st = fn(a_ptr or a.data_ptr(), b_ptr or b.data_ptr(), n, k, fmt, topk, vals.data_ptr(), ids.data_ptr(), s)
    torch.cuda.synchronize()
    return st, vals.cpu().numpy(), ids.cpu().numpy()


@pytest.mark.parametrize("fmt", [F16, Q8, Q4], ids=["f16", "q8_0", "q4_0"])
def test_noalloc_equals_allocating_entry_point(fmt):
    """LM head 151936 x 2048 at k = 50, then 5000 x 512 at k = 8: the allocation-free
    call returns exactly what wq_lm_head_topk returns, and the top-k the oracle's
    logits allow."""
    for (n, k, topk, seed) in ((151936, 2048, 50, 1), (5000, 512, 8, 2)):
        say(f"noalloc fmt={fmt} n={n} k={k} topk={topk}")
        b = weights(n, k, fmt, seed)
        a = torch.from_numpy(wqgen.activations(1, k, seed)).cuda()
        st0, v0, i0 = call("wq_lm_head_topk", a, b, n, k, fmt, topk)
        st1, v1, i1 = call("wq_lm_head_topk_noalloc", a, b, n, k, fmt, topk)
        assert st0 == wq.WQ_OK and st1 == wq.WQ_OK, (st0, st1)
        assert np.array_equal(v0, v1) and np.array_equal(i0, i1)
        ref_b = wqgen.q4_0_bytes(n, k, seed) if fmt == Q4 else oracle.encode(wqgen.weights(n, k, seed), fmt)
        _, _, logits, bound = oracle.lm_head_topk(wqgen.activations(1, k, seed), ref_b, fmt, n, k, topk)
        got = i1.astype(np.int64)
        assert len(set(got.tolist())) == topk
        assert np.all(np.abs(v1 - logits[got]) <= bound[got])
        kth = v1[-1]
        # No row whose oracle logit is clearly above the k-th returned value is left out.
        left = np.setdiff1d(np.arange(n), got)
        assert np.all(logits[left] - bound[left] <= kth + bound[got].max())


def test_noalloc_unaligned_f16_rows_take_the_list_route():
    """K = 1001 (f16 rows that take the plain kernel and its per-wave lists) matches
    the allocating entry point."""
    n, k, topk = 20000, 1001, 16
    b = weights(n, k, F16, 3)
    a = torch.from_numpy(wqgen.activations(1, k, 3)).cuda()
    say("noalloc f16 K=1001")
    st0, v0, i0 = call("wq_lm_head_topk", a, b, n, k, F16, topk)
    st1, v1, i1 = call("wq_lm_head_topk_noalloc", a, b, n, k, F16, topk)
    assert st0 == st1 == wq.WQ_OK
    assert np.array_equal(v0, v1) and np.array_equal(i0, i1)


def test_noalloc_rejects_requests_beyond_the_workspace():
    """f16 logits of 1.1 M rows need more than the 4 MiB workspace: WQ_ERR_WORKSPACE,
    nothing written."""
    assert wq.wq_noalloc_workspace_bytes() == 4 << 20
    n, k, topk = 1_100_000, 8, 4
    b = torch.zeros((n, k), dtype=torch.uint16, device="cuda")
    a = torch.zeros(k, device="cuda")
    say("noalloc oversized")
    st, v, i = call("wq_lm_head_topk_noalloc", a, b, n, k, F16, topk)
    assert st == wq.WQ_ERR_WORKSPACE
    assert np.isnan(v).all() and (i == -7).all()
    with pytest.raises(wq.WQError):
        wq.wq_lm_head_topk_noalloc(a, b, n, k, F16, topk, torch.empty(topk, device="cuda"),
                                   torch.empty(topk, dtype=torch.int32, device="cuda"))
