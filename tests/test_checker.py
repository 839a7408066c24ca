"""The comparison rules can fail: correct results pass, planted errors fail."""
import numpy as np
import pytest

import oracle
from checker import Mismatch, check_sfa, check_topk_row


def _ref(seed=0, n=500, k=64):
    r = np.random.default_rng(seed)
    s = r.standard_normal(n)
    idx = oracle.topk_select(s, k)
    return dict(t=n - 1, scores=s, idx=idx, kth=np.sort(s)[::-1][k - 1])


def test_topk_exact_passes_in_any_order():
    ref = _ref()
    row = np.random.default_rng(1).permutation(ref["idx"])
    assert check_topk_row(row, ref, 64) == 0


def test_topk_swap_far_from_boundary_fails():
    ref = _ref()
    row = ref["idx"].copy()
    worst = int(np.argmin(ref["scores"]))
    row[0] = worst
    with pytest.raises(Mismatch):
        check_topk_row(row, ref, 64)


def test_topk_swap_within_band_passes():
    s = np.arange(100, dtype=float)
    s[50] = 90.0 + 1e-5          # nearly tied with the k-th (90.0)
    idx = oracle.topk_select(s, 10)
    ref = dict(t=99, scores=s, idx=idx, kth=np.sort(s)[::-1][9])
    assert 50 in idx and 90 not in idx
    row = idx.copy()
    row[row == 50] = 90
    assert check_topk_row(row, ref, 10) == 2


def test_topk_padding_and_duplicates_fail():
    ref = dict(t=5, scores=np.arange(6.0), idx=np.arange(6), kth=0.0)
    ok = np.array([5, 4, 3, 2, 1, 0, -1, -1])
    assert check_topk_row(ok, ref, 8) == 0
    with pytest.raises(Mismatch):
        check_topk_row(np.array([5, 4, 3, 2, 1, 0, 0, -1]), ref, 8)
    with pytest.raises(Mismatch):
        check_topk_row(np.array([5, 5, 3, 2, 1, 0, -1, -1]), ref, 8)
    with pytest.raises(Mismatch):
        check_topk_row(np.array([5, 4, 3, 2, 1, 6, -1, -1]), ref, 8)


def test_sfa_rules():
    r = np.random.default_rng(3)
    ref = r.standard_normal((8, 16)) * 0.01
    check_sfa(ref + 1e-5, ref, "bf16")
    with pytest.raises(Mismatch):
        check_sfa(ref + 3e-2, ref, "bf16")          # absolute bar
    with pytest.raises(Mismatch):
        check_sfa(np.zeros_like(ref), ref, "bf16")  # passes 2e-2 abs, fails rel-L2
    big = ref.copy(); big[0, 0] = 20.0
    check_sfa(np.where(big > 16, big + 0.06, big), big, "bf16")   # bf16 rounding of a large output
    with pytest.raises(Mismatch):
        check_sfa(np.where(big > 16, big + 0.2, big), big, "bf16")
    with pytest.raises(Mismatch):
        bad = ref.copy(); bad[0, 0] = np.nan
        check_sfa(bad, ref, "bf16")
