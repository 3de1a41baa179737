"""Pins of the oracle's top-k: pure-Python brute force, closed forms and the
defining property. CPU only."""
import math

import numpy as np
import pytest

import oracle


def _brute_topk(row, L, k):
    """Sort positions with Python's sorted() on the key (NaN last, larger
    score first, lower index first), keep min(k, L), list them ascending."""
    def key(i):
        x = float(row[i])
        return (1, 0.0, i) if math.isnan(x) else (0, -x, i)

    chosen = sorted(sorted(range(L), key=key)[:min(k, L)])
    return chosen + [-1] * (k - len(chosen))


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_random_with_ties(seed):
    rng = np.random.default_rng(seed)
    B, N = 4, 200
    x = rng.integers(-6, 7, size=(B, N)).astype(np.float32)  # many exact ties
    x[0, 5] = -0.0
    x[0, 9] = 0.0
    x[1, 3] = np.nan
    lens = rng.integers(0, N + 1, size=B)
    for k in (1, 7, 64, 199, 250):
        got = oracle.topk(x, lens, k)
        for b in range(B):
            assert got[b].tolist() == _brute_topk(x[b], int(lens[b]), k), (b, k)


def test_selected_dominate_unselected():
    rng = np.random.default_rng(42)
    x = rng.standard_normal((3, 1000))
    lens = np.array([1000, 517, 3])
    idx = oracle.topk(x, lens, 100)
    for b in range(3):
        L = lens[b]
        sel = idx[b][idx[b] >= 0]
        assert sel.size == min(100, L) and np.all(sel < L) and np.all(np.diff(sel) > 0)
        rest = np.setdiff1d(np.arange(L), sel)
        if rest.size and sel.size:
            assert x[b, sel].min() >= x[b, rest].max()


def test_all_equal_takes_lowest_indices():
    x = np.full((1, 300), 1.5)
    assert oracle.topk(x, [300], 10)[0].tolist() == list(range(10))


def test_monotone_rows():
    inc = np.arange(100, dtype=np.float64)[None]
    assert oracle.topk(inc, [100], 5)[0].tolist() == [95, 96, 97, 98, 99]
    assert oracle.topk(inc, [60], 5)[0].tolist() == [55, 56, 57, 58, 59]
    dec = -inc
    assert oracle.topk(dec, [100], 5)[0].tolist() == [0, 1, 2, 3, 4]


def test_padding_and_empty_rows():
    x = np.arange(10, dtype=np.float64)[None].repeat(2, 0)
    got = oracle.topk(x, [0, 4], 6)
    assert got[0].tolist() == [-1] * 6
    assert got[1].tolist() == [0, 1, 2, 3, -1, -1]


def test_signed_zeros_tie_and_nan_last():
    x = np.array([[-0.0, 0.0, -0.0, np.nan, -1.0]])
    assert oracle.topk(x, [5], 1)[0].tolist() == [0]
    assert oracle.topk(x, [5], 3)[0].tolist() == [0, 1, 2]
    assert oracle.topk(x, [5], 4)[0].tolist() == [0, 1, 2, 4]
    assert oracle.topk(x, [5], 5)[0].tolist() == [0, 1, 2, 3, 4]


def test_masked_tail_never_selected():
    x = np.concatenate([np.full(10, -5.0), np.full(10, -np.inf)])[None]
    assert oracle.topk(x, [10], 15)[0].tolist() == list(range(10)) + [-1] * 5


def test_values_follow_indices():
    x = np.array([[3.0, 1.0, 2.0, 5.0]])
    idx = oracle.topk(x, [4], 3)
    assert idx[0].tolist() == [0, 2, 3]
    assert oracle.topk_values(x, idx)[0].tolist() == [3.0, 2.0, 5.0]
