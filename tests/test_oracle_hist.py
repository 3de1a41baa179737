"""CPU pins of the oracle's key map and first-digit histogram (the fused
score + top-k pair): the IEEE-754 layout fixes some keys outright, the key
order must be the ranking the oracle's top-k uses (checked against sorting
floats, not against the map itself), and the histogram must place the k-th
largest score of every row in the bin its prefix counts name."""
import numpy as np
import pytest

import oracle


def test_keys_of_known_bit_patterns():
    # 1.0 is 0x3F800000 and -1.0 is 0xBF800000 in IEEE-754 binary32
    k = oracle.order_keys(np.array([1.0, -1.0, 0.0, -0.0, np.inf, -np.inf, np.nan], np.float32))
    assert k[0] == 0xBF800000 and k[0] >> 21 == 1532
    assert k[1] == 0x407FFFFF and k[1] >> 21 == 515
    assert k[2] == k[3] == 0x80000000
    assert k[4] == 0xFF800000 and k[5] == 0x007FFFFF
    assert k[6] == 1


def test_key_order_is_the_float_order():
    f = np.finfo(np.float32)
    tiny_sub = np.float32(1e-45)  # smallest subnormal
    ladder = np.array([-np.inf, -f.max, -1e10, -1.5, -1.0, -f.tiny, -tiny_sub, -0.0, 0.0, tiny_sub, f.tiny,
                       1.0, 1.5, 1e10, f.max, np.inf], np.float32)
    k = oracle.order_keys(ladder).astype(np.int64)
    d = np.diff(k)
    assert np.all(d[:7] > 0) and d[7] == 0 and np.all(d[8:] > 0)  # -0 and +0 share a key
    assert oracle.order_keys(np.array([np.nan], np.float32))[0] < k.min()
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(5000) * np.exp2(rng.integers(-30, 30, 5000))).astype(np.float32)
    x[::50] = np.round(x[::50])  # ties, zeros of both signs
    x[::77] = -0.0
    order = np.argsort(oracle.order_keys(x), kind="stable")
    assert np.all(np.diff(x[order].astype(np.float64)) >= 0)


def test_histogram_counts_valid_positions():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 300)).astype(np.float32)
    x[2, 5:9] = [0.0, -0.0, np.nan, -np.inf]
    lens = np.array([0, 1, 300, 1000, -4])
    h = oracle.key_histogram(x, lens)
    assert h.shape == (5, 2048) and h.dtype == np.uint32
    assert h.sum(axis=1).tolist() == [0, 1, 300, 300, 0]
    # -0 and +0 in one bin, NaN in bin 0, -inf in bin 0x007FFFFF >> 21 = 3
    h1 = oracle.key_histogram(np.array([[0.0, -0.0, np.nan, -np.inf]], np.float32), [4])[0]
    assert h1[1024] == 2 and h1[0] == 1 and h1[3] == 1


@pytest.mark.parametrize("k", [1, 7, 64, 299, 300])
def test_kth_largest_lies_in_the_bin_the_prefix_counts_name(k):
    """With t the bin of each row's k-th ranked score (by the oracle's own
    top-k, a lexsort), fewer than k keys lie above bin t and at least k in or
    above it."""
    rng = np.random.default_rng(k)
    x = rng.standard_normal((6, 300)).astype(np.float32)
    x[1] = np.round(x[1] * 2) / 2                 # heavy ties
    x[2] = -np.abs(x[2])                          # all negative
    x[3, ::4] = np.nan
    x[4] *= np.float32(1e-30)                     # tiny magnitudes
    lens = np.array([300, 300, 250, 300, 300, 120])
    h = oracle.key_histogram(x, lens).astype(np.int64)
    sel = oracle.topk(x, lens, k)
    for b in range(6):
        chosen = sel[b][sel[b] >= 0]
        if chosen.size < k:
            continue
        worst = x[b, chosen]
        kth = np.nan if np.isnan(worst).any() else worst.min()
        t = int(oracle.order_keys(np.array([kth], np.float32))[0] >> 21)
        above, at_or_above = h[b, t + 1:].sum(), h[b, t:].sum()
        assert above < k <= at_or_above, (b, t, above, at_or_above)
