"""Pins of the oracle's sparse attention over the selected positions (CPU):
a pure-Python brute force, closed forms, invariance to the order of the
selection, and the log-sum-exp merge of a split selection."""
import math

import numpy as np
import pytest

import oracle
from sparse_attention_kv_indexer_amd import workloads as wl


def _case(seed, B=3, H=4, KD=8, S=3, k=10):
    rng = np.random.default_rng(seed)
    inp = wl.random_case(seed, B, S, lens=[S * 64] * B)
    q = wl.round_to_bf16_bits(rng.standard_normal((B, H, KD)).astype(np.float32))
    kv = wl.round_to_bf16_bits(rng.standard_normal((inp.num_pages, wl.PAGE, KD)).astype(np.float32))
    idx = np.stack([rng.choice(S * 64, size=k, replace=False) for _ in range(B)]).astype(np.int64)
    return inp, q, kv, idx


def test_brute_force_small():
    inp, q, kv, idx = _case(0)
    scale, vd = 0.37, 6
    out, lse = oracle.sparse_attention(q, kv, inp.page_table, idx, scale, vd)
    qf = oracle.bf16_bits_to_f64(q)
    kf = oracle.bf16_bits_to_f64(kv)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            rows = [kf[inp.page_table[b, s // 64], s % 64] for s in idx[b]]
            sc = [scale * math.fsum(float(qf[b, h, d]) * float(r[d]) for d in range(q.shape[2])) for r in rows]
            m = max(sc)
            ws = [math.exp(x - m) for x in sc]
            tot = math.fsum(ws)
            assert lse[b, h] == pytest.approx(m + math.log(tot), rel=1e-13, abs=1e-13)
            for d in range(vd):
                ref = math.fsum(w_ * float(r[d]) for w_, r in zip(ws, rows)) / tot
                assert out[b, h, d] == pytest.approx(ref, rel=1e-12, abs=1e-13)


def test_single_position_returns_its_value():
    inp, q, kv, idx = _case(1, k=10)
    idx[:, 1:] = -1
    out, lse = oracle.sparse_attention(q, kv, inp.page_table, idx, 0.5, 6)
    kf = oracle.bf16_bits_to_f64(kv)
    qf = oracle.bf16_bits_to_f64(q)
    for b in range(idx.shape[0]):
        s = idx[b, 0]
        lat = kf[inp.page_table[b, s // 64], s % 64]
        assert np.array_equal(out[b], np.broadcast_to(lat[:6], out[b].shape))
        assert np.allclose(lse[b], 0.5 * (qf[b] @ lat), rtol=0, atol=1e-12)


def test_zero_query_averages_the_values():
    inp, q, kv, idx = _case(2)
    q[:] = 0
    out, lse = oracle.sparse_attention(q, kv, inp.page_table, idx, 1.0, 8)
    kf = oracle.bf16_bits_to_f64(kv)
    for b in range(idx.shape[0]):
        lat = np.stack([kf[inp.page_table[b, s // 64], s % 64] for s in idx[b]])
        assert np.allclose(out[b], lat.mean(axis=0), rtol=0, atol=1e-13)
        assert np.allclose(lse[b], math.log(idx.shape[1]), rtol=0, atol=1e-13)


def test_order_of_selection_does_not_matter():
    inp, q, kv, idx = _case(3)
    a = oracle.sparse_attention(q, kv, inp.page_table, idx, 0.3, 8)
    rev = idx[:, ::-1].copy()
    b = oracle.sparse_attention(q, kv, inp.page_table, rev, 0.3, 8)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-13) and np.allclose(a[1], b[1], rtol=0, atol=1e-13)


def test_split_selection_merges_by_log_sum_exp():
    """Attention over a union equals the LSE-weighted merge of its parts."""
    inp, q, kv, idx = _case(4, k=12)
    full = oracle.sparse_attention(q, kv, inp.page_table, idx, 0.4, 8)
    p1 = oracle.sparse_attention(q, kv, inp.page_table, np.where(np.arange(12) < 5, idx, -1), 0.4, 8)
    p2 = oracle.sparse_attention(q, kv, inp.page_table, np.where(np.arange(12) >= 5, idx, -1), 0.4, 8)
    m = np.maximum(p1[1], p2[1])
    w1, w2 = np.exp(p1[1] - m), np.exp(p2[1] - m)
    merged = (w1[..., None] * p1[0] + w2[..., None] * p2[0]) / (w1 + w2)[..., None]
    assert np.allclose(merged, full[0], rtol=0, atol=1e-13)
    assert np.allclose(m + np.log(w1 + w2), full[1], rtol=0, atol=1e-13)


def test_empty_selection():
    inp, q, kv, idx = _case(5)
    idx[1] = -1
    out, lse = oracle.sparse_attention(q, kv, inp.page_table, idx, 1.0, 8)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(lse[0]))


def test_generator_shapes():
    inp = wl.generate("tiny")
    att = wl.attention_inputs(inp, 0)
    assert att.q_bits.shape == (1, wl.ATT_HEADS, wl.ATT_KD) and att.q_bits.dtype == np.uint16
    assert att.kv_bits.shape == (inp.num_pages, wl.PAGE, wl.ATT_KD)
    assert att.scale == pytest.approx(1 / math.sqrt(192))


def test_positions_off_the_table_or_pool_poison_only_their_request():
    inp, q, kv, idx = _case(6, B=4)
    pt = inp.page_table.copy()
    idx[1, 3] = pt.shape[1] * 64          # past the page table
    pt[2, idx[2, 0] // 64] = kv.shape[0]  # page id outside the pool
    pt[3, idx[3, 0] // 64] = -5
    out, lse = oracle.sparse_attention(q, kv, pt, idx, 0.5, 8)
    for b in (1, 2, 3):
        assert np.all(np.isnan(out[b])) and np.all(np.isnan(lse[b]))
    assert np.all(np.isfinite(out[0])) and np.all(np.isfinite(lse[0]))
    # a negative entry is never looked up, whatever its page would be
    idx2 = idx.copy()
    idx2[0, 0] = -7
    out2, _ = oracle.sparse_attention(q, kv, inp.page_table, idx2, 0.5, 8)
    assert np.all(np.isfinite(out2[0]))


def test_selection_recipe():
    inp = wl.random_case(7, 5, 4, lens=[0, 10, 64, 256, 300])
    sel = wl.random_selection(inp, 100, 0)
    assert sel.dtype == np.int32 and sel.shape == (5, 100)
    for b, L in enumerate([0, 10, 64, 256, 256]):
        n = min(100, L)
        row = sel[b]
        assert np.all(row[n:] == -1)
        assert np.all(np.diff(row[:n]) > 0) and (n == 0 or (row[0] >= 0 and row[n - 1] < L))


def test_a_repeated_position_counts_twice():
    """Selection [s, s, t]: weights e^a, e^a, e^b (closed form with two distinct latents)."""
    inp, q, kv, idx = _case(8, B=1, k=3)
    s_, t_ = int(idx[0, 0]), int(idx[0, 1])
    sel = np.array([[s_, s_, t_]], dtype=np.int64)
    out, lse = oracle.sparse_attention(q, kv, inp.page_table, sel, 0.3, 8)
    qf = oracle.bf16_bits_to_f64(q)[0]
    kf = oracle.bf16_bits_to_f64(kv)
    vs = kf[inp.page_table[0, s_ // 64], s_ % 64]
    vt = kf[inp.page_table[0, t_ // 64], t_ % 64]
    a, b = 0.3 * (qf @ vs), 0.3 * (qf @ vt)  # [H]
    want = (2 * np.exp(a)[:, None] * vs[None, :8] + np.exp(b)[:, None] * vt[None, :8]) / (2 * np.exp(a) + np.exp(b))[:, None]
    assert np.allclose(out[0], want, rtol=0, atol=1e-12)
    assert np.allclose(lse[0], np.log(2 * np.exp(a) + np.exp(b)), rtol=0, atol=1e-12)
