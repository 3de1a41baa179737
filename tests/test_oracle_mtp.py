"""Pins of the oracle's multi-token scores (CPU): one token is the plain
step, a pure-Python brute force on a tiny case, token independence, and the
causal structure of the input recipe."""
import math

import numpy as np

import oracle
from sparse_attention_kv_indexer_amd import workloads as wl


def test_one_token_is_the_plain_step():
    inp = wl.random_case(21, 3, 4, lens=[0, 100, 256])
    q = inp.q_bits[:, None]
    w = inp.w[:, None]
    got = oracle.score_mtp(q, w, inp.k_bits, inp.page_table, inp.seq_lens[:, None])
    want = oracle.score(inp.q_bits, inp.w, inp.k_bits, inp.page_table, inp.seq_lens)
    assert np.array_equal(got[:, 0], want, equal_nan=True)


def test_brute_force_tiny():
    inp = wl.random_case(22, 2, 2, lens=[128, 128])
    mt = wl.mtp_inputs(inp, 3, 5)
    mt.seq_lens[:] = np.array([[0, 70, 128], [128, 1, 64]], np.int32)
    got = oracle.score_mtp(mt.q_bits, mt.w, inp.k_bits, inp.page_table, mt.seq_lens)
    q = oracle.bf16_bits_to_f64(mt.q_bits)
    k = oracle.bf16_bits_to_f64(inp.k_bits)
    for b in range(2):
        for t in range(3):
            L = int(mt.seq_lens[b, t])
            for s in range(128):
                if s >= L:
                    assert got[b, t, s] == -np.inf
                    continue
                key = k[inp.page_table[b, s // 64], s % 64]
                terms = []
                for h in range(32):
                    dot = math.fsum(float(q[b, t, h, d]) * float(key[d]) for d in range(64))
                    terms.append(float(mt.w[b, t, h]) * max(dot, 0.0))
                assert abs(got[b, t, s] - math.fsum(terms)) <= 1e-12 * (1 + abs(math.fsum(terms)))


def test_tokens_are_independent_rows():
    inp = wl.random_case(23, 2, 3, lens=[150, 192])
    mt = wl.mtp_inputs(inp, 4, 6)
    a = oracle.score_mtp(mt.q_bits, mt.w, inp.k_bits, inp.page_table, mt.seq_lens)
    perm = [2, 0, 3, 1]
    b = oracle.score_mtp(mt.q_bits[:, perm], mt.w[:, perm], inp.k_bits, inp.page_table, mt.seq_lens[:, perm])
    assert np.array_equal(a[:, perm], b, equal_nan=True)
    # the same query with a shorter length is the longer row cut off with -inf
    q2 = np.repeat(mt.q_bits[:, :1], 2, axis=1)
    w2 = np.repeat(mt.w[:, :1], 2, axis=1)
    lens = np.array([[150, 90], [192, 0]], np.int32)
    c = oracle.score_mtp(q2, w2, inp.k_bits, inp.page_table, lens)
    for b_ in range(2):
        L = lens[b_, 1]
        assert np.array_equal(c[b_, 1, :L], c[b_, 0, :L]) and np.all(np.isneginf(c[b_, 1, L:]))


def test_recipe_is_causal():
    inp = wl.generate("c2")
    mt = wl.mtp_inputs(inp, 4, 0)
    assert mt.q_bits.shape == (16, 4, 32, 64) and mt.w.shape == (16, 4, 32) and mt.seq_lens.shape == (16, 4)
    assert np.all(mt.seq_lens[:, -1] == inp.seq_lens)
    assert np.all(np.diff(mt.seq_lens, axis=1) >= 0)
    assert np.all(mt.seq_lens[:, 0] >= inp.seq_lens - 1)
