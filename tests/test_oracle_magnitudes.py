"""Pins of the oracle's tolerance scales (CPU): M and A fix the size of every
score tolerance the GPU parity tests apply, so each is checked from both
sides against a pure-Python computation of its definition, not only bounded.

    M_s = sum_h |w_h| * |q_h . k_s|              (size of the head terms)
    A_s = sum_h |w_h| * sum_d |q_hd * k_sd|      (size of the products)

Each dot product is a correctly rounded sum of exact products (math.fsum of
bfloat16 x bfloat16, or bfloat16 x scaled-e4m3 values, both exact in float64),
then the head sum is taken in exact rationals. The fp8 keys are decoded by
torch's float8_e4m3fn conversion, not by the oracle's own decoder. The
accuracy claim these scales stand in for is the relative error the page "The
Final Piece: Documenting a ~17x Throughput Breakthrough on Blackwell GPUs"
quotes in its section "What the Message Actually Contains".
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_attention_kv_indexer_amd import workloads as wl

H, D, P = wl.HEADS, wl.DIM, wl.PAGE
REL = 1e-12


def _bf16(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _brute_mag(qrows, wrow, key):
    """(M, A) of one key against one query block, by definition."""
    m, a = Fraction(0), Fraction(0)
    for h in range(H):
        wh = Fraction(abs(float(wrow[h])))
        dot = math.fsum(qrows[h][d] * key[d] for d in range(D))
        m += wh * Fraction(abs(dot))
        a += wh * Fraction(math.fsum(abs(qrows[h][d] * key[d]) for d in range(D)))
    return float(m), float(a)


def _assert_close(got, want, where):
    assert abs(got - want) <= REL * abs(want) + 1e-300, (where, got, want)


def _check(M, A, lens, qrows_of, wrow_of, key_of, rows):
    """M, A [rows..., N] against brute force at every position of every row;
    exactly 0 at and past the row's length."""
    for r in rows:
        L = int(lens[r])
        qrows, wrow = qrows_of(r), wrow_of(r)
        for s in range(M[r].shape[-1]):
            if s >= L:
                assert M[r][s] == 0 and A[r][s] == 0, (r, s)
                continue
            m, a = _brute_mag(qrows, wrow, key_of(r, s))
            _assert_close(M[r][s], m, ("M", r, s))
            _assert_close(A[r][s], a, ("A", r, s))


def _bf16_case(seed):
    lens = [[70, 128, 1], [130, 0, 192], [64, 65, 191]][seed]
    return wl.random_case(seed + 40, batch=3, max_pages=3, lens=lens, pool_extra=2)


def check_bf16_magnitudes(seed):
    inp = _bf16_case(seed)
    M, A = oracle.score_magnitudes(inp.q_bits, inp.w, inp.k_bits, inp.page_table, inp.seq_lens)
    assert M.shape == A.shape == (inp.batch, inp.max_c4)
    N = inp.max_c4
    lens = np.clip(inp.seq_lens, 0, N)
    qs = [[[_bf16(x) for x in inp.q_bits[b][h]] for h in range(H)] for b in range(inp.batch)]

    def key_of(b, s):
        return [_bf16(x) for x in inp.k_bits[int(inp.page_table[b][s // P])][s % P]]

    _check(M, A, lens, lambda b: qs[b], lambda b: inp.w[b], key_of, range(inp.batch))


@pytest.mark.parametrize("seed", range(3))
def test_bf16_magnitudes_equal_their_definition(seed):
    check_bf16_magnitudes(seed)


def check_fp8_magnitudes(seed):
    torch = pytest.importorskip("torch")
    inp = wl.random_case(seed + 50, 2, 3, lens=[150, 64])
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(inp.num_pages, P, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30  # no NaN codes
    scale = rng.uniform(0.05, 3.0, size=(inp.num_pages, P)).astype(np.float32)
    scale[0, :4] = [-0.5, 0.0, 1.0, 2.0 ** -12]
    M, A = oracle.score_magnitudes_fp8(inp.q_bits, inp.w, codes, scale, inp.page_table, inp.seq_lens)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    lens = np.clip(inp.seq_lens, 0, inp.max_c4)
    qs = [[[_bf16(x) for x in inp.q_bits[b][h]] for h in range(H)] for b in range(inp.batch)]

    def key_of(b, s):
        p, i = int(inp.page_table[b][s // P]), s % P
        return [float(dec[p, i, d]) * float(scale[p, i]) for d in range(D)]

    _check(M, A, lens, lambda b: qs[b], lambda b: inp.w[b], key_of, range(inp.batch))


@pytest.mark.parametrize("seed", range(2))
def test_fp8_magnitudes_equal_their_definition(seed):
    check_fp8_magnitudes(seed)


def check_mtp_magnitudes(seed):
    inp = wl.random_case(seed + 60, 2, 2, lens=[128, 100])
    mt = wl.mtp_inputs(inp, 3, seed + 7)
    mt.seq_lens[:] = np.array([[0, 70, 128], [100, 1, 64]], np.int32)
    M, A = oracle.score_magnitudes_mtp(mt.q_bits, mt.w, inp.k_bits, inp.page_table, mt.seq_lens)
    assert M.shape == A.shape == (2, 3, inp.max_c4)
    Mf, Af = M.reshape(6, -1), A.reshape(6, -1)
    lens = mt.seq_lens.reshape(6)
    qs = [[[_bf16(x) for x in mt.q_bits[r // 3, r % 3, h]] for h in range(H)] for r in range(6)]

    def key_of(r, s):
        return [_bf16(x) for x in inp.k_bits[int(inp.page_table[r // 3][s // P])][s % P]]

    _check(Mf, Af, lens, lambda r: qs[r], lambda r: mt.w[r // 3, r % 3], key_of, range(6))


@pytest.mark.parametrize("seed", range(2))
def test_mtp_magnitudes_equal_their_definition(seed):
    check_mtp_magnitudes(seed)


def test_magnitudes_closed_form():
    """One head, q = e_0 and w_h = -2: a key with k[0] = -3 and k[1] = 5 has
    q . k = -3, so M = 2 * 3 = 6 and A = 2 * 3 = 6; with q = e_0 + e_1 the dot
    is 2 while the products are -3 and 5: M = 2 * 2 = 4 but A = 2 * 8 = 16."""
    q = np.zeros((1, H, D), np.float32)
    w = np.zeros((1, H), np.float32)
    k = np.zeros((1, P, D), np.float32)
    table = np.zeros((1, 1), np.int32)
    w[0, 3] = -2.0
    k[0, 0, 0], k[0, 0, 1] = -3.0, 5.0
    q[0, 3, 0] = 1.0
    bits = wl.round_to_bf16_bits
    M, A = oracle.score_magnitudes(bits(q), w, bits(k), table, np.array([1], np.int32))
    assert (M[0, 0], A[0, 0]) == (6.0, 6.0)
    q[0, 3, 1] = 1.0
    M, A = oracle.score_magnitudes(bits(q), w, bits(k), table, np.array([1], np.int32))
    assert (M[0, 0], A[0, 0]) == (4.0, 16.0)
