"""Pins of the oracle's fp8-key path (CPU): the e4m3fn decode against torch's
float8_e4m3fn conversion and closed forms, the fp8 score against the pinned
bf16 score on keys both formats hold exactly, and the exact scaling law."""
import numpy as np
import pytest

import oracle
from sparse_attention_kv_indexer_amd import workloads as wl

torch = pytest.importorskip("torch")


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(mine[fin], ref[fin])
    assert np.array_equal(np.signbit(mine[fin]), np.signbit(ref[fin]))


@pytest.mark.parametrize("code,value", [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
                                        (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0), (0x80, -0.0),
                                        (0xB8, -1.0), (0xFE, -448.0)])
def test_e4m3_decode_closed_forms(code, value):
    got = oracle.e4m3_to_f64(np.array([code], np.uint8))[0]
    assert got == value and np.signbit(got) == np.signbit(value)


def test_e4m3_nan_codes():
    assert np.all(np.isnan(oracle.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))))


def _fp8_case(seed, B=3, S=4, lens=(200, 64, 1), pow2_scales=True):
    inp = wl.random_case(seed, B, S, lens=list(lens))
    rng = np.random.default_rng(seed)
    P = inp.num_pages
    codes = rng.integers(0, 256, size=(P, wl.PAGE, wl.DIM)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes
    if pow2_scales:
        scale = (2.0 ** rng.integers(-6, 4, size=(P, wl.PAGE)) * rng.choice([-1.0, 1.0], size=(P, wl.PAGE))).astype(np.float32)
    else:
        scale = rng.uniform(0.01, 2.0, size=(P, wl.PAGE)).astype(np.float32)
    return inp, codes, scale


def _bf16_keys_by_torch(codes, scale):
    """The same keys as bfloat16 bits, built through torch (exact when every
    scaled value fits bfloat16's 8 significant bits)."""
    k = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(scale)[..., None]
    return k.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("seed", range(3))
def test_fp8_score_equals_bf16_score_on_shared_keys(seed):
    inp, codes, scale = _fp8_case(seed)
    kb = _bf16_keys_by_torch(codes, scale)
    a = oracle.score_fp8(inp.q_bits, inp.w, codes, scale, inp.page_table, inp.seq_lens)
    b = oracle.score(inp.q_bits, inp.w, kb, inp.page_table, inp.seq_lens)
    assert np.array_equal(a, b, equal_nan=True)
    Ma, Aa = oracle.score_magnitudes_fp8(inp.q_bits, inp.w, codes, scale, inp.page_table, inp.seq_lens)
    Mb, Ab = oracle.score_magnitudes(inp.q_bits, inp.w, kb, inp.page_table, inp.seq_lens)
    assert np.array_equal(Ma, Mb) and np.array_equal(Aa, Ab)


def test_fp8_score_scales_exactly_with_positive_power_of_two():
    inp, codes, scale = _fp8_case(5, pow2_scales=False)
    a = oracle.score_fp8(inp.q_bits, inp.w, codes, scale, inp.page_table, inp.seq_lens)
    b = oracle.score_fp8(inp.q_bits, inp.w, codes, scale * np.float32(8.0), inp.page_table, inp.seq_lens)
    fin = np.isfinite(a)
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    assert np.array_equal(b[fin], 8.0 * a[fin])


def test_fp8_score_of_zero_scale_is_zero():
    inp, codes, scale = _fp8_case(6)
    a = oracle.score_fp8(inp.q_bits, inp.w, codes, np.zeros_like(scale), inp.page_table, inp.seq_lens)
    L = np.clip(inp.seq_lens, 0, inp.max_c4)
    for b in range(inp.batch):
        assert np.all(a[b, :L[b]] == 0.0) and np.all(np.isneginf(a[b, L[b]:]))


def test_fp8_keys_from_generator_round_trip():
    """Quantized keys decode to within half a code step of key / scale."""
    inp = wl.to_fp8(wl.random_case(7, 2, 3, lens=[150, 30]))
    src = wl.random_case(7, 2, 3, lens=[150, 30]).k_bits
    x = oracle.bf16_bits_to_f64(src)
    dec = oracle.e4m3_to_f64(inp.k8) * inp.k_scale.astype(np.float64)[..., None]
    rel = np.abs(dec - x) / np.maximum(np.abs(x), 2.0 ** -6 * inp.k_scale.astype(np.float64)[..., None])
    assert rel.max() <= 2.0 ** -4 + 1e-12  # 3 mantissa bits: half an ulp is 2^-4 relative
    assert np.all(np.abs(oracle.e4m3_to_f64(inp.k8)).max(axis=-1) <= 448.0)
