"""The seeded input generator: determinism, layout, and the bf16 rounding of
its draws (pinned against torch's own float32 -> bfloat16 conversion). CPU only."""
import os

import numpy as np
import pytest

import oracle
from sparse_attention_kv_indexer_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_same_seed_same_bytes():
    a, b = wl.generate("c2"), wl.generate("c2")
    for f in ("q_bits", "w", "k_bits", "page_table", "seq_lens"):
        assert getattr(a, f).tobytes() == getattr(b, f).tobytes()
    c = wl.generate("c2", seed=99)
    assert c.k_bits.tobytes() != a.k_bits.tobytes()


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32),
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40])])
    # ties: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7 and must round to even (1.0)
    mine = wl.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


@pytest.mark.parametrize("name", ["tiny", "c2", "stress8k"])
def test_layout(name):
    cfg = wl.CONFIGS[name]
    inp = wl.generate(name)
    B, S = cfg.batch, cfg.max_pages
    assert inp.q_bits.shape == (B, wl.HEADS, wl.DIM) and inp.q_bits.dtype == np.uint16
    assert inp.w.shape == (B, wl.HEADS) and inp.w.dtype == np.float32
    assert inp.k_bits.shape[1:] == (wl.PAGE, wl.DIM) and inp.k_bits.dtype == np.uint16
    assert inp.page_table.shape == (B, S) and inp.page_table.dtype == np.int32
    assert inp.seq_lens.shape == (B,) and inp.seq_lens.dtype == np.int32
    assert np.all(inp.seq_lens >= cfg.len_lo) and np.all(inp.seq_lens <= cfg.len_hi)
    need = wl.pages_needed(inp.seq_lens)
    used = np.concatenate([inp.page_table[b, :need[b]] for b in range(B)])
    assert len(np.unique(used)) == used.size  # every valid slot names a distinct page
    assert used.min() >= 0 and used.max() < inp.num_pages
    if cfg.pool == "shared":
        assert inp.num_pages == need.sum()
        for b in range(B):
            assert np.all(inp.page_table[b, need[b]:] == wl.POISON)
    else:
        assert sorted(inp.page_table[0].tolist()) == sorted(set(inp.page_table[0].tolist()))
    if cfg.w_kind == "abs":
        assert np.all(inp.w >= 0)


def test_value_distributions():
    inp = wl.generate("c2")
    q = oracle.bf16_bits_to_f64(inp.q_bits)
    k = oracle.bf16_bits_to_f64(inp.k_bits)
    assert abs(q.mean()) < 0.05 and abs(q.std() - 1) < 0.05
    assert abs(k.mean()) < 0.01 and abs(k.std() - 1) < 0.01
    assert abs(inp.w.std() - 1 / np.sqrt(32)) < 0.02


def test_golden_geometry():
    """Row width = page slots x 64 c4 positions, as printed on the pages."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "geometry.txt")) if l.strip() and not l.startswith("#")]
    for slots, positions in rows:
        slots, positions = int(slots), int(positions)
        table = np.full((1, slots), -1, np.int32)
        out = oracle.score(np.zeros((1, wl.HEADS, wl.DIM), np.uint16), np.zeros((1, wl.HEADS), np.float32),
                           np.zeros((1, wl.PAGE, wl.DIM), np.uint16), table, np.zeros(1, np.int32))
        assert out.shape == (1, positions)
    assert 262144 // 8192 == 32  # the work cut by capping 262144 -> 8192 tokens
    assert wl.CONFIGS["stress1m"].max_c4 == 262144 and wl.CONFIGS["stress8k"].max_c4 == 2048


def test_e4m3_encoding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    mags = wl._e4m3_magnitudes()
    mids = (mags[1:] + mags[:-1]) / 2
    x = np.concatenate([rng.standard_normal(20000) * 60, mags, -mags, mids, -mids, [0.0, -0.0, 448.0]]).astype(np.float32)
    mine = wl.round_to_e4m3_codes(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_encoding_saturates():
    assert wl.round_to_e4m3_codes(np.array([449.0, 1e6, -1e6]))[0] == 0x7E
    assert wl.round_to_e4m3_codes(np.array([-1e6]))[0] == 0xFE


def test_fp8_inputs_layout():
    inp = wl.to_fp8(wl.generate("tiny"))
    assert inp.fp8 and inp.k_bits is None
    assert inp.k8.dtype == np.uint8 and inp.k8.shape == (inp.num_pages, wl.PAGE, wl.DIM)
    assert inp.k_scale.dtype == np.float32 and inp.k_scale.shape == (inp.num_pages, wl.PAGE)
    assert np.all(inp.k_scale > 0)
