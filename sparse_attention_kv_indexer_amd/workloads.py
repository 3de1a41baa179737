"""Seeded synthetic inputs for the DSA indexer decode step.

This module only draws random numbers and lays them out; it performs none of
the indexer's arithmetic. Both the HIP path (through the binding) and the CPU
oracle consume what it returns, so it imports neither of them.

Geometry (page "The O(Actual) Indexer", section "The Bottleneck That Was";
page "The Moment of Breakthrough", section "The Context"): keys are kept in
c4-compressed form, one key per 4 tokens, in pages of 64 c4 positions
(256 tokens / 4). A request's logical c4 position s lives in page slot s // 64
of its page-table row, at offset s % 64 inside that physical page, and the
widest row of logits is ``max_pages * 64`` positions.

Value recipe (same for every config): q and k are standard normal draws in
float32 rounded to bfloat16 with round-to-nearest-even; w is float32, either
N(0, 1/32) or |N(0, 1)| / sqrt(32). Lengths are drawn directly in c4 positions,
uniform over the integer range, which equals a uniform token length that is a
multiple of 4. Draw order from ``numpy.random.Generator(PCG64(seed))``:
lengths, page permutation, q, w, k.

fp8 keys (an input format, not a step of the method): the same bfloat16 keys
are quantized per position to OCP FP8 E4M3 (``e4m3fn``: 4 exponent bits with
bias 7, 3 mantissa bits, no infinities, largest finite value 448) with a
float32 scale per position, scale = max_d |k_d| / 448 (1 for an all-zero
key), codes = round-to-nearest-even(k / scale).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HEADS = 32  # indexer heads
DIM = 64  # indexer head dimension
PAGE = 64  # c4 positions per page (256 tokens / 4)
POISON = -1  # page-table value in slots no valid position maps to


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    max_pages: int  # page slots per request; max_c4 = max_pages * PAGE
    len_lo: int  # c4 positions, inclusive
    len_hi: int  # c4 positions, inclusive
    topk: int
    w_kind: str  # "signed": N(0, 1/32); "abs": |N(0,1)| / sqrt(32)
    pool: str  # "shared": pool = total valid pages; "perm64": tiny's 64-page pool
    seed: int
    description: str = ""

    @property
    def max_c4(self) -> int:
        return self.max_pages * PAGE


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny", 1, 32, 128, 128, 64, "abs", "perm64", 0,
               "B=1, 8K-token max context (2048 c4), seq_len 512 tokens (128 c4), top-k 64"),
        Config("c2", 16, 32, 64, 2048, 512, "signed", "shared", 1,
               "B=16, 8K-token max context, seq_lens uniform in [256, 8192] tokens, top-k 512"),
        Config("c3", 64, 512, 128, 32768, 2048, "signed", "shared", 2,
               "B=64, 128K-token max context, seq_lens uniform in [512, 131072] tokens, top-k 2048"),
        Config("stress1m", 64, 4096, 128, 128, 64, "signed", "shared", 3,
               "B=64, ~1M-token max context (262144 c4), every seq_len 512 tokens, top-k 64"),
        Config("stress8k", 64, 32, 128, 128, 64, "signed", "shared", 3,
               "B=64, 8K-token max context (2048 c4), every seq_len 512 tokens, top-k 64"),
        Config("full", 64, 512, 32768, 32768, 2048, "signed", "shared", 4,
               "B=64, 128K-token max context, every seq_len 131072 tokens (all 512 pages valid), top-k 2048"),
    ]
}


@dataclasses.dataclass
class Inputs:
    """Host buffers of one decode step, in the layout the library takes.

    q_bits   uint16 [B, HEADS, DIM]        bfloat16 bit patterns
    w        float32 [B, HEADS]
    k_bits   uint16 [num_pages, PAGE, DIM] bfloat16 bit patterns, dim fastest
    page_table int32 [B, max_pages]        physical page per slot, POISON where unused
    seq_lens int32 [B]                     valid c4 positions per request
    """

    q_bits: np.ndarray
    w: np.ndarray
    k_bits: np.ndarray | None  # None when the keys are fp8
    page_table: np.ndarray
    seq_lens: np.ndarray
    topk: int
    k8: np.ndarray | None = None  # uint8 [num_pages, PAGE, DIM] e4m3fn codes, dim fastest
    k_scale: np.ndarray | None = None  # float32 [num_pages, PAGE] scale of each key

    @property
    def batch(self) -> int:
        return int(self.q_bits.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def max_c4(self) -> int:
        return self.max_pages * PAGE

    @property
    def num_pages(self) -> int:
        return int((self.k_bits if self.k_bits is not None else self.k8).shape[0])

    @property
    def fp8(self) -> bool:
        return self.k8 is not None


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    Inputs here are finite draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


E4M3_MAX = 448.0


def _e4m3_magnitudes() -> np.ndarray:
    """The 127 non-negative finite e4m3fn values, by code 0x00..0x7E
    (exponent field e, mantissa m: (m / 8) 2^-6 if e = 0, else (1 + m / 8) 2^(e - 7))."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


def round_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Finite reals -> e4m3fn codes, round to nearest, ties to the even code;
    magnitudes above 448 saturate to 448 (the encoding has no infinity)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    mags = _e4m3_magnitudes()
    hi = np.clip(np.searchsorted(mags, a, side="left"), 1, 126)  # mags[hi - 1] < a <= mags[hi], or the ends
    lo = hi - 1
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a <= 0.0, 0, code)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def quantize_keys_fp8(k_bits: np.ndarray):
    """bfloat16 keys [P, PAGE, DIM] -> (e4m3fn codes, per-key float32 scales)."""
    x = (np.asarray(k_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    codes = round_to_e4m3_codes(x.astype(np.float64) / scale[..., None].astype(np.float64))
    return codes, scale


def to_fp8(inp: "Inputs") -> "Inputs":
    """The same step with its keys quantized to e4m3fn with per-key scales."""
    codes, scale = quantize_keys_fp8(inp.k_bits)
    return Inputs(inp.q_bits, inp.w, None, inp.page_table, inp.seq_lens, inp.topk, codes, scale)


def pages_needed(seq_lens: np.ndarray) -> np.ndarray:
    """Page slots a request of the given c4 length occupies."""
    return (np.asarray(seq_lens, dtype=np.int64) + PAGE - 1) // PAGE


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return round_to_bf16_bits(rng.standard_normal(n, dtype=np.float32)).reshape(shape)


def generate(cfg: Config | str, seed: int | None = None) -> Inputs:
    """Draw one decode step's inputs for ``cfg`` (deterministic in the seed)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    B, S = cfg.batch, cfg.max_pages

    # 1. lengths
    if cfg.len_lo == cfg.len_hi:
        lens = np.full(B, cfg.len_lo, dtype=np.int32)
    else:
        lens = rng.integers(cfg.len_lo, cfg.len_hi, size=B, endpoint=True).astype(np.int32)
    need = pages_needed(lens)

    # 2. page permutation -> page table
    table = np.full((B, S), POISON, dtype=np.int32)
    if cfg.pool == "perm64":
        num_pages = 64
        perm = rng.permutation(num_pages).astype(np.int32)
        table[:, :] = perm[:S]
    else:
        num_pages = int(need.sum())
        perm = rng.permutation(num_pages).astype(np.int32)
        off = 0
        for b in range(B):
            n = int(need[b])
            table[b, :n] = perm[off:off + n]
            off += n

    # 3. q, 4. w, 5. k
    q = _normal_bf16(rng, (B, HEADS, DIM))
    if cfg.w_kind == "abs":
        w = (np.abs(rng.standard_normal(B * HEADS, dtype=np.float32))
             / np.float32(math.sqrt(HEADS))).reshape(B, HEADS)
    else:
        w = (rng.standard_normal(B * HEADS, dtype=np.float32)
             * np.float32(1.0 / math.sqrt(HEADS))).reshape(B, HEADS)
    k = _normal_bf16(rng, (num_pages, PAGE, DIM))
    return Inputs(q, w.astype(np.float32), k, table, lens, cfg.topk)


def random_case(seed: int, batch: int, max_pages: int, lens=None, topk: int = 16,
                signed_w: bool = True, pool_extra: int = 3, poison: int = POISON) -> Inputs:
    """A small randomized case for parity sweeps: arbitrary lengths (may be 0,
    a partial page, or exactly the row width), a pool with spare pages, and
    unused slots filled with ``poison``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    N = max_pages * PAGE
    if lens is None:
        lens = rng.integers(0, N, size=batch, endpoint=True)
    lens = np.asarray(lens, dtype=np.int32)
    need = pages_needed(np.clip(lens, 0, N))
    num_pages = int(need.sum()) + pool_extra
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((batch, max_pages), poison, dtype=np.int32)
    off = 0
    for b in range(batch):
        n = int(need[b])
        table[b, :n] = perm[off:off + n]
        off += n
    q = _normal_bf16(rng, (batch, HEADS, DIM))
    w = rng.standard_normal(batch * HEADS, dtype=np.float32).reshape(batch, HEADS)
    w = w * np.float32(1.0 / math.sqrt(HEADS))
    if not signed_w:
        w = np.abs(w)
    k = _normal_bf16(rng, (num_pages, PAGE, DIM))
    return Inputs(q, w.astype(np.float32), k, table, lens, topk)


# Sparse attention after the indexer (an input recipe for the step that reads
# the selected positions): per position one bfloat16 latent of ATT_KD dims
# (the first ATT_VD of which are the value), ATT_HEADS bfloat16 queries of
# ATT_KD dims per request, all N(0, 1); scale 1 / sqrt(192). Drawn from their
# own stream, PCG64(seed + ATT_SEED_OFFSET): queries, then latents, so the
# indexer's inputs are unchanged.
ATT_HEADS = 32
ATT_KD = 576
ATT_VD = 512
ATT_SCALE = 1.0 / math.sqrt(192.0)
ATT_SEED_OFFSET = 1000


@dataclasses.dataclass
class AttentionInputs:
    """q_bits uint16 [B, ATT_HEADS, ATT_KD]; kv_bits uint16 [num_pages, PAGE, ATT_KD]
    (same pages and page table as the indexer's keys); scale float."""

    q_bits: np.ndarray
    kv_bits: np.ndarray
    scale: float


def attention_inputs(inp: Inputs, seed: int) -> AttentionInputs:
    rng = np.random.Generator(np.random.PCG64(seed + ATT_SEED_OFFSET))
    q = _normal_bf16(rng, (inp.batch, ATT_HEADS, ATT_KD))
    kv = _normal_bf16(rng, (inp.num_pages, PAGE, ATT_KD))
    return AttentionInputs(q, kv, ATT_SCALE)



def random_selection(inp: Inputs, k: int, seed: int) -> np.ndarray:
    """A selection shaped like the top-k output, int32 [B, k]: for each request
    min(k, L) distinct positions drawn uniformly from [0, L) (L its c4 length,
    clamped to the row width), ascending, then -1. PCG64(seed + ATT_SEED_OFFSET + 1)."""
    rng = np.random.Generator(np.random.PCG64(seed + ATT_SEED_OFFSET + 1))
    out = np.full((inp.batch, k), -1, dtype=np.int32)
    for b in range(inp.batch):
        L = int(np.clip(inp.seq_lens[b], 0, inp.max_c4))
        n = min(k, L)
        if n:
            out[b, :n] = np.sort(rng.choice(L, size=n, replace=False))
    return out


# Several query tokens per request (an input recipe for speculative steps):
# T bf16 query blocks and T weight vectors per request, drawn like the
# indexer's (N(0, 1) rounded to bf16; N(0, 1/32)) from PCG64(seed + 2000);
# token t of a request whose last token sees n = 4 L tokens sees n - (T-1-t)
# tokens, so its c4 length is (4 L - (T-1-t)) // 4 (the earlier tokens miss
# the newest c4 position).
MTP_SEED_OFFSET = 2000


@dataclasses.dataclass
class MtpInputs:
    """q_bits uint16 [B, T, HEADS, DIM]; w float32 [B, T, HEADS]; seq_lens int32 [B, T]."""

    q_bits: np.ndarray
    w: np.ndarray
    seq_lens: np.ndarray

    @property
    def tokens(self) -> int:
        return self.q_bits.shape[1]


def mtp_inputs(inp: Inputs, tokens: int, seed: int) -> MtpInputs:
    rng = np.random.Generator(np.random.PCG64(seed + MTP_SEED_OFFSET))
    B = inp.batch
    q = _normal_bf16(rng, (B, tokens, HEADS, DIM))
    w = (rng.standard_normal(B * tokens * HEADS, dtype=np.float32) * np.float32(1.0 / math.sqrt(HEADS)))
    w = w.reshape(B, tokens, HEADS).astype(np.float32)
    L = np.asarray(inp.seq_lens, dtype=np.int64)
    lens = np.stack([np.maximum(4 * L - (tokens - 1 - t), 0) // 4 for t in range(tokens)], axis=1)
    return MtpInputs(q, w, lens.astype(np.int32))

